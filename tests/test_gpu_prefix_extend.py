"""GPU parity of the prefix + extend layout (va_run_prefix_extend) against the
oracle, and its agreement with the paged path on the same keys (bit for bit
where both layouts run the same kernel).

The layout is the sglang PR #34517 summary page's shared-KV verify layout:
prefix K/V gathered by per-token slots, draft K/V in separate buffers.  Cases
cover FP8 and bf16 caches, G 4/8/16, one and two kv heads, empty and
one-token prefixes, prefixes that end on and off a 16-key boundary, query
lengths 0..4, token-granular and page-granular slots (unused rows poisoned
with NaN), forced split grids, and the window / softcap / sink options.
"""
import numpy as np
import pytest

import oracle
import va_inputs as vi
from gpu_util import as_f64, compare, note, run, to_device

pytestmark = pytest.mark.gpu

CASES = [
    dict(q=[4, 2, 3], pre=[300, 40, 17], hq=16, hkv=1, dt="fp8", slots="tokens"),
    dict(q=[1, 3, 0, 2], pre=[16, 33, 5, 64], hq=32, hkv=2, dt="bf16", slots="pages"),
    dict(q=[4, 4, 1], pre=[0, 1, 15], hq=8, hkv=1, dt="fp8", slots="tokens"),
    dict(q=[2, 3], pre=[1000, 2047], hq=4, hkv=1, dt="bf16", slots="tokens"),
    dict(q=[3, 3, 3, 3, 3], pre=[700, 16, 17, 31, 32], hq=16, hkv=1, dt="fp8", slots="tokens",
         window_left=50),
    dict(q=[4, 2], pre=[500, 90], hq=16, hkv=1, dt="bf16", slots="tokens", softcap=20.0,
         sinks=list(np.linspace(-2.0, 3.0, 16))),
    dict(q=[4, 1, 2], pre=[4000, 3, 260], hq=16, hkv=2, dt="fp8", slots="pages", softcap=10.0,
         window_left=300, sinks=list(np.linspace(1.0, -1.0, 16))),
]


def _problem(c, seed=11):
    return vi.prefix_extend(c["q"], c["pre"], c["hq"], c["hkv"], c["dt"], seed=seed, slots=c["slots"],
                            extra_rows=37, window_left=c.get("window_left", -1),
                            softcap=c.get("softcap", 0.0), sinks=c.get("sinks"),
                            k_descale=0.8, v_descale=1.25, name="pe")


def to_device_pe(p, device="cuda"):
    import torch

    def kv(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if p.kv_dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)
    return dict(
        q=torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(device),
        kb=kv(p.k_buffer), vb=kv(p.v_buffer), ke=kv(p.k_extend), ve=kv(p.v_extend),
        indptr=torch.from_numpy(p.kv_indptr).to(device),
        indices=torch.from_numpy(p.kv_indices).to(device),
        cu=torch.from_numpy(p.cu_seqlens_q).to(device),
        kd=torch.tensor([p.k_descale], dtype=torch.float32, device=device),
        vd=torch.tensor([p.v_descale], dtype=torch.float32, device=device),
        sinks=None if p.sinks is None else torch.from_numpy(p.sinks).to(device),
    )


def run_pe(p, dev=None, **plan_kw):
    import torch
    import paged_gqa_attention_va_amd as va
    if dev is None:
        dev = to_device_pe(p)
    plan = va.Plan.for_prefix_extend(p, **plan_kw)
    note(f"  run {p.name}: B={p.num_seqs} Hq={p.num_q_heads} Hkv={p.num_kv_heads} kv={p.kv_dtype} "
         f"prefix={list(p.prefix_lens)[:8]} grid={plan.grid}")
    out = plan.run_prefix_extend(dev["q"], dev["kb"], dev["vb"], dev["indptr"], dev["indices"], dev["ke"],
                                 dev["ve"], dev["cu"], p.scale, dev["kd"], dev["vd"], sinks=dev["sinks"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("grid", [0, 7, 300])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_prefix_extend_matches_oracle(i, grid):
    p = _problem(CASES[i])
    ref, _ = oracle.attn_prefix_extend_problem(p)
    got = as_f64(run_pe(p, force_grid=grid))
    compare(got, ref, f"case{i} grid{grid}")


@pytest.mark.parametrize("dt,hq,hkv", [("fp8", 16, 1), ("bf16", 32, 2), ("fp8", 8, 1)])
@pytest.mark.parametrize("grid", [0, 7])
def test_prefix_extend_agrees_with_paged_path(dt, hq, hkv, grid):
    """The same keys in the two layouts.  With a bf16 cache both layouts run the
    same kernel, split and merge order, so the outputs must be identical.  With
    an FP8 cache the paged layout runs the one-wave-per-SIMD kernel (each wave
    takes a contiguous quarter of a piece) and the prefix + extend layout the
    two-waves-per-SIMD kernel (interleaved steps), which add the same terms in
    another order: both must match the oracle, and each other, to the parity
    bar."""
    import torch
    p = vi.custom([4, 2, 3, 1], [300, 40, 17, 1024], hq, hkv, dt, seed=5)
    paged = run(p, force_grid=grid)
    pe = vi.prefix_extend_from_paged(p)
    other = run_pe(pe, force_grid=grid)
    if dt == "bf16":
        assert torch.equal(paged.view(torch.int16), other.view(torch.int16))
    else:
        ref, _ = oracle.attn_problem(p)
        compare(as_f64(paged), ref, "paged")
        compare(as_f64(other), ref, "prefix + extend")
        compare(as_f64(other), as_f64(paged), "prefix + extend vs paged")


def test_prefix_extend_long_context_sampled():
    """16 sequences x 32764 prefix tokens in token-granular random rows + 4
    draft tokens each (the long-context verify shape), FP8, G 16: sampled rows
    against the oracle."""
    p = vi.prefix_extend([4] * 16, [32764] * 16, 16, 1, "fp8", seed=21, slots="tokens",
                         name="long-context-prefix-extend")
    rows = vi.sample_rows(p, 96, seed=3)
    got = as_f64(run_pe(p))
    ref, _ = oracle.attn_prefix_extend_problem(p, rows=rows)
    compare(got[rows], ref, p.name)
