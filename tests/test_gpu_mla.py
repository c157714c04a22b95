"""GPU parity of the absorbed-MLA path (PE_DIM split) against the oracle.

The PE_DIM split of the sglang PR #34517 summary page: one kv head whose cache
row is [latent (512) | RoPE part (64)], logits over the whole 576-wide row,
values = the latent.  Cases cover FP8 and bf16 caches, 4/8/16 heads, query
lengths 0..4, KV lengths on and off page boundaries (page tails and unused
pages poisoned with NaN), per-tensor descales, forced split grids, and a
sampled long-context case.
"""
import numpy as np
import pytest

import oracle
import va_inputs as vi
from gpu_util import as_f64, compare, note

pytestmark = pytest.mark.gpu

CASES = [
    dict(q=[4, 2, 3], kv=[300, 40, 17], hq=16, dt="fp8"),
    dict(q=[1, 3, 0, 2], kv=[16, 33, 5, 64], hq=8, dt="bf16"),
    dict(q=[4, 4], kv=[4, 129], hq=4, dt="fp8"),
    dict(q=[2, 3, 1], kv=[1000, 2047, 16], hq=16, dt="bf16"),
    dict(q=[3, 3, 3, 3, 3], kv=[700, 16, 17, 31, 32], hq=8, dt="fp8"),
    dict(q=[1, 1], kv=[1, 2], hq=16, dt="bf16"),
]


def _problem(c, seed=13):
    return vi.mla(c["q"], c["kv"], c["hq"], c["dt"], seed=seed, k_descale=0.8, v_descale=1.25)


def run_mla(p, **plan_kw):
    import torch
    import paged_gqa_attention_va_amd as va
    pool = torch.from_numpy(p.k)
    if p.kv_dtype == "bf16":
        pool = pool.view(torch.int16).view(torch.bfloat16)
    pool = pool.cuda()
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(p.block_table).cuda()
    cu = torch.from_numpy(p.cu_seqlens_q).cuda()
    sk = torch.from_numpy(p.seqused_k).cuda()
    kd = torch.tensor([p.k_descale], dtype=torch.float32, device="cuda")
    vd = torch.tensor([p.v_descale], dtype=torch.float32, device="cuda")
    plan = va.Plan.for_problem(p, **plan_kw)
    note(f"  run {p.name}: B={p.num_seqs} Hq={p.num_q_heads} kv={p.kv_dtype} "
         f"kv_lens={list(p.seqused_k)[:8]} grid={plan.grid}")
    out = plan.run(q, pool, pool, bt, cu, sk, p.scale, kd, vd)     # V is the latent of the K rows
    torch.cuda.synchronize()
    assert tuple(out.shape) == (p.total_q, p.num_q_heads, vi.MLA_LATENT)
    return out


@pytest.mark.parametrize("grid", [0, 7, 300])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_mla_matches_oracle(i, grid):
    p = _problem(CASES[i])
    ref, _ = oracle.attn_mla_problem(p)
    got = as_f64(run_mla(p, force_grid=grid))
    compare(got, ref, f"mla case{i} grid{grid}")


def test_mla_run_to_run_bitwise():
    import torch
    p = _problem(CASES[0])
    a = run_mla(p, force_grid=7)
    b = run_mla(p, force_grid=7)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mla_rejects_separate_value_pool_and_sinks():
    import torch
    import paged_gqa_attention_va_amd as va
    p = _problem(CASES[2])
    pool = torch.from_numpy(p.k).cuda()
    other = pool.clone()
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    args = (torch.from_numpy(p.block_table).cuda(), torch.from_numpy(p.cu_seqlens_q).cuda(),
            torch.from_numpy(p.seqused_k).cuda(), p.scale)
    plan = va.Plan.for_problem(p)
    with pytest.raises(va.VaError) as e:
        plan.run(q, pool, other, *args)
    assert e.value.status == va.VA_ERR_INVALID_ARG
    sinks = torch.zeros(p.num_q_heads, dtype=torch.float32, device="cuda")
    with pytest.raises(va.VaError) as e:
        plan.run(q, pool, pool, *args, sinks=sinks)
    assert e.value.status == va.VA_ERR_INVALID_ARG


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_mla_long_context_sampled(dt):
    """16 sequences x 32768 keys, 4 draft tokens, 16 heads: sampled rows."""
    p = vi.mla([4] * 16, [32768] * 16, 16, dt, seed=23, name=f"mla-long-{dt}")
    rows = vi.sample_rows(p, 96, seed=5)
    got = as_f64(run_mla(p))
    ref, _ = oracle.attn_mla_problem(p, rows=rows)
    compare(got[rows], ref, p.name)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_mla_long_pieces(dt):
    """Two sequences of 9000 keys on a 3-workgroup split: each piece spans
    several hundred pages (the kernel reads its block-table entries in chunks
    of 256 pages)."""
    p = vi.mla([4, 3], [9000, 8190], 16, dt, seed=29, name=f"mla-long-pieces-{dt}")
    ref, _ = oracle.attn_mla_problem(p)
    compare(as_f64(run_mla(p, force_grid=3)), ref, p.name)
