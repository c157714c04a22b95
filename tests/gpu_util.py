"""Helpers shared by the GPU tests: device copies, running the library through
its C ABI, and the comparison rules against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_va_amd as va

# Judge rule for bf16 output vs the fp64 oracle: |gpu - ref| <= ATOL + RTOL*|ref|
# (the atol=rtol=1e-2 of the page test's assert_close).
ATOL = 1e-2
RTOL = 1e-2
# Stricter internal bar: relative RMS error.  bf16 output rounding alone is
# about 2^-9 / sqrt(3) ~ 1.1e-3; P is rounded to bf16 once more inside the kernel.
REL_RMS = 5e-3


# The two split-KV kernels of paged FP8 GQA (va_problem.kernel): 1 runs one
# wave per SIMD, 2 two row groups.  The plan picks one by pages per workgroup;
# tests force each so both stay covered at every shape.
FP8_KERNELS = (1, 2)


def kernel_for(dt: str, k: int) -> int:
    """The kernel value to force for a paged GQA case: k for an FP8 cache,
    0 (the only choice) for bf16."""
    return k if dt == "fp8" else 0


def with_kernels(cases, dt_of):
    """pytest params: each FP8 case once per FP8 kernel, each other case once."""
    out = []
    for i, c in enumerate(cases):
        ks = FP8_KERNELS if dt_of(c) == "fp8" else (0,)
        out += [pytest.param(c, k, id=f"{i}-k{k}") for k in ks]
    return out


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_device(p, device="cuda"):
    kv_t = torch.uint8 if p.kv_dtype == "fp8" else torch.bfloat16
    def kv(a):
        t = torch.from_numpy(a)
        if p.kv_dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)
    d = dict(
        q=torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(device),
        k=kv(p.k), v=kv(p.v),
        bt=torch.from_numpy(p.block_table).to(device),
        cu=torch.from_numpy(p.cu_seqlens_q).to(device),
        sk=torch.from_numpy(p.seqused_k).to(device),
        kd=torch.tensor([p.k_descale], dtype=torch.float32, device=device),
        vd=torch.tensor([p.v_descale], dtype=torch.float32, device=device),
        sinks=None if getattr(p, "sinks", None) is None else torch.from_numpy(p.sinks).to(device),
    )
    assert d["k"].dtype == kv_t
    return d


def run(p, dev=None, plan=None, out=None, workspace=None, **plan_kw):
    """Run the library on problem p; returns the bf16 output tensor (device)."""
    if dev is None:
        dev = to_device(p)
    if plan is None:
        plan = va.Plan.for_problem(p, **plan_kw)
    note(f"  run {p.name}: B={p.num_seqs} Hq={p.num_q_heads} Hkv={p.num_kv_heads} "
         f"kv={p.kv_dtype} grid={plan.grid} ws={plan.workspace_bytes}")
    out = plan.run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale,
                   dev["kd"], dev["vd"], out=out, workspace=workspace, sinks=dev["sinks"])
    torch.cuda.synchronize()
    return out


def as_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64).reshape(-1, out.shape[-1])


def compare(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Assert the judge rule and the rel-RMS bar; return (max_abs_err, rel_rms)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    rel_rms = float(np.sqrt(np.mean((got - ref) ** 2)) / max(1e-30, np.sqrt(np.mean(ref ** 2))))
    note(f"  {what}: max|err|={err.max():.3e} rel_rms={rel_rms:.3e}")
    assert np.all(err <= bound), (f"{what}: max excess at {worst}: got {got[worst]} ref {ref[worst]}")
    assert rel_rms <= REL_RMS, f"{what}: rel_rms {rel_rms}"
    return float(err.max()), rel_rms


def check_problem(p, rows=None, **plan_kw):
    """Run p on the GPU and compare to the oracle (all rows or a sample)."""
    out = as_f64(run(p, **plan_kw))
    ref, _ = oracle.attn_problem(p, rows=rows)
    got = out if rows is None else out[rows]
    return compare(got, ref, p.name), out
