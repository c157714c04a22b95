"""GPU parity of the optional features against the fp64 oracle: sliding
window, logit softcap and attention sinks (the verify call of the sglang PR
#30105 summary page, "Key source snippets", passes all three to the attention
kernel).  Same bar as test_gpu_parity.py: |gpu - ref| <= 1e-2 + 1e-2 |ref| on
every element and rel-RMS <= 5e-3.  Forced grids split sequences into many
pieces so the segment reduce (where the sink joins the denominator) runs.
"""
import numpy as np
import pytest

import oracle
import va_inputs
from gpu_util import as_f64, check_problem, compare, run

pytestmark = pytest.mark.gpu

CASES = [
    # q_lens, kv_lens, Hq, Hkv, dtype, window_left, softcap, sinks
    ([4, 2], [1024, 769], 16, 1, "fp8", 0, 0.0, False),
    ([4, 2, 3], [1024, 769, 100], 16, 1, "fp8", 37, 0.0, False),
    ([4, 1, 3], [2000, 33, 517], 16, 1, "fp8", 256, 0.0, False),
    ([3, 4], [1500, 90], 8, 2, "bf16", 100, 0.0, False),
    ([4, 2], [1024, 769], 16, 1, "fp8", -1, 0.5, False),
    ([2, 3], [700, 1100], 4, 1, "fp8", -1, 30.0, False),
    ([4, 4], [900, 65], 16, 4, "bf16", -1, 2.0, False),
    ([4, 2], [1024, 769], 16, 1, "fp8", -1, 0.0, True),
    ([1, 4, 2], [3000, 48, 700], 8, 1, "bf16", -1, 0.0, True),
    ([4, 3, 2], [1500, 640, 77], 16, 1, "fp8", 127, 1.5, True),
    ([4, 2], [2048, 300], 32, 2, "bf16", 511, 5.0, True),
]


def _problem(case):
    ql, kl, hq, hkv, dt, wl, cap, use_sinks = case
    sinks = np.linspace(-2.0, 3.0, hq).astype(np.float32) if use_sinks else None
    return va_inputs.custom(ql, kl, hq, hkv, dt, seed=sum(kl) + hq + max(wl, 0), window_left=wl,
                            softcap=cap, sinks=sinks, name=f"feat-w{wl}-c{cap}-s{int(use_sinks)}-{dt}")


@pytest.mark.parametrize("grid", [0, 7, 300])
@pytest.mark.parametrize("case", CASES, ids=[f"f{i}" for i in range(len(CASES))])
def test_features_all_rows(case, grid):
    check_problem(_problem(case), force_grid=grid)


def test_sink_dominates_closed_form():
    """A sink far above every logit drives the output to ~0 (and a far-below
    one changes nothing): a check of the denominator that needs no oracle."""
    p = va_inputs.custom([4, 2], [1024, 769], 16, 1, "fp8", seed=11)
    base = as_f64(run(p))
    p.sinks = np.full(16, 60.0, dtype=np.float32)
    big = as_f64(run(p, force_grid=64))
    assert np.max(np.abs(big)) < 1e-6
    p.sinks = np.full(16, -60.0, dtype=np.float32)
    small = as_f64(run(p, force_grid=64))
    assert np.max(np.abs(small - base)) <= 2 ** -8 * np.max(np.abs(base))


def test_long_context_with_every_feature_sampled():
    """The long-context batch shape (16 x 32768, fp8, 16q/1kv) with a 4096-key
    window, softcap 30 and sinks, on sampled rows."""
    sinks = np.linspace(-1.0, 1.0, 16).astype(np.float32)
    p = va_inputs.custom([4] * 16, [32768] * 16, 16, 1, "fp8", seed=2, window_left=4095,
                         softcap=30.0, sinks=sinks, name="long-context-features")
    rows = va_inputs.sample_rows(p, 96, seed=5)
    out = as_f64(run(p))
    ref, _ = oracle.attn_problem(p, rows=rows)
    compare(out[rows], ref, p.name)
