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
from gpu_util import FP8_KERNELS, as_f64, check_problem, compare, run, with_kernels

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
@pytest.mark.parametrize("case,kernel", with_kernels(CASES, lambda c: c[4]))
def test_features_all_rows(case, kernel, grid):
    check_problem(_problem(case), force_grid=grid, kernel=kernel)


def test_sink_dominates_closed_form():
    """A sink far above every logit drives the output to ~0 (and a far-below
    one changes nothing): a check of the denominator that needs no oracle."""
    for k in FP8_KERNELS:
        p = va_inputs.custom([4, 2], [1024, 769], 16, 1, "fp8", seed=11)
        base = as_f64(run(p, kernel=k))
        p.sinks = np.full(16, 60.0, dtype=np.float32)
        big = as_f64(run(p, force_grid=64, kernel=k))
        assert np.max(np.abs(big)) < 1e-6
        p.sinks = np.full(16, -60.0, dtype=np.float32)
        small = as_f64(run(p, force_grid=64, kernel=k))
        assert np.max(np.abs(small - base)) <= 2 ** -8 * np.max(np.abs(base))


def test_long_context_with_every_feature_sampled():
    """The long-context batch shape (16 x 32768, fp8, 16q/1kv) with a 4096-key
    window, softcap 30 and sinks, on sampled rows."""
    sinks = np.linspace(-1.0, 1.0, 16).astype(np.float32)
    p = va_inputs.custom([4] * 16, [32768] * 16, 16, 1, "fp8", seed=2, window_left=4095,
                         softcap=30.0, sinks=sinks, name="long-context-features")
    rows = va_inputs.sample_rows(p, 96, seed=5)
    ref, _ = oracle.attn_problem(p, rows=rows)
    for k in FP8_KERNELS:
        compare(as_f64(run(p, kernel=k))[rows], ref, f"{p.name} kernel {k}")


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_window_ignores_released_pages_of_a_separate_page_table(dt):
    """A sliding-window layer's own page table (swa_page_table) passed as the
    block table: entries of pages that lie wholly before the window are stale
    (here out-of-range ids and, for one sequence, ids of live pages of another
    sequence); the result must equal the oracle's, which never reads them."""
    wl = 300
    p = va_inputs.custom([4, 2, 3], [5000, 2100, 64], 16, 1, dt, seed=77, window_left=wl,
                         name=f"swa-table-{dt}")
    for b in range(p.num_seqs):
        lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        first = max(0, int(p.seqused_k[b]) - lq - wl) // 16     # first page any query sees
        p.block_table[b, :first] = p.num_blocks + 7 + np.arange(first)
    first1 = (2100 - 2 - wl) // 16
    p.block_table[0, :5] = p.block_table[1, first1:first1 + 5]               # live pages of sequence 1
    for k in (FP8_KERNELS if dt == "fp8" else (0,)):
        for grid in (0, 7):
            check_problem(p, force_grid=grid, kernel=k)
