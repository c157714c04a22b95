"""GPU parity at the edges of the work split and of the plan's domain.

- More than 64 (sequence, kv head) pairs: the work split then scans the page
  counts in several 64-wide passes (the one-pass case covers up to 64 pairs).
- The largest pair count the plan accepts (65536), with tiny sequences.
- Eight kv heads (G = 4 with 32 query heads, G = 8 with 64).
- The same edges through the prefix + extend layout and the absorbed-MLA path.
Every case is a valid input; results are checked against the oracle (all rows,
or a seeded sample where the oracle would take long).
"""
import numpy as np
import pytest

import oracle
import va_inputs
from gpu_util import as_f64, check_problem, compare

pytestmark = pytest.mark.gpu


def _lens(n, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


@pytest.mark.parametrize("grid", [0, 7, 1000])
def test_many_pairs_fp8(grid):
    n = 100                                           # 100 pairs: two scan passes
    p = va_inputs.custom(_lens(n, 0, 4, 1), _lens(n, 4, 300, 2), 16, 1, "fp8", seed=3, name="many-pairs-fp8")
    check_problem(p, force_grid=grid)


@pytest.mark.parametrize("grid", [0, 300])
def test_many_pairs_bf16_four_kv_heads(grid):
    n = 40                                            # 160 pairs
    p = va_inputs.custom(_lens(n, 1, 4, 4), _lens(n, 4, 700, 5), 32, 4, "bf16", seed=6,
                         name="many-pairs-bf16")
    check_problem(p, force_grid=grid)


@pytest.mark.parametrize("hq,dt", [(32, "fp8"), (64, "bf16")])
def test_eight_kv_heads(hq, dt):
    p = va_inputs.custom([4, 1, 3], [900, 17, 260], hq, 8, dt, seed=7, name=f"hkv8-{dt}")
    check_problem(p)


def test_largest_pair_count():
    """16384 sequences x 4 kv heads = 65536 pairs (the plan's maximum), 1..32
    keys each, one query token each: sampled rows."""
    n = 16384
    p = va_inputs.custom([1] * n, _lens(n, 1, 32, 8), 16, 4, "fp8", seed=9, name="max-pairs")
    rows = va_inputs.sample_rows(p, 256, seed=1)
    check_problem(p, rows=rows)


def test_many_pairs_prefix_extend():
    from test_gpu_prefix_extend import run_pe
    n = 90
    pe = va_inputs.prefix_extend(_lens(n, 1, 4, 10), _lens(n, 0, 500, 11), 16, 1, "fp8", seed=12,
                                 slots="tokens", name="many-pairs-pe")
    ref, _ = oracle.attn_prefix_extend_problem(pe)
    compare(as_f64(run_pe(pe, force_grid=300)), ref, pe.name)


def test_many_pairs_mla():
    from test_gpu_mla import run_mla
    n = 80
    p = va_inputs.mla(_lens(n, 0, 4, 13), _lens(n, 1, 400, 14), 8, "fp8", seed=15, name="many-pairs-mla")
    ref, _ = oracle.attn_mla_problem(p)
    compare(as_f64(run_mla(p, force_grid=7)), ref, p.name)
