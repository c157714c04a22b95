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
from gpu_util import FP8_KERNELS, as_f64, check_problem, compare

pytestmark = pytest.mark.gpu


def _lens(n, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


@pytest.mark.parametrize("kernel", FP8_KERNELS)
@pytest.mark.parametrize("grid", [0, 7, 1000])
def test_many_pairs_fp8(grid, kernel):
    n = 100                                           # 100 pairs: two scan passes
    p = va_inputs.custom(_lens(n, 0, 4, 1), _lens(n, 4, 300, 2), 16, 1, "fp8", seed=3, name="many-pairs-fp8")
    check_problem(p, force_grid=grid, kernel=kernel)


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
    p = va_inputs.mla(_lens(n, 0, 4, 13), _lens(n, 4, 400, 14), 8, "fp8", seed=15, name="many-pairs-mla")
    ref, _ = oracle.attn_mla_problem(p)
    compare(as_f64(run_mla(p, force_grid=7)), ref, p.name)


# ---- pools beyond 4 GiB: every copy address is a 64-bit offset ----------
#
# A small problem's pages (or token rows) are placed near the end of a device
# pool of more than 4 GiB, with the block table (or kv_indices) remapped, so
# every page offset needs more than 32 bits.  The output must equal the oracle's
# on the compact problem.  Unreferenced pool bytes are never read.

_BIG = (5 << 30) + (1 << 20)                          # bytes per pool: just over 5 GiB


class _WithBlocks:
    """The problem p seen with another pool size (the plan takes num_blocks)."""

    def __init__(self, p, num_blocks):
        self._p, self.num_blocks = p, num_blocks

    def __getattr__(self, a):
        return getattr(self._p, a)


def _spread(pool, idx, n_big):
    import torch
    big = torch.empty((n_big,) + tuple(pool.shape[1:]), dtype=pool.dtype, device=pool.device)
    big[idx] = pool
    return big


def _remap_table(bt, n_small, idx):
    """Entries < n_small (real pages) -> idx[entry]; the out-of-range padding
    entries stay out of range of the big pool."""
    import torch
    big_n = int(idx.max().item()) + 1
    valid = bt < n_small
    mapped = idx[bt.clamp(0, n_small - 1).long()].to(torch.int32)
    return torch.where(valid, mapped, bt - n_small + big_n + 7)


def _high_indices(n_small, n_big):
    """Page i -> n_big - 1 - 3 i (the first page kept at index 0, so both ends
    of the pool are read)."""
    import torch
    idx = n_big - 1 - 3 * torch.arange(n_small, dtype=torch.int64)
    idx[0] = 0
    assert int(idx.min()) >= 0
    return idx.cuda()


@pytest.mark.parametrize("dt,hq,hkv", [("fp8", 16, 1), ("bf16", 32, 2)])
def test_pool_beyond_4gib(dt, hq, hkv):
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import note, to_device
    p = va_inputs.custom([4, 2, 3], [1000, 517, 2048], hq, hkv, dt, seed=21, name=f"big-pool-{dt}")
    dev = to_device(p)
    page_bytes = dev["k"][0].numel() * dev["k"].element_size()
    n_big = _BIG // page_bytes
    idx = _high_indices(p.num_blocks, n_big)
    note(f"  big pool {dt}: {n_big} pages of {page_bytes} B, highest byte offset "
         f"{int(idx.max()) * page_bytes}")
    k, v = _spread(dev["k"], idx, n_big), _spread(dev["v"], idx, n_big)
    bt = _remap_table(dev["bt"], p.num_blocks, idx)
    outs = []
    for kern in (FP8_KERNELS if dt == "fp8" else (0,)):
        plan = va.Plan.for_problem(_WithBlocks(p, n_big), kernel=kern)
        outs.append(plan.run(dev["q"], k, v, bt, dev["cu"], dev["sk"], p.scale, dev["kd"], dev["vd"]))
    torch.cuda.synchronize()
    del k, v
    torch.cuda.empty_cache()
    ref, _ = oracle.attn_problem(p)
    for out in outs:
        compare(as_f64(out), ref, p.name)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_pool_beyond_4gib_mla(dt):
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import note
    p = va_inputs.mla([4, 1, 2], [700, 1234, 33], 16, dt, seed=22, name=f"big-pool-mla-{dt}")
    pool = torch.from_numpy(p.k)
    if dt == "bf16":
        pool = pool.view(torch.int16).view(torch.bfloat16)
    pool = pool.cuda()
    page_bytes = pool[0].numel() * pool.element_size()
    n_big = _BIG // page_bytes
    idx = _high_indices(p.num_blocks, n_big)
    note(f"  big MLA pool {dt}: {n_big} pages of {page_bytes} B")
    big = _spread(pool, idx, n_big)
    bt = _remap_table(torch.from_numpy(p.block_table).cuda(), p.num_blocks, idx)
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(p.cu_seqlens_q).cuda()
    sk = torch.from_numpy(p.seqused_k).cuda()
    kd = torch.tensor([p.k_descale], dtype=torch.float32, device="cuda")
    vd = torch.tensor([p.v_descale], dtype=torch.float32, device="cuda")
    plan = va.Plan.for_problem(_WithBlocks(p, n_big))
    out = plan.run(q, big, big, bt, cu, sk, p.scale, kd, vd)
    torch.cuda.synchronize()
    del big
    torch.cuda.empty_cache()
    ref, _ = oracle.attn_mla_problem(p)
    compare(as_f64(out), ref, p.name)


def test_token_buffer_beyond_4gib_prefix_extend():
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import note
    from test_gpu_prefix_extend import to_device_pe
    pe = va_inputs.prefix_extend([4, 3], [900, 1500], 16, 1, "fp8", seed=23, slots="tokens",
                                 name="big-buffer-pe")
    dev = to_device_pe(pe)
    row_bytes = dev["kb"][0].numel() * dev["kb"].element_size()
    n_big = _BIG // row_bytes
    idx = _high_indices(pe.num_rows, n_big)
    note(f"  big token buffer: {n_big} rows of {row_bytes} B")
    kb, vb = _spread(dev["kb"], idx, n_big), _spread(dev["vb"], idx, n_big)
    indices = idx[dev["indices"].long()].to(torch.int32)
    plan = va.Plan.for_prefix_extend(_WithRows(pe, n_big))
    out = plan.run_prefix_extend(dev["q"], kb, vb, dev["indptr"], indices, dev["ke"], dev["ve"],
                                 dev["cu"], pe.scale, dev["kd"], dev["vd"])
    torch.cuda.synchronize()
    del kb, vb
    torch.cuda.empty_cache()
    ref, _ = oracle.attn_prefix_extend_problem(pe)
    compare(as_f64(out), ref, pe.name)


class _WithRows(_WithBlocks):
    """The prefix + extend problem seen with another token-buffer size."""

    def __init__(self, p, num_rows):
        self._p, self.num_rows = p, num_rows
