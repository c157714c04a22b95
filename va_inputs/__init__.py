"""Seeded synthetic inputs for paged GQA verify attention.

This module only draws and lays out input data.  It holds none of the
attention arithmetic, so both the HIP path (tests, bench) and the CPU oracle can
take their inputs from it.

The construction follows the unit test printed on the sglang PR #36330 summary
page ("Key source snippets", ``_check_matches_aiter``).  Q is bf16 N(0,1). K and
V are N(0,1) cast to fp8 e4m3. The pool layout is [num_blocks, page=16, Hkv, D=256].
cu_seqlens_q is the prefix sum of the query lengths. seqused_k is the total KV
length including the verify tokens. Descales are per tensor, and the scale is
head_dim**-0.5.
The five named workloads are the synthetic verify shapes this library is
measured on. ``config(i)`` builds them.  ``custom()`` builds any other shape
for tests.

Memory that no query may see is poisoned by default. That covers page-tail
slots at or beyond seqused_k, pages no sequence references, and block-table
entries past a sequence's last page. Poison is an fp8/bf16 NaN pattern and
out-of-range page ids, so a kernel that reads such memory gives a visibly wrong
answer.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

HEAD_DIM = 256
PAGE = 16
FP8_NAN = 0x7F          # e4m3fn NaN byte (S.1111.111)
BF16_NAN = 0x7FC0       # bf16 quiet NaN


@dataclasses.dataclass
class Problem:
    """Host copy of one verify-attention call (raw bit patterns)."""
    name: str
    q: np.ndarray                # uint16 bf16 bits, [total_q, Hq, D]
    k: np.ndarray                # uint8 fp8 bytes or uint16 bf16 bits, [num_blocks, page, Hkv, D]
    v: np.ndarray
    kv_dtype: str                # "fp8" | "bf16"
    block_table: np.ndarray      # int32 [B, max_blocks_per_seq]
    cu_seqlens_q: np.ndarray     # int32 [B+1]
    seqused_k: np.ndarray        # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    scale: float                 # fp32 value
    k_descale: float             # fp32 value
    v_descale: float             # fp32 value
    head_dim: int = HEAD_DIM
    page_size: int = PAGE
    window_left: int = -1                  # sliding window: keys from i - window_left (-1 = none)
    softcap: float = 0.0                   # logit softcap (0 = none)
    sinks: Optional[np.ndarray] = None     # float32 [Hq] sink logits, or None
    v_head_dim: Optional[int] = None       # absorbed MLA: V = the first v_head_dim dims of
                                           # the K row (v is k); None = head_dim, separate V

    @property
    def num_seqs(self) -> int:
        return int(self.seqused_k.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q.astype(np.int64))

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seqused_k.max()) if self.num_seqs else 0

    @property
    def num_blocks(self) -> int:
        return int(self.k.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _f32(x: float) -> float:
    return float(np.float32(x))


def _randn_bf16_bits(gen: torch.Generator, shape) -> np.ndarray:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _randn_kv_bits(gen: torch.Generator, shape, kv_dtype: str) -> np.ndarray:
    """N(0,1) drawn in float32, cast with torch's round-to-nearest-even cast,
    generated in slabs of pages to bound the temporary float32 memory."""
    nblk = shape[0]
    per = max(1, (1 << 24) // max(1, int(np.prod(shape[1:]))))
    out = np.empty(shape, dtype=np.uint8 if kv_dtype == "fp8" else np.uint16)
    for s in range(0, nblk, per):
        e = min(nblk, s + per)
        t = torch.randn(e - s, *shape[1:], generator=gen, dtype=torch.float32)
        if kv_dtype == "fp8":
            out[s:e] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            out[s:e] = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def custom(q_lens: Sequence[int], kv_lens: Sequence[int], num_q_heads: int,
           num_kv_heads: int, kv_dtype: str = "fp8", seed: int = 0,
           table: str = "perm", k_descale: float = 1.0, v_descale: float = 1.0,
           scale: Optional[float] = None, poison: bool = True,
           extra_blocks: int = 0, name: str = "custom",
           max_blocks_per_seq: Optional[int] = None, window_left: int = -1,
           softcap: float = 0.0, sinks: Optional[Sequence[float]] = None,
           head_dim: int = HEAD_DIM, v_head_dim: Optional[int] = None) -> Problem:
    """Build one problem.

    head_dim / v_head_dim: with v_head_dim < head_dim the call is absorbed MLA
    (one kv head; a key's value is the first v_head_dim dims of its K row, and
    the problem's v is the same array as k).

    table: "perm"     -- pages of all sequences are a seeded random permutation
                         of a pool that holds exactly the pages in use (+extra);
           "identity" -- sequence b owns pool pages b*mbps .. b*mbps+mbps-1
                         (the arange(...).view(B, mbps) table of the page test).
    """
    assert kv_dtype in ("fp8", "bf16")
    q_lens = [int(x) for x in q_lens]
    kv_lens = [int(x) for x in kv_lens]
    B = len(q_lens)
    assert B == len(kv_lens) and B >= 1
    assert num_q_heads % num_kv_heads == 0
    if any(q > k for q, k in zip(q_lens, kv_lens)):
        # kv_lens count the verify tokens themselves
        raise ValueError(f"q_lens {q_lens} exceed kv_lens {kv_lens}")
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    pages = [math.ceil(k / PAGE) for k in kv_lens]
    mbps = max(1, max(pages)) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    assert mbps >= max(pages)
    if table == "identity":
        num_blocks = B * mbps + extra_blocks
    else:
        num_blocks = sum(pages) + extra_blocks
    num_blocks = max(num_blocks, 1)
    total_q = sum(q_lens)
    mla = v_head_dim is not None and v_head_dim < head_dim
    assert not mla or num_kv_heads == 1
    q = _randn_bf16_bits(gen, (total_q, num_q_heads, head_dim))
    k = _randn_kv_bits(gen, (num_blocks, PAGE, num_kv_heads, head_dim), kv_dtype)
    v = k if mla else _randn_kv_bits(gen, (num_blocks, PAGE, num_kv_heads, head_dim), kv_dtype)

    bt = np.zeros((B, mbps), dtype=np.int32)
    if table == "identity":
        bt[:] = np.arange(B * mbps, dtype=np.int32).reshape(B, mbps)
    else:
        perm = torch.randperm(num_blocks, generator=gen).numpy().astype(np.int32)
        off = 0
        for b in range(B):
            bt[b, :pages[b]] = perm[off:off + pages[b]]
            off += pages[b]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    seqused = np.asarray(kv_lens, dtype=np.int32)

    if poison:
        nan = FP8_NAN if kv_dtype == "fp8" else BF16_NAN
        used = np.zeros(num_blocks, dtype=bool)
        for b in range(B):
            used[bt[b, :pages[b]]] = True
            tail = kv_lens[b] % PAGE
            if pages[b] and tail:
                last = bt[b, pages[b] - 1]
                k[last, tail:] = nan
                v[last, tail:] = nan                 # no-op when v is k
            # entries past the last page point outside the pool
            bt[b, pages[b]:] = num_blocks + np.arange(mbps - pages[b], dtype=np.int32)
        k[~used] = nan
        v[~used] = nan

    if scale is None:
        scale = head_dim ** -0.5
    sk_arr = None if sinks is None else np.asarray(sinks, dtype=np.float32)
    if sk_arr is not None:
        assert sk_arr.shape == (num_q_heads,)
    return Problem(name=name, q=q, k=k, v=v, kv_dtype=kv_dtype, block_table=bt, head_dim=head_dim,
                   v_head_dim=v_head_dim if mla else None,
                   cu_seqlens_q=cu, seqused_k=seqused, num_q_heads=num_q_heads,
                   num_kv_heads=num_kv_heads, scale=_f32(scale),
                   k_descale=_f32(k_descale), v_descale=_f32(v_descale),
                   window_left=int(window_left), softcap=_f32(softcap), sinks=sk_arr)


# ----------------------------------------------------------------- workloads --

CONFIG_NAMES = {
    0: "tiny verify 2 seqs q[4,2] kv[1024,769] 16q/1kv fp8",
    1: "tiny verify 2 seqs q[4,2] kv[1024,769] 32q/2kv fp8",
    2: "long context 16 seqs q4 kv32768 16q/1kv fp8",
    3: "high concurrency 64 seqs q3 kv U[8192,65536] 16q/1kv fp8 descale U[0.5,2]",
    4: "shape sweep 8 seqs q{1,2,3} kv131072 G{4,8,16}/1kv fp8|bf16",
}

SWEEP_VARIANTS = [(g, dt) for dt in ("fp8", "bf16") for g in (16, 8, 4)]


def config(i: int, variant: int = 0, poison: bool = True,
           seed: Optional[int] = None) -> Problem:
    """The named workloads.  Config 4 has six variants (group size x KV dtype,
    see SWEEP_VARIANTS); ``variant`` picks one."""
    if i in (0, 1):
        hq, hkv = (16, 1) if i == 0 else (32, 2)
        return custom([4, 2], [1024, 769], hq, hkv, "fp8",
                      seed=0 if seed is None else seed, table="identity",
                      max_blocks_per_seq=math.ceil(1024 / PAGE), poison=poison,
                      name=f"config{i}")
    if i == 2:
        return custom([4] * 16, [32768] * 16, 16, 1, "fp8",
                      seed=2 if seed is None else seed, poison=poison, name="config2")
    if i == 3:
        s = 3 if seed is None else seed
        gen = torch.Generator(device="cpu")
        gen.manual_seed(1000 + s)
        kv = torch.randint(8192, 65536 + 1, (64,), generator=gen).tolist()
        kd, vd = (0.5 + 1.5 * torch.rand(2, generator=gen, dtype=torch.float64)).tolist()
        return custom([3] * 64, kv, 16, 1, "fp8", seed=s, k_descale=kd,
                      v_descale=vd, poison=poison, name="config3")
    if i == 4:
        g, dt = SWEEP_VARIANTS[variant]
        s = (4 if seed is None else seed) + 10 * variant
        gen = torch.Generator(device="cpu")
        gen.manual_seed(2000 + s)
        ql = torch.randint(1, 4, (8,), generator=gen).tolist()
        return custom(ql, [131072] * 8, g, 1, dt, seed=s, poison=poison,
                      name=f"config4-g{g}-{dt}")
    raise ValueError(f"unknown config {i}")


# Absorbed-MLA shape of the PR #34517 page's Kimi-K3 path: a 512-wide latent
# plus a 64-wide RoPE part per key row, one kv head.
MLA_LATENT = 512
MLA_ROPE = 64


def mla(q_lens: Sequence[int], kv_lens: Sequence[int], num_q_heads: int, kv_dtype: str = "fp8",
        seed: int = 0, **kw) -> Problem:
    """An absorbed-MLA verify problem: Q rows [q_nope (512) | q_pe (64)], one kv
    head whose cache row is [latent (512) | k_pe (64)], V = the latent.  The
    scale defaults to 192**-0.5 (a 128-wide no-RoPE head plus the 64-wide RoPE
    part before absorption)."""
    kw.setdefault("scale", (128 + MLA_ROPE) ** -0.5)
    kw.setdefault("name", "mla")
    return custom(q_lens, kv_lens, num_q_heads, 1, kv_dtype, seed=seed,
                  head_dim=MLA_LATENT + MLA_ROPE, v_head_dim=MLA_LATENT, **kw)


def sample_rows(p: Problem, n: int, seed: int = 0) -> np.ndarray:
    """A seeded sample of flat output rows (q_row * Hq + head): n rows drawn
    at random, plus, for every sequence with query tokens, one row of its
    first query token and one of its last (each at a seeded head), so that
    every sequence's boundaries are checked.  All rows when n covers them."""
    rng = np.random.default_rng(seed)
    hq = p.num_q_heads
    total = p.total_q * hq
    if n >= total:
        return np.arange(total, dtype=np.int64)
    pick = set(rng.choice(total, size=n, replace=False).tolist())
    cu = np.asarray(p.cu_seqlens_q)
    for b in range(p.num_seqs):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        if q1 > q0:
            pick.add(q0 * hq + int(rng.integers(hq)))
            pick.add((q1 - 1) * hq + int(rng.integers(hq)))
    return np.array(sorted(pick), dtype=np.int64)


# ------------------------------------------------- prefix + extend layout --

@dataclasses.dataclass
class PrefixExtendProblem:
    """Host copy of one verify call in the prefix + extend layout: the prefix
    K/V of each sequence sit in a token-row buffer addressed by per-token slots
    (kv_indptr / kv_indices), the draft tokens' K/V in separate buffers with
    one row per query token (the layout of the sglang PR #34517 summary page's
    shared-KV verify kernel: prefix through kv_indices, k_extend / v_extend)."""
    name: str
    q: np.ndarray                # uint16 bf16 bits, [total_q, Hq, D]
    k_buffer: np.ndarray         # uint8 fp8 bytes or uint16 bf16 bits, [num_rows, Hkv, D]
    v_buffer: np.ndarray
    k_extend: np.ndarray         # [total_q, Hkv, D], same dtype as the buffers
    v_extend: np.ndarray
    kv_dtype: str
    kv_indptr: np.ndarray        # int32 [B+1], prefix sums of the prefix lengths
    kv_indices: np.ndarray       # int32 [kv_indptr[B]], row of every prefix token
    cu_seqlens_q: np.ndarray     # int32 [B+1]
    num_q_heads: int
    num_kv_heads: int
    scale: float
    k_descale: float
    v_descale: float
    head_dim: int = HEAD_DIM
    window_left: int = -1
    softcap: float = 0.0
    sinks: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens_q.shape[0] - 1)

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def prefix_lens(self) -> np.ndarray:
        return np.diff(self.kv_indptr)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int((self.prefix_lens + self.q_lens).max()) if self.num_seqs else 0

    @property
    def num_rows(self) -> int:
        return int(self.k_buffer.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def prefix_extend(q_lens: Sequence[int], prefix_lens: Sequence[int], num_q_heads: int,
                  num_kv_heads: int, kv_dtype: str = "fp8", seed: int = 0,
                  slots: str = "tokens", extra_rows: int = 0, k_descale: float = 1.0,
                  v_descale: float = 1.0, scale: Optional[float] = None, poison: bool = True,
                  name: str = "prefix_extend", window_left: int = -1, softcap: float = 0.0,
                  sinks: Optional[Sequence[float]] = None) -> PrefixExtendProblem:
    """Build one prefix + extend problem.

    slots: "tokens" -- every prefix token gets its own seeded random row (a
                       token-granular allocator, the worst case for gathering);
           "pages"  -- prefix tokens fill 16-row pages in order, pages in a
                       seeded random order (a paged allocator).
    Rows no prefix token uses are poisoned with NaN (when ``poison``).
    """
    assert kv_dtype in ("fp8", "bf16") and slots in ("tokens", "pages")
    q_lens = [int(x) for x in q_lens]
    prefix_lens = [int(x) for x in prefix_lens]
    B = len(q_lens)
    assert B == len(prefix_lens) and B >= 1
    assert num_q_heads % num_kv_heads == 0
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    total_q = sum(q_lens)
    n_prefix = sum(prefix_lens)
    q = _randn_bf16_bits(gen, (total_q, num_q_heads, HEAD_DIM))
    if slots == "tokens":
        num_rows = max(1, n_prefix + extra_rows)
        perm = torch.randperm(num_rows, generator=gen).numpy().astype(np.int64)
        indices = perm[:n_prefix]
    else:
        pages = [math.ceil(n / PAGE) for n in prefix_lens]
        num_pages = sum(pages) + math.ceil(extra_rows / PAGE)
        num_rows = max(1, num_pages * PAGE)
        pperm = torch.randperm(max(1, num_pages), generator=gen).numpy().astype(np.int64)
        parts, off = [], 0
        for n, npg in zip(prefix_lens, pages):
            j = np.arange(n)
            parts.append(pperm[off + j // PAGE] * PAGE + j % PAGE)
            off += npg
        indices = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    k_buf = _randn_kv_bits(gen, (num_rows, num_kv_heads, HEAD_DIM), kv_dtype)
    v_buf = _randn_kv_bits(gen, (num_rows, num_kv_heads, HEAD_DIM), kv_dtype)
    k_ext = _randn_kv_bits(gen, (total_q, num_kv_heads, HEAD_DIM), kv_dtype)
    v_ext = _randn_kv_bits(gen, (total_q, num_kv_heads, HEAD_DIM), kv_dtype)
    if poison:
        nan = FP8_NAN if kv_dtype == "fp8" else BF16_NAN
        used = np.zeros(num_rows, dtype=bool)
        used[indices] = True
        k_buf[~used] = nan
        v_buf[~used] = nan
    indptr = np.zeros(B + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(prefix_lens)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    if scale is None:
        scale = HEAD_DIM ** -0.5
    sk_arr = None if sinks is None else np.asarray(sinks, dtype=np.float32)
    return PrefixExtendProblem(
        name=name, q=q, k_buffer=k_buf, v_buffer=v_buf, k_extend=k_ext, v_extend=v_ext,
        kv_dtype=kv_dtype, kv_indptr=indptr, kv_indices=indices.astype(np.int32),
        cu_seqlens_q=cu, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        scale=_f32(scale), k_descale=_f32(k_descale), v_descale=_f32(v_descale),
        window_left=int(window_left), softcap=_f32(softcap), sinks=sk_arr)


def prefix_extend_from_paged(p: Problem, name: Optional[str] = None) -> PrefixExtendProblem:
    """The same call as paged problem ``p`` in the prefix + extend layout: the
    first seqused_k - q_len keys of each sequence stay in the pool (viewed as
    token rows, slot = page * 16 + offset), its last q_len keys move to
    k_extend / v_extend.  Pure data movement."""
    B = p.num_seqs
    rows_k = p.k.reshape(-1, p.num_kv_heads, p.head_dim)
    rows_v = p.v.reshape(-1, p.num_kv_heads, p.head_dim)
    indptr = np.zeros(B + 1, dtype=np.int32)
    idx, ext_k, ext_v = [], [], []
    for b in range(B):
        lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        lk = int(p.seqused_k[b])
        pre = lk - lq
        j = np.arange(lk)
        slot = p.block_table[b, j // p.page_size].astype(np.int64) * p.page_size + j % p.page_size
        idx.append(slot[:pre])
        ext_k.append(rows_k[slot[pre:]])
        ext_v.append(rows_v[slot[pre:]])
        indptr[b + 1] = indptr[b] + pre
    return PrefixExtendProblem(
        name=name or p.name + "-prefix-extend", q=p.q, k_buffer=rows_k.copy(), v_buffer=rows_v.copy(),
        k_extend=np.concatenate(ext_k), v_extend=np.concatenate(ext_v), kv_dtype=p.kv_dtype,
        kv_indptr=indptr, kv_indices=np.concatenate(idx).astype(np.int32),
        cu_seqlens_q=p.cu_seqlens_q.copy(), num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
        scale=p.scale, k_descale=p.k_descale, v_descale=p.v_descale, window_left=p.window_left,
        softcap=p.softcap, sinks=p.sinks)
