"""fp64 CPU oracle for paged GQA target-verify attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  It
shares no code with the HIP library in ``paged_gqa_attention_va_amd`` and
imports nothing from it.  The C source ``va_oracle.c`` states the definition it
follows and cites the passages it comes from.

``attn()`` takes the raw bit patterns of the inputs (uint16 bf16 bits, uint8
fp8 bytes) and returns the attention output and its log-sum-exp in float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "va_oracle.c")
_LIB = os.path.join(_HERE, "libva_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no GPU toolchain)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-shared",
                               "-fPIC", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open an oracle shared library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB)
    return _lib


def _declare(lib) -> None:
    P = ctypes.c_void_p
    lib.va_oracle_fp8e4m3fn_to_double.restype = ctypes.c_double
    lib.va_oracle_fp8e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    lib.va_oracle_bf16_to_double.restype = ctypes.c_double
    lib.va_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.va_oracle_attn.restype = ctypes.c_int
    lib.va_oracle_attn.argtypes = [
        P, P, P, ctypes.c_int, P, ctypes.c_int64, P, P,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, ctypes.c_double, ctypes.c_double,
        P, P, P, ctypes.c_int64, P, P, ctypes.c_int]
    lib.va_oracle_attn_ex.restype = ctypes.c_int
    lib.va_oracle_attn_ex.argtypes = [
        P, P, P, ctypes.c_int, P, ctypes.c_int64, P, P,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_double, P,
        P, P, P, ctypes.c_int64, P, P, ctypes.c_int]


def fp8_e4m3fn_to_float(code: int) -> float:
    return _load().va_oracle_fp8e4m3fn_to_double(int(code))


def bf16_to_float(bits: int) -> float:
    return _load().va_oracle_bf16_to_double(int(bits))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_dtype: str,
         block_table: np.ndarray, cu_seqlens_q: np.ndarray, seqused_k: np.ndarray,
         num_kv_heads: int, scale: float, k_descale: float = 1.0,
         v_descale: float = 1.0, rows: Optional[Sequence[int]] = None,
         segments: Optional[Sequence[Sequence[int]]] = None,
         threads: Optional[int] = None, lib=None, window_left: int = -1,
         softcap: float = 0.0, sinks: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention output [n_rows, D] and natural-log LSE [n_rows], float64.

    q: uint16 [total_q, Hq, D]; k, v: uint8 (fp8 e4m3fn) or uint16 (bf16)
    [num_blocks, page, Hkv, D].  rows: flat (q_row * Hq + head) indices, default
    all rows in order.  segments: per sequence, the ascending start keys of a
    contiguous split of [0, seqused_k) (first start 0); the oracle then merges
    per-segment partials by log-sum-exp instead of one pass.  lib: an
    alternative build of the oracle (tests that plant mistakes use this).
    window_left (-1 = none), softcap (0 = none) and sinks ([Hq] logits or None)
    select the optional sliding window, logit softcap and attention sinks.
    Raises ValueError when a sequence has more query tokens than keys
    (q_len > seqused_k), a call outside the operation's domain.
    """
    if lib is None:
        lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    if kv_dtype == "fp8":
        k = np.ascontiguousarray(k, dtype=np.uint8)
        v = np.ascontiguousarray(v, dtype=np.uint8)
    elif kv_dtype == "bf16":
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
    else:
        raise ValueError(kv_dtype)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sk = np.ascontiguousarray(seqused_k, dtype=np.int32)
    total_q, hq, d = q.shape
    page = k.shape[1]
    assert k.shape[2] == num_kv_heads and k.shape[3] == d
    if rows is None:
        rows_arr = None
        n = total_q * hq
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = int(rows_arr.shape[0])
    seg_start = seg_ptr = None
    if segments is not None:
        assert len(segments) == sk.shape[0]
        starts, ptr = [], [0]
        for s in segments:
            starts.extend(int(x) for x in s)
            ptr.append(len(starts))
        seg_start = np.asarray(starts if starts else [0], dtype=np.int32)
        seg_ptr = np.asarray(ptr, dtype=np.int32)
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    sk_arr = None
    if sinks is not None:
        sk_arr = np.ascontiguousarray(sinks, dtype=np.float64)
        assert sk_arr.shape == (hq,)
    st = lib.va_oracle_attn_ex(
        _ptr(q), _ptr(k), _ptr(v), 1 if kv_dtype == "fp8" else 0,
        _ptr(bt), bt.shape[1], _ptr(cu), _ptr(sk), sk.shape[0], hq, num_kv_heads,
        d, page, float(scale), float(k_descale), float(v_descale),
        int(window_left), float(softcap), _ptr(sk_arr),
        _ptr(seg_start), _ptr(seg_ptr), _ptr(rows_arr), n, _ptr(out), _ptr(lse),
        default_threads() if threads is None else int(threads))
    if st == -4:
        raise ValueError("a sequence has more query tokens than keys (q_len > seqused_k): "
                         "seqused_k counts the verify tokens, so the call has no defined result")
    if st != 0:
        raise RuntimeError(f"va_oracle_attn failed with status {st}")
    return out, lse


def attn_problem(p, rows=None, segments=None, threads=None, lib=None):
    """``attn`` on a ``va_inputs.Problem``-like object (duck typed)."""
    return attn(p.q, p.k, p.v, p.kv_dtype, p.block_table, p.cu_seqlens_q,
                p.seqused_k, p.num_kv_heads, p.scale, p.k_descale, p.v_descale,
                rows=rows, segments=segments, threads=threads, lib=lib,
                window_left=getattr(p, "window_left", -1), softcap=getattr(p, "softcap", 0.0),
                sinks=None if getattr(p, "sinks", None) is None else p.sinks.astype(np.float64))


def spec_block_table(kv_indptr, kv_indices, page_size: int, max_blocks_per_seq: int):
    """Block table and KV lengths of a draft-extend (KV catch-up) call, from
    speculative-decoding metadata.

    The PR #30105 summary page ("Key source snippets", draft_extend_v2 routed to
    the verify kernel) builds a 2D page table from the spec metadata and takes
    each sequence's KV length as the kv_indptr difference.  Reading: kv_indices
    lists, per sequence, the pool slot of every KV token in order (slot = page *
    page_size + offset, pages filled from offset 0), so page p of sequence b is
    the slot of its token p * page_size divided by page_size.  Plain loops;
    entries past a sequence's last page are 0.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    B = kv_indptr.shape[0] - 1
    bt = np.zeros((B, max_blocks_per_seq), dtype=np.int32)
    seqused = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(kv_indptr[b + 1] - kv_indptr[b])
        seqused[b] = n
        for pg in range(-(-n // page_size)):
            bt[b, pg] = int(kv_indices[kv_indptr[b] + pg * page_size]) // page_size
    return bt, seqused


# Rules of the call's device metadata (bits of ``validate``'s result).
BAD_CU_SEQLENS_Q, BAD_Q_LEN, BAD_SEQUSED_K, BAD_Q_GT_K, BAD_PAGE = 1, 2, 4, 8, 16


def validate(block_table, cu_seqlens_q, seqused_k, num_blocks: int, total_q: int,
             max_seqlen_q: int, max_seqlen_k: int, window_left: int = -1,
             page_size: int = 16) -> Tuple[int, int]:
    """Check one call's metadata; returns (OR of the broken rules' bits, the
    smallest sequence that breaks one, or num_seqs).

    The rules restate what the verify call's inputs mean on the PR #36330
    summary page ("Key source snippets": cu_seqlens_q, seqused_k and
    block_table of the unified_attention_3d_mtp_func call, and the paged cache
    the test builds):
      - cu_seqlens_q holds prefix sums of the query lengths from 0, inside the
        total_q rows of q (BAD_CU_SEQLENS_Q);
      - no sequence has more than max_seqlen_q queries (BAD_Q_LEN);
      - 0 <= seqused_k <= max_seqlen_k (BAD_SEQUSED_K);
      - the query tokens are the last q_len of the seqused_k keys, so
        q_len <= seqused_k (BAD_Q_GT_K; q_len counts 0 where cu is broken);
      - every page holding a key some query of the sequence sees is a pool page
        (BAD_PAGE).  The first query sits at position seqused_k - q_len and with
        a sliding window sees keys from that position - window_left on.
    Plain loops over sequences and pages.
    """
    bt = np.asarray(block_table)
    cu = [int(x) for x in np.asarray(cu_seqlens_q).ravel()]
    sk = [int(x) for x in np.asarray(seqused_k).ravel()]
    B = len(sk)
    mbps = bt.shape[1]
    bits, first_bad = 0, B
    for b in range(B):
        q0, q1, lk = cu[b], cu[b + 1], sk[b]
        bad = 0
        cu_ok = (b > 0 or q0 == 0) and q0 <= q1 <= total_q
        lq = q1 - q0 if cu_ok else 0
        if not cu_ok:
            bad |= BAD_CU_SEQLENS_Q
        if lq > max_seqlen_q:
            bad |= BAD_Q_LEN
        if lk < 0 or lk > max_seqlen_k:
            bad |= BAD_SEQUSED_K
        if lq > lk:
            bad |= BAD_Q_GT_K
        if lk > 0:
            first_key = 0 if window_left < 0 else max(0, lk - lq - window_left)
            last_page = (lk - 1) // page_size
            for pg in range(first_key // page_size, min(last_page + 1, mbps)):
                if not 0 <= int(bt[b, pg]) < num_blocks:
                    bad |= BAD_PAGE
        if bad:
            bits |= bad
            first_bad = min(first_bad, b)
    return bits, first_bad


def prefix_extend_to_paged(k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend,
                           cu_seqlens_q, page_size: int = 16):
    """The paged cache, block table and KV lengths of a prefix + extend call.

    Reading of the sglang PR #34517 summary page ("Key source snippets", the
    shared-KV verify kernel and its entry guards): the prefix keys of sequence
    b are the rows kv_indices[kv_indptr[b] + j], j < P_b, of the K/V buffers;
    its q_len draft tokens' keys are rows cu[b] .. cu[b+1]-1 of k_extend /
    v_extend and come after the prefix.  Query token t sits at position
    P_b + t and sees the whole prefix and draft tokens 0..t, which is the
    bottom-right causal rule of the paged call with seqused_k = P_b + q_len.
    So the call is the paged call over a cache that holds each sequence's
    keys in that order.  Plain loops copy them into fresh pages; buffers are
    [rows, Hkv, D], the result is (k_pool, v_pool, block_table, seqused_k).
    """
    k_buffer = np.asarray(k_buffer)
    v_buffer = np.asarray(v_buffer)
    k_extend = np.asarray(k_extend)
    v_extend = np.asarray(v_extend)
    indptr = [int(x) for x in np.asarray(kv_indptr).ravel()]
    cu = [int(x) for x in np.asarray(cu_seqlens_q).ravel()]
    B = len(cu) - 1
    hkv, d = k_buffer.shape[1], k_buffer.shape[2]
    lens = [(indptr[b + 1] - indptr[b]) + (cu[b + 1] - cu[b]) for b in range(B)]
    pages = [-(-n // page_size) for n in lens]
    mbps = max(1, max(pages))
    k_pool = np.zeros((max(1, sum(pages)), page_size, hkv, d), dtype=k_buffer.dtype)
    v_pool = np.zeros_like(k_pool)
    bt = np.zeros((B, mbps), dtype=np.int32)
    page = 0
    for b in range(B):
        keys_k, keys_v = [], []
        for j in range(indptr[b], indptr[b + 1]):
            keys_k.append(k_buffer[int(kv_indices[j])])
            keys_v.append(v_buffer[int(kv_indices[j])])
        for r in range(cu[b], cu[b + 1]):
            keys_k.append(k_extend[r])
            keys_v.append(v_extend[r])
        for i in range(len(keys_k)):
            if i % page_size == 0:
                bt[b, i // page_size] = page
                page += 1
            k_pool[bt[b, i // page_size], i % page_size] = keys_k[i]
            v_pool[bt[b, i // page_size], i % page_size] = keys_v[i]
    return k_pool, v_pool, bt, np.asarray(lens, dtype=np.int32)


def attn_prefix_extend(q, k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend,
                       kv_dtype: str, cu_seqlens_q, num_kv_heads: int, scale: float,
                       k_descale: float = 1.0, v_descale: float = 1.0, rows=None,
                       threads=None, window_left: int = -1, softcap: float = 0.0,
                       sinks=None) -> Tuple[np.ndarray, np.ndarray]:
    """``attn`` of a prefix + extend call (see ``prefix_extend_to_paged``)."""
    k_pool, v_pool, bt, seqused = prefix_extend_to_paged(
        k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend, cu_seqlens_q)
    return attn(q, k_pool, v_pool, kv_dtype, bt, cu_seqlens_q, seqused, num_kv_heads, scale,
                k_descale, v_descale, rows=rows, threads=threads, window_left=window_left,
                softcap=softcap, sinks=sinks)


def attn_prefix_extend_problem(p, rows=None, threads=None):
    """``attn_prefix_extend`` on a ``va_inputs.PrefixExtendProblem``-like object."""
    return attn_prefix_extend(
        p.q, p.k_buffer, p.v_buffer, p.kv_indptr, p.kv_indices, p.k_extend, p.v_extend,
        p.kv_dtype, p.cu_seqlens_q, p.num_kv_heads, p.scale, p.k_descale, p.v_descale,
        rows=rows, threads=threads, window_left=getattr(p, "window_left", -1),
        softcap=getattr(p, "softcap", 0.0),
        sinks=None if getattr(p, "sinks", None) is None else p.sinks.astype(np.float64))


def attn_mla(q, kv_pool, kv_dtype: str, block_table, cu_seqlens_q, seqused_k, scale: float,
             v_head_dim: int, k_descale: float = 1.0, v_descale: float = 1.0, rows=None,
             threads=None, window_left: int = -1, softcap: float = 0.0,
             sinks=None) -> Tuple[np.ndarray, np.ndarray]:
    """Absorbed-MLA verify attention: the PE_DIM split of the sglang PR #34517
    summary page ("Key source snippets", verify_shared_kv_fwd: q_nope.k_nope
    plus, when PE_DIM > 0, q_pe.k_pe; NOPE_DIM is the latent width of the
    absorbed-MLA layout).

    One kv head.  A cache row is [latent (v_head_dim) | RoPE part]; a query
    row is [q_nope | q_pe] over the same widths.  The logit is the sum of the
    two partial dot products, i.e. the dot product over the whole row, scaled
    as in ``attn``.  Reading: the value of a key is its latent (the absorbed
    layout keeps one cached vector per token; the page's output width is the
    latent width).  So this is ``attn`` with V = the cache rows with their
    RoPE part set to zero, keeping the first v_head_dim output dims.
    Returns out [n_rows, v_head_dim] and the natural-log LSE, float64.
    """
    kv_pool = np.asarray(kv_pool)
    v = kv_pool.copy()
    v[..., v_head_dim:] = 0                 # +0.0 in both encodings
    out, lse = attn(q, kv_pool, v, kv_dtype, block_table, cu_seqlens_q, seqused_k, 1, scale,
                    k_descale, v_descale, rows=rows, threads=threads, window_left=window_left,
                    softcap=softcap, sinks=sinks)
    return np.ascontiguousarray(out[:, :v_head_dim]), lse


def attn_mla_problem(p, rows=None, threads=None):
    """``attn_mla`` on a ``va_inputs.Problem`` built by ``va_inputs.mla``."""
    return attn_mla(p.q, p.k, p.kv_dtype, p.block_table, p.cu_seqlens_q, p.seqused_k, p.scale,
                    p.v_head_dim, p.k_descale, p.v_descale, rows=rows, threads=threads,
                    window_left=getattr(p, "window_left", -1), softcap=getattr(p, "softcap", 0.0),
                    sinks=None if getattr(p, "sinks", None) is None else p.sinks.astype(np.float64))
