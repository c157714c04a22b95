"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each check below compares the oracle to one of these:
  * a library routine (torch's fp8 / bf16 decoders);
  * an independent dense numpy formulation of the attention definition
    (gather through the block table, full score matrix, explicit mask);
  * a closed form the definition implies;
  * an invariant the definition implies.
The checks are chosen so that a dropped term, a wrong sign, a wrong index or
a transposed operand in the oracle fails at least one of them.
test_oracle_mutants.py plants such mistakes in a copy of the oracle to show
that they are caught.

Sources for the definition: the sglang PR #36330 summary page, "Key source
snippets" (the verify-attention call, causal=True, seqused_k counting the verify
tokens, descales as [1] tensors, scale head_size**-0.5), and the sglang PR #34517
summary page, "Key source snippets" (logits times sm_scale * k_scale, masked
logits to -inf).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import va_inputs

# ------------------------------------------------------------ helpers ------


def dec_fp8(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dec_bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def dec_kv(a: np.ndarray, kv_dtype: str) -> np.ndarray:
    return dec_fp8(a) if kv_dtype == "fp8" else dec_bf16(a)


def dense_reference(p):
    """Independent dense formulation: returns out [total_q*Hq, D], lse [.]"""
    G = p.num_q_heads // p.num_kv_heads
    D = p.q.shape[2]
    K = dec_kv(p.k, p.kv_dtype)
    V = dec_kv(p.v, p.kv_dtype)
    Q = dec_bf16(p.q)
    outs = np.zeros((p.total_q, p.num_q_heads, D))
    lses = np.zeros((p.total_q, p.num_q_heads))
    for b in range(p.num_seqs):
        q0, q1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(p.seqused_k[b])
        if Lq == 0:
            continue
        npg = -(-Lk // p.page_size)
        pages = p.block_table[b, :npg]
        Kb = K[pages].reshape(npg * p.page_size, p.num_kv_heads, D)[:Lk]   # [Lk, Hkv, D]
        Vb = V[pages].reshape(npg * p.page_size, p.num_kv_heads, D)[:Lk]
        kv_of_head = np.arange(p.num_q_heads) // G
        Kh = Kb[:, kv_of_head, :]                                          # [Lk, Hq, D]
        Vh = Vb[:, kv_of_head, :]
        Qb = Q[q0:q1]                                                      # [Lq, Hq, D]
        S = np.einsum("thd,jhd->thj", Qb, Kh) * (p.scale * p.k_descale)    # [Lq, Hq, Lk]
        t = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        visible = j <= (Lk - Lq) + t                                       # [Lq, Lk]
        S = np.where(visible[:, None, :], S, -np.inf)
        m = S.max(axis=2, keepdims=True)
        W = np.exp(S - m)
        L = W.sum(axis=2, keepdims=True)
        outs[q0:q1] = p.v_descale * np.einsum("thj,jhd->thd", W / L, Vh)
        lses[q0:q1] = (m + np.log(L))[..., 0]
    return outs.reshape(-1, D), lses.reshape(-1)


def small_problem(rng, q_lens, kv_lens, hq, hkv, d=256, kv_dtype="fp8", kd=1.0, vd=1.0,
                  table="perm", scale=None, seed=0, poison=True):
    """A small random problem with arbitrary head_dim (the generator module is fixed at
    D=256, so D != 256 cases are built here)."""
    if d == 256:
        return va_inputs.custom(q_lens, kv_lens, hq, hkv, kv_dtype, seed=seed, table=table,
                                k_descale=kd, v_descale=vd, scale=scale, poison=poison)
    p = va_inputs.custom(q_lens, kv_lens, hq, hkv, kv_dtype, seed=seed, table=table,
                         k_descale=kd, v_descale=vd, scale=d ** -0.5 if scale is None else scale,
                         poison=poison)
    p.q = np.ascontiguousarray(p.q[:, :, :d])
    p.k = np.ascontiguousarray(p.k[:, :, :, :d])
    p.v = np.ascontiguousarray(p.v[:, :, :, :d])
    p.head_dim = d
    return p


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


# ------------------------------------------------------------- P1 codecs ----

def test_fp8_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = dec_fp8(codes)
    got = np.array([oracle.fp8_e4m3fn_to_float(c) for c in range(256)])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    # the format facts the pages' dtype implies: max finite 448, min subnormal 2^-9
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_bf16_decoder_matches_torch_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = dec_bf16(bits)
    got = np.array([oracle.bf16_to_float(int(b)) for b in bits])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])


def test_every_finite_fp8_value_is_exact_in_bf16():
    # the dequant step (fp8 -> bf16 in registers) loses nothing
    vals = dec_fp8(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    as_bf16 = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, fin)


# ---------------------------------------------------- P2 brute force -------

BRUTE_CASES = [
    # q_lens, kv_lens, Hq, Hkv, D, dtype, kd, vd
    ([1], [1], 1, 1, 8, "fp8", 1.0, 1.0),
    ([4], [4], 4, 1, 8, "fp8", 1.0, 1.0),
    ([2, 3], [17, 80], 4, 2, 8, "fp8", 1.5, 0.75),
    ([4, 1, 3], [16, 33, 79], 16, 1, 8, "bf16", 1.0, 1.0),
    ([3, 4], [5, 64], 2, 2, 256, "fp8", 0.5, 2.0),
    ([4, 2], [47, 31], 16, 1, 256, "fp8", 1.0, 1.0),
    ([1, 4, 2], [1, 48, 15], 8, 2, 256, "bf16", 1.25, 0.5),
    ([0, 3], [20, 3], 4, 1, 256, "fp8", 1.0, 1.0),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_dense_brute_force(case):
    ql, kl, hq, hkv, d, dt, kd, vd = case
    p = small_problem(None, ql, kl, hq, hkv, d=d, kv_dtype=dt, kd=kd, vd=vd, seed=sum(kl) + hq)
    out, lse = oracle.attn_problem(p, threads=2)
    ref_out, ref_lse = dense_reference(p)
    rows = np.arange(p.total_q * p.num_q_heads)
    assert np.all(np.isfinite(out))
    assert rel_err(out, ref_out) <= 1e-12
    assert np.max(np.abs(lse[rows] - ref_lse[rows])) <= 1e-12 * max(1.0, np.max(np.abs(ref_lse)))


def test_oracle_row_selection_matches_full():
    p = small_problem(None, [4, 2], [100, 37], 16, 2, seed=7)
    full, full_lse = oracle.attn_problem(p, threads=3)
    rows = np.array([0, 5, 17, 40, p.total_q * p.num_q_heads - 1])
    sub, sub_lse = oracle.attn_problem(p, rows=rows, threads=2)
    assert np.array_equal(sub, full[rows]) and np.array_equal(sub_lse, full_lse[rows])


# -------------------------------------------------- P3 closed forms --------

def test_zero_query_gives_mean_of_visible_values():
    p = small_problem(None, [4, 2], [37, 20], 8, 2, seed=3, vd=1.5)
    p.q[:] = 0
    out, lse = oracle.attn_problem(p)
    V = dec_fp8(p.v)
    G = p.num_q_heads // p.num_kv_heads
    out = out.reshape(p.total_q, p.num_q_heads, -1)
    for b in range(p.num_seqs):
        q0, q1 = p.cu_seqlens_q[b], p.cu_seqlens_q[b + 1]
        Lq, Lk = q1 - q0, p.seqused_k[b]
        for t in range(Lq):
            n = Lk - Lq + t + 1
            keys = np.arange(n)
            pages = p.block_table[b, keys // 16]
            for h in range(p.num_q_heads):
                mean = V[pages, keys % 16, h // G].mean(axis=0) * p.v_descale
                assert np.max(np.abs(out[q0 + t, h] - mean)) <= 1e-12
                assert abs(lse.reshape(p.total_q, p.num_q_heads)[q0 + t, h] - math.log(n)) <= 1e-12


def test_first_query_of_full_verify_sees_exactly_one_key():
    # Lk == Lq: token 0 of the verify block sees key 0 only -> O = v_descale * V[key 0]
    p = small_problem(None, [4, 3], [4, 3], 16, 1, seed=11, vd=1.75, kd=0.5)
    out, _ = oracle.attn_problem(p)
    V = dec_fp8(p.v)
    out = out.reshape(p.total_q, p.num_q_heads, -1)
    for b in range(p.num_seqs):
        q0 = p.cu_seqlens_q[b]
        page = p.block_table[b, 0]
        for h in range(p.num_q_heads):
            assert np.array_equal(out[q0, h], p.v_descale * V[page, 0, 0])


def test_query_tokens_beyond_the_keys_are_refused():
    # seqused_k counts the verify tokens themselves, so a sequence with more
    # query tokens than keys is outside the operation's domain
    p = small_problem(None, [4, 3], [20, 3], 8, 1, seed=23)
    oracle.attn_problem(p)                         # q_len == seqused_k is in the domain
    p.seqused_k[1] = 2                             # 3 query tokens, 2 keys
    with pytest.raises(ValueError):
        oracle.attn_problem(p)
    with pytest.raises(ValueError):                # also when only other rows are asked for
        oracle.attn_problem(p, rows=[0, 1])
    p.seqused_k[1] = 0
    with pytest.raises(ValueError):
        oracle.attn_problem(p)


def test_identical_keys_give_mean_of_visible_values():
    p = small_problem(None, [3], [50], 4, 1, seed=5)
    K = p.k
    pages = p.block_table[0, :4]
    K[pages] = K[pages[0], 0]          # every key row of the sequence identical
    out, _ = oracle.attn_problem(p)
    V = dec_fp8(p.v)
    out = out.reshape(p.total_q, p.num_q_heads, -1)
    for t in range(3):
        n = 50 - 3 + t + 1
        keys = np.arange(n)
        mean = V[p.block_table[0, keys // 16], keys % 16, 0].mean(axis=0)
        for h in range(4):
            assert np.max(np.abs(out[t, h] - mean)) <= 1e-12


def test_one_dominant_key_closed_form():
    # all keys zero except key j*: logits are 0 except s* -> O is the two-term blend
    p = small_problem(None, [1], [40], 4, 1, seed=9, kv_dtype="bf16")
    pages = p.block_table[0, :3]
    p.k[pages] = 0
    jstar = 21
    pg, sl = p.block_table[0, jstar // 16], jstar % 16
    qrow = dec_bf16(p.q[0, 0])
    kvec = np.sign(qrow) * 2.0            # exact in bf16
    p.k[pg, sl, 0] = torch.from_numpy(kvec).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    p.q[0, 1:] = p.q[0, 0]
    out, lse = oracle.attn_problem(p)
    V = dec_bf16(p.v)
    n = 40
    keys = np.arange(n)
    Vs = V[p.block_table[0, keys // 16], keys % 16, 0]
    sstar = p.scale * float(np.dot(qrow, kvec))
    w = np.ones(n)
    w[jstar] = math.exp(sstar)
    expect = (w[:, None] * Vs).sum(0) / w.sum()
    for h in range(4):
        assert np.max(np.abs(out[h] - expect)) <= 1e-12
        assert abs(lse[h] - math.log(w.sum())) <= 1e-12
    # and it approaches V[j*] as the gap grows (monotone in the gap)
    assert np.max(np.abs(out[0] - Vs[jstar])) < np.max(np.abs(Vs.mean(0) - Vs[jstar]))


def test_constant_values_give_constant_output():
    p = small_problem(None, [4, 2], [70, 18], 16, 2, seed=13, vd=0.625)
    p.v[:] = 0x44          # fp8 e4m3fn 0x44 = 3.0
    out, _ = oracle.attn_problem(p)
    assert np.max(np.abs(out - 3.0 * 0.625)) <= 1e-12


# ------------------------------------------- P4 causal invariants ----------

def test_row_t_equals_truncated_single_query_decode():
    p = small_problem(None, [4], [45], 8, 1, seed=17)
    out, lse = oracle.attn_problem(p)
    out = out.reshape(4, 8, -1)
    for t in range(4):
        single = va_inputs.Problem(
            name="single", q=np.ascontiguousarray(p.q[t:t + 1]), k=p.k, v=p.v,
            kv_dtype=p.kv_dtype, block_table=p.block_table,
            cu_seqlens_q=np.array([0, 1], np.int32),
            seqused_k=np.array([45 - 4 + t + 1], np.int32), num_q_heads=8,
            num_kv_heads=1, scale=p.scale, k_descale=p.k_descale, v_descale=p.v_descale)
        o1, _ = oracle.attn_problem(single)
        assert np.array_equal(o1, out[t])


def test_poisoned_invisible_memory_changes_nothing():
    a = va_inputs.custom([4, 2, 3], [33, 17, 64], 16, 2, "fp8", seed=21, poison=False)
    b = va_inputs.custom([4, 2, 3], [33, 17, 64], 16, 2, "fp8", seed=21, poison=True)
    assert not np.array_equal(a.k, b.k)         # poison did land somewhere
    oa, la = oracle.attn_problem(a)
    ob, lb = oracle.attn_problem(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_relabelling_physical_pages_changes_nothing():
    p = va_inputs.custom([3, 4], [90, 41], 8, 2, "fp8", seed=23, extra_blocks=5)
    o1, _ = oracle.attn_problem(p)
    perm = np.random.default_rng(0).permutation(p.num_blocks)     # new id of old page i
    q = va_inputs.Problem(**{**p.__dict__})
    q.k = np.empty_like(p.k)
    q.v = np.empty_like(p.v)
    q.k[perm] = p.k
    q.v[perm] = p.v
    bt = p.block_table.copy()
    inside = bt < p.num_blocks
    bt[inside] = perm[bt[inside]]
    q.block_table = bt
    o2, _ = oracle.attn_problem(q)
    assert np.array_equal(o1, o2)


def test_two_kv_heads_equal_two_single_head_problems():
    p = va_inputs.custom([4, 2], [64, 29], 32, 2, "fp8", seed=29)
    full, _ = oracle.attn_problem(p)
    full = full.reshape(p.total_q, 32, -1)
    for g in range(2):
        sub = va_inputs.Problem(**{**p.__dict__})
        sub.q = np.ascontiguousarray(p.q[:, 16 * g:16 * (g + 1)])
        sub.k = np.ascontiguousarray(p.k[:, :, g:g + 1])
        sub.v = np.ascontiguousarray(p.v[:, :, g:g + 1])
        sub.num_q_heads, sub.num_kv_heads = 16, 1
        o, _ = oracle.attn_problem(sub)
        assert np.array_equal(o.reshape(p.total_q, 16, -1), full[:, 16 * g:16 * (g + 1)])


def test_group_one_is_plain_multi_head_attention():
    p = small_problem(None, [2, 3], [30, 12], 4, 4, seed=31)
    out, _ = oracle.attn_problem(p)
    ref, _ = dense_reference(p)
    assert rel_err(out, ref) <= 1e-12


# --------------------------------------------------- P5 split = unsplit ----

@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    kv = [int(x) for x in rng.integers(1, 120, size=3)]
    ql = [int(min(k, x)) for k, x in zip(kv, rng.integers(1, 5, size=3))]
    p = va_inputs.custom(ql, kv, 8, 2, "fp8", seed=100 + seed)
    segs = []
    for Lk in kv:
        cuts = sorted(set(rng.integers(1, Lk, size=min(Lk - 1, 6)).tolist())) if Lk > 1 else []
        starts = [0] + cuts
        if Lk > 1:
            starts.append(Lk - 1)          # a one-key last segment: invisible to early rows
        segs.append(sorted(set(starts)))
    o1, l1 = oracle.attn_problem(p)
    o2, l2 = oracle.attn_problem(p, segments=segs)
    assert rel_err(o2, o1) <= 1e-12
    assert np.max(np.abs(l2 - l1)) <= 1e-12 * max(1.0, np.max(np.abs(l1)))


def test_split_with_fully_masked_segment():
    # config-0 shape: sequence 1 has 769 = 48*16 + 1 keys; a page-aligned last
    # segment [768, 769) is invisible to every row but the last one
    p = va_inputs.config(0)
    segs = [list(range(0, 1024, 256)), [0, 384, 768]]
    o1, _ = oracle.attn_problem(p)
    o2, _ = oracle.attn_problem(p, segments=segs)
    assert rel_err(o2, o1) <= 1e-12


# ------------------------------------------------------- P6 descale -------

def test_descale_factorisation():
    base = small_problem(None, [4, 2], [55, 30], 16, 1, seed=37)
    a = va_inputs.Problem(**{**base.__dict__})
    a.k_descale, a.v_descale = 1.5, 0.75
    b = va_inputs.Problem(**{**base.__dict__})
    b.scale, b.k_descale, b.v_descale = base.scale * 1.5, 1.0, 1.0
    oa, la = oracle.attn_problem(a)
    ob, lb = oracle.attn_problem(b)
    assert rel_err(oa, 0.75 * ob) <= 1e-13
    assert np.max(np.abs(la - lb)) <= 1e-13 * max(1.0, np.max(np.abs(lb)))
