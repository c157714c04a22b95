"""Pins for the oracle's optional features: sliding window, logit softcap and
attention sinks (the verify call of the sglang PR #30105 summary page, "Key
source snippets", passes window_size = (sliding_window - 1, 0), softcap and
sinks to the attention kernel).

Each feature is checked against
  * an independent dense numpy formulation with the feature written out
    (explicit window mask, explicit tanh cap, the sink as an extra softmax
    column without a value);
  * closed forms and limits: window 0 sees only the query's own key, a window
    at least as long as the sequence changes nothing, a huge softcap is no cap,
    a -inf sink is no sink, Q = 0 with a sink gives a known fraction of the mean;
  * split = unsplit with every feature on.
test_oracle_mutants.py plants mistakes in these paths too.
"""
import numpy as np
import pytest

import oracle
import va_inputs
from test_oracle_pins import dec_bf16, dec_kv, rel_err


def dense_reference_ex(p, window_left=-1, softcap=0.0, sinks=None):
    """out [total_q*Hq, D], lse [.] with the features written out densely."""
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
        Kb = K[pages].reshape(npg * p.page_size, p.num_kv_heads, D)[:Lk]
        Vb = V[pages].reshape(npg * p.page_size, p.num_kv_heads, D)[:Lk]
        kvh = np.arange(p.num_q_heads) // G
        S = np.einsum("thd,jhd->thj", Q[q0:q1], Kb[:, kvh, :]) * (p.scale * p.k_descale)
        if softcap > 0:
            S = softcap * np.tanh(S / softcap)
        pos = (Lk - Lq) + np.arange(Lq)[:, None]          # absolute query positions
        j = np.arange(Lk)[None, :]
        vis = j <= pos
        if window_left >= 0:
            vis &= j >= pos - window_left
        S = np.where(vis[:, None, :], S, -np.inf)
        if sinks is not None:                               # extra column, no value
            col = np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None], (Lq, p.num_q_heads, 1))
            S = np.concatenate([S, col], axis=2)
        m = S.max(axis=2, keepdims=True)
        W = np.exp(S - m)
        L = W.sum(axis=2, keepdims=True)
        Wk = W[:, :, :Lk]
        outs[q0:q1] = p.v_descale * np.einsum("thj,jhd->thd", Wk / L, Vb[:, kvh, :])
        lses[q0:q1] = (m + np.log(L))[..., 0]
    return outs.reshape(-1, D), lses.reshape(-1)


def _problem(q_lens, kv_lens, hq, hkv, kv_dtype="fp8", seed=0):
    return va_inputs.custom(q_lens, kv_lens, hq, hkv, kv_dtype, seed=seed)


FEATURE_CASES = [
    # q_lens, kv_lens, hq, hkv, kv, window_left, softcap, sinks?
    ([4, 2], [70, 33], 4, 1, "fp8", 0, 0.0, False),
    ([4, 2], [70, 33], 4, 1, "fp8", 5, 0.0, False),
    ([3, 1, 4], [17, 80, 40], 8, 2, "bf16", 16, 0.0, False),
    ([4, 2], [70, 33], 4, 1, "fp8", -1, 0.3, False),
    ([2, 3], [48, 65], 16, 1, "fp8", -1, 1.5, False),
    ([4, 2], [70, 33], 4, 1, "fp8", -1, 0.0, True),
    ([1, 4], [16, 79], 4, 2, "bf16", 31, 0.5, True),
    ([4, 4], [64, 100], 16, 1, "fp8", 20, 2.0, True),
]


@pytest.mark.parametrize("case", FEATURE_CASES, ids=lambda c: f"w{c[5]}-cap{c[6]}-sink{int(c[7])}-{c[4]}")
def test_features_match_dense_reference(case):
    ql, kl, hq, hkv, dt, wl, cap, use_sinks = case
    p = _problem(ql, kl, hq, hkv, dt, seed=sum(kl) + hq)
    sinks = np.linspace(-1.5, 2.5, hq) if use_sinks else None
    out, lse = oracle.attn(
        p.q, p.k, p.v, p.kv_dtype, p.block_table, p.cu_seqlens_q, p.seqused_k, p.num_kv_heads,
        p.scale, p.k_descale, p.v_descale, threads=2, window_left=wl, softcap=cap, sinks=sinks)
    ref_out, ref_lse = dense_reference_ex(p, wl, cap, sinks)
    assert rel_err(out, ref_out) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12 * max(1.0, np.max(np.abs(ref_lse)))


def _run(p, **kw):
    return oracle.attn(p.q, p.k, p.v, p.kv_dtype, p.block_table, p.cu_seqlens_q, p.seqused_k,
                       p.num_kv_heads, p.scale, p.k_descale, p.v_descale, threads=2, **kw)


def test_window_zero_sees_only_own_key():
    p = _problem([4, 3], [50, 21], 4, 1, "fp8", seed=3)
    out, _ = _run(p, window_left=0)
    V = dec_kv(p.v, "fp8")
    D = p.q.shape[2]
    out = out.reshape(p.total_q, p.num_q_heads, D)
    for b in range(p.num_seqs):
        q0, q1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(p.seqused_k[b])
        for t in range(Lq):
            j = Lk - Lq + t
            row = V[p.block_table[b, j // 16], j % 16, 0]
            assert np.array_equal(out[q0 + t], np.broadcast_to(row * p.v_descale, (p.num_q_heads, D)))


def test_window_covering_the_sequence_changes_nothing():
    p = _problem([4, 2], [70, 33], 8, 2, "bf16", seed=4)
    a, la = _run(p)
    b, lb = _run(p, window_left=70)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_huge_softcap_is_no_softcap():
    p = _problem([4, 2], [70, 33], 4, 1, "fp8", seed=5)
    a, _ = _run(p)
    b, _ = _run(p, softcap=1e9)
    assert rel_err(b, a) <= 1e-12


def test_minus_infinite_sinks_are_no_sinks():
    p = _problem([4, 2], [70, 33], 4, 1, "fp8", seed=6)
    a, la = _run(p)
    b, lb = _run(p, sinks=np.full(4, -np.inf))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_zero_query_with_sink_closed_form():
    """Q = 0: every visible logit is 0, so out = n/(n + e^sink) * mean(V) per row."""
    p = _problem([3], [40], 4, 1, "fp8", seed=7)
    p.q[:] = 0
    sinks = np.array([-1.0, 0.0, 0.5, 3.0])
    out, lse = _run(p, sinks=sinks, softcap=0.7)          # the cap keeps 0 at 0
    V = dec_kv(p.v, "fp8")
    D = p.q.shape[2]
    out = out.reshape(3, 4, D)
    lse = lse.reshape(3, 4)
    keys = V[p.block_table[0, :3]].reshape(48, 1, D)[:40, 0]
    for t in range(3):
        n = 40 - 3 + t + 1
        for h in range(4):
            expect = keys[:n].mean(axis=0) * n / (n + np.exp(sinks[h]))
            assert rel_err(out[t, h], expect) <= 1e-12
            assert abs(lse[t, h] - np.log(n + np.exp(sinks[h]))) <= 1e-12


def test_softcap_bounds_every_logit():
    """With a tiny cap every logit lies in (-cap, cap): weights within e^(2 cap)."""
    p = _problem([2], [64], 4, 1, "fp8", seed=8)
    cap = 1e-3
    out, _ = _run(p, softcap=cap)
    q_zero = va_inputs.custom([2], [64], 4, 1, "fp8", seed=8)
    q_zero.q[:] = 0
    mean, _ = _run(q_zero)
    assert rel_err(out, mean) <= 3 * cap


@pytest.mark.parametrize("wl,cap,use_sinks", [(7, 0.0, False), (-1, 0.9, True), (12, 1.7, True)])
def test_split_equals_unsplit_with_features(wl, cap, use_sinks):
    p = _problem([4, 2, 3], [70, 33, 90], 8, 2, "fp8", seed=9)
    sinks = np.linspace(-0.5, 1.5, 8) if use_sinks else None
    a, la = _run(p, window_left=wl, softcap=cap, sinks=sinks)
    segs = [[0, 16, 17, 64], [0, 32], [0, 5, 48, 80]]
    b, lb = _run(p, window_left=wl, softcap=cap, sinks=sinks, segments=segs)
    assert rel_err(b, a) <= 1e-12
    assert np.max(np.abs(la - lb)) <= 1e-12
