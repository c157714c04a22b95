"""Pins of the oracle's prefix + extend layout (oracle.attn_prefix_extend).

The layout is the sglang PR #34517 summary page's: prefix K/V gathered by
per-token slots (kv_indptr / kv_indices), the draft tokens' K/V in separate
k_extend / v_extend rows.  The oracle re-lays such a call out as a paged call
and runs the pinned paged oracle.  Pinned here against things other than that
re-layout:
  - a paged problem moved into the prefix + extend layout by pure data
    movement (va_inputs.prefix_extend_from_paged) gives the paged oracle's
    result bit for bit, with and without window, softcap and sinks;
  - the result does not depend on which buffer rows hold the prefix;
  - with Q = 0 and no prefix, every visible draft key gets the same weight,
    so the output is the running mean of the draft V rows (closed form);
  - planted mistakes in the re-layout (draft keys first, draft rows shifted by
    one, the last prefix key dropped) each fail one of these pins.
"""
import numpy as np
import pytest

import oracle
import va_inputs as vi


ROUND_TRIP_CASES = [
    dict(q_lens=[4, 2, 3], kv_lens=[300, 40, 17], hq=16, hkv=1, dt="fp8"),
    dict(q_lens=[1, 3, 0, 2], kv_lens=[16, 33, 5, 64], hq=32, hkv=2, dt="bf16"),
    dict(q_lens=[4, 4], kv_lens=[4, 129], hq=8, hkv=1, dt="fp8", window_left=20),
    dict(q_lens=[2, 3], kv_lens=[90, 47], hq=4, hkv=1, dt="bf16", softcap=5.0,
         sinks=[0.5, -1.0, 2.0, 0.0]),
]


def _paged(c, seed=0):
    return vi.custom(c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["dt"], seed=seed,
                     window_left=c.get("window_left", -1), softcap=c.get("softcap", 0.0),
                     sinks=c.get("sinks"))


@pytest.mark.parametrize("c", ROUND_TRIP_CASES, ids=lambda c: f"{c['dt']}-hq{c['hq']}-hkv{c['hkv']}")
def test_round_trip_equals_paged_oracle(c):
    p = _paged(c)
    pe = vi.prefix_extend_from_paged(p)
    want, want_lse = oracle.attn_problem(p)
    got, got_lse = oracle.attn_prefix_extend_problem(pe)
    assert np.array_equal(got, want)
    assert np.array_equal(got_lse, want_lse)


def test_prefix_rows_can_sit_anywhere():
    p = vi.prefix_extend([4, 1, 3], [70, 0, 33], 16, 1, "fp8", seed=7, slots="tokens", extra_rows=9)
    base, _ = oracle.attn_prefix_extend_problem(p)
    rng = np.random.default_rng(1)
    perm = rng.permutation(p.num_rows)           # new row of old row r is perm[r]
    kb = np.empty_like(p.k_buffer)
    vb = np.empty_like(p.v_buffer)
    kb[perm] = p.k_buffer
    vb[perm] = p.v_buffer
    moved, _ = oracle.attn_prefix_extend(
        p.q, kb, vb, p.kv_indptr, perm[p.kv_indices].astype(np.int32), p.k_extend, p.v_extend,
        p.kv_dtype, p.cu_seqlens_q, p.num_kv_heads, p.scale)
    assert np.array_equal(moved, base)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_no_prefix_zero_q_is_running_mean_of_draft_values(dt):
    q_lens = [4, 2]
    p = vi.prefix_extend(q_lens, [0, 0], 8, 1, dt, seed=3, v_descale=0.75, poison=False)
    p.q[:] = 0
    out, _ = oracle.attn_prefix_extend_problem(p)
    dec = (np.vectorize(oracle.fp8_e4m3fn_to_float) if dt == "fp8"
           else np.vectorize(oracle.bf16_to_float))
    v = dec(p.v_extend[:, 0, :]).astype(np.float64)          # [total_q, D]
    hq = p.num_q_heads
    for b in range(2):
        c0 = int(p.cu_seqlens_q[b])
        for t in range(q_lens[b]):
            want = 0.75 * v[c0:c0 + t + 1].mean(axis=0)
            for h in range(hq):
                np.testing.assert_allclose(out[(c0 + t) * hq + h], want, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------- planted mistakes --

def _mutant_relayout(kind):
    """prefix_extend_to_paged with one planted mistake (test-only copy)."""
    def f(k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend, cu_seqlens_q, page_size=16):
        B = len(cu_seqlens_q) - 1
        hkv, d = k_buffer.shape[1], k_buffer.shape[2]
        seqs = []
        for b in range(B):
            pre = [int(kv_indices[j]) for j in range(kv_indptr[b], kv_indptr[b + 1])]
            ext = list(range(int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])))
            if kind == "drop_last_prefix" and pre:
                pre = pre[:-1]
            if kind == "shift_draft_rows":
                ext = [min(r + 1, len(k_extend) - 1) for r in ext]
            ks = [k_buffer[r] for r in pre] + [k_extend[r] for r in ext]
            vs = [v_buffer[r] for r in pre] + [v_extend[r] for r in ext]
            if kind == "draft_first":
                n = len(ext)
                ks = ks[len(pre):] + ks[:len(pre)]
                vs = vs[len(pre):] + vs[:len(pre)]
                assert n == len(ks) - len(pre)
            seqs.append((ks, vs))
        pages = [max(1, -(-len(ks) // page_size)) for ks, _ in seqs]
        k_pool = np.zeros((sum(pages), page_size, hkv, d), dtype=k_buffer.dtype)
        v_pool = np.zeros_like(k_pool)
        bt = np.zeros((B, max(pages)), dtype=np.int32)
        pg = 0
        lens = []
        for b, (ks, vs) in enumerate(seqs):
            for i in range(pages[b]):
                bt[b, i] = pg + i
            for i, (kk, vv) in enumerate(zip(ks, vs)):
                k_pool[pg + i // page_size, i % page_size] = kk
                v_pool[pg + i // page_size, i % page_size] = vv
            pg += pages[b]
            lens.append(len(ks))
        return k_pool, v_pool, bt, np.asarray(lens, dtype=np.int32)
    return f


def _pins_pass():
    try:
        for c in ROUND_TRIP_CASES[:2]:
            test_round_trip_equals_paged_oracle(c)
        test_prefix_rows_can_sit_anywhere()
        for dt in ("fp8", "bf16"):
            test_no_prefix_zero_q_is_running_mean_of_draft_values(dt)
    except AssertionError:
        return False
    return True


def test_pins_pass_with_the_real_relayout():
    assert _pins_pass()


@pytest.mark.parametrize("kind", ["draft_first", "shift_draft_rows", "drop_last_prefix"])
def test_planted_relayout_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "prefix_extend_to_paged", _mutant_relayout(kind))
    assert not _pins_pass()
