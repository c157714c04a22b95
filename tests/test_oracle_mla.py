"""Pins of the oracle's absorbed-MLA attention (oracle.attn_mla), the PE_DIM
split of the sglang PR #34517 summary page: logits q_nope.k_nope + q_pe.k_pe,
value = the latent part of the key row.

Pinned against things other than its own code path:
  - with q_pe = 0 it equals the plain oracle on the 512-wide latent alone with
    V = K (another head width, another V);
  - with q_nope = 0 it equals the plain oracle on rows whose latent is zeroed
    for the keys and whose RoPE part is zeroed for the values;
  - permuting the latent dims of Q and of the cache permutes the output dims the
    same way; permuting the RoPE dims changes nothing;
  - one visible key: the output is that key's latent times v_descale;
  - a constant added to one RoPE dim of every key shifts all logits of a row
    equally and changes nothing, while flipping q_pe changes the result;
  - planted mistakes (value from the wrong dims, RoPE part left out of the
    logits or entering with the wrong sign) each fail one of these pins.
"""
import numpy as np
import pytest

import oracle
import va_inputs as vi

L, R = vi.MLA_LATENT, vi.MLA_ROPE


def _mla(dt="fp8", q_lens=(4, 2, 1), kv_lens=(70, 33, 16), hq=8, seed=1, **kw):
    return vi.mla(list(q_lens), list(kv_lens), hq, dt, seed=seed, k_descale=0.9, v_descale=1.2, **kw)


def _run(p, q=None, k=None):
    return oracle.attn_mla(p.q if q is None else q, p.k if k is None else k, p.kv_dtype, p.block_table,
                           p.cu_seqlens_q, p.seqused_k, p.scale, p.v_head_dim, p.k_descale, p.v_descale)[0]


def _plain(p, q, k, v):
    return oracle.attn(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v), p.kv_dtype,
                       p.block_table, p.cu_seqlens_q, p.seqused_k, 1, p.scale, p.k_descale, p.v_descale)[0]


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_no_rope_query_equals_plain_oracle_on_latent(dt):
    p = _mla(dt)
    q = p.q.copy()
    q[..., L:] = 0
    lat = p.k[..., :L]
    assert np.array_equal(_run(p, q=q), _plain(p, q[..., :L], lat, lat))


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_no_latent_query_equals_plain_oracle_on_split_rows(dt):
    p = _mla(dt, seed=2)
    q = p.q.copy()
    q[..., :L] = 0
    k = p.k.copy()
    k[..., :L] = 0                      # keys: RoPE part only
    v = p.k.copy()
    v[..., L:] = 0                      # values: latent only
    assert np.array_equal(_run(p, q=q), _plain(p, q, k, v)[:, :L])


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_dim_permutations(dt):
    p = _mla(dt, seed=4)
    base = _run(p)
    rng = np.random.default_rng(0)
    pl = rng.permutation(L)
    perm = np.concatenate([pl, np.arange(L, L + R)])
    moved = _run(p, q=np.ascontiguousarray(p.q[..., perm]), k=np.ascontiguousarray(p.k[..., perm]))
    assert np.array_equal(moved, base[:, pl])
    perm2 = np.concatenate([np.arange(L), L + rng.permutation(R)])
    moved2 = _run(p, q=np.ascontiguousarray(p.q[..., perm2]), k=np.ascontiguousarray(p.k[..., perm2]))
    np.testing.assert_allclose(moved2, base, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_single_visible_key_gives_its_latent(dt):
    p = _mla(dt, q_lens=(1, 1), kv_lens=(1, 1), poison=False)
    out = _run(p)
    dec = np.vectorize(oracle.fp8_e4m3fn_to_float if dt == "fp8" else oracle.bf16_to_float)
    hq = p.num_q_heads
    for b in range(2):
        lat = dec(p.k[p.block_table[b, 0], 0, 0, :L]).astype(np.float64)
        for h in range(hq):
            np.testing.assert_allclose(out[b * hq + h], p.v_descale * lat, rtol=1e-12, atol=0)


def test_rope_part_enters_the_logits():
    p = _mla("bf16", seed=6, poison=False)
    q = p.q.copy()
    q[..., L:] = 0
    q[..., L] = 0x3F80                  # q_pe = e_0 (1.0)
    k1 = p.k.copy()
    k1[..., L] = 0x3F80                 # every key's first RoPE dim = 1.0: all logits + 1
    k2 = p.k.copy()
    k2[..., L] = 0x4000                 # = 2.0: all logits + 2
    np.testing.assert_allclose(_run(p, q=q, k=k1), _run(p, q=q, k=k2), rtol=1e-12, atol=1e-14)
    qn = q.copy()
    qn[..., L] = 0xBF80                 # q_pe = -e_0 on the original cache
    assert not np.allclose(_run(p, q=qn), _run(p, q=q), rtol=1e-6, atol=1e-9)


# ------------------------------------------------------- planted mistakes --

def _mutant(kind):
    """attn_mla with one planted mistake (test-only copy)."""
    def f(q, kv_pool, kv_dtype, bt, cu, sk, scale, v_head_dim, kd=1.0, vd=1.0, **kw):
        q = np.array(q)
        k = np.array(kv_pool)
        v = k.copy()
        v[..., v_head_dim:] = 0
        if kind == "value_from_shifted_dims":
            v = np.zeros_like(k)
            v[..., :v_head_dim] = k[..., 1:v_head_dim + 1]
        elif kind == "rope_dropped":
            q[..., v_head_dim:] = 0
        elif kind == "rope_sign":
            k = k.copy()
            if kv_dtype == "fp8":
                k[..., v_head_dim:] ^= 0x80
            else:
                k[..., v_head_dim:] ^= 0x8000
        out, lse = oracle.attn(q, k, v, kv_dtype, bt, cu, sk, 1, scale, kd, vd, **kw)
        return out[:, :v_head_dim], lse
    return f


def _pins_pass():
    try:
        for dt in ("fp8", "bf16"):
            test_no_rope_query_equals_plain_oracle_on_latent(dt)
            test_no_latent_query_equals_plain_oracle_on_split_rows(dt)
            test_dim_permutations(dt)
            test_single_visible_key_gives_its_latent(dt)
        test_rope_part_enters_the_logits()
    except AssertionError:
        return False
    return True


def test_pins_pass_with_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("kind", ["value_from_shifted_dims", "rope_dropped", "rope_sign"])
def test_planted_mla_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "attn_mla", _mutant(kind))
    assert not _pins_pass()
