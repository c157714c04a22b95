"""Planted mistakes in a copy of the oracle must be caught by the pins.

Each mutant is one plausible slip in a textual copy of oracle/va_oracle.c:
an off-by-one causal limit, a wrong GQA head mapping, the wrong fp8 bias, a
dropped descale, a flipped sign, a transposed pool index, and so on.  The copy
is compiled with gcc into a temporary directory.  The pins from
test_oracle_pins.py (dense brute force and codec) then have to reject it.  The
real oracle is never modified.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_features import FEATURE_CASES, dense_reference_ex
from test_oracle_pins import BRUTE_CASES, dec_fp8, dense_reference, rel_err, small_problem
import va_inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "va_oracle.c")

MUTANTS = {
    "causal_off_by_one": ("visible = Lk - Lq + t + 1;", "visible = Lk - Lq + t;"),
    "causal_top_left": ("visible = Lk - Lq + t + 1;", "visible = t + 1;"),
    "gqa_mapping": ("int g = h / G, d;", "int g = h % p->num_kv_heads, d;"),
    "fp8_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "fp8_subnormal": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "k_descale_dropped": ("p->scale * p->k_descale * dot", "p->scale * dot"),
    "v_descale_dropped": ("out[d] = p->v_descale * acc[d] / L;", "out[d] = acc[d] / L;"),
    "softmax_sign": ("double w = exp(logits[j] - m);", "double w = exp(m - logits[j]);"),
    "slot_index": ("int64_t slot = j % p->page_size;", "int64_t slot = (j + 1) % p->page_size;"),
    "pool_transposed": ("((page * p->page_size + slot) * p->num_kv_heads + g)",
                        "((page * p->num_kv_heads + g) * p->page_size + slot)"),
    "bf16_shift": ("uint32_t u = (uint32_t)x << 16;", "uint32_t u = (uint32_t)x << 15;"),
    "q_k_same_operand": ("va_oracle_bf16_to_double(qrow[d]) * kv_at(p, p->k_pool, base + d)",
                         "va_oracle_bf16_to_double(qrow[d]) * kv_at(p, p->v_pool, base + d)"),
    "lse_log_dropped": ("*lse = m + log(L);", "*lse = m;"),
    # optional features (sliding window, softcap, sinks)
    "feat_window_off_by_one": ("first = visible - 1 - p->window_left;", "first = visible - p->window_left;"),
    "feat_window_ignored": ("if (lo < first)\n                lo = first;", "if (0)\n                lo = first;"),
    "feat_softcap_unscaled": ("logits[j] = p->softcap * tanh(logits[j] / p->softcap);",
                              "logits[j] = tanh(logits[j] / p->softcap);"),
    "feat_sink_kv_head": ("sink = p->sinks[h];", "sink = p->sinks[g];"),
    "feat_sink_dropped": ("L = L * f + exp(sink - mm);", "L = L * f;"),
    "feat_sink_in_split_dropped": ("                denom += exp(sink - lse_max);", "                ;"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-D_DEFAULT_SOURCE", "-shared", "-fPIC",
                           str(c), "-o", str(so), "-lm", "-lpthread"])
    return oracle.load_library(str(so))


def _pins_pass(lib) -> bool:
    # codec pin
    got = np.array([lib.va_oracle_fp8e4m3fn_to_double(c) for c in range(256)])
    ref = dec_fp8(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(ref)
    if not (np.array_equal(np.isnan(got), ~fin) and np.array_equal(got[fin], ref[fin])):
        return False
    # dense brute-force pin, outputs and LSE
    for case in BRUTE_CASES:
        ql, kl, hq, hkv, d, dt, kd, vd = case
        p = small_problem(None, ql, kl, hq, hkv, d=d, kv_dtype=dt, kd=kd, vd=vd, seed=sum(kl) + hq)
        out, lse = oracle.attn_problem(p, threads=2, lib=lib)
        ref_out, ref_lse = dense_reference(p)
        if not np.all(np.isfinite(out)) or rel_err(out, ref_out) > 1e-12:
            return False
        if np.max(np.abs(lse - ref_lse)) > 1e-12 * max(1.0, np.max(np.abs(ref_lse))):
            return False
    return True


def _feature_pins_pass(lib) -> bool:
    """Dense brute force with window / softcap / sinks, unsplit and split."""
    for ql, kl, hq, hkv, dt, wl, cap, use_sinks in FEATURE_CASES:
        p = va_inputs.custom(ql, kl, hq, hkv, dt, seed=sum(kl) + hq)
        sinks = np.linspace(-1.5, 2.5, hq) if use_sinks else None
        ref_out, ref_lse = dense_reference_ex(p, wl, cap, sinks)
        for segs in (None, [[0] + list(range(7, k, 23)) for k in kl]):
            out, lse = oracle.attn(p.q, p.k, p.v, p.kv_dtype, p.block_table, p.cu_seqlens_q,
                                   p.seqused_k, p.num_kv_heads, p.scale, p.k_descale, p.v_descale,
                                   threads=2, lib=lib, window_left=wl, softcap=cap, sinks=sinks,
                                   segments=segs)
            if not np.all(np.isfinite(out)) or rel_err(out, ref_out) > 1e-12:
                return False
            if np.max(np.abs(lse - ref_lse)) > 1e-12 * max(1.0, np.max(np.abs(ref_lse))):
                return False
    return True


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "libclean.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-D_DEFAULT_SOURCE", "-shared", "-fPIC",
                           SRC, "-o", str(so), "-lm", "-lpthread"])
    lib = oracle.load_library(str(so))
    assert _pins_pass(lib) and _feature_pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    assert not (_pins_pass(lib) and _feature_pins_pass(lib)), f"pins failed to catch mutant {name}"
