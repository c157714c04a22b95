"""Stored fixtures under tests/golden/.

- page_verify_case.json holds the test case printed on the sglang PR #36330
  summary page ("Key source snippets": _check_matches_aiter and its two
  callers): its shapes, lengths, descales, scale and assert_close tolerance.
  The named tiny workloads must be exactly that case, and the GPU tests'
  element bar must be that tolerance.
- config0_oracle_digest.txt is written by tests/golden/make_oracle_digest.py,
  which calls only the oracle and the seeded input generator.  It is a
  regression pin: a later change to the oracle's arithmetic shows up here.
"""
import importlib.util
import json
import math
import os

import numpy as np

import va_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _case():
    with open(os.path.join(GOLDEN, "page_verify_case.json")) as f:
        return json.load(f)


def test_tiny_workloads_are_the_page_test_case():
    c = _case()
    ql, kl, d, page = c["query_lens"], c["kv_lens"], c["head_size"], c["block_size"]
    mbps = math.ceil(max(kl) / page)
    for i, (hq, hkv) in enumerate(c["head_configs"]):
        p = va_inputs.config(i)
        assert p.num_q_heads == hq and p.num_kv_heads == hkv
        assert list(p.q_lens) == ql and list(p.seqused_k) == kl
        assert list(p.cu_seqlens_q) == [0] + list(np.cumsum(ql))
        assert p.q.shape == (sum(ql), hq, d) and p.k.shape[1:] == (page, hkv, d)
        assert p.kv_dtype == "fp8"
        assert p.scale == np.float32(d ** -0.5)
        assert p.k_descale == c["k_descale"] and p.v_descale == c["v_descale"]
        # arange(num_blocks).view(num_seqs, mbps), over the pages each sequence uses
        assert p.block_table.shape == (len(ql), mbps)
        full = np.arange(len(ql) * mbps).reshape(len(ql), mbps)
        for b, n in enumerate(kl):
            used = math.ceil(n / page)
            assert np.array_equal(p.block_table[b, :used], full[b, :used])


def test_gpu_element_bar_is_the_page_tolerance():
    import gpu_util
    c = _case()
    assert gpu_util.ATOL == c["atol"] and gpu_util.RTOL == c["rtol"]


def test_oracle_matches_its_stored_digest():
    spec = importlib.util.spec_from_file_location("make_oracle_digest",
                                                  os.path.join(GOLDEN, "make_oracle_digest.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    now = [ln for ln in mod.digest_lines() if not ln.startswith("#")]
    with open(os.path.join(GOLDEN, "config0_oracle_digest.txt")) as f:
        stored = [ln for ln in f.read().splitlines() if ln and not ln.startswith("#")]
    assert len(now) == len(stored) == 6 * 16
    a = np.array([[float(x) for x in ln.split()] for ln in now])
    b = np.array([[float(x) for x in ln.split()] for ln in stored])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
