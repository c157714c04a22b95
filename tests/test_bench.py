"""bench.py: the byte count behind `value` and `roofline.achieved`, checked
against closed forms on small hand-made shapes, and the output contract.

- Algorithmic bytes: every KV page a sequence references within seqused_k
  once (K and V, per kv head; a partial last page counts whole), plus the
  bf16 Q rows read and O rows written.  Absorbed MLA reads one 576-wide cache
  row per key (K and V share it).  A sliding window drops the pages below the
  first key any query row can see.
- One GPU only: --gpus N > 1 exits with status 2 before touching a device.
- On a GPU, one short run prints one JSON line with the documented keys.
"""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _shape(q_lens, kv_lens, hq=16, hkv=1, dt="fp8", head_dim=256, v_head_dim=None, window_left=-1):
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return SimpleNamespace(cu_seqlens_q=cu, seqused_k=np.asarray(kv_lens, dtype=np.int32),
                           num_seqs=len(q_lens), num_q_heads=hq, num_kv_heads=hkv, kv_dtype=dt,
                           head_dim=head_dim, v_head_dim=v_head_dim, page_size=16,
                           window_left=window_left)


def test_long_context_bytes():
    # 16 sequences x 2048 pages x 4 KiB, K and V; Q and O: 16 x 4 rows x 16 heads x 512 B each
    p = _shape([4] * 16, [32768] * 16)
    assert bench.algorithmic_bytes(p) == 16 * 2048 * 4096 * 2 + 2 * 16 * 4 * 16 * 512 == 269484032


def test_partial_pages_empty_queries_and_kv_heads():
    # 17 keys -> 2 pages; a sequence with no query rows reads nothing; 2 kv heads
    p = _shape([3, 0, 1], [17, 5000, 16], hq=8, hkv=2)
    kv = (2 + 1) * 2 * 16 * 256 * 2                    # pages x kv heads x page rows x 256 B x (K, V)
    qo = (3 + 1) * 8 * 256 * 2 * 2
    assert bench.algorithmic_bytes(p) == kv + qo


def test_bf16_doubles_the_cache_bytes():
    f8 = bench.algorithmic_bytes(_shape([2], [100]))
    b16 = bench.algorithmic_bytes(_shape([2], [100], dt="bf16"))
    qo = 2 * 16 * 256 * 2 * 2
    assert b16 - qo == 2 * (f8 - qo)


def test_window_drops_pages_below_the_first_visible_key():
    # lk 1000, lq 4, window 100: the first visible key is 1000 - 4 - 100 = 896 -> page 56 of 63
    p = _shape([4], [1000], window_left=100)
    assert bench.algorithmic_bytes(p) == (63 - 56) * 16 * 256 * 2 + 4 * 16 * 256 * 4


def test_mla_reads_one_row_per_key():
    p = _shape([4, 2], [300, 32], head_dim=576, v_head_dim=512)
    pages = 19 + 2
    assert bench.algorithmic_bytes(p) == pages * 16 * 576 + 6 * 16 * (576 + 512) * 2


def test_prefix_extend_counts_keys_not_pages():
    pe = SimpleNamespace(cu_seqlens_q=np.array([0, 4, 6], np.int32), kv_indptr=np.array([0, 17, 20], np.int32),
                         num_seqs=2, num_q_heads=16, num_kv_heads=1, head_dim=256, kv_dtype="fp8",
                         window_left=-1)
    keys = (17 + 4) + (3 + 2)
    assert bench.algorithmic_bytes_pe(pe) == keys * 256 * 2 + 6 * 16 * 256 * 4


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "0", "--steps", "3",
                        "--warmup", "1", "--warmup-seconds", "0", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["unit"] == "GB/s" and d["value"] > 0
    assert d["config"]["workload"] and d["config"]["algorithmic_bytes"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and 0 < rf["frac"] == pytest.approx(rf["achieved"] / 8000.0,
                                                                                             abs=1e-3)


def test_stamp_report_phases_and_low_32_bit_slots():
    # Two workgroups x four waves of a VA_STAMPS run: clock ticks of 10 ns.
    # Slots 4, 5 and 16..21 hold only the low 32 bits; the report rebuilds them
    # from the page-loop end (slot 6) and returns phase medians in us.
    grid, base = 2, (7 << 32) - 500                  # the low 32 bits wrap inside the call
    w = np.zeros((grid, 4, 32), dtype=np.int64)
    full = {0: 0, 1: 150, 2: 560, 3: 760, 4: 940, 5: 1250, 6: 4700, 7: 5200, 8: 5210}
    for k, v in full.items():
        w[:, :, k] = base + v
    w[:, :, 9] = 16                                  # steps of the first piece
    w[:, :, 10] = 1
    w[:, :, 12] = 1
    for k, v in ((16, 2000), (17, 2128), (18, 2136), (19, 2220)):
        w[:, :, k] = (base + v) & 0xFFFFFFFF
    w[:, :, 4] = (base + full[4]) & 0xFFFFFFFF
    w[:, :, 5] = (base + full[5]) & 0xFFFFFFFF
    w[:, :, 20] = 0xFFFFFF00                         # shader clock: 3960 cycles over 2.2 us
    w[:, :, 21] = (0xFFFFFF00 + 3960) & 0xFFFFFFFF
    rep = bench.stamp_report(w.reshape(-1), grid)
    assert rep["workgroups"] == grid
    assert rep["step0_landed"] == 9.4 and rep["step1_landed"] == 12.5
    assert rep["page_loop_done"] == 47.0 and rep["exit_last"] == 52.1
    assert rep["us_per_step_median"] == round((4700 - 940) / 15 / 100, 2)
    assert rep["mid_step_qk_softmax_us"] == 1.28 and rep["mid_step_v_wait_us"] == 0.08
    assert rep["mid_step_pv_us"] == 0.84 and rep["mid_step_us"] == 2.2
    assert rep["shader_clock_mhz"] == 1800.0
