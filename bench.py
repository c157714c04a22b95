#!/usr/bin/env python3
"""Benchmark of the verify-attention hot path on one MI355X.

One step is one va_run over one batch of synthetic input: the split-KV main
kernel and then the segment-reduce kernel.  The default workload is the
long-context batch: 16 sequences x 4 verify tokens, 32768 KV tokens each,
16 query heads per kv head, head_dim 256, FP8 e4m3 KV in 16-token pages with a
random block table.  It is the one the metric is quoted on: 16:1 GQA, FP8 KV,
32K+ context.

  value        effective HBM GB/s over the whole step, computed from the
               algorithmic bytes.  Those are the unique KV pages within
               seqused_k (K and V) plus the Q and O bytes.
  roofline     the main kernel: the same algorithmic bytes over its average
               duration inside the timed whole calls, against the 8 TB/s
               peak.  The duration comes from HIP events that the main
               kernel's own dispatch records (va_run_timed) on the stream it
               runs on, in every one of the timed steps.
  cpu_baseline the fp64 oracle, timed on this host's cores on a bounded
               sample of the same workload.

Inputs are resident in HBM before timing starts.  The KV pools rotate over
several copies, so the 256 MiB memory-side cache cannot serve a step from
the previous one.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0                 # dense MFMA, MI355X
PEAK_FP8_TFLOPS = 5000.0
def main_kernel(kv_dtype: str, plan_kernel: int) -> str:
    """Name of the split-KV kernel a plan launches (plan_kernel as va_plan_kernel
    reports it: 1 or 2 for paged FP8 GQA, 0 otherwise)."""
    if kv_dtype == "bf16":
        return "va_split_kv_bf16_w8_kernel"
    return "va_split_kv_fp8_w4_kernel" if plan_kernel == 1 else "va_split_kv_fp8_w8_kernel"

MLA_KERNEL = "va_mla_split_kernel"
# Arithmetic of the path: FP8 KV runs QK^T on fp8 MFMA (Q as an exact hi/lo fp8
# pair) and PV on bf16 MFMA; bf16 KV runs both on bf16 MFMA; fp32 accumulation.
COMPUTE_DTYPE = {"fp8": "fp8/bf16", "bf16": "bf16"}


def algorithmic_bytes(p, seqs=None) -> int:
    """Unique KV pages referenced within seqused_k (K and V, each page once per
    kv head) plus Q and O bytes, optionally restricted to some sequences.  With
    a sliding window only the pages some query row can see count."""
    elt = 1 if p.kv_dtype == "fp8" else 2
    idx = np.arange(p.num_seqs) if seqs is None else np.asarray(seqs)
    wl = getattr(p, "window_left", -1)
    dv = getattr(p, "v_head_dim", None)
    pages = 0
    rows = 0
    for b in idx:
        lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        lk = int(p.seqused_k[b])
        if lq > 0:
            first = 0 if wl < 0 else max(0, lk - lq - wl) // p.page_size
            pages += -(-lk // p.page_size) - first
            rows += lq
    if dv:                                 # absorbed MLA: one cache row serves K and V
        kv = pages * p.page_size * p.head_dim * elt
        qo = rows * p.num_q_heads * (p.head_dim + dv) * 2
        return int(kv + qo)
    kv = pages * p.num_kv_heads * p.page_size * p.head_dim * elt * 2
    qo = rows * p.num_q_heads * p.head_dim * 2 * 2
    return int(kv + qo)


def algorithmic_bytes_pe(pe, seqs=None) -> int:
    """The same count for a prefix + extend call: every key row some query row
    can see (prefix rows gathered by slot and draft rows, K and V, per kv head)
    plus Q and O bytes.  There are no pages, so no partial-page rounding."""
    elt = 1 if pe.kv_dtype == "fp8" else 2
    idx = np.arange(pe.num_seqs) if seqs is None else np.asarray(seqs)
    wl = getattr(pe, "window_left", -1)
    keys = rows = 0
    for b in idx:
        lq = int(pe.cu_seqlens_q[b + 1] - pe.cu_seqlens_q[b])
        lk = int(pe.kv_indptr[b + 1] - pe.kv_indptr[b]) + lq
        if lq > 0:
            keys += lk - (0 if wl < 0 else max(0, lk - lq - wl))
            rows += lq
    kv = keys * pe.num_kv_heads * pe.head_dim * elt * 2
    qo = rows * pe.num_q_heads * pe.head_dim * 2 * 2
    return int(kv + qo)


def pe_head(pe, n):
    """The first n sequences of a prefix + extend problem (slices of its metadata;
    the row buffers are shared)."""
    import dataclasses
    e = int(pe.kv_indptr[n])
    c = int(pe.cu_seqlens_q[n])
    return dataclasses.replace(pe, q=pe.q[:c], k_extend=pe.k_extend[:c], v_extend=pe.v_extend[:c],
                               kv_indptr=pe.kv_indptr[:n + 1].copy(), kv_indices=pe.kv_indices[:e].copy(),
                               cu_seqlens_q=pe.cu_seqlens_q[:n + 1].copy())


def source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "paged_gqa_attention_va_amd", "csrc", "va.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_launch")


def host_cpu():
    """CPU model and core counts of this host (for the cpu_baseline record)."""
    model, phys = None, set()
    try:
        cur = {}
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k in ("physical id", "core id"):
                    cur[k] = v
                elif not k and cur:
                    phys.add((cur.get("physical id"), cur.get("core id")))
                    cur = {}
            if cur:
                phys.add((cur.get("physical id"), cur.get("core id")))
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(phys) or None, "logical_cpus_available": avail}


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the library torch already loaded),
    for va_run_timed, whose main-kernel dispatch records them itself."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.ev = []


def stamp_report(st: np.ndarray, grid: int) -> dict:
    """Phase times (us, from the earliest kernel entry) of one traced call, from the
    per-wave timestamps of a VA_STAMPS library (32 words per wave, see va.h)."""
    w = st.reshape(grid, 4, 32).astype(np.int64)
    live = w[:, 0, 1] > 0                                  # workgroups that found work
    if not live.any():                                     # the kernel that ran records no stamps
        return None
    w = w[live].copy()
    # slots 4, 5 and 16..19 hold the low 32 bits of the 100 MHz clock (taken
    # inside the page loop); the full value is the page-loop end (slot 6, full)
    # minus the 32-bit distance back to it
    for k in (4, 5, 16, 17, 18, 19):
        w[:, :, k] = w[:, :, 6] - ((w[:, :, 6] - w[:, :, k]) & 0xFFFFFFFF)
    t0 = w[:, :, 0].min()
    us = lambda x: (x - t0) / 100.0                        # 100 MHz clock -> us
    med = lambda a: round(float(np.median(a)), 2)
    first = w[:, :, 6] > 0
    steps = w[:, :, 9]
    per_step = (w[:, :, 6] - w[:, :, 4]) / np.maximum(steps - 1, 1) / 100.0
    rep = {"workgroups": int(live.sum()),
           "entry": med(us(w[:, :, 0])),
           "located": med(us(w[:, :, 1])),
           "q_landed": med(us(w[:, :, 2][first])),
           "q_operands_loaded": med(us(w[:, :, 3][first])),
           "step0_landed": med(us(w[:, :, 4][first])),
           "step1_landed": med(us(w[:, :, 5][first])),
           "page_loop_done": med(us(w[:, :, 6][first])),
           "epilogue_states_out": med(us(w[:, :, 13][first])),
           "epilogue_o_published": med(us(w[:, :, 14][first])),
           "epilogue_all_published": med(us(w[:, :, 15][first])),
           "epilogue_done": med(us(w[:, :, 7][first])),
           "exit_median": med(us(w[:, :, 8])),
           "exit_last": round(float(us(w[:, :, 8]).max()), 2),
           "steps_first_piece_median": int(np.median(steps[first])),
           "us_per_step_median": med(per_step[first & (steps > 1)]),
           "pieces_max": int(w[:, :, 10].max()),
           "second_passes": int((w[:, :, 12] > 1).sum())}
    # the middle step of the first piece: its phases and the shader clock
    mid = first & (steps >= 2)
    if mid.any():
        ph = lambda a, b: med((w[:, :, b] - w[:, :, a])[mid] / 100.0)
        span = (w[:, :, 19] - w[:, :, 16])[mid] / 100.0             # us, K landed .. PV done
        cyc = ((w[:, :, 21] - w[:, :, 20]) & 0xFFFFFFFF)[mid]
        rep.update({"mid_step_us": med(span), "mid_step_qk_softmax_us": ph(16, 17),
                    "mid_step_v_wait_us": ph(17, 18), "mid_step_pv_us": ph(18, 19),
                    "shader_clock_mhz": round(float(np.median(cyc / np.maximum(span, 1e-3))), 0)})
    return rep


def cpu_baseline_pe(pe, budget_s: float = 12.0):
    """Time the oracle on the first sequences of a prefix + extend call, one
    more sequence per round, until about budget_s of work."""
    import oracle
    threads = oracle.default_threads()
    n, secs = 0, 0.0
    while n < pe.num_seqs and secs < budget_s:
        n += 1
        sub = pe_head(pe, n)
        t0 = time.perf_counter()
        oracle.attn_prefix_extend_problem(sub, threads=threads)
        secs = time.perf_counter() - t0
    nbytes = algorithmic_bytes_pe(pe, range(n))
    rec = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the first {n} of {pe.num_seqs} sequences (all their rows, re-layout included), "
                     f"{nbytes} algorithmic bytes in {secs:.2f} s"}
    rec.update(host_cpu())
    return rec


def cpu_baseline(p, budget_s: float = 12.0):
    """Time the oracle on whole sequences of p until about budget_s of work."""
    import oracle
    threads = oracle.default_threads()
    G = p.num_q_heads
    done_seqs, secs = [], 0.0
    for b in range(p.num_seqs):
        q0, q1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        rows = np.arange(q0 * G, q1 * G, dtype=np.int64)
        if len(rows) == 0:
            continue
        t0 = time.perf_counter()
        run = oracle.attn_mla_problem if getattr(p, "v_head_dim", None) else oracle.attn_problem
        run(p, rows=rows, threads=threads)
        secs += time.perf_counter() - t0
        done_seqs.append(b)
        if secs >= budget_s:
            break
    nbytes = algorithmic_bytes(p, done_seqs)
    if not done_seqs:
        return None
    # the same oracle on one thread, over the first sequence with query rows
    b1 = done_seqs[0]
    rows1 = np.arange(int(p.cu_seqlens_q[b1]) * G, int(p.cu_seqlens_q[b1 + 1]) * G, dtype=np.int64)
    t0 = time.perf_counter()
    run(p, rows=rows1, threads=1)
    secs1 = time.perf_counter() - t0
    nbytes1 = algorithmic_bytes(p, [b1])
    rec = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{len(done_seqs)} of {p.num_seqs} sequences (all their rows), "
                     f"{nbytes} algorithmic bytes in {secs:.2f} s",
           "value_1_thread": round(nbytes1 / secs1 / 1e9, 4),
           "sample_1_thread": f"sequence {b1} (all its rows), {nbytes1} algorithmic bytes in {secs1:.2f} s"}
    rec.update(host_cpu())
    return rec


def mfma_bound(p, main_ms):
    """The matrix-core bound of the main kernel: the MFMA work it executes
    (every key of every streamed page against every row of the 16-row tiles),
    at MI355X's dense peaks.  QK^T on an FP8 cache runs as two fp8 MFMAs per
    product (Q split into exact e4m3 hi and lo parts, 5.0 PFLOP/s); on a bf16
    cache as bf16 MFMAs (2.5 PFLOP/s); PV always in bf16.  frac is the time at
    those peaks over the measured main-kernel time (1 = bound by MFMA)."""
    qk_w = p.head_dim
    pv_w = getattr(p, "v_head_dim", None) or p.head_dim
    g = p.num_q_heads // p.num_kv_heads
    qk_fl = pv_fl = 0
    for b in range(p.num_seqs):
        lq, lk = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b]), int(p.seqused_k[b])
        if lq <= 0 or lk <= 0:
            continue
        rows = -(-lq * g // 16) * 16                      # rows in 16-row MFMA tiles
        keys = -(-lk // p.page_size) * p.page_size        # every key of the streamed pages
        qk_fl += 2 * rows * keys * qk_w * p.num_kv_heads
        pv_fl += 2 * rows * keys * pv_w * p.num_kv_heads
    fp8 = p.kv_dtype == "fp8"
    t_qk = qk_fl * (2 if fp8 else 1) / ((PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS) * 1e12)
    t_pv = pv_fl / (PEAK_BF16_TFLOPS * 1e12)
    return {"qk_flops": qk_fl, "pv_flops": pv_fl, "qk_mfma": "fp8 hi + lo" if fp8 else "bf16",
            "pv_mfma": "bf16", "us_at_peak": round((t_qk + t_pv) * 1e6, 3),
            "frac": round((t_qk + t_pv) / (main_ms * 1e-3), 4)}


def ceiling(args):
    """Streaming ceiling of the copy path alone: va_stream_pages over the
    long-context workload's bytes (2 x 32768 pages of 4 KiB = 268 MB per
    launch), pages in a seeded random order, four disjoint page sets of a
    1 GiB pool so that no launch finds the previous one's data in a cache.
    One line of JSON per ring depth."""
    import torch
    import paged_gqa_attention_va_amd as va
    dev = torch.device("cuda:0")
    n_pool = 1 << 18                                      # 4 KiB pages: 1 GiB
    n_launch = 2 * 32768                                  # K and V pages of the long-context workload
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    pool = torch.randint(0, 256, (n_pool * 4096,), dtype=torch.uint8, generator=g).to(dev)
    order = torch.randperm(n_pool, generator=g).to(torch.int32)
    sets = [order[i * n_launch:(i + 1) * n_launch].contiguous().to(dev) for i in range(4)]
    grid = torch.cuda.get_device_properties(dev).multi_processor_count
    sums = torch.zeros(grid * 4, dtype=torch.int32, device=dev)
    for depth in (2, 4, 6, 8, 10):
        t_w = time.perf_counter()
        i = 0
        while time.perf_counter() - t_w < args.warmup_seconds or i < 20:
            va.stream_pages(pool, sets[i % 4], depth, grid, sums)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for j in range(args.steps):
            va.stream_pages(pool, sets[j % 4], depth, grid, sums)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.steps
        gbps = n_launch * 4096 / (us * 1e-6) / 1e9
        print(json.dumps({"ceiling": "va_stream_pages", "depth_pages_per_wave": depth, "grid": grid,
                          "bytes_per_launch": n_launch * 4096, "launches": args.steps,
                          "us_per_launch": round(us, 3), "GBps": round(gbps, 1),
                          "pct_of_8TBps": round(100.0 * gbps / PEAK_HBM_GBPS, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls (default 200; 2000 for a workload under 64 MB, whose call is launch-bound)")
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps before timing")
    ap.add_argument("--warmup-seconds", type=float, default=3.0,
                    help="keep running untimed steps for at least this long (memory and core "
                         "clocks take about a second of sustained load to settle)")
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = the headline)")
    ap.add_argument("--variant", type=int, default=0, help="sweep variant of workload 4")
    ap.add_argument("--copies", type=int, default=4, help="KV pool copies to rotate over")
    ap.add_argument("--grid", type=int, default=0, help="force the split-KV grid (0 = plan)")
    ap.add_argument("--kernel", type=int, default=0, choices=[0, 1, 2],
                    help="paged FP8 GQA split-KV kernel: 0 = plan's choice, 1 = one wave per SIMD, "
                         "2 = two row groups")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, default=-1,
                    help="sliding window size (keys a query sees, itself included; -1 = none)")
    ap.add_argument("--softcap", type=float, default=0.0, help="logit softcap (0 = none)")
    ap.add_argument("--sinks", action="store_true", help="add one sink logit per query head")
    ap.add_argument("--draft-extend", action="store_true",
                    help="draft-extend call: each step first builds the block table and seqused_k "
                         "from kv_indptr / kv_indices on the device (va_spec_block_table)")
    ap.add_argument("--prefix-extend", choices=["tokens", "pages"], default=None,
                    help="prefix + extend layout (va_run_prefix_extend): the same lengths with the "
                         "prefix in a token-row buffer (slots one per token, or 16-row pages) and "
                         "the draft tokens' K/V in separate buffers")
    ap.add_argument("--mla", choices=["fp8", "bf16"], default=None,
                    help="absorbed-MLA call of the same batch shape: 576-wide cache rows "
                         "(512 latent + 64 RoPE), one kv head, the workload's query heads")
    ap.add_argument("--stage", choices=["all", "split", "merge"], default="all",
                    help="profiling aid: time only one kernel per step")
    ap.add_argument("--stamps", action="store_true",
                    help="load the VA_STAMPS build (libva_stamps.so) and report the main kernel's "
                         "per-phase times of one call after the timed steps")
    ap.add_argument("--stamps-out", default=None, metavar="NPY",
                    help="with --stamps: also save the raw per-wave timestamps (.npy)")
    ap.add_argument("--warm", action="store_true",
                    help="warm-cache run: one copy of the KV pools, so steps may find the previous "
                         "step's data in the memory-side cache (the default rotates 4 copies)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the streaming ceiling of the FP8 kernel's copy path "
                         "(va_stream_pages): the long-context workload's 268 MB of 4 KiB pages, "
                         "random order, from a 1 GiB pool rotated over four page sets, no compute")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}), flush=True)
        return

    if args.ceiling:
        if args.steps is None:
            args.steps = 200
        ceiling(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the kernels run on a single device)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_gqa_attention_va_amd as va
    import va_inputs

    if args.warm:
        args.copies = 1
    if args.stamps:                       # the diagnostic build replaces the library
        from paged_gqa_attention_va_amd import _build as va_build
        if not os.path.exists(va_build.LIB_STAMPS):
            raise RuntimeError(f"{va_build.LIB_STAMPS} is not built (paged_gqa_attention_va_amd._build)")
        va._lib = va.library(va_build.LIB_STAMPS)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    p = va_inputs.config(args.config, args.variant)
    workload = va_inputs.CONFIG_NAMES[args.config] if args.config != 4 else p.name
    if args.mla:
        q_lens = np.diff(p.cu_seqlens_q)
        p = va_inputs.mla(q_lens, p.seqused_k, p.num_q_heads // p.num_kv_heads, args.mla,
                          seed=200 + args.config, k_descale=p.k_descale, v_descale=p.v_descale,
                          name=p.name + "-mla")
        workload = (f"absorbed MLA {p.num_seqs} seqs q{int(p.max_seqlen_q)} kv{int(p.max_seqlen_k)} "
                    f"{p.num_q_heads}q/1kv 512+64 {args.mla}")
    features = []
    if args.window > 0:
        p.window_left = args.window - 1
        features.append(f"window {args.window}")
    if args.softcap > 0:
        p.softcap = float(np.float32(args.softcap))
        features.append(f"softcap {args.softcap:g}")
    if args.sinks:
        p.sinks = np.linspace(-1.0, 1.0, p.num_q_heads).astype(np.float32)
        features.append("sinks")
    if args.draft_extend:
        features.append("draft-extend metadata")
    pe = None
    if args.mla and (args.prefix_extend or args.draft_extend or features):
        ap.error("--mla runs the paged causal call without window, softcap, sinks or other layouts")
    if args.prefix_extend:
        if args.draft_extend:
            ap.error("--prefix-extend and --draft-extend are different layouts")
        q_lens = np.diff(p.cu_seqlens_q)
        pe = va_inputs.prefix_extend(q_lens, p.seqused_k - q_lens, p.num_q_heads, p.num_kv_heads,
                                     p.kv_dtype, seed=100 + args.config, slots=args.prefix_extend,
                                     k_descale=p.k_descale, v_descale=p.v_descale,
                                     window_left=p.window_left, softcap=p.softcap, sinks=p.sinks,
                                     name=p.name + "-prefix-extend")
        features.append(f"prefix + extend layout ({args.prefix_extend} slots)")
    if features:
        workload += " + " + ", ".join(features)
    log(f"bench: generated {p.name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(dev)

    def kv(a):
        t = torch.from_numpy(a)
        if p.kv_dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    if pe is not None:                    # rotate over copies of the row buffers instead
        k0, v0 = kv(pe.k_buffer), kv(pe.v_buffer)
        ke, ve = kv(pe.k_extend), kv(pe.v_extend)
        pe_indptr = torch.from_numpy(pe.kv_indptr).to(dev)
        pe_indices = torch.from_numpy(pe.kv_indices).to(dev)
    else:
        k0, v0 = kv(p.k), kv(p.v)
    ks = [k0] + [k0.clone() for _ in range(args.copies - 1)]
    vs = ks if getattr(p, "v_head_dim", None) else [v0] + [v0.clone() for _ in range(args.copies - 1)]
    bt = torch.from_numpy(p.block_table).to(dev)
    cu = torch.from_numpy(p.cu_seqlens_q).to(dev)
    sk = torch.from_numpy(p.seqused_k).to(dev)
    kd = torch.tensor([p.k_descale], dtype=torch.float32, device=dev)
    vd = torch.tensor([p.v_descale], dtype=torch.float32, device=dev)
    sinks = None if p.sinks is None else torch.from_numpy(p.sinks).to(dev)
    if args.draft_extend:                 # every KV token's pool slot, sequence by sequence
        indptr = np.zeros(p.num_seqs + 1, dtype=np.int32)
        slots = []
        for b in range(p.num_seqs):
            n = int(p.seqused_k[b])
            indptr[b + 1] = indptr[b] + n
            j = np.arange(n)
            slots.append(p.block_table[b, j // p.page_size].astype(np.int64) * p.page_size + j % p.page_size)
        kv_indptr = torch.from_numpy(indptr).to(dev)
        kv_indices = torch.from_numpy(np.concatenate(slots).astype(np.int32)).to(dev)
    make_plan = ((lambda: va.Plan.for_prefix_extend(pe, force_grid=args.grid)) if pe is not None
                 else (lambda: va.Plan.for_problem(p, force_grid=args.grid, kernel=args.kernel)))
    plan = make_plan()
    t_plan = []
    for _ in range(50):                   # host cost of a plan (once per shape, never per call)
        t0 = time.perf_counter()
        make_plan()
        t_plan.append(time.perf_counter() - t0)
    plan_us = round(float(np.median(t_plan)) * 1e6, 1)
    ws = plan.workspace(dev)
    out = torch.empty((q.shape[0], q.shape[1], plan.v_head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    log(f"bench: plan grid={plan.grid} workspace={plan.workspace_bytes} B, "
        f"{args.copies} pool copies of {2 * k0.numel() * k0.element_size() / 2**20:.0f} MiB")

    if args.steps is None:
        alg0 = algorithmic_bytes_pe(pe) if pe is not None else algorithmic_bytes(p)
        args.steps = 2000 if alg0 < (64 << 20) else 200
    stages = {"all": (va.VA_STAGE_SPLIT_KV, va.VA_STAGE_MERGE), "split": (va.VA_STAGE_SPLIT_KV,),
              "merge": (va.VA_STAGE_MERGE,)}[args.stage]

    def step(i, stage_list=stages):
        c = i % args.copies
        bt_i, sk_i = bt, sk
        if args.draft_extend:
            bt_i, sk_i = va.spec_block_table(kv_indptr, kv_indices, p.block_table.shape[1],
                                             p.page_size, stream=stream)
        for s in stage_list:
            if pe is not None:
                plan.run_prefix_extend(q, ks[c], vs[c], pe_indptr, pe_indices, ke, ve, cu, p.scale, kd, vd,
                                       out=out, workspace=ws, stream=stream, stage=s, sinks=sinks)
            else:
                plan.run(q, ks[c], vs[c], bt_i, cu, sk_i, p.scale, kd, vd, out=out, workspace=ws,
                         stream=stream, stage=s, sinks=sinks)

    def step_timed(i, ev_a, ev_b):
        """One whole call whose main-kernel dispatch records ev_a / ev_b."""
        c = i % args.copies
        bt_i, sk_i = bt, sk
        if args.draft_extend:
            bt_i, sk_i = va.spec_block_table(kv_indptr, kv_indices, p.block_table.shape[1],
                                             p.page_size, stream=stream)
        plan.run_timed(q, ks[c], vs[c], bt_i, cu, sk_i, p.scale, kd, vd, out, ws, stream, ev_a, ev_b,
                       sinks=sinks)

    def timed(n, first, stage_list=stages):
        """Average ms per step over n back-to-back steps, HIP events on `stream`
        recorded only around the whole run (no per-step synchronisation)."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            step(first + i, stage_list)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    if args.stage == "merge":      # the merge reads what a split pass left in the workspace
        step(0, (va.VA_STAGE_SPLIT_KV,))
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step(n_warm)
        n_warm += 1
        if n_warm % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    log(f"bench: {n_warm} warmup steps done in {warm_s:.1f} s")

    ms_step = timed(args.steps, n_warm)
    alg = algorithmic_bytes_pe(pe) if pe is not None else algorithmic_bytes(p)
    value = alg / (ms_step * 1e-3) / 1e9
    log(f"bench: {args.steps} steps, {ms_step * 1e3:.2f} us/step, {value:.1f} GB/s effective")

    # Spread of single calls: events around every call of a back-to-back run
    # (a pass of its own; value above comes from the undisturbed run).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (ea, eb) in enumerate(ev):
        ea.record(stream)
        step(n_warm + args.steps + i)
        eb.record(stream)
    torch.cuda.synchronize()
    per_call = np.array([ea.elapsed_time(eb) * 1e3 for ea, eb in ev])
    spread = {"p10": round(float(np.percentile(per_call, 10)), 3),
              "median": round(float(np.median(per_call)), 3),
              "p90": round(float(np.percentile(per_call, 90)), 3),
              "method": "HIP events around each call, back to back"}

    roofline = None
    if va.VA_STAGE_SPLIT_KV in stages:
        # Main-only launches back to back: a labelled extra, not the roofline.
        main_only_ms = ms_step if stages == (va.VA_STAGE_SPLIT_KV,) else \
            timed(args.steps, n_warm, (va.VA_STAGE_SPLIT_KV,))
        main_ms, ms_step_ev = None, None
        if args.stage == "all" and pe is None:
            # The roofline time: the main kernel inside whole calls, from events its
            # own dispatch records in every one of a second run of timed steps.
            evs = HipEvents(2 * args.steps)
            a = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for i in range(args.steps):
                step_timed(n_warm + i, evs.ev[2 * i], evs.ev[2 * i + 1])
            e.record(stream)
            torch.cuda.synchronize()
            ms_step_ev = a.elapsed_time(e) / args.steps
            durs = [evs.elapsed_ms(evs.ev[2 * i], evs.ev[2 * i + 1]) for i in range(args.steps)]
            evs.close()
            main_ms = float(np.mean(durs))
            log(f"bench: main kernel inside whole calls {main_ms * 1e3:.2f} us (whole calls of that run "
                f"{ms_step_ev * 1e3:.2f} us); main-only launches {main_only_ms * 1e3:.2f} us")
        else:
            main_ms = main_only_ms
            log(f"bench: main kernel {main_ms * 1e3:.2f} us/launch (main-only launches)")
        achieved = alg / (main_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": load_traffic(workload),
                    "kernel": MLA_KERNEL if args.mla else main_kernel((pe if pe is not None else p).kv_dtype, plan.kernel),
                    "us_per_launch": round(main_ms * 1e3, 3),
                    "timing": ("events recorded by the main kernel's own dispatch, in every step of a "
                               "run of timed whole calls" if ms_step_ev is not None
                               else "back-to-back main-kernel launches"),
                    "us_per_call_of_that_run": None if ms_step_ev is None else round(ms_step_ev * 1e3, 3),
                    "us_per_launch_main_only": round(main_only_ms * 1e3, 3)}
        if pe is None:
            roofline["mfma_bound"] = mfma_bound(p, main_ms)

    stamps = None
    if args.stamps and pe is None:
        # every call of a back-to-back run overwrites the buffer: it ends up holding
        # the last call, in steady state
        buf = torch.zeros(plan.grid * 4 * 32, dtype=torch.int64, device=dev)
        va.set_stamp_buffer(buf)
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(n_warm + 3 * args.steps + i)
        torch.cuda.synchronize()
        va.set_stamp_buffer(None)
        raw = buf.cpu().numpy()
        stamps = stamp_report(raw, plan.grid)
        log(f"bench: phase stamps (last of {args.steps} back-to-back calls) {stamps}")
        if args.stamps_out:
            np.save(args.stamps_out, raw)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_pe(pe) if pe is not None else cpu_baseline(p)
        log(f"bench: cpu baseline {cpu}")

    rec = {
        "metric": "verify-attn effective HBM GB/s (% of peak) and us/call at 16:1 GQA, FP8 KV",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "warmup_seconds": round(warm_s, 2),
        "ms_per_step": round(ms_step, 6),
        "us_per_call": round(ms_step * 1e3, 3),
        "us_per_call_spread": spread,
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": COMPUTE_DTYPE[p.kv_dtype],
        "data": "synthetic",
        "config": {"workload": workload,
                   "num_seqs": p.num_seqs, "q_len": int(p.max_seqlen_q),
                   "kv_len_max": int(p.max_seqlen_k), "q_heads": p.num_q_heads,
                   "kv_heads": p.num_kv_heads, "head_dim": p.head_dim, "page": p.page_size,
                   "kv_dtype": p.kv_dtype, "algorithmic_bytes": alg, "grid": plan.grid,
                   "pool_copies": args.copies, "cache": "warm" if args.warm else "cold",
                   "stage": args.stage},
        "plan_host_us": plan_us,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if stamps is not None:
        rec["stamps"] = stamps
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
