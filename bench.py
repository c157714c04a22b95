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
               launch time, measured with HIP events on the stream it runs on
               around a run of back-to-back launches, against the 8 TB/s peak.
  cpu_baseline the fp64 oracle, timed on this host's cores on a bounded
               sample of the same workload.

Inputs are resident in HBM before timing starts.  The KV pools rotate over
several copies, so the 256 MiB memory-side cache cannot serve a step from
the previous one.
"""
import argparse
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
MAIN_KERNEL = {"fp8": "va_split_kv_fp8_w8_kernel", "bf16": "va_split_kv_bf16_w8_kernel"}
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
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the first {n} of {pe.num_seqs} sequences (all their rows, re-layout included), "
                      f"{nbytes} algorithmic bytes in {secs:.2f} s"}


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
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(done_seqs)} of {p.num_seqs} sequences (all their rows), "
                      f"{nbytes} algorithmic bytes in {secs:.2f} s",
            "value_1_thread": round(nbytes1 / secs1 / 1e9, 4),
            "sample_1_thread": f"sequence {b1} (all its rows), {nbytes1} algorithmic bytes in {secs1:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps before timing")
    ap.add_argument("--warmup-seconds", type=float, default=3.0,
                    help="keep running untimed steps for at least this long (memory and core "
                         "clocks take about a second of sustained load to settle)")
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = the headline)")
    ap.add_argument("--variant", type=int, default=0, help="sweep variant of workload 4")
    ap.add_argument("--copies", type=int, default=4, help="KV pool copies to rotate over")
    ap.add_argument("--grid", type=int, default=0, help="force the split-KV grid (0 = plan)")
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

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the kernels run on a single device)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_gqa_attention_va_amd as va
    import va_inputs

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
    plan = (va.Plan.for_prefix_extend(pe, force_grid=args.grid) if pe is not None
            else va.Plan.for_problem(p, force_grid=args.grid))
    ws = plan.workspace(dev)
    out = torch.empty((q.shape[0], q.shape[1], plan.v_head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    log(f"bench: plan grid={plan.grid} workspace={plan.workspace_bytes} B, "
        f"{args.copies} pool copies of {2 * k0.numel() * k0.element_size() / 2**20:.0f} MiB")

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
    log(f"bench: {n_warm} warmup steps done in {time.perf_counter() - t_w:.1f} s")

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
        # The main kernel is timed in a run of its own launches.
        if stages == (va.VA_STAGE_SPLIT_KV,):
            main_ms = ms_step
        else:
            main_ms = timed(args.steps, n_warm, (va.VA_STAGE_SPLIT_KV,))
        achieved = alg / (main_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": load_traffic(workload),
                    "kernel": MLA_KERNEL if args.mla else MAIN_KERNEL[p.kv_dtype],
                    "us_per_launch": round(main_ms * 1e3, 3)}
        log(f"bench: main kernel {main_ms * 1e3:.2f} us/launch, {achieved:.1f} GB/s")

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
        "warmup": args.warmup,
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
                   "pool_copies": args.copies, "stage": args.stage},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
