#!/usr/bin/env python3
"""Benchmark of the fused MaxSim hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

Prints ONE JSON line.  A step is one pass of the hot path over one batch of
seeded synthetic input already resident in HBM.  With no --workload the line
is the ColPali-scale forward (the largest configuration that fits one GPU),
and its "configs" object holds every configuration measured in the same run:
  colbert_tiny:  1 query x 32 tokens against 1,000 documents of 180 tokens,
      fp16, scores + argmax (maxsim_fwd_varlen);
  colbert_rerank_varlen: 64 queries x 32 tokens against a 10,000 document
      corpus, lengths uniform in [32, 300], packed by cu_seqlens, fp16, scores;
  colbert_rerank_padded: the same corpus padded to 300 tokens with d_lens
      (maxsim_fwd), for the packed-vs-padded speedup;
  colpali_fwd:   4 queries x 10,000 documents, Lq = Ld = 1024, bf16, scores +
      argmax (the headline);
  contrastive_train: 64 x 64 in-batch pairs, Lq = Ld = 1024, bf16: forward
      with argmax, InfoNCE gradient (tau = 0.02), backward (CSR, dD, dQ);
  int8_varlen:   32 queries x 32 tokens against 100,000 int8 documents,
      lengths uniform in [32, 512], scores (maxsim_fwd_i8).
--workload NAME prints that workload's own line instead (also
contrastive_train_varlen, two_stage_topk, ooc_colpali, chamfer_100k,
chamfer_batch).  `value` is the algorithmic TFLOP/s (TOP/s for int8) of the
step: 2*Nq*Lq*d per (query, document token) pair, real tokens only.  The
roofline object reports the dominant kernel against MI355X's published dense
peaks, timed with HIP events on the stream it is launched on; the CPU
baseline is the oracle timed on the host's cores on a bounded sample of the
same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MaxSim fwd/bwd TFLOP/s + doc-tokens/s; % of MFMA or HBM roofline; peak mem"
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0}  # dense, MI355X
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "fwd": ["late_interaction_retrieval_amd/csrc/fwd.hip"],
    "bwd": ["late_interaction_retrieval_amd/csrc/bwd.hip"],
}
HEADLINE = "colpali_fwd"
ALL_CONFIGS = ["colbert_tiny", "colbert_rerank_varlen", "colbert_rerank_padded", "colpali_fwd",
               "contrastive_train", "int8_varlen"]
FWD_WORKLOADS = ALL_CONFIGS + ["contrastive_train_varlen"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all",
                    choices=["all"] + FWD_WORKLOADS + ["two_stage_topk", "ooc_colpali", "chamfer_100k",
                                                       "chamfer_batch"])
    ap.add_argument("--argmax", choices=["auto", "on", "off"], default="auto",
                    help="save the argmax in inference workloads (auto: as the workload specifies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained", action="store_true", help="no effect (accepted for older command lines)")
    ap.add_argument("--no-graph", action="store_true",
                    help="tiny workload: time eager launches instead of HIP-graph replays")
    ap.add_argument("--bwd-dispatch-sweep", action="store_true",
                    help="instead of the workload, time the CSR and the atomic-scatter backward over a grid "
                         "of contention levels (sources per dD row) and print one JSON line per shape")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="target oracle time of each CPU baseline (default 10 s for one workload; with all "
                         "configurations 8 s for the headline and 4 s for each other one)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the workload, run 5 device-to-device copies of MIB MiB: the counter "
                         "reading of a copy of known size scales the rocprofv3 byte counters")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "reads_per_copy": n, "writes_per_copy": n}), flush=True)


PROBE_KIND = {"f16": 0, "bf16": 1, "i8": 2}


def fwd_kernel_name(Nq, Lq, el, packed, argmax):
    """The forward kernel the library launches for this shape (its dispatch
    rule): a single 32-row query block runs one workgroup per document;
    32-token queries over a packed corpus without argmax run the kernel that
    tiles across document boundaries; everything else the slab kernel."""
    if Nq * Lq <= 32 and el != "i8":
        return "fwd_tiny_kernel"
    if packed and not argmax and Lq == 32 and el != "i8":
        return "fwd_flat_kernel"
    return "fwd_kernel"


def source_sha(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def auto_counts(est, args, target_s=0.5):
    """Timed steps K and warmup W: the command line's, else about target_s
    seconds of GPU work (at least 10 steps)."""
    steps = args.steps if args.steps is not None else int(min(2000, max(10, target_s / est)))
    warmup = args.warmup if args.warmup is not None else int(min(50, max(3, 0.1 / est)))
    return steps, warmup


def run_workload(name, args, cpu_seconds, want_argmax=None):
    """Time one forward (or training) workload; returns its JSON object.

    Inputs are generated on the host, copied to HBM once, and stay resident;
    the timed region holds only library calls (plus the InfoNCE gradient in
    torch for the training step).  The dominant kernel is timed with HIP
    events on the launch stream around every timed launch."""
    import torch
    from late_interaction_retrieval_amd import binding as bd
    from late_interaction_retrieval_amd import inputs

    dev = torch.device("cuda:0")
    padded = name == "colbert_rerank_padded"
    w = inputs.make("colbert_rerank_varlen" if padded else name)
    Nq, Lq, B, d, T = w["Nq"], w["Lq"], w["B"], w["d"], w["T"]
    dtn = w["dtype"]
    if want_argmax is None:
        want_argmax = {"colbert_rerank_varlen": False, "colbert_rerank_padded": False, "colbert_tiny": True,
                       "colpali_fwd": True, "contrastive_train": True, "int8_varlen": False,
                       "contrastive_train_varlen": True}[name]
    train = name.startswith("contrastive_train")

    def dev_t(a, bf16=False):
        a = np.ascontiguousarray(a)
        if bf16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    isbf = dtn == inputs.BF16
    Q = dev_t(w["Q"], isbf)
    cu = dev_t(w["cu_seqlens"])
    lens_d = dev_t(w["lens"])
    max_ld = int(w["lens"].max())
    pair_flops = 2.0 * Nq * Lq * d  # per real document token
    fwd_flops = pair_flops * T
    extra = {}
    stream = torch.cuda.current_stream(dev)

    # D copies: the small tiny workload fits the 256 MB MALL, so it rotates
    # 12 copies (>= 550 MB) between steps to time HBM, not the cache.
    ncopies = 12 if name == "colbert_tiny" else 1
    if name == "int8_varlen":
        Ds = [dev_t(w["D_packed"]) for _ in range(ncopies)]
        q_scale = dev_t(w["q_scale"])
        d_scale = dev_t(w["d_scale"])
    elif name == "contrastive_train":
        Ds = [dev_t(w["D_packed"].reshape(B, w["Ld_max"], d), isbf)]
    elif padded:
        Ds = [dev_t(inputs.pad_packed(w["D_packed"], w["cu_seqlens"], w["Ld_max"]), isbf)]
    else:
        Ds = [dev_t(w["D_packed"], isbf) for _ in range(ncopies)]

    scores = torch.empty((Nq, B), dtype=torch.float32, device=dev)
    amax = torch.empty((Nq, B, Lq), dtype=torch.int32, device=dev) if want_argmax else None
    ev_pool = []

    if train:
        Dd = Ds[0]
        Ld = w["Ld_max"]
        rows = B * Ld if name == "contrastive_train" else T
        if name == "contrastive_train":
            ws = torch.empty(max(16, bd.maxsim_bwd_workspace_bytes(Nq, B, Lq, Ld)), dtype=torch.uint8, device=dev)
        else:
            ws = torch.empty(max(256, bd.maxsim_bwd_varlen_workspace_bytes(Nq, B, Lq, max_ld)), dtype=torch.uint8,
                             device=dev)
        dQ = torch.empty((Nq, Lq, d), dtype=torch.float32, device=dev)
        dD = torch.empty((rows, d), dtype=torch.float32, device=dev)
        rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        ci = torch.empty(Nq * B * Lq, dtype=torch.int32, device=dev)
        tau = w["tau"]
        eye = torch.eye(Nq, device=dev, dtype=torch.float32)

        def step(i, timed):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
            if timed:
                ev[0].record(stream)
            if name == "contrastive_train":
                bd.maxsim_fwd(Q, Dd, scores=scores, argmax=amax)
            else:
                bd.maxsim_fwd_varlen(Q, Dd, cu, max_ld, scores=scores, argmax=amax)
            if timed:
                ev[1].record(stream)
            # InfoNCE over scores / tau with the diagonal as positives (harness, torch)
            p = torch.softmax(scores / tau, dim=1)
            g = ((p - eye) / (tau * Nq)).contiguous()
            if timed:
                ev[2].record(stream)
            if name == "contrastive_train":
                bd.maxsim_bwd(Q, Dd, amax, g, dQ=dQ, dD=dD.view(B, Ld, d), row_ptr=rp, col_idx=ci, workspace=ws)
            else:
                bd.maxsim_bwd_varlen(Q, Dd, cu, max_ld, amax, g, dQ=dQ, dD=dD, row_ptr=rp, col_idx=ci,
                                     workspace=ws)
            if timed:
                ev[3].record(stream)
                ev_pool.append(ev)

        bwd_flops = 4.0 * d * Nq * B * Lq
        step_flops = fwd_flops + bwd_flops
    elif name == "int8_varlen":
        def step(i, timed):
            Dc = Ds[i % ncopies]
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            bd.maxsim_fwd_i8(Q, q_scale, Dc, d_scale, cu, max_ld, scores=scores, argmax=amax,
                             with_argmax=want_argmax)
            if timed:
                e1.record(stream)
                ev_pool.append((e0, e1))

        step_flops = fwd_flops
    elif padded:
        def step(i, timed):
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            bd.maxsim_fwd(Q, Ds[0], lens_d, scores=scores, argmax=amax, with_argmax=want_argmax)
            if timed:
                e1.record(stream)
                ev_pool.append((e0, e1))

        step_flops = fwd_flops
    else:
        def step(i, timed):
            Dc = Ds[i % ncopies]
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            bd.maxsim_fwd_varlen(Q, Dc, cu, max_ld, scores=scores, argmax=amax, with_argmax=want_argmax)
            if timed:
                e1.record(stream)
                ev_pool.append((e0, e1))

        step_flops = fwd_flops

    # The tiny workload's kernel (about 10 microseconds) is shorter than the
    # host time to launch it, so eager launches leave the GPU idle between
    # them and events around one launch time the launch latency too.  There a
    # HIP graph holds one launch per D copy and is replayed; a launch's
    # duration is the replay's event time divided by the launches in it.
    graph = None
    graph_ms = []
    if name == "colbert_tiny" and not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        for i in range(ncopies):  # warm the allocator and the code object outside capture
            step(i, False)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(ncopies):
                step(i, False)
        torch.cuda.synchronize()

        def step_graph(i, timed):
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            graph.replay()
            if timed:
                e1.record(stream)
                graph_ms.append((e0, e1))

    for i in range(3):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(0, False)
    torch.cuda.synchronize()
    est = max(1e-5, time.perf_counter() - t0)
    steps, warmup = auto_counts(est, args)
    if graph is not None:  # whole replays only: K becomes a multiple of the launches per replay
        steps = max(ncopies, (steps + ncopies - 1) // ncopies * ncopies)
        warmup = max(ncopies, (warmup + ncopies - 1) // ncopies * ncopies)
    for i in range(warmup if graph is None else warmup // ncopies):
        (step if graph is None else step_graph)(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is None:
        for i in range(steps):
            step(i, True)
    else:
        for i in range(steps // ncopies):
            step_graph(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_mem = torch.cuda.max_memory_allocated(dev)

    kernel_ms, bwd_ms = [], []
    for ev in ev_pool:
        kernel_ms.append(ev[0].elapsed_time(ev[1]))
        if len(ev) == 4:
            bwd_ms.append(ev[2].elapsed_time(ev[3]))
    if graph is not None:
        kernel_ms = [e0.elapsed_time(e1) / ncopies for e0, e1 in graph_ms]
    k_avg_ms = float(np.mean(kernel_ms))
    k_med_ms = float(np.median(kernel_ms))
    ms_per_step = elapsed * 1e3 / steps
    value = step_flops * steps / elapsed / 1e12

    # roofline of the dominant kernel: the forward
    el = {"f16": "f16", "bf16": "bf16", "i8": "i8"}[dtn]
    peak = MFMA_PEAK_TFLOPS[el]
    achieved = fwd_flops / (k_avg_ms * 1e-3) / 1e12
    rowb = 128 if el == "i8" else 256
    fwd_bytes = T * rowb + Nq * Lq * rowb + 4 * (B + 1) + 4 * Nq * B
    if el == "i8":
        fwd_bytes += 4 * T + 4 * Nq * Lq
    if want_argmax:
        fwd_bytes += 4 * Nq * B * Lq
    traffic = read_traffic("fwd", name)
    hbm_gbs = fwd_bytes / (k_avg_ms * 1e-3) / 1e9
    # the binding roof: arithmetic intensity against the ridge point peak / HBM
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if fwd_flops / fwd_bytes >= ridge:
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TOP/s" if el == "i8" else "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    roofline.update({"traffic": traffic,
                     "kernel": fwd_kernel_name(Nq, Lq, el, not (padded or name == "contrastive_train"), want_argmax),
                     "kernel_avg_ms": round(k_avg_ms, 5),
                     "kernel_median_ms": round(k_med_ms, 5), "algorithmic_flops_per_launch": fwd_flops,
                     "algorithmic_bytes_per_launch": fwd_bytes, "arithmetic_intensity": round(fwd_flops / fwd_bytes, 1),
                     "mfma_frac": round(achieved / peak, 4), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4)})
    if padded:
        roofline["executed_flops_per_launch"] = pair_flops * B * w["Ld_max"]
    if bwd_ms:
        b_avg = float(np.mean(bwd_ms))
        rows = T if name == "contrastive_train_varlen" else B * w["Ld_max"]
        # argmax read, Q and D read (bf16), dQ and dD written (fp32), col_idx written
        # and read back, row_ptr, upstream gradient
        bwd_bytes = (4 * Nq * B * Lq + 2 * d * (Nq * Lq + rows) + 4 * d * (Nq * Lq + rows)
                     + 2 * 4 * Nq * B * Lq + 4 * (rows + 1) + 4 * Nq * B)
        # What actually moves: every source gathers one Q row (for dD) and one D row
        # (for dQ), 2 * d bytes each, from L2 or the memory-side cache.
        gathered = 2 * (2 * d) * Nq * B * Lq
        extra["bwd"] = {"avg_ms": round(b_avg, 5), "algorithmic_bytes": bwd_bytes,
                        "hbm_gbs": round(bwd_bytes / (b_avg * 1e-3) / 1e9, 1),
                        "hbm_frac": round(bwd_bytes / (b_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "bound": "hbm", "timed": "HIP events around the backward's launches",
                        "row_gather_bytes": gathered,
                        "row_gather_gbs": round(gathered / (b_avg * 1e-3) / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline and cpu_seconds > 0:
        cpu = cpu_baseline(w, cpu_seconds, padded=padded)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOP/s" if el == "i8" else "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": el,
        "data": "synthetic (seeded N(0,1) rows, l2-normalised; stands in for ColBERT/ColPali embeddings)",
        "config": {"workload": name, "Nq": Nq, "Lq": Lq, "B": B, "T_doc_tokens": T, "d": d,
                   "Ld_range": [int(w["lens"].min()), int(w["lens"].max())], "argmax_saved": want_argmax,
                   "layout": "padded" if (padded or name == "contrastive_train") else "cu_seqlens",
                   "launch": "hip_graph_replay_of_%d" % ncopies if graph is not None else "eager",
                   "d_copies_rotated": ncopies},
        "doc_tokens_per_s": round(T * steps / elapsed, 1),
        "query_doc_token_pairs_per_s": round(Nq * T * steps / elapsed, 1),
        "peak_mem_bytes": int(peak_mem),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if extra:
        out["extra"] = extra
    del Ds, Q, scores, amax
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def summary(o):
    """The per-configuration entry of the headline line."""
    r = o["roofline"]
    s = {"workload": o["config"]["workload"], "kernel": r["kernel"], "kernel_avg_ms": r["kernel_avg_ms"],
         "value": o["value"], "unit": o["unit"], "dtype": o["dtype"], "bound": r["bound"], "frac": r["frac"],
         "mfma_frac": r["mfma_frac"], "hbm_frac": r["hbm_frac"], "traffic": r["traffic"],
         "doc_tokens_per_s": o["doc_tokens_per_s"], "peak_mem_bytes": o["peak_mem_bytes"], "steps": o["steps"],
         "ms_per_step": o["ms_per_step"], "config": o["config"], "cpu_baseline": o["cpu_baseline"]}
    if "extra" in o:
        s.update(o["extra"])
    return s


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this benchmark measures one GPU only (one process, one MI355X); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    wall0 = time.perf_counter()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    if args.bwd_dispatch_sweep:
        bwd_dispatch_sweep()
        return
    if args.workload == "two_stage_topk":
        bench_two_stage(args)
        return
    if args.workload == "ooc_colpali":
        bench_ooc(args)
        return
    if args.workload.startswith("chamfer"):
        bench_chamfer(args)
        return

    lib_path = os.path.join(ROOT, "late_interaction_retrieval_amd", "libmaxsim.so")
    if not os.path.exists(lib_path):
        from late_interaction_retrieval_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    want = None if args.argmax == "auto" else args.argmax == "on"
    if args.workload != "all":
        out = run_workload(args.workload, args, 10.0 if args.cpu_seconds is None else args.cpu_seconds, want)
        print(json.dumps(out), flush=True)
        return

    # every configuration, the headline last so nothing runs after its timing
    cpu_other = 4.0 if args.cpu_seconds is None else args.cpu_seconds
    cpu_head = 8.0 if args.cpu_seconds is None else args.cpu_seconds
    configs = {}
    for name in ALL_CONFIGS:
        if name == HEADLINE:
            continue
        # the padded comparison repeats the packed workload's arithmetic: its CPU
        # baseline is the packed one's
        o = run_workload(name, args, 0.0 if name == "colbert_rerank_padded" else cpu_other)
        configs[name] = summary(o)
        print("bench: %s %.4f ms (%s %.3f of the %s roof)" % (name, o["roofline"]["kernel_avg_ms"],
              o["unit"], o["roofline"]["frac"], o["roofline"]["bound"]), file=sys.stderr, flush=True)
    pk, pd = configs["colbert_rerank_varlen"], configs["colbert_rerank_padded"]
    pd["speedup_packed_vs_padded"] = round(pd["kernel_avg_ms"] / pk["kernel_avg_ms"], 4)
    pd["fill_ratio"] = round(pk["config"]["T_doc_tokens"] / (pk["config"]["B"] * pk["config"]["Ld_range"][1]), 4)
    pd["cpu_baseline"] = "the oracle's work is that of colbert_rerank_varlen"
    out = run_workload(HEADLINE, args, cpu_head, want)
    configs[HEADLINE] = summary(out)
    out["configs"] = configs
    out["bench_wall_s"] = round(time.perf_counter() - wall0, 1)
    print(json.dumps(out), flush=True)


def bwd_dispatch_sweep(reps=20):
    """CSR backward (maxsim_bwd) against the atomic-scatter backward
    (maxsim_bwd_scatter) on padded fp16 documents, seeded uniform argmax and
    upstream gradient, over shapes whose mean number of sources per dD row
    (Nq*Lq/Ld) spans 0.03 .. 64.  Each time is the mean of `reps` launches
    between HIP events on the launch stream, after one warm-up call."""
    import torch
    from late_interaction_retrieval_amd import binding as bd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    shapes = [(nq, 32, 1000, 180) for nq in (1, 2, 4, 8, 16, 32, 64)]
    shapes += [(nq, 32, 64, 1024) for nq in (1, 8, 32)]
    shapes += [(nq, 1024, 64, 1024) for nq in (1, 4, 16, 64)]
    for Nq, Lq, B, Ld in shapes:
        Q = torch.randn((Nq, Lq, 128), device=dev, generator=gen).to(torch.float16)
        D = torch.randn((B, Ld, 128), device=dev, generator=gen).to(torch.float16)
        A = torch.randint(0, Ld, (Nq, B, Lq), device=dev, generator=gen, dtype=torch.int32)
        g = torch.randn((Nq, B), device=dev, generator=gen)
        dQ = torch.empty((Nq, Lq, 128), device=dev)
        dD = torch.empty((B, Ld, 128), device=dev)
        rp = torch.empty(B * Ld + 1, dtype=torch.int32, device=dev)
        ci = torch.empty(Nq * B * Lq, dtype=torch.int32, device=dev)
        ws = torch.empty(max(16, bd.maxsim_bwd_workspace_bytes(Nq, B, Lq, Ld)), dtype=torch.uint8, device=dev)
        runs = {"csr": lambda: bd.maxsim_bwd(Q, D, A, g, dQ=dQ, dD=dD, row_ptr=rp, col_idx=ci, workspace=ws),
                "scatter": lambda: bd.maxsim_bwd_scatter(Q, D, A, g, dQ=dQ, dD=dD)}
        ms = {}
        for k, fn in runs.items():
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms[k] = e0.elapsed_time(e1) / reps
        per_row = Nq * Lq / Ld
        print(json.dumps({"Nq": Nq, "Lq": Lq, "B": B, "Ld": Ld, "sources_per_row": round(per_row, 4),
                          "csr_ms": round(ms["csr"], 4), "scatter_ms": round(ms["scatter"], 4),
                          "faster": min(ms, key=ms.get),
                          "rule_picks": "scatter" if bd.maxsim_bwd_prefer_scatter(Nq, Lq, B, B * Ld) else "csr"}),
              flush=True)
        del Q, D, A, g, dQ, dD, rp, ci, ws


# Vector ALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# lane-instructions per second (packed fp32 instructions are not used).
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
FP32_VALU_PEAK_TFLOPS = 2 * VALU_LANE_OPS / 1e12  # FMA = 2 flop: 78.6
CHAMFER_VALU_PER_PAIR = 9  # 3 sub, 1 mul, 2 fma, 1 compare, 2 select (inner loop of nn_kernel)
CHAMFER_FLOP_PER_PAIR = 8  # 3 sub, 3 mul, 2 add


def bench_chamfer(args):
    """Chamfer distance (a next step beyond the hot path): forward (nearest
    neighbours both ways, saved indices) and backward (two CSR maps and the
    gradient rows) of the page's loss on two noisy unit-sphere clouds.  A step
    is one forward + backward.  The forward is bound by the vector ALU: the
    roofline counts its inner-loop VALU instructions per point pair against
    the chip's issue rate."""
    import torch
    from late_interaction_retrieval_amd import binding as bd
    from late_interaction_retrieval_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.make_chamfer(args.workload)
    Bt, N, M = w["Bt"], w["N"], w["M"]
    P = torch.from_numpy(w["P"]).to(dev)
    Q = torch.from_numpy(w["Q"]).to(dev)
    gp = torch.full((Bt, N), 1.0 / N, dtype=torch.float32, device=dev)
    gq = torch.full((Bt, M), 1.0 / M, dtype=torch.float32, device=dev)
    wsf = torch.empty(max(256, bd.lib().maxsim_chamfer_fwd_workspace_bytes(Bt, N, M)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(256, bd.lib().maxsim_chamfer_bwd_workspace_bytes(Bt, N, M)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    pool = []

    def step(timed):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            ev[0].record(stream)
        dp, ip, dq, iq = bd.maxsim_chamfer_fwd(P, Q, workspace=wsf)
        if timed:
            ev[1].record(stream)
        bd.maxsim_chamfer_bwd(P, Q, ip, iq, gp, gq, workspace=wsb)
        if timed:
            ev[2].record(stream)
            pool.append(ev)

    steps = args.steps if args.steps is not None else (20 if N >= 50000 else 200)
    warmup = args.warmup if args.warmup is not None else 3
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_mem = torch.cuda.max_memory_allocated(dev)
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pool]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in pool]))
    pairs = 2.0 * Bt * N * M  # both directions
    flops = CHAMFER_FLOP_PER_PAIR * pairs
    valu = CHAMFER_VALU_PER_PAIR * pairs / (fwd_ms * 1e-3)
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    roofline = {"bound": "alu", "achieved": round(achieved, 2), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP32_VALU_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "nn_kernel (both directions, with the chunk merge)", "kernel_avg_ms": round(fwd_ms, 4),
                "flop_per_pair": CHAMFER_FLOP_PER_PAIR, "valu_instr_per_pair": CHAMFER_VALU_PER_PAIR,
                "valu_lane_instr_per_s_implied": round(valu, 1),
                "valu_lane_instr_per_s_at_2p4ghz": VALU_LANE_OPS,
                "peak_note": "fp32 vector rate without packed instructions (which this library does not emit): "
                             "256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz = 78.6 TFLOP/s, half the "
                             "published 157.3 that counts packed fp32",
                "bwd_ms": round(bwd_ms, 4)}
    cpu = None
    cpu_s = 10.0 if args.cpu_seconds is None else args.cpu_seconds
    if not args.no_cpu_baseline:
        import oracle
        n = 64
        while True:
            t1 = time.perf_counter()
            oracle.chamfer_nn(w["P"][:, :n], w["Q"])
            tc = time.perf_counter() - t1
            if tc > 0.5 * cpu_s or n >= N:
                break
            n = int(min(N, n * max(2.0, 0.8 * cpu_s / max(tc, 1e-3))))
        cpu = {"value": round(CHAMFER_FLOP_PER_PAIR * Bt * n * M / tc / 1e12, 6), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "nearest neighbours of the first %d points of P in all of Q (per item), %.1f s" % (n, tc),
               "pairs_per_s": round(Bt * n * M / tc, 1)}
    out = {
        "metric": METRIC, "value": round(flops * steps / elapsed / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(elapsed * 1e3 / steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded noisy samples of the unit sphere, sigma 0.01)",
        "config": {"workload": args.workload, "Bt": Bt, "N": N, "M": M, "loss": "mean dist_p + mean dist_q"},
        "point_pairs_per_s": round(pairs * steps / elapsed, 1),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "peak_mem_bytes": int(peak_mem),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


PCIE5_X16_GBS = 64.0  # PCIe 5.0 x16, one direction, published (32 GT/s x 16 lanes, 128b/130b)


def bench_ooc(args, B=40960, block_docs=4096, chunk=2048):
    """Out-of-core scoring (a next step beyond the hot path): one ColPali query
    (Lq = Ld = 1024, bf16) against a corpus of B documents held in pinned host
    memory and streamed to the GPU in blocks of block_docs documents through
    two device buffers (maxsim_fwd_host_stream).  A step scores the whole
    corpus.  The host corpus repeats a seeded chunk of `chunk` documents
    (values do not change the copy or the arithmetic).  The bound is the
    host-to-device link: the roofline compares the corpus bytes per step with
    PCIe 5.0 x16 and with a plain pinned host-to-device copy measured here."""
    import torch
    from late_interaction_retrieval_amd import binding as bd
    from late_interaction_retrieval_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.make("colpali_fwd", Nq=1, B=chunk)
    Nq, Lq, d, Ld = w["Nq"], w["Lq"], w["d"], w["Ld_max"]
    doc_bytes = Ld * d * 2
    host = torch.empty((B, Ld, d), dtype=torch.bfloat16, pin_memory=True)
    src = torch.from_numpy(w["D_packed"].view(np.int16)).view(torch.bfloat16).reshape(chunk, Ld, d)
    for b0 in range(0, B, chunk):
        n = min(chunk, B - b0)
        host[b0:b0 + n].copy_(src[:n])
    Q = torch.from_numpy(w["Q"].view(np.int16)).view(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    staging = torch.empty(bd.maxsim_fwd_host_stream_staging_bytes(Nq, Lq, Ld, block_docs, False),
                          dtype=torch.uint8, device=dev)
    scores = torch.empty((Nq, B), dtype=torch.float32, device=dev)

    def step(pool):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bd.maxsim_fwd_host_stream(Q, host, block_docs, scores=scores, staging=staging)
        e1.record(stream)
        pool.append((e0, e1))

    steps = args.steps if args.steps is not None else 5
    warmup = args.warmup if args.warmup is not None else 1
    for _ in range(warmup):
        step([])
    torch.cuda.synchronize()
    pool = []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(pool)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_mem = torch.cuda.max_memory_allocated(dev)
    pass_ms = float(np.mean([a.elapsed_time(b) for a, b in pool]))
    # a plain pinned host-to-device copy of one block, on the same stream
    dst = torch.empty((block_docs, Ld, d), dtype=torch.bfloat16, device=dev)
    cp = []
    for i in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(host[(i % (B // block_docs)) * block_docs:][:block_docs], non_blocking=True)
        e1.record(stream)
        cp.append((e0, e1))
    torch.cuda.synchronize()
    copy_gbs = block_docs * doc_bytes / (float(np.mean([a.elapsed_time(b) for a, b in cp[1:]])) * 1e-3) / 1e9
    # the forward alone on one resident block (what the stream hides behind the copies)
    s_blk = torch.empty((Nq, block_docs), dtype=torch.float32, device=dev)
    fw = []
    for i in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bd.maxsim_fwd(Q, dst, scores=s_blk, with_argmax=False)
        e1.record(stream)
        fw.append((e0, e1))
    torch.cuda.synchronize()
    fwd_block_ms = float(np.mean([a.elapsed_time(b) for a, b in fw[1:]]))
    flops = 2.0 * Nq * Lq * d * Ld * B
    h2d_gbs = B * doc_bytes / (pass_ms * 1e-3) / 1e9
    roofline = {"bound": "pcie", "achieved": round(h2d_gbs, 2), "peak": PCIE5_X16_GBS, "unit": "GB/s",
                "frac": round(h2d_gbs / PCIE5_X16_GBS, 4), "traffic": None,
                "kernel": "host-to-device block copies (maxsim_fwd_host_stream)", "pass_event_ms": round(pass_ms, 3),
                "algorithmic_bytes_per_pass": B * doc_bytes,
                "pinned_copy_gbs": round(copy_gbs, 2), "frac_of_pinned_copy": round(h2d_gbs / copy_gbs, 4),
                "pinned_copy_kind": "plain pinned host-to-device copy of one block, same stream",
                "fwd_ms_per_block_resident": round(fwd_block_ms, 3)}
    cpu = None
    cpu_s = 10.0 if args.cpu_seconds is None else args.cpu_seconds
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cpu_s)
    out = {
        "metric": METRIC, "value": round(flops * steps / elapsed / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(elapsed * 1e3 / steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rows, l2-normalised; a %d-document seeded chunk repeated to %d documents "
                "in pinned host memory)" % (chunk, B),
        "config": {"workload": "ooc_colpali", "Nq": Nq, "Lq": Lq, "B": B, "Ld": Ld, "d": d,
                   "block_docs": block_docs, "corpus_bytes_host": B * doc_bytes, "layout": "padded, host-resident"},
        "docs_per_s": round(B * steps / elapsed, 1),
        "doc_tokens_per_s": round(B * Ld * steps / elapsed, 1),
        "h2d_gbs": round(h2d_gbs, 2),
        "peak_mem_bytes": int(peak_mem),
        "pages_context": "52K documents/s on A100-80GB in 20K-document blocks (other hardware)",
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_two_stage(args, B=30000, K1=100, K2=10):
    """The two-stage scan (a next step beyond the hot path): 32 ColBERT-length
    queries against an INT8 corpus shaped like the int8 workload (B documents of
    32..512 tokens), each query's K1 best re-scored in fp16, K2 kept.  A step is
    one maxsim_two_stage_topk call.  The roofline is that of its INT8 stage
    (timed alone on the same data)."""
    import torch
    from late_interaction_retrieval_amd import binding as bd
    from late_interaction_retrieval_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.make("int8_varlen", B=B)
    Q16h, D16h = inputs.fp16_of_int8_workload(w)
    Nq, Lq, d, T = w["Nq"], w["Lq"], w["d"], w["T"]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    Q8, qs, D8, ds, cu = t(w["Q"]), t(w["q_scale"]), t(w["D_packed"]), t(w["d_scale"]), t(w["cu_seqlens"])
    Q16, D16 = t(Q16h), t(D16h)
    max_ld = int(w["lens"].max())
    ws = torch.empty(max(256, bd.maxsim_two_stage_workspace_bytes(Nq, B, K1)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    s8 = torch.empty((Nq, B), dtype=torch.float32, device=dev)

    def step(timed, pool):
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        out = bd.maxsim_two_stage_topk(Q8, qs, D8, ds, Q16, D16, cu, max_ld, K1, K2, workspace=ws)
        if timed:
            e1.record(stream)
            pool.append((e0, e1))
        return out

    def int8_stage(timed, pool):
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        bd.maxsim_fwd_i8(Q8, qs, D8, ds, cu, max_ld, scores=s8, with_argmax=False)
        if timed:
            e1.record(stream)
            pool.append((e0, e1))

    for _ in range(3):
        cand = step(False, None)[0]
    torch.cuda.synchronize()
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 10
    for _ in range(warmup):
        step(False, None)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    pool, pool8 = [], []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True, pool)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_mem = torch.cuda.max_memory_allocated(dev)
    for _ in range(steps):
        int8_stage(True, pool8)
    torch.cuda.synchronize()
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in pool]))
    i8_ms = float(np.mean([a.elapsed_time(b) for a, b in pool8]))
    lens = np.diff(w["cu_seqlens"])
    cand_tokens = int(lens[cand.cpu().numpy()].sum())  # doc tokens the rescoring pass reads
    ops8 = 2.0 * Nq * Lq * d * T
    ops16 = 2.0 * Lq * d * cand_tokens
    value = (ops8 + ops16) * steps / elapsed / 1e12
    i8_bytes = T * (d + 4) + Nq * Lq * (d + 4) + 4 * (B + 1) + 4 * Nq * B
    achieved = ops8 / (i8_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS["i8"], "unit": "TOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS["i8"], 4), "traffic": None,
                "kernel": "fwd_kernel (INT8 stage)", "kernel_avg_ms": round(i8_ms, 5),
                "algorithmic_flops_per_launch": ops8, "algorithmic_bytes_per_launch": i8_bytes,
                "stage_share_of_step": round(i8_ms / step_ms, 4)}
    cpu = None
    cpu_s = 10.0 if args.cpu_seconds is None else args.cpu_seconds
    if not args.no_cpu_baseline:
        import oracle
        n = 200
        while True:
            sub = inputs.make("int8_varlen", B=n)
            q16s, d16s = inputs.fp16_of_int8_workload(sub)
            t1 = time.perf_counter()
            oracle.two_stage_topk(sub["Q"], sub["q_scale"], sub["D_packed"], sub["d_scale"], q16s, d16s,
                                  sub["cu_seqlens"], oracle.F16, min(K1, n), min(K2, n))
            tc = time.perf_counter() - t1
            if tc > 0.5 * cpu_s or n >= B:
                break
            n = int(min(B, n * max(2.0, 0.8 * cpu_s / max(tc, 1e-3))))
        ops_c = 2.0 * Nq * Lq * d * int(sub["T"]) + 2.0 * Lq * d * int(np.diff(sub["cu_seqlens"]).mean() * Nq * min(K1, n))
        cpu = {"value": round(ops_c / tc / 1e12, 6), "unit": "TOP/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d queries x first %d documents of the same corpus, K1=%d, K2=%d, %.1f s" %
                         (Nq, n, min(K1, n), min(K2, n), tc)}
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(elapsed * 1e3 / steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8+f16",
        "data": "synthetic (seeded N(0,1) rows, l2-normalised; int8 per-token quantised, fp16 of the same rows)",
        "config": {"workload": "two_stage_topk", "Nq": Nq, "Lq": Lq, "B": B, "T_doc_tokens": T, "d": d,
                   "Ld_range": [int(lens.min()), int(lens.max())], "K1": K1, "K2": K2,
                   "rescored_doc_tokens": cand_tokens, "layout": "cu_seqlens"},
        "queries_per_s": round(Nq * steps / elapsed, 1),
        "doc_tokens_per_s": round(T * steps / elapsed, 1),
        "step_event_ms": round(step_ms, 5),
        "peak_mem_bytes": int(peak_mem),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def host_cpu():
    """(CPU model name, logical CPUs this process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count()
    return model, n


def cpu_baseline(w, target_s, padded=False):
    """The oracle as it stands, on the host's cores, on a bounded sample of the
    same workload: the first n documents, then the first nq queries, then whole
    repeats of that, grown until one measurement takes about target_s seconds.
    For the training workloads the sample is the forward (the backward's
    arithmetic is about 0.2 % of the step's)."""
    import oracle

    Q, Dp, cu = w["Q"], w["D_packed"], w["cu_seqlens"]
    Nq, Lq, d, B = w["Nq"], w["Lq"], w["d"], w["B"]
    isi8 = w["dtype"] == "i8"
    odt = oracle.BF16 if w["dtype"] == "bf16" else oracle.F16

    def run(nq, n, reps):
        sub = Dp[:cu[n]]
        subcu = np.ascontiguousarray(cu[:n + 1])
        q = np.ascontiguousarray(Q[:nq])
        t0 = time.perf_counter()
        for _ in range(reps):
            if isi8:
                oracle.fwd_i8(q, np.ascontiguousarray(w["q_scale"][:nq]), sub, w["d_scale"][:cu[n]], subcu)
            else:
                oracle.fwd_varlen(q, sub, subcu, odt)
        return time.perf_counter() - t0

    wall0 = time.perf_counter()
    nq, n, reps = (1 if w["name"].startswith("contrastive_train") else Nq), 1, 1
    t = run(nq, n, reps)
    while t < 0.5 * target_s:
        scale = max(2.0, min(16.0, 0.8 * target_s / max(t, 1e-6)))
        if n < B:
            n = int(min(B, max(n + 1, n * scale)))
        elif nq < Nq:
            nq = int(min(Nq, max(nq + 1, nq * scale)))
        else:
            reps = int(max(reps + 1, reps * scale))
        t = run(nq, n, reps)
    toks = int(cu[n])
    flops = 2.0 * nq * Lq * d * toks * reps
    model, ncpu = host_cpu()
    return {"value": round(flops / t / 1e12, 6), "unit": "TOP/s" if isi8 else "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d queries x first %d documents (%d doc tokens) of the same workload, forward, "
                      "%d pass(es), %.1f s" % (nq, n, toks, reps, t),
            "doc_tokens_per_s": round(toks * reps / t, 1),
            "cpu_model": model, "nproc": ncpu, "wall_s": round(time.perf_counter() - wall0, 1)}


if __name__ == "__main__":
    main()
