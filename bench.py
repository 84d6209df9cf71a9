#!/usr/bin/env python3
"""Benchmark of the group-quantized fused-dequant path on one MI355X.

Headline step (the workload the metric is quoted on): one fp32 activation
vector through a dense INT4 group-64 4096x4096 projection and an INT8
group-64 vocab projection 4096x129280 (dsq_gemv twice).  `value` is the
effective weight bandwidth of the step: canonical bytes moved (codes + fp32
scale + fp32 zero point + activations + outputs) / wall time per step, with
every input resident in HBM when timing starts.  The step streams ~607 MB,
more than the 256 MB Infinity Cache, so no input stays cached across steps.

`roofline` is for the dominant kernel (the vocab GEMV), timed per launch with
HIP events on the stream it runs on.  `secondary` reports the other workloads
(INT8 GEMV, MoE decode, batched MoE decode, dense and MoE prefill) with
their own timings; `cpu_baseline` times the CPU oracle (the pages' own
OpenMP fused-dequant loop) on the whole headline workload, in a child process
after the GPU phase, pinned one thread per physical core with one core left
to the GPU thread.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published

# Workload shape: the model constants "ds4 code walkthrough" prints (DeepSeek
# V4 Flash architecture constants and the RMSNorm epsilon): hidden size,
# vocabulary, routed experts, experts per token.  The expert FFN width (2048)
# is the benchmark workload's own; the pages do not print one.
N_EMBD = 4096
N_VOCAB = 129280
N_EXPERT = 256
N_EXPERT_USED = 6
RMS_EPS = 1e-6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def qbytes(bits, group, K, N):
    """Canonical bytes of a quantized matrix: codes + fp32 (scale, zp), or for
    the super-block format (group 256) codes + a 16-byte header per block."""
    return N * K * bits // 8 + N * (K // group) * (16 if group == 256 else 8)


RECORDS = os.path.join(ROOT, "profiles", "records.json")
CSRC = os.path.join(ROOT, "group_quantized_moe_dsq_amd", "csrc")


def library_source_hash():
    """Hash of every kernel source: a profile record counts for the sources
    it was taken on only."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def load_records():
    if not os.path.exists(RECORDS):
        return {}
    with open(RECORDS) as fh:
        return json.load(fh)


def kernel_record(workload, prefix):
    """(name, record) of the kernel of workload's committed rocprofv3 profile
    whose name starts with `prefix` and which took the most GPU time, with the
    counter calibration (fetch scale, write scale); None when there is no
    record for the current sources."""
    recs = load_records()
    w = recs.get("workloads", {}).get(workload)
    cal = recs.get("calibration") or {}
    if not w or w.get("source_hash") != library_source_hash():
        return None
    cands = [(k, v) for k, v in w.get("kernels", {}).items() if k.startswith(prefix)]
    if not cands:
        return None
    name, k = max(cands, key=lambda kv: kv[1].get("calls", 0) * kv[1].get("avg_us", 0.0))
    return name, k, cal.get("fetch_scale"), cal.get("write_scale")


def roofline_entry(workload, kernel, bound, work, unit_work, graph_us=None):
    """Roofline of the workload's dominant kernel from its committed profile
    record: achieved = algorithmic work per launch (bytes or flops) / the
    kernel's average rocprof duration; traffic = FETCH_SIZE + WRITE_SIZE per
    dispatch scaled by the plain-copy calibration.  Fields are null when no
    record was taken on the current sources."""
    peak = HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS
    unit = "GB/s" if bound == "hbm" else "TFLOP/s"
    e = {"kernel": kernel, "bound": bound, "peak": peak, "unit": unit,
         unit_work: work, "kernel_us": None, "achieved": None, "frac": None, "traffic": None}
    if graph_us is not None:
        e["graph_us_per_call"] = graph_us
    r = kernel_record(workload, kernel)
    if r is None:
        e["note"] = "no rocprofv3 record of this workload on the current sources"
        return e
    e["kernel"], k, fs, ws = r
    us = k.get("avg_us")
    if us:
        e["kernel_us"] = us
        scale = 1e9 if bound == "hbm" else 1e12
        e["achieved"] = round(work / (us * 1e-6) / scale, 1)
        e["frac"] = round(e["achieved"] / peak, 4)
    if k.get("FETCH_SIZE") is not None and k.get("WRITE_SIZE") is not None and fs and ws:
        e["traffic"] = int(k["FETCH_SIZE"] * 1024 * fs + k["WRITE_SIZE"] * 1024 * ws)
    return e


def time_calls(fn, iters, warmup, torch, graph=True, replays=5):
    """Average ms per call.  With graph=True the `iters` calls are captured
    once into a HIP graph and replayed, so host launch overhead does not hide
    short kernels; HIP events on the replay stream bracket the replays."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / (iters * replays)
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters  # ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cases", default="head,gemv8,gemv4,sb4,gemv4vocab,sb4vocab,moe1,block1,"
                                       "cache,moe32,"
                                       "gemm256,moe256",
                    help="secondary workloads to run (comma list)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="run just these secondary workloads (comma list, names as in "
                         "--cases) and print their records: the command the per-kernel "
                         "profiles are taken with")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB a few times: the reference "
                         "kernel of known traffic for scaling the FETCH_SIZE / WRITE_SIZE "
                         "counters")
    ap.add_argument("--cpu-reps", type=int, default=5,
                    help="timed passes of the CPU baseline (median reported)")
    ap.add_argument("--cpu-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="print the per-kernel mean of every counter in rocprofv3 --pmc "
                         "CSV files (library kernels only) and exit")
    ap.add_argument("--record", metavar="WORKLOAD",
                    help="store the library kernels' rocprofv3 figures of WORKLOAD (the "
                         "--only name, or 'calibration' for --calibrate-copy) from --kt / --pmc "
                         "CSV files into profiles/records.json, keyed to the current sources")
    ap.add_argument("--kt", metavar="CSV", help="rocprofv3 --stats kernel statistics CSV")
    ap.add_argument("--pmc", nargs="*", default=[], metavar="CSV",
                    help="rocprofv3 --pmc counter collection CSVs")
    args = ap.parse_args()
    if args.record:
        store_record(args.record, args.kt, args.pmc)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.cpu_child:
        cpu_baseline_child(args.cpu_reps)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library's hot path runs on one device; it has no multi-GPU leg).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from group_quantized_moe_dsq_amd import dsq, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        x = synth.normal((N_EMBD,), 1.0, 0, synth.X, 21, device=dev)
        recs = secondary(dsq, synth, torch, np, dev, set(args.only.split(",")), x, floor=False)
        print(json.dumps({"only": args.only, "records": recs}), flush=True)
        return
    if args.calibrate_copy:
        n = 1 << 28  # fp32 elements: 1 GiB read and 1 GiB written per copy
        a = torch.ones(n, device=dev)
        b = torch.empty(n, device=dev)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4,
                          "copies": 4}), flush=True)
        return
    K = N_EMBD
    NV = N_VOCAB

    # ---------------- headline workload ----------------
    log("setup: INT4 g64 4096x4096 and INT8 g64 4096x129280")
    w4 = synth.normal((4096, K), 0.02, 0, synth.W, 21, device=dev)
    W4 = dsq.QWeight(4, 64, K, 4096)
    dsq.pack_weights(w4, W4)
    del w4
    wv = synth.normal((NV, K), 0.02, 0, synth.W, 22, device=dev)
    WV = dsq.QWeight(8, 64, K, NV)
    dsq.pack_weights(wv, WV)
    del wv
    torch.cuda.empty_cache()
    x = synth.normal((K,), 1.0, 0, synth.X, 21, device=dev)
    y4 = torch.empty(4096, device=dev)
    yv = torch.empty(NV, device=dev)
    bytes4 = qbytes(4, 64, K, 4096) + K * 4 + 4096 * 4
    bytesv = qbytes(8, 64, K, NV) + K * 4 + NV * 4
    step_bytes = bytes4 + bytesv

    def step():
        dsq.gemv(W4, x, y4)
        dsq.gemv(WV, x, yv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # the dominant kernel alone: back-to-back vocab GEMVs replayed from a HIP
    # graph on one stream, bracketed by HIP events on that stream (the 596 MB
    # matrix exceeds the Infinity Cache, so every launch streams from HBM).
    # A graph of 100 launches: the first replay (untimed) then warms the
    # series as long as the timed ones run (with 20 launches the first timed
    # replays of a fresh process ran ~15% slow)
    vocab_ms = time_calls(lambda i: dsq.gemv(WV, x, yv), 100, 2, torch)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = bytesv / (vocab_ms * 1e-3) / 1e9
    log(f"headline: {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s; vocab gemv "
        f"{vocab_ms * 1e3:.1f} us = {achieved:.0f} GB/s")
    prof = roofline_entry("gemv8vocab", "dsq::gemv_kernel<8", "hbm", bytesv, "algorithmic_bytes")

    result = {
        "metric": "effective weight GB/s (% of HBM peak) for INT4/INT8 GEMV + MoE FFN; "
                  "prefill TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "dense INT4 g64 GEMV 4096x4096 + INT8 g64 vocab GEMV "
                               "4096x129280, M=1, fp32 activations ~N(0,1), weights "
                               "~N(0,0.02), seed 0",
                   "step_bytes": step_bytes, "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": prof["traffic"],
                     "kernel": (prof["kernel"] if prof["kernel_us"] else "dsq::gemv_kernel<8, ...>")
                     + " (INT8 g64 vocab GEMV 4096x129280)",
                     "kernel_us": round(vocab_ms * 1e3, 2), "algorithmic_bytes": bytesv,
                     "timing": "HIP events on the launch stream around replays of a graph of 100 "
                               "back-to-back launches",
                     "kernel_us_rocprof": prof["kernel_us"],
                     "frac_rocprof": prof["frac"]},
    }
    del W4
    torch.cuda.empty_cache()

    head = []
    if not args.no_secondary and "head" in args.cases.split(","):
        # the output head: the same vocab GEMV followed by the top-k selection
        # over its 129280 logits (graph-replayed, like the roofline series)
        for k in (1, 50):
            hidx = torch.empty(k, dtype=torch.int32, device=dev)
            hval = torch.empty(k, device=dev)
            hws = torch.empty(dsq.topk_workspace_bytes(NV, k) + 256, dtype=torch.uint8, device=dev)
            hms = time_calls(lambda i: dsq.gemv_topk(WV, x, k, y=yv, idx=hidx, values=hval,
                                                     workspace=hws), 100, 2, torch)
            gbs = bytesv / (hms * 1e-3) / 1e9
            head.append({"workload": f"output head: INT8 g64 vocab GEMV 4096x129280 + top-{k} "
                                     "of the logits", "us": round(hms * 1e3, 2),
                         "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "selection_us": round((hms - vocab_ms) * 1e3, 2)})
            log(head[-1])
    if not args.no_secondary and args.cases:
        result["secondary"] = head + secondary(dsq, synth, torch, np, dev,
                                               set(args.cases.split(",")), x)
    del WV
    torch.cuda.empty_cache()

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_reps)
    print(json.dumps(result), flush=True)


def secondary(dsq, synth, torch, np, dev, cases, x, floor=True):
    out = []
    K = 4096

    def rotated_gemv(bits, group, name, copies, case, kname):
        Ws = []
        for c in range(copies):
            w = synth.normal((4096, K), 0.02, 0, synth.W, 100 + c, device=dev)
            q = dsq.QWeight(bits, group, K, 4096)
            dsq.pack_weights(w, q)
            Ws.append(q)
        del w
        y = torch.empty(4096, device=dev)
        ms = time_calls(lambda i: dsq.gemv(Ws[i % copies], x, y), 400, 64, torch)
        b = qbytes(bits, group, K, 4096) + K * 4 + 4096 * 4
        gbs = b / (ms * 1e-3) / 1e9
        rec = {"workload": name, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
               "note": f"rotating {copies} weight copies ({copies * b / 1e6:.0f} MB) "
                       "so the Infinity Cache cannot hold them"}
        if floor:
            # per-launch floor of back-to-back graph launches of this kernel:
            # the same GEMV format on a 64x256 matrix (a few KB, cache
            # resident); left out of the single-workload (profiled) runs so
            # that the profile holds the 4096x4096 launches only
            wt = synth.normal((64, 256), 0.02, 0, synth.W, 99, device=dev)
            qt = dsq.QWeight(bits, group, 256, 64)
            dsq.pack_weights(wt, qt)
            xt = synth.normal((256,), 1.0, 0, synth.X, 99, device=dev)
            yt = torch.empty(64, device=dev)
            floor_ms = time_calls(lambda i: dsq.gemv(qt, xt, yt), 400, 64, torch)
            rec["launch_floor_us"] = round(floor_ms * 1e3, 2)
        rec["roofline"] = roofline_entry(case, kname, "hbm", b, "algorithmic_bytes",
                                         graph_us=rec["us"])
        out.append(rec)
        log(out[-1])

    if "gemv8" in cases:
        rotated_gemv(8, 64, "INT8 g64 GEMV 4096x4096 (M=1)", 64, "gemv8", "dsq::gemv_kernel<8")
    if "gemv4" in cases:
        rotated_gemv(4, 64, "INT4 g64 GEMV 4096x4096 (M=1)", 64, "gemv4", "dsq::gemv_kernel<4")
    if "sb4" in cases:
        rotated_gemv(4, 256, "super-block 4-bit GEMV 4096x4096 (M=1)", 64, "sb4",
                     "dsq::gemv_sb4_kernel")
    torch.cuda.empty_cache()
    def vocab_gemv(bits, group, name, case, kname):
        # the vocab projection, 298-331 MB: cold by size
        NV = N_VOCAB
        w = synth.normal((NV, K), 0.02, 0, synth.W, 2, device=dev)
        q = dsq.QWeight(bits, group, K, NV)
        dsq.pack_weights(w, q)
        del w
        torch.cuda.empty_cache()
        y = torch.empty(NV, device=dev)
        ms = time_calls(lambda i: dsq.gemv(q, x, y), 100, 1, torch)
        b = qbytes(bits, group, K, NV) + K * 4 + NV * 4
        gbs = b / (ms * 1e-3) / 1e9
        out.append({"workload": name, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": b,
                    "roofline": roofline_entry(case, kname, "hbm", b, "algorithmic_bytes",
                                               graph_us=round(ms * 1e3, 2))})
        log(out[-1])
        del q
        torch.cuda.empty_cache()

    if "gemv8vocab" in cases:  # the headline's dominant kernel alone (for its profile)
        vocab_gemv(8, 64, "INT8 g64 vocab GEMV 4096x129280 (M=1)", "gemv8vocab", "dsq::gemv_kernel<8")
    if "gemv4vocab" in cases:
        vocab_gemv(4, 64, "INT4 g64 vocab GEMV 4096x129280 (M=1)", "gemv4vocab", "dsq::gemv_kernel<4")
    if "sb4vocab" in cases:
        vocab_gemv(4, 256, "super-block 4-bit vocab GEMV 4096x129280 (M=1)", "sb4vocab",
                   "dsq::gemv_sb4_kernel")

    # MoE decode layers: 256 experts, H=4096, I=2048, top-6
    def build_moe(bits, group, bias_std):
        E, H, I = N_EXPERT, N_EMBD, 2048
        router = synth.normal((E, H), 0.02, 0, synth.ROUTER, 0, device=dev)
        bias = None if bias_std is None else synth.normal((E,), bias_std, 0, synth.BIAS, 0,
                                                          device=dev)
        g, u, d = dsq.QWeight(bits, group, H, I, E), dsq.QWeight(bits, group, H, I, E), \
            dsq.QWeight(bits, group, I, H, E)
        for e in range(E):
            wg, wu, wd = synth.expert_weights(e, H, I, 0, device=dev)
            dsq.pack_weights(wg, g, first=e)
            dsq.pack_weights(wu, u, first=e)
            dsq.pack_weights(wd, d, first=e)
        torch.cuda.synchronize()
        return router, bias, g, u, d

    def moe_case(name, layer, T, nsets, math, bits, group, iters, block=False, case=None,
                 kernels=None):
        # block: the MoE step with its RMSNorm and residual (dsq_moe_block)
        H = N_EMBD
        Xs = [synth.normal((T, H), 1.0, 0, synth.X, 1000 + T * 100 + s, device=dev)
              for s in range(nsets)]
        gamma = synth.normal((H,), 0.25, 0, synth.X, 900, device=dev) + 1.0
        wsq = dsq.moe_block_workspace_bytes if block else dsq.moe_workspace_bytes
        ws = torch.empty(wsq(T, N_EXPERT, N_EXPERT_USED, H, 2048, math) + 256, dtype=torch.uint8,
                         device=dev)
        Y = torch.empty((T, H), device=dev)
        counts = torch.empty(256, dtype=torch.int32, device=dev)

        def run(X, **kw):
            if block:
                return dsq.moe_block(layer, X, gamma, RMS_EPS, math=math, Y=Y, workspace=ws, **kw)
            return dsq.moe_ffn(layer, X, math=math, Y=Y, workspace=ws, **kw)
        touched = []
        for s in range(nsets):
            run(Xs[s], counts_out=counts)
            touched.append(int((counts > 0).sum().item()))
        D = float(np.mean(touched))
        ms = time_calls(lambda i: run(Xs[i % nsets]), iters, 4, torch)
        eb = 3 * qbytes(bits, group, H, 2048)
        b = N_EXPERT * H * 4 + D * eb + 2 * T * H * 4 + (H * 4 if block else 0)
        flops = 2 * T * N_EXPERT * H + 2 * T * N_EXPERT_USED * 3 * H * 2048
        gbs = b / (ms * 1e-3) / 1e9
        rec = {"workload": name, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "experts_touched": D,
               "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 3)}
        if case and kernels:
            # the weight-streaming kernels: gate/up reads the touched experts'
            # gate and up matrices, down their down matrices (codes + fp32
            # scale and zero point); the dominant one is gate/up
            gu_bytes = int(D * 2 * qbytes(bits, group, H, 2048))
            dn_bytes = int(D * qbytes(bits, group, 2048, H))
            rec["roofline"] = roofline_entry(case, kernels[0], "hbm", gu_bytes, "algorithmic_bytes")
            rec["roofline_down"] = roofline_entry(case, kernels[1], "hbm", dn_bytes,
                                                  "algorithmic_bytes")
            w = load_records().get("workloads", {}).get(case)
            if w and w.get("source_hash") == library_source_hash():
                rec["kernels_us"] = {k: v.get("avg_us") for k, v in sorted(w["kernels"].items())
                                     if not k.startswith("dsq::pack")}
        out.append(rec)
        log(rec)

    if "moe1" in cases or "moe32" in cases or "block1" in cases or "cache" in cases:
        r, b, g, u, d = build_moe(4, 64, None)
        if "moe1" in cases:
            moe_case("MoE decode T=1, 256 experts top-6, INT4 g64 SwiGLU",
                     dsq.MoeLayer(r, g, u, d, None, N_EXPERT_USED), 1, 64, dsq.MATH_FP32, 4, 64, 64,
                     case="moe1", kernels=("dsq::dec_gateup_kernel", "dsq::dec_down_kernel"))
        if "block1" in cases:
            moe_case("MoE block decode T=1 (RMSNorm + MoE + residual), INT4 g64 SwiGLU",
                     dsq.MoeLayer(r, g, u, d, None, N_EXPERT_USED), 1, 64, dsq.MATH_FP32, 4, 64, 64,
                     block=True)
        if "cache" in cases:
            expert_cache_case(dsq, synth, torch, dev, r, (g, u, d), out)
        if "moe32" in cases:
            bias = synth.normal((256,), 1.0, 0, synth.BIAS, 0, device=dev)
            moe_case("MoE batched decode T=32 skewed (router bias ~N(0,1)), INT4 g64",
                     dsq.MoeLayer(r, g, u, d, bias, N_EXPERT_USED), 32, 8, dsq.MATH_FP32, 4, 64, 64,
                     case="moe32", kernels=("dsq::gmm_kernel<4, 2, 2, true>",
                                            "dsq::gmm_kernel<4, 2, 2, false>"))
        del g, u, d
        torch.cuda.empty_cache()
    if "gemm256" in cases:
        out.append(dense_prefill(dsq, synth, torch, dev))
    if "gemm256lib" in cases:
        out.append(dense_prefill_library(synth, torch, dev))
    if "moe256" in cases:
        r, b, g, u, d = build_moe(8, 128, None)
        moe_case("MoE prefill T=256, 256 experts top-6, INT8 g128 SwiGLU, bf16 MFMA",
                 dsq.MoeLayer(r, g, u, d, None, N_EXPERT_USED), 256, 1, dsq.MATH_BF16_MFMA, 8, 128, 24,
                 case="moe256", kernels=("dsq::gmm_kernel<8, 4, 1, true>",
                                         "dsq::gmm_kernel<8, 4, 1, false>"))
        del g, u, d
        torch.cuda.empty_cache()
    return out


def expert_cache_case(dsq, synth, torch, dev, router, layer, out):
    """Decode tokens through the full MoE layer with its 256 experts in
    pinned host memory and an HBM cache of `slots` experts (least recently
    used out): time per token, hit rate, host-to-device copy rate.  The
    routing of random activations is spread over all experts, so the hit
    rate follows the cache's share of them."""
    import time
    H, I, E, k = N_EMBD, 2048, N_EXPERT, N_EXPERT_USED
    for slots in (16, 64, 256):
        c = dsq.ExpertCache(4, 64, H, I, E, slots, device=dev)
        for m, q in enumerate(layer):
            c.host[m].copy_(q.buf)
        ws = torch.empty(dsq.moe_cached_workspace_bytes(1, E, slots, k, H, I, dsq.MATH_FP32) + 256,
                         dtype=torch.uint8, device=dev)
        Y = torch.empty((1, H), device=dev)
        Xs = [synth.normal((1, H), 1.0, 0, synth.X, 5000 + t, device=dev) for t in range(96)]
        torch.cuda.synchronize()
        for t in range(32):                    # fill the cache
            dsq.moe_ffn_cached(router, None, c, Xs[t], k, math=dsq.MATH_FP32, Y=Y, workspace=ws)
        h0, m0, b0 = c.hits, c.misses, c.bytes_copied
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(32, 96):
            dsq.moe_ffn_cached(router, None, c, Xs[t], k, math=dsq.MATH_FP32, Y=Y, workspace=ws)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 64
        hits, misses, nbytes = c.hits - h0, c.misses - m0, c.bytes_copied - b0
        rec = {"workload": f"MoE decode T=1 with the experts behind an HBM cache of {slots} of 256 "
                           "(pinned host store, LRU), INT4 g64",
               "us_per_token": round(dt * 1e6, 1),
               "hit_rate": round(hits / max(hits + misses, 1), 3),
               "h2d_GB_per_token": round(nbytes / 64 / 1e9, 4),
               "h2d_GB/s": round(nbytes / (dt * 64) / 1e9, 1)}
        out.append(rec)
        log(rec)
        del c, ws
        torch.cuda.empty_cache()


def dense_prefill(dsq, synth, torch, dev):
    K = 4096
    # dense prefill GEMM M=256, INT8 g128, bf16 MFMA, rotating 32 weight copies
    Ws = []
    for c in range(32):
        w = synth.normal((4096, K), 0.02, 0, synth.W, 200 + c, device=dev)
        q = dsq.QWeight(8, 128, K, 4096)
        dsq.pack_weights(w, q)
        Ws.append(q)
    del w
    X = synth.normal((256, K), 1.0, 0, synth.X, 5, device=dev)
    Y = torch.empty((256, 4096), device=dev)
    wsb = torch.empty(dsq.gemm_workspace_bytes(256, 4096, K, dsq.MATH_BF16_MFMA) + 256,
                      dtype=torch.uint8, device=dev)
    ms = time_calls(lambda i: dsq.gemm(Ws[i % 32], X, Y, math=dsq.MATH_BF16_MFMA, workspace=wsb),
                    128, 16, torch)
    flops = 2 * 256 * 4096 * K
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"workload": "dense prefill GEMM M=256 K=N=4096 INT8 g128 bf16 MFMA",
           "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
           "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
           "GB/s": round((qbytes(8, 128, K, 4096) + 2 * 256 * K * 4) / (ms * 1e-3) / 1e9, 1),
           "roofline": roofline_entry("gemm256", "dsq::gemm_mfma_kernel", "mfma", flops,
                                      "algorithmic_flops", graph_us=round(ms * 1e3, 2))}
    w = load_records().get("workloads", {}).get("gemm256")
    if w and w.get("source_hash") == library_source_hash():
        rec["kernels_us"] = {k: v.get("avg_us") for k, v in sorted(w["kernels"].items())
                             if not k.startswith("dsq::pack")}
    log(rec)
    del Ws
    torch.cuda.empty_cache()
    return rec



def dense_prefill_library(synth, torch, dev):
    """Context for the quantized prefill GEMM, not part of the path: the
    platform's own bf16 GEMM (torch.matmul, i.e. hipBLASLt) on the same shape,
    M=256, K=N=4096, with plain bf16 weights (twice the bytes of INT8 codes,
    nothing to dequantize) stored as [N][K] like the packed rows, 32 rotating
    copies, bf16 output.  Run only when named (--only gemm256lib)."""
    K = N = 4096
    Ws = [synth.normal((N, K), 0.02, 0, synth.W, 200 + c, device=dev).to(torch.bfloat16)
          for c in range(32)]
    X = synth.normal((256, K), 1.0, 0, synth.X, 5, device=dev).to(torch.bfloat16)
    Y = torch.empty((256, N), device=dev, dtype=torch.bfloat16)
    ms = time_calls(lambda i: torch.matmul(X, Ws[i % 32].t(), out=Y), 128, 16, torch)
    tf = 2 * 256 * N * K / (ms * 1e-3) / 1e12
    rec = {"workload": "library bf16 GEMM (torch.matmul) M=256 K=N=4096, bf16 weights",
           "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
           "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
           "note": "platform library on unquantized weights, for comparison only"}
    log(rec)
    del Ws
    torch.cuda.empty_cache()
    return rec


def _kernel_name(raw):
    """'void dsq::gmm_kernel<8, 4, 1, true>(dsq::GmmArgs)' -> 'dsq::gmm_kernel<8, 4, 1, true>'."""
    import re
    name = raw.replace("void ", "", 1) if raw.startswith("void ") else raw
    m = re.match(r"^([^(]*?(?:<.*?>)?)\(", name)
    return (m.group(1) if m else name).strip()


def _pmc_means(paths):
    import collections
    import csv
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if "dsq::" not in name and "copyBuffer" not in name:
                    continue
                vals[_kernel_name(name)][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}, \
        {k: max(len(v) for v in cs.values()) for k, cs in vals.items()}


def store_record(workload, kt, pmc):
    """Merge one workload's rocprofv3 figures into profiles/records.json."""
    import csv
    recs = load_records()
    means, counts = _pmc_means(pmc)
    counters = sorted({c for m in means.values() for c in m})
    if workload == "calibration":
        copy = next((v for k, v in means.items() if "copyBuffer" in k), None)
        if copy is None:
            sys.exit("no buffer copy kernel in the counter files")
        n = 1 << 30  # bytes read and written by the --calibrate-copy copy
        cal = recs.get("calibration", {})
        if "FETCH_SIZE" in copy:
            cal["fetch_scale"] = round(n / 1024 / copy["FETCH_SIZE"], 5)
            cal["FETCH_SIZE_KiB"] = copy["FETCH_SIZE"]
        if "WRITE_SIZE" in copy:
            cal["write_scale"] = round(n / 1024 / copy["WRITE_SIZE"], 5)
            cal["WRITE_SIZE_KiB"] = copy["WRITE_SIZE"]
        cal["reference"] = "device copy of 1 GiB fp32 (bench.py --calibrate-copy), bytes read " \
                           "and written known"
        cal["commands"] = sorted(set(cal.get("commands", [])) | {
            f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o r -- python3 -u bench.py "
            "--calibrate-copy" for c in counters})
        recs["calibration"] = cal
    else:
        w = recs.setdefault("workloads", {}).get(workload, {})
        if w.get("source_hash") != library_source_hash():
            w = {}
        w["source_hash"] = library_source_hash()
        kernels = w.setdefault("kernels", {})
        cmds = set(w.get("commands", []))
        if kt:
            with open(kt) as fh:
                for r in csv.DictReader(fh):
                    if "dsq::" not in r["Name"]:
                        continue
                    k = kernels.setdefault(_kernel_name(r["Name"]), {})
                    k["calls"] = int(r["Calls"])
                    k["avg_us"] = round(float(r["AverageNs"]) / 1000, 3)
                    k["min_us"] = round(float(r["MinNs"]) / 1000, 3)
                    k["max_us"] = round(float(r["MaxNs"]) / 1000, 3)
            cmds.add("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o r -- "
                     f"python3 -u bench.py --only {workload}")
        for name, m in means.items():
            if "copyBuffer" in name:
                continue
            k = kernels.setdefault(name, {})
            k.update({c: round(v, 3) for c, v in m.items()})
            k["dispatches_counted"] = counts[name]
        for path in pmc:
            with open(path) as fh:
                import csv as _csv
                names = sorted({r["Counter_Name"] for r in _csv.DictReader(fh)})
            cmds.add(f"rocprofv3 --pmc {' '.join(names)} --output-format csv -d <dir> -o r -- "
                     f"python3 -u bench.py --only {workload}")
        w["commands"] = sorted(cmds)
        recs["workloads"][workload] = w
    os.makedirs(os.path.dirname(RECORDS), exist_ok=True)
    with open(RECORDS, "w") as fh:
        json.dump(recs, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(f"recorded {workload} into {RECORDS}")


def pmc_summary(paths):
    """Mean of each counter per dispatch of each library kernel, from the
    per-dispatch rows rocprofv3 --pmc writes (*_counter_collection.csv); the
    runtime's buffer copy is kept too, as the reference of known traffic."""
    import collections
    import csv
    import re
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    info = {}
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if "dsq::" not in name and "copyBuffer" not in name:
                    continue
                name = re.sub(r"\(dsq::.*|\(float const.*|\(.*", "", name).replace("void ", "")
                vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
                info[name] = (r["Grid_Size"], r["Workgroup_Size"], r["VGPR_Count"],
                              r.get("Accum_VGPR_Count", ""), r["LDS_Block_Size"])
    for name in sorted(vals):
        cs = vals[name]
        n = max(len(v) for v in cs.values())
        g, wg, vg, ag, lds = info[name]
        print(f"{name}  dispatches={n} grid={g} wg={wg} vgpr={vg} agpr={ag} lds={lds}")
        for c in sorted(cs):
            v = cs[c]
            print(f"    {c:28s} mean {sum(v) / len(v):.6g}")


def cpu_topology():
    """Physical cores this process may use, read at run time: the CPUs in the
    affinity mask grouped by (package, core), capped by the cgroup's CPU
    quota; one is left to the thread that drives the GPU ("Running a
    284B-parameter LLM from 3.2 GB of RAM in plain C": CPU matmul throughput
    collapsed while the GPU thread competed for cores), and hyperthreads are
    not used ("Hand-writing a DeepSeek inference engine in pure C" §4.2: 32
    threads on 16 cores ran ~10% slower than 16)."""
    cpus = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in cpus:
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        try:
            with open(base + "physical_package_id") as fh:
                pkg = fh.read().strip()
            with open(base + "core_id") as fh:
                core = fh.read().strip()
            cores.add((pkg, core))
        except OSError:
            cores.add(("?", str(c)))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            q, per = fh.read().split()[:2]
            if q != "max":
                quota = max(1, -(-int(q) // int(per)))
    except (OSError, ValueError):
        pass
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    physical = len(cores) if quota is None else min(len(cores), quota)
    return {"cpu_model": model, "logical_cpus": len(cpus), "physical_cores": physical,
            "cgroup_cpu_quota": quota, "threads": max(1, physical - 1)}


def cpu_baseline_child(reps):
    """Runs in its own process (OpenMP pinned by the parent's environment):
    the oracle's fp32 fused-dequant OpenMP GEMV (the pages' CPU method) on the
    whole headline workload, one warm-up pass, then the median of `reps`."""
    import statistics

    import oracle
    from group_quantized_moe_dsq_amd import synth

    K, NV = N_EMBD, N_VOCAB
    # the same shapes, seeds and distributions as the GPU phase, drawn with
    # the CPU generator
    w4 = synth.normal((4096, K), 0.02, 0, synth.W, 21).numpy()
    m4 = oracle.quantize(w4, 4, 64)
    del w4
    wv = synth.normal((NV, K), 0.02, 0, synth.W, 22).numpy()
    mv = oracle.quantize(wv, 8, 64)
    del wv
    x = synth.normal((1, K), 1.0, 0, synth.X, 21).numpy()
    step_bytes = qbytes(4, 64, K, 4096) + qbytes(8, 64, K, NV) + 2 * K * 4 + (4096 + NV) * 4

    def step():
        oracle.qmatmul_f32(x, m4)
        oracle.qmatmul_f32(x, mv)

    # torch (the input generator) sets the process's OpenMP thread count
    # when it starts its own pool, from its environment: the parent's count
    # is applied here, after the last torch call and before the timed passes
    if os.environ.get("OMP_NUM_THREADS"):
        oracle.set_threads(int(os.environ["OMP_NUM_THREADS"]))
    step()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    print(json.dumps({"ms_per_step": med * 1e3, "times_ms": [t * 1e3 for t in times],
                      "step_bytes": step_bytes, "threads": oracle.max_threads()}), flush=True)


def cpu_baseline(reps):
    """The CPU oracle timed on the host's physical cores in a phase after the
    GPU phase (never concurrently with GPU work), in a child process pinned
    with OMP_PROC_BIND=close / OMP_PLACES=cores."""
    import subprocess

    topo = cpu_topology()
    env = dict(os.environ, OMP_NUM_THREADS=str(topo["threads"]),
               MKL_NUM_THREADS=str(topo["threads"]), OMP_PROC_BIND="close", OMP_PLACES="cores")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child",
                        "--cpu-reps", str(reps)], env=env, capture_output=True, text=True,
                       timeout=900)
    if r.returncode != 0:
        raise RuntimeError("cpu baseline child failed:\n" + r.stderr[-2000:])
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    gbs = rec["step_bytes"] / (rec["ms_per_step"] * 1e-3) / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": rec["threads"], "kind": "oracle",
            "sample": "the whole headline step (INT4 g64 4096x4096 + INT8 g64 4096x129280 GEMV, "
                      f"M=1, {rec['step_bytes']} bytes), fp32 fused dequant, OpenMP "
                      f"{rec['threads']} threads pinned one per physical core "
                      "(OMP_PROC_BIND=close, OMP_PLACES=cores), one core left to the GPU "
                      f"thread; 1 warm-up pass, median of {reps}",
            "ms_per_step": round(rec["ms_per_step"], 3),
            "times_ms": [round(t, 3) for t in rec["times_ms"]], **topo}


if __name__ == "__main__":
    main()
