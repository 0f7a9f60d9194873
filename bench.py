"""Benchmark of the fused W4A4 + rank-32 linear (SVDQuant layer) on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload flux_qkv]

One step = the whole hot path on one batch already resident in HBM: the activation kernel
(smoothing, group quantization, down projection X̂·L1) followed by the fused 4-bit GEMM with the
low-rank up projection. Prints ONE JSON line on stdout (diagnostics go to stderr):

  value      effective TOPS = (2·M·N·K + 2·M·r·(K+N)) / time per step (whole job, one GPU)
  roofline   the GEMM kernel: algorithmic ops per launch / its average launch time (HIP events on
             the launch stream around each GEMM launch of `steps` further steps, right after the
             timed region) against the MI355X dense int8/fp8 MFMA peak (5.0 POP/s) for INT4 and
             W8A8, or the MXFP4 peak (10.1 PFLOP/s) for the FP4 variant; also against the peak
             measured on this GPU by register-only MFMA chains (libw4a4_peak.so)
  cpu_baseline  the numpy oracle's forward pass on a bounded sample of rows of the same layer
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = {"int4_g64": 5000.0, "mxfp4_b32": 10100.0, "w8a8": 5000.0}   # dense MFMA peaks (int8/fp8; fp4)
DTYPE = {"int4_g64": "int4", "mxfp4_b32": "fp4", "w8a8": "int8"}
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_ops(M, N, K, r):
    return 2.0 * M * N * K + 2.0 * M * r * (K + N)


def quantize_bytes(M, K, r, fmt):
    """Algorithmic HBM bytes of the activation side of one step: read X (bf16) and 1/λ, read L1,
    write codes, scales and t."""
    if fmt == "w8a8":
        return M * K * 2 + K * 4 + r * K * 2 + M * (K + 4 + r * 4)
    scale_bytes = (K // 64) * 2 if fmt == "int4_g64" else (K // 32)
    return M * K * 2 + K * 4 + r * K * 2 + M * (K // 2 + scale_bytes + r * 4)


def gemm_kernel_name(fmt, rank_pad, M, N):
    """The GEMM kernel the library launches for this layer (as rocprofv3 names it)."""
    nt = rank_pad // 16
    if fmt == "w8a8":
        return f"gemm_w8a8_kernel<{nt}, false>"
    if fmt == "int4_g64":
        return f"gemm_kernel<0, {nt}, -1>"
    small = ((M + 255) // 256 * 2) * ((N + 255) // 256 * 2) <= 512   # grid of 128 x 128 blocks
    return f"gemm_mx_small_kernel<{nt}>" if small else f"gemm_w8a8_kernel<{nt}, true>"


def time_layer(lay, x, y, M, steps, warmup):
    """ms per step (quantize + GEMM) by wall clock over `steps` steps, and the GEMM's average
    launch time by HIP events on the launch stream (a separate pass)."""
    import torch
    stream = torch.cuda.current_stream()
    acts = lay.act_buffers(M)
    for _ in range(warmup):
        lay.quantize(x)
        lay.gemm(acts, M, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lay.quantize(x)
        lay.gemm(acts, M, y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        lay.quantize(x)
        e[0].record(stream)
        lay.gemm(acts, M, y)
        e[1].record(stream)
    torch.cuda.synchronize()
    return ms, float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))


def traffic_from_profile(kernel_src: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", "gemm_int4_flux_qkv_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if kv.get("source_sha256") != sha or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def unfused_lowrank_factors(prep, inv, device):
    """The low-rank factors for the unfused ablation: L1' = diag(1/λ)·L1 [K, r] (the smoothing folded
    into the down projection, so it needs no separate pass over X) and L2 [r, N], bf16."""
    import torch
    K, N, r, rp = prep["K"], prep["N"], prep["rank"], prep["rank_pad"]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    l1 = bf(prep["l1t"].reshape(rp, K)[:r]).float().t() * torch.from_numpy(np.asarray(inv, np.float32))[:, None]
    l2 = bf(prep["l2t"].reshape(-1, rp)[:N, :r]).t()
    return l1.to(torch.bfloat16).contiguous().to(device), l2.contiguous().to(device)


def unfused_layer(prep, inv, device):
    """The same layer with its low-rank branch left out of this library's kernels: the residual's
    codes and scales, run at rank 0 (the branch is added by `unfused_step`)."""
    import w4a4_quantized_gemm_smooth_amd as w4
    return w4.W4A4Linear(dict(prep, rank=0), inv, device=device)


def unfused_step(layer_u, acts_u, x, y, l1s, l2):
    """One step of the unfused baseline: the 4-bit main branch (this library's kernels at rank 0),
    then the low-rank branch as separate library GEMMs (hipBLASLt through torch) that re-read X and
    read-modify-write Y: t = bf16(X·L1'), Y = bf16(Y + t·L2)."""
    import torch
    M = x.shape[0]
    layer_u.quantize(x)
    layer_u.gemm(acts_u, M, y)
    t = torch.matmul(x, l1s)
    y.addmm_(t, l2)


def measured_peaks(dev):
    """Measured MFMA peaks (TOPS) from libw4a4_peak.so: register-only chains of one instruction per
    kind on every SIMD; None when the helper library is absent."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "w4a4_quantized_gemm_smooth_amd", "libw4a4_peak.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.w4a4_peak_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.w4a4_peak_mfma_launch.restype = ctypes.c_int
    L.w4a4_peak_mfma_macs.argtypes = [ctypes.c_int]
    L.w4a4_peak_mfma_macs.restype = ctypes.c_longlong
    blocks, iters = 2048, 1000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for kind, name in ((0, "int8"), (1, "fp6"), (2, "fp4"), (3, "bf16")):
        launch = lambda: L.w4a4_peak_mfma_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                                 ctypes.c_void_p(stream.cuda_stream))
        assert launch() == 0
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert launch() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        ops = 2.0 * blocks * 4 * iters * 8 * L.w4a4_peak_mfma_macs(kind)
        res[name] = round(ops / (best * 1e-3) / 1e12, 1)
    del out
    return res


def copy_bandwidth(dev, mib=256):
    """Read + write GB/s of a device-to-device copy of `mib` MiB (best of 3)."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2.0 * (mib << 20) / (best * 1e-3) / 1e9


def pct(v, q):
    return round(float(np.percentile(np.asarray(v), q)), 5)


def mlp_bench(args):
    """The FLUX MLP pair fc1 (4608 x 3072 -> 12288) -> GELU -> fc2 (12288 -> 3072), r 32, INT4. One
    step = both layers. Fused: fc1's activation kernel, fc1's GEMM with fc2's activation side in its
    epilogue (+ the t2 reduction), fc2's GEMM. Unfused: fc1's two kernels writing Y1, fc2's
    activation kernel applying the GELU as it reads Y1, fc2's GEMM."""
    import torch
    import synth
    import w4a4_quantized_gemm_smooth_amd as w4
    dev = torch.device("cuda:0")
    d1, d2 = synth.workload("flux_mlp_fc1"), synth.workload("flux_mlp_fc2")
    M, K, N, N2, r = d1["M"], d1["K"], d1["N"], d2["N"], d1["rank"]
    log(f"[bench] flux_mlp: fc1 {M}x{K}->{N}, fc2 ->{N2}, r={r}")
    lam1, inv1 = w4.smooth_factors(w4.column_absmax(d1["x"]), w4.column_absmax(d1["w"]))
    lam2, inv2 = w4.smooth_factors(w4.column_absmax(d2["x"]), w4.column_absmax(d2["w"]))
    fc1 = w4.W4A4Linear(w4.prepare_weights(d1["w"], lam1, r), inv1, device=dev)
    fc2 = w4.W4A4Linear(w4.prepare_weights(d2["w"], lam2, r), inv2, device=dev)
    pair = w4.MLPPair(fc1, fc2)
    x = torch.from_numpy(np.ascontiguousarray(d1["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    y2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
    ops = layer_ops(M, N, K, r) + layer_ops(M, N2, N, r)
    stream = torch.cuda.current_stream()
    b = pair.buffers(M)
    f1, f2, a2 = fc1, fc2, b["act2"]

    def fused_parts():
        a1 = f1.quantize(x)
        yield
        w4.lowrank_linear_gelu_quant(a1["xq"], a1["xscale"], a1["xl1"], f1.wq, f1.wscale, f1.l2t, f1.bias, M, N, K, r,
                                     f1.fmt, f2.inv_lambda, f2.l1t, f2.rank, a2["xq"], a2["xscale"], b["xl1_2_fused"])
        yield
        f2.gemm(dict(a2, xl1=b["xl1_2_fused"]), M, y2)
        yield

    def unfused_parts():
        a1 = f1.quantize(x)
        yield
        f1.gemm(a1, M, b["y1"])
        yield
        w4.gelu_quantize_act(b["y1"], f2.inv_lambda, f2.l1t, f2.rank, f2.fmt, a2["xq"], a2["xscale"], a2["xl1"])
        yield
        f2.gemm(a2, M, y2)
        yield

    def run(parts, n):
        for _ in range(n):
            for _ in parts():
                pass

    def timed(parts):
        run(parts, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(parts, args.steps)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        per = []   # per-kernel event times, in a separate pass
        for _ in range(args.steps):
            evs = [torch.cuda.Event(enable_timing=True)]
            evs[0].record(stream)
            for _ in parts():
                evs.append(torch.cuda.Event(enable_timing=True))
                evs[-1].record(stream)
            per.append(evs)
        torch.cuda.synchronize()
        kern = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in per])) for i in range(len(per[0]) - 1)]
        return ms, kern

    ms_f, k_f = timed(fused_parts)
    ms_u, k_u = timed(unfused_parts)
    fc1_ops = layer_ops(M, N, K, r)
    out = {
        "metric": "effective TOPS of fused W4A4+rank-32 linear at FLUX shapes; % MFMA peak",
        "value": round(ops / (ms_f * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_f, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4", "data": "synthetic (seeded FLUX-shaped MLP pair; random weights)",
        "config": {"workload": "flux_mlp", "M": M, "K": K, "N": N, "N2": N2, "rank": r, "format": "int4_g64",
                   "ops_per_step": ops, "path": "fc2's activation side fused into fc1's GEMM epilogue"},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel<0,2,2>", "achieved": round(fc1_ops / (k_f[1] * 1e-3) / 1e12, 2),
                     "peak": PEAK_TOPS["int4_g64"], "unit": "TFLOP/s",
                     "frac": round(fc1_ops / (k_f[1] * 1e-3) / 1e12 / PEAK_TOPS["int4_g64"], 4), "traffic": None,
                     "avg_launch_ms": round(k_f[1], 5), "algorithmic_ops_per_launch": fc1_ops},
        "kernels_fused_ms": {"fc1_quantize": round(k_f[0], 5), "fc1_gemm_gelu_quant_and_t2_reduce": round(k_f[1], 5),
                             "fc2_gemm": round(k_f[2], 5)},
        "kernels_unfused_ms": {"fc1_quantize": round(k_u[0], 5), "fc1_gemm": round(k_u[1], 5),
                               "fc2_gelu_quantize": round(k_u[2], 5), "fc2_gemm": round(k_u[3], 5)},
        "ablation": {"unfused_ms_per_step": round(ms_u, 5), "fused_ms_per_step": round(ms_f, 5),
                     "fusion_gain_pct": round(100.0 * (ms_u - ms_f) / ms_u, 2)},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(d, lam, inv, budget_s=20.0):
    """Time the oracle's forward (quantize X, 4-bit main branch, low-rank branch) on a sample of
    rows; the oracle's weight preparation is offline and not timed."""
    import oracle as O
    t0 = time.perf_counter()
    prep = O.prepare_weights(d["w"], lam, d["rank"], d["fmt"])
    log(f"[cpu] oracle weight prep {time.perf_counter() - t0:.1f}s (not timed)")
    M = d["x"].shape[0]
    rows, spent = 64, 0.0
    while True:  # grow the sample (up to all of X) until one forward takes a quarter of the budget
        t0 = time.perf_counter()
        O.linear(d["x"][:rows], inv, prep)
        dt = time.perf_counter() - t0
        spent += dt
        if dt >= budget_s / 4 or spent >= budget_s or rows == M:
            break
        rows = min(rows * 2, M)
    times = [dt]
    while spent < budget_s / 2:  # repeat the final sample to about half the budget in all
        t0 = time.perf_counter()
        O.linear(d["x"][:rows], inv, prep)
        times.append(time.perf_counter() - t0)
        spent += times[-1]
    dt = float(np.mean(times))
    ops = layer_ops(rows, d["N"], d["K"], d["rank"])
    try:  # threads the BLAS behind numpy ran with (the oracle's matmuls), bounded by the CPU set
        from threadpoolctl import threadpool_info
        cores = max([p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except ImportError:
        cores = 1
    cores = min(cores, len(os.sched_getaffinity(0)))
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {M} rows of X, {len(times)} run(s) of {dt:.2f}s each (numpy fp64 forward incl. "
                      f"quantization; {spent:.1f}s of CPU work in all)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux_qkv")
    ap.add_argument("--batch", type=int, default=0, help="rows of X for the mxfp4 sweep (default: all)")
    ap.add_argument("--format", default="", choices=["", "int4_g64", "mxfp4_b32", "w8a8"],
                    help="run the workload's layer in another format (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the rank-0 (plain W4A4) comparison run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy a MIB-sized device buffer 3 times (a plain copy of known size, "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU sharding "
              "is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import w4a4_quantized_gemm_smooth_amd as w4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "flux_mlp":
        return mlp_bench(args)
    dev = torch.device("cuda:0")
    d = synth.workload(args.workload)
    if args.batch:
        d = dict(d, x=d["x"][: args.batch], M=args.batch)
    if args.format:
        d = dict(d, fmt=args.format)
    M, K, N, r, fmt = d["x"].shape[0], d["K"], d["N"], d["rank"], d["fmt"]
    log(f"[bench] {args.workload}: M={M} K={K} N={N} r={r} fmt={fmt}")

    t0 = time.perf_counter()
    lam, inv = w4.smooth_factors(w4.column_absmax(d["x"]), w4.column_absmax(d["w"]))
    prep = w4.prepare_weights(d["w"], lam, r, fmt)          # library's own SVD, offline
    log(f"[bench] host weight prep {time.perf_counter() - t0:.1f}s")
    layer = w4.W4A4Linear(prep, inv, device=dev)
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acts = layer.act_buffers(M)
    stream = torch.cuda.current_stream()

    def step():
        layer.quantize(x)
        layer.gemm(acts, M, y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps, nothing else on the stream
    e_begin, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_begin.record(stream)
    for i in range(args.steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms_step = e_begin.elapsed_time(e_end) / args.steps

    # per-kernel launch durations: the same steps again, with HIP events on the launch stream
    # between the kernels (outside the timed region: the events themselves cost a little time)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        layer.quantize(x)
        evs[i][1].record(stream)
        layer.gemm(acts, M, y)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    q_avg = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    g_avg = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # cold-cache view: overwrite a 1 GiB buffer (> 256 MB MALL + L2) before each step, kernels timed by events
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cq, cg = [], []
    for i in range(min(args.steps, 20)):
        flush.fill_(float(i))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        layer.quantize(x)
        ev[1].record(stream)
        layer.gemm(acts, M, y)
        ev[2].record(stream)
        torch.cuda.synchronize()
        cq.append(ev[0].elapsed_time(ev[1]))
        cg.append(ev[1].elapsed_time(ev[2]))
    del flush

    ops = layer_ops(M, N, K, r)
    ms_step = wall * 1e3 / args.steps
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (g_avg * 1e-3) / 1e12
    peak = PEAK_TOPS[fmt]
    peaks = measured_peaks(dev)
    peak_meas = None if peaks is None else peaks["fp4" if fmt == "mxfp4_b32" else "int8"]
    copy_gbs = copy_bandwidth(dev)
    qbytes = quantize_bytes(M, K, r, fmt)
    traffic = traffic_from_profile(os.path.join(ROOT, "w4a4_quantized_gemm_smooth_amd", "csrc", "w4a4_device.hip")) \
        if args.workload == "flux_qkv" and fmt == "int4_g64" else None
    out = {
        "metric": "effective TOPS of fused W4A4+rank-32 linear at FLUX shapes; % MFMA peak",
        "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "event_ms_per_step": round(ev_ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[fmt], "data": "synthetic (seeded FLUX-shaped layer; random weights)",
        "config": {"workload": args.workload, "M": M, "K": K, "N": N, "rank": r, "format": fmt,
                   "ops_per_step": ops, "peak_frac_of_step": round(value / peak, 4)},
        "roofline": {"bound": "mfma", "kernel": gemm_kernel_name(fmt, prep["rank_pad"], M, prep["N"]),
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "avg_launch_ms": round(g_avg, 5), "algorithmic_ops_per_launch": ops,
                     "peak_measured": peak_meas,
                     "frac_measured": None if not peak_meas else round(achieved / peak_meas, 4),
                     "measured_mfma_peaks_TOPS": peaks},
        "kernels": {
            "quantize_act": {"avg_ms_warm": round(q_avg, 5), "avg_ms_cold": round(float(np.mean(cq)), 5),
                             "cold_median_p10_p90_ms": [pct(cq, 50), pct(cq, 10), pct(cq, 90)],
                             "algorithmic_bytes": qbytes,
                             "GB/s_cold": round(qbytes / (np.median(cq) * 1e-3) / 1e9, 1),
                             "hbm_frac_cold": round(qbytes / (np.median(cq) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "copy_GB/s_measured": round(copy_gbs, 1),
                             "frac_of_copy_cold": round(qbytes / (np.median(cq) * 1e-3) / 1e9 / copy_gbs, 4)},
            "gemm": {"avg_ms_warm": round(g_avg, 5), "avg_ms_cold": round(float(np.mean(cg)), 5),
                     "cold_median_p10_p90_ms": [pct(cg, 50), pct(cg, 10), pct(cg, 90)],
                     "TOPS_cold": round(ops / (np.median(cg) * 1e-3) / 1e12, 2)},
        },
    }
    if not args.no_ablation and r > 0:
        # the same layer without the low-rank branch (rank 0: plain W4A4 on the smoothed weight),
        # to report the branch's overhead (§4.3: fused, it should add only a few percent)
        prep0 = w4.prepare_weights(d["w"], lam, 0, fmt)
        layer0 = w4.W4A4Linear(prep0, inv, device=dev)
        acts0 = layer0.act_buffers(M)
        for _ in range(args.warmup):
            layer0.quantize(x)
            layer0.gemm(acts0, M, y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer0.quantize(x)
            layer0.gemm(acts0, M, y)
        torch.cuda.synchronize()
        ms0 = (time.perf_counter() - t0) * 1e3 / args.steps
        # the same branch unfused: separate library GEMMs that re-read X and Y (the pages' baseline)
        l1s, l2 = unfused_lowrank_factors(prep, inv, dev)
        layer_u = unfused_layer(prep, inv, dev)
        acts_u = layer_u.act_buffers(M)
        for _ in range(args.warmup):
            unfused_step(layer_u, acts_u, x, y, l1s, l2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            unfused_step(layer_u, acts_u, x, y, l1s, l2)
        torch.cuda.synchronize()
        msu = (time.perf_counter() - t0) * 1e3 / args.steps
        out["ablation"] = {"rank0_ms_per_step": round(ms0, 5),
                           "lowrank_overhead_pct": round(100.0 * (ms_step - ms0) / ms0, 2),
                           "unfused_ms_per_step": round(msu, 5),
                           "unfused_lowrank_overhead_pct": round(100.0 * (msu - ms0) / ms0, 2)}
        del layer0, acts0, layer_u, acts_u, l1s, l2
        if fmt != "w8a8":
            # the 8-bit setting of App. D (per-token / per-channel INT8, rank 16) on the same layer:
            # its rank-16 factors are the leading 16 of this layer's SVD factors
            r8 = min(16, r)
            prep8 = w4.prepare_weights(d["w"], lam, r8, "w8a8", prep["l1"][:, :r8], prep["l2"][:r8])
            layer8 = w4.W4A4Linear(prep8, inv, device=dev)
            ms8, g8 = time_layer(layer8, x, y, M, args.steps, args.warmup)
            ops8 = layer_ops(M, N, K, r8)
            out["ablation"].update({"w8a8_rank": r8, "w8a8_ms_per_step": round(ms8, 5),
                                    "w8a8_gemm_avg_ms": round(g8, 5),
                                    "w8a8_gemm_TOPS": round(ops8 / (g8 * 1e-3) / 1e12, 2),
                                    "speedup_vs_w8a8": round(ms8 / ms_step, 3)})
            del layer8, prep8
    if args.copy_calibration:
        n = args.copy_calibration << 18   # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            log(f"[bench] copy {args.copy_calibration} MiB: {ms * 1e3:.1f} us, {2 * n * 4 / ms / 1e6:.0f} GB/s (read+write)")
        out["copy_calibration_mib"] = args.copy_calibration
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, lam, inv)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
