"""Benchmark of the fused W4A4 + rank-32 linear (SVDQuant layer) on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload flux_qkv]

One step = the whole hot path on one batch already resident in HBM: the activation kernel
(smoothing, group quantization, down projection X̂·L1) followed by the fused 4-bit GEMM with the
low-rank up projection. Prints ONE JSON line on stdout (diagnostics go to stderr):

  value      effective TOPS = (2·M·N·K + 2·M·r·(K+N)) / time per step, the step's time being the
             median over the `steps` timed steps of the step's HIP-event time with cold caches (a
             1 GiB buffer is overwritten before every step, outside the events, so no input is in
             the 256 MB MALL or the L2s); the warm (back-to-back) step is reported beside it
  roofline   the GEMM kernel: algorithmic ops per launch / its average launch time (HIP events on
             the launch stream around each GEMM launch of the timed steps) against the MI355X
             dense int8/fp8 MFMA peak (5.0 POP/s) for INT4 and W8A8, or the MXFP4 peak
             (10.1 PFLOP/s) for the FP4 variant; also against the peak measured on this GPU by
             register-only MFMA chains (libw4a4_peak.so)
  configs    the other workloads of the pages' kernel-level claims, same protocol: the FLUX MLP
             pair (fc2's activation side fused into fc1's GEMM, and consumer-side), the QKV layer
             with a merged rank-16 LoRA (rank 48), and the MXFP4 layer at three batch sizes
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


def new_flush(dev):
    """A 1 GiB buffer; overwriting it evicts everything from the 256 MB MALL and the L2s."""
    import torch
    return torch.empty(1 << 28, dtype=torch.float32, device=dev)


def cold_run(parts, n, flush, read_flush=False):
    """`n` steps of the callables `parts` (run in order on the current stream). Before each step the
    flush buffer is overwritten (not timed); HIP events on the stream time every part. Returns the
    per-step, per-part times [n, len(parts)] in ms and the wall-clock seconds of the whole loop
    (flushes included). With `read_flush` the buffer is read instead (a sum over it): the caches are
    as cold, but the MALL then holds clean lines, so the step does not pay for writing back the
    flush's dirty ones."""
    import torch
    stream = torch.cuda.current_stream()
    out = np.zeros((n, len(parts)))
    sink = torch.zeros((), dtype=torch.float32, device=flush.device)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        if read_flush:
            sink.copy_(flush.sum())
        else:
            flush.fill_(float(i & 7))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
        ev[0].record(stream)
        for k, f in enumerate(parts):
            f()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        out[i] = [ev[k].elapsed_time(ev[k + 1]) for k in range(len(parts))]
    return out, time.perf_counter() - t0


def warm_run(parts, n):
    """`n` back-to-back steps (no flush, no synchronization between them): wall-clock ms per step,
    and per-part event times [n, len(parts)] from a second such pass."""
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        for f in parts:
            f()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(n)]
    for e in evs:
        e[0].record(stream)
        for k, f in enumerate(parts):
            f()
            e[k + 1].record(stream)
    torch.cuda.synchronize()
    return ms, np.array([[e[k].elapsed_time(e[k + 1]) for k in range(len(parts))] for e in evs])


def layer_parts(lay, x, y, M):
    acts = lay.act_buffers(M)
    return [lambda: lay.quantize(x), lambda: lay.gemm(acts, M, y)]


def cold_summary(t, ops_step, gemm_col, gemm_ops, peak):
    """Step and kernel figures of a cold run (t: [n, parts] ms)."""
    step = t.sum(axis=1)
    g = t[:, gemm_col]
    return {"step_ms_cold": round(float(np.median(step)), 5),
            "step_ms_cold_p10_p90": [pct(step, 10), pct(step, 90)],
            "TOPS": round(ops_step / (np.median(step) * 1e-3) / 1e12, 2),
            "kernels_ms_cold": [round(float(np.median(t[:, k])), 5) for k in range(t.shape[1])],
            "gemm_ms_cold_mean": round(float(g.mean()), 5),
            "roofline_frac": round(gemm_ops / (g.mean() * 1e-3) / 1e12 / peak, 4)}


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


def mlp_setup(dev):
    """The FLUX MLP pair fc1 (4608 x 3072 -> 12288) -> GELU -> fc2 (12288 -> 3072), r 32, INT4, and
    the kernel lists of one step. Fused: fc1's activation kernel, fc1's GEMM with fc2's activation
    side in its epilogue (+ the t2 reduction), fc2's GEMM. Consumer-side: fc1's two kernels writing
    Y1, fc2's activation kernel applying the GELU as it reads Y1, fc2's GEMM."""
    import torch
    import synth
    import w4a4_quantized_gemm_smooth_amd as w4
    d1, d2 = synth.workload("flux_mlp_fc1"), synth.workload("flux_mlp_fc2")
    M, K, N, N2, r = d1["M"], d1["K"], d1["N"], d2["N"], d1["rank"]
    log(f"[bench] flux_mlp: fc1 {M}x{K}->{N}, fc2 ->{N2}, r={r}")
    lam1, inv1 = w4.smooth_factors(w4.column_absmax(d1["x"]), w4.column_absmax(d1["w"]))
    lam2, inv2 = w4.smooth_factors(w4.column_absmax(d2["x"]), w4.column_absmax(d2["w"]))
    f1 = w4.W4A4Linear(w4.prepare_weights(d1["w"], lam1, r), inv1, device=dev)
    f2 = w4.W4A4Linear(w4.prepare_weights(d2["w"], lam2, r), inv2, device=dev)
    pair = w4.MLPPair(f1, f2)
    x = torch.from_numpy(np.ascontiguousarray(d1["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    y2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
    b = pair.buffers(M)
    a2 = b["act2"]
    a1 = f1.act_buffers(M)
    fused = [lambda: f1.quantize(x),
             lambda: w4.lowrank_linear_gelu_quant(a1["xq"], a1["xscale"], a1["xl1"], f1.wq, f1.wscale, f1.l2t,
                                                  f1.bias, M, N, K, r, f1.fmt, f2.inv_lambda, f2.l1t, f2.rank,
                                                  a2["xq"], a2["xscale"], b["xl1_2_fused"]),
             lambda: f2.gemm(dict(a2, xl1=b["xl1_2_fused"]), M, y2)]
    unfused = [lambda: f1.quantize(x),
               lambda: f1.gemm(a1, M, b["y1"]),
               lambda: w4.gelu_quantize_act(b["y1"], f2.inv_lambda, f2.l1t, f2.rank, f2.fmt, a2["xq"], a2["xscale"],
                                            a2["xl1"]),
               lambda: f2.gemm(a2, M, y2)]
    ops1, ops2 = layer_ops(M, N, K, r), layer_ops(M, N2, N, r)
    return dict(M=M, K=K, N=N, N2=N2, r=r, fused=fused, unfused=unfused, ops1=ops1, ops2=ops2)


def mlp_entries(mlp, n, warmup, flush):
    """configs entries of the MLP pair: fused and consumer-side, cold, per kernel."""
    out = {}
    peak = PEAK_TOPS["int4_g64"]
    ops = mlp["ops1"] + mlp["ops2"]
    for name, parts, g1, g2 in (("flux_mlp_fused", mlp["fused"], 1, 2), ("flux_mlp_consumer_side", mlp["unfused"], 1, 3)):
        for _ in range(warmup):
            for f in parts:
                f()
        t, _ = cold_run(parts, n, flush)
        e = cold_summary(t, ops, g1, mlp["ops1"], peak)
        e["kernel"] = "gemm_kernel<0, 2, 2>" if g1 == 1 and name.endswith("fused") else "gemm_kernel<0, 2, -1>"
        e["kernels"] = (["fc1_quantize_act", "fc1_gemm_with_fc2_activation_side", "fc2_gemm"] if g2 == 2 else
                        ["fc1_quantize_act", "fc1_gemm", "fc2_gelu_quantize_act", "fc2_gemm"])
        e["fc2_gemm_roofline_frac"] = round(mlp["ops2"] / (t[:, g2].mean() * 1e-3) / 1e12 / peak, 4)
        e["ops_per_step"] = ops
        out[name] = e
    f, u = out["flux_mlp_fused"]["step_ms_cold"], out["flux_mlp_consumer_side"]["step_ms_cold"]
    out["flux_mlp_fused"]["fusion_gain_pct"] = round(100.0 * (u - f) / u, 2)
    return out


def mlp_bench(args):
    """--workload flux_mlp: the fused MLP pair as the headline, with the consumer-side pair beside it."""
    import torch
    dev = torch.device("cuda:0")
    mlp = mlp_setup(dev)
    flush = new_flush(dev)
    ent = mlp_entries(mlp, args.steps, args.warmup, flush)
    f = ent["flux_mlp_fused"]
    ops = f["ops_per_step"]
    gemm_ms = f["gemm_ms_cold_mean"]
    out = {
        "metric": "effective TOPS of fused W4A4+rank-32 linear at FLUX shapes; % MFMA peak",
        "value": f["TOPS"], "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": f["step_ms_cold"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4", "data": "synthetic (seeded FLUX-shaped MLP pair; random weights)",
        "config": {"workload": "flux_mlp", "M": mlp["M"], "K": mlp["K"], "N": mlp["N"], "N2": mlp["N2"],
                   "rank": mlp["r"], "format": "int4_g64", "ops_per_step": ops, "caches": "cold",
                   "path": "fc2's activation side fused into fc1's GEMM epilogue"},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel<0, 2, 2>",
                     "achieved": round(mlp["ops1"] / (gemm_ms * 1e-3) / 1e12, 2), "peak": PEAK_TOPS["int4_g64"],
                     "unit": "TOPS", "frac": f["roofline_frac"], "traffic": None, "avg_launch_ms": gemm_ms,
                     "algorithmic_ops_per_launch": mlp["ops1"]},
        "configs": ent,
    }
    print(json.dumps(out), flush=True)


def lora_layer(dev):
    """The FLUX QKV layer with a rank-16 LoRA merged into its low-rank branch (rank 32 + 16 = 48)."""
    import synth
    import w4a4_quantized_gemm_smooth_amd as w4
    d = synth.workload("flux_qkv_lora")
    lam, inv = w4.smooth_factors(w4.column_absmax(d["x"]), w4.column_absmax(d["w"]))
    prep = w4.prepare_weights(d["w"], lam, 32, "int4_g64")
    l1t, l2t, r2 = w4.append_lowrank(prep["l1t"], prep["l2t"], d["K"], d["N"], 32, d["lora_a"], d["lora_b"])
    return d, w4.W4A4Linear(dict(prep, l1t=l1t, l2t=l2t, rank=r2, rank_pad=48), inv, device=dev)


def configs_block(dev, n, warmup, flush):
    """The configs entries beyond the headline layer (cold protocol, `n` steps each)."""
    import torch
    import synth
    import w4a4_quantized_gemm_smooth_amd as w4
    out = {}
    t0 = time.perf_counter()
    out.update(mlp_entries(mlp_setup(dev), n, warmup, flush))
    log(f"[bench] configs: MLP pair done ({time.perf_counter() - t0:.0f}s)")
    d, lay = lora_layer(dev)
    M, K, N = d["M"], d["K"], d["N"]
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    parts = layer_parts(lay, x, y, M)
    warm_run(parts, warmup)
    t, _ = cold_run(parts, n, flush)
    ops = layer_ops(M, N, K, 48)
    out["flux_qkv_lora_r48"] = dict(cold_summary(t, ops, 1, ops, PEAK_TOPS["int4_g64"]), kernel="gemm_kernel<0, 3, -1>",
                                    kernels=["quantize_act", "gemm"], ops_per_step=ops)
    del lay, x, y
    d = synth.workload("mxfp4_sweep")
    K, N, r = d["K"], d["N"], d["rank"]
    lam, inv = w4.smooth_factors(w4.column_absmax(d["x"]), w4.column_absmax(d["w"]))
    lay = w4.W4A4Linear(w4.prepare_weights(d["w"], lam, r, "mxfp4_b32"), inv, device=dev)
    xall = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    for M in d["batches"]:
        x = xall[:M]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        parts = layer_parts(lay, x, y, M)
        warm_run(parts, warmup)
        t, _ = cold_run(parts, n, flush)
        ops = layer_ops(M, N, K, r)
        out[f"mxfp4_m{M}"] = dict(cold_summary(t, ops, 1, ops, PEAK_TOPS["mxfp4_b32"]),
                                 kernel=gemm_kernel_name("mxfp4_b32", 32, M, N), kernels=["quantize_act", "gemm"],
                                 ops_per_step=ops)
    log(f"[bench] configs done ({time.perf_counter() - t0:.0f}s)")
    return out


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (MLP pair, LoRA r48, MXFP4 sweep)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy a MIB-sized device buffer 3 times (a plain copy of known size, "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer's multi-GPU sharding "
              "(token-, column- or row-parallel) is not built.", file=sys.stderr)
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
    stream = torch.cuda.current_stream()

    parts = layer_parts(layer, x, y, M)
    warm_run(parts, args.warmup)
    flush = new_flush(dev)

    # the timed region: exactly `steps` steps, each preceded by a cache flush outside its events
    torch.cuda.synchronize()
    tc, wall = cold_run(parts, args.steps, flush)
    torch.cuda.synchronize()
    step_c = tc.sum(axis=1)
    ms_step = float(np.median(step_c))
    q_c, g_c = tc[:, 0], tc[:, 1]
    g_avg = float(g_c.mean())   # the GEMM's average launch time over the timed steps
    # the warm view: back-to-back steps, inputs left in the MALL by the previous step
    warm_ms, tw = warm_run(parts, args.steps)
    # cold caches without the write-back of the flush's dirty lines (a read sweep of the buffer)
    tr = cold_run(parts, min(args.steps, 20), flush, read_flush=True)[0]

    ops = layer_ops(M, N, K, r)
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (g_avg * 1e-3) / 1e12
    peak = PEAK_TOPS[fmt]
    peaks = measured_peaks(dev)
    peak_meas = None if peaks is None else peaks["fp4" if fmt == "mxfp4_b32" else "int8"]
    copy_gbs = copy_bandwidth(dev)
    qbytes = quantize_bytes(M, K, r, fmt)
    traffic = traffic_from_profile(os.path.join(ROOT, "w4a4_quantized_gemm_smooth_amd", "csrc", "w4a4_device.hip")) \
        if args.workload == "flux_qkv" and fmt == "int4_g64" else None
    q_med = float(np.median(q_c))
    out = {
        "metric": "effective TOPS of fused W4A4+rank-32 linear at FLUX shapes; % MFMA peak",
        "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[fmt], "data": "synthetic (seeded FLUX-shaped layer; random weights)",
        "config": {"workload": args.workload, "M": M, "K": K, "N": N, "rank": r, "format": fmt,
                   "ops_per_step": ops, "caches": "cold (1 GiB overwritten before each step, not timed)",
                   "peak_frac_of_step": round(value / peak, 4)},
        "timing": {"ms_per_step_cold_median": round(ms_step, 5),
                   "ms_per_step_cold_p10_p90": [pct(step_c, 10), pct(step_c, 90)],
                   "ms_per_step_cold_readflush_median": round(float(np.median(tr.sum(axis=1))), 5),
                   "ms_per_step_warm": round(warm_ms, 5),
                   "TOPS_warm": round(ops / (warm_ms * 1e-3) / 1e12, 2),
                   "wall_s_timed_loop_incl_flushes": round(wall, 4)},
        "roofline": {"bound": "mfma", "kernel": gemm_kernel_name(fmt, prep["rank_pad"], M, prep["N"]),
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TOPS",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "avg_launch_ms": round(g_avg, 5), "algorithmic_ops_per_launch": ops,
                     "peak_measured": peak_meas,
                     "frac_measured": None if not peak_meas else round(achieved / peak_meas, 4),
                     "measured_mfma_peaks_TOPS": peaks},
        "kernels": {
            "quantize_act": {"ms_cold_median_p10_p90": [round(q_med, 5), pct(q_c, 10), pct(q_c, 90)],
                             "ms_warm_mean": round(float(tw[:, 0].mean()), 5),
                             "ms_cold_readflush_median": pct(tr[:, 0], 50),
                             "algorithmic_bytes": qbytes,
                             "GB/s_cold": round(qbytes / (q_med * 1e-3) / 1e9, 1),
                             "hbm_frac_cold": round(qbytes / (q_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "copy_GB/s_measured": round(copy_gbs, 1),
                             "frac_of_copy_cold": round(qbytes / (q_med * 1e-3) / 1e9 / copy_gbs, 4)},
            "gemm": {"ms_cold_median_p10_p90": [pct(g_c, 50), pct(g_c, 10), pct(g_c, 90)],
                     "ms_cold_mean": round(g_avg, 5), "ms_warm_mean": round(float(tw[:, 1].mean()), 5),
                     "ms_cold_readflush_median": pct(tr[:, 1], 50),
                     "TOPS_cold": round(ops / (np.median(g_c) * 1e-3) / 1e12, 2)},
        },
    }
    if not args.no_ablation and r > 0:
        # the same layer without the low-rank branch (rank 0: plain W4A4 on the smoothed weight),
        # to report the branch's overhead (§4.3: fused, it should add only a few percent)
        n_ab = min(args.steps, 20)
        prep0 = w4.prepare_weights(d["w"], lam, 0, fmt)
        layer0 = w4.W4A4Linear(prep0, inv, device=dev)
        p0 = layer_parts(layer0, x, y, M)
        warm_run(p0, args.warmup)
        ms0 = float(np.median(cold_run(p0, n_ab, flush)[0].sum(axis=1)))
        # the same branch unfused: separate library GEMMs that re-read X and Y (the pages' baseline)
        l1s, l2 = unfused_lowrank_factors(prep, inv, dev)
        layer_u = unfused_layer(prep, inv, dev)
        acts_u = layer_u.act_buffers(M)
        pu = [lambda: unfused_step(layer_u, acts_u, x, y, l1s, l2)]
        warm_run(pu, args.warmup)
        msu = float(np.median(cold_run(pu, n_ab, flush)[0].sum(axis=1)))
        out["ablation"] = {"caches": "cold", "rank0_ms_per_step": round(ms0, 5),
                           "lowrank_overhead_pct": round(100.0 * (ms_step - ms0) / ms0, 2),
                           "unfused_ms_per_step": round(msu, 5),
                           "unfused_lowrank_overhead_pct": round(100.0 * (msu - ms0) / ms0, 2)}
        del layer0, layer_u, acts_u, l1s, l2
        if fmt != "w8a8":
            # the 8-bit setting of App. D (per-token / per-channel INT8, rank 16) on the same layer:
            # its rank-16 factors are the leading 16 of this layer's SVD factors
            r8 = min(16, r)
            prep8 = w4.prepare_weights(d["w"], lam, r8, "w8a8", prep["l1"][:, :r8], prep["l2"][:r8])
            layer8 = w4.W4A4Linear(prep8, inv, device=dev)
            p8 = layer_parts(layer8, x, y, M)
            warm_run(p8, args.warmup)
            t8 = cold_run(p8, n_ab, flush)[0]
            ms8 = float(np.median(t8.sum(axis=1)))
            ops8 = layer_ops(M, N, K, r8)
            out["ablation"].update({"w8a8_rank": r8, "w8a8_ms_per_step": round(ms8, 5),
                                    "w8a8_gemm_ms": round(float(t8[:, 1].mean()), 5),
                                    "w8a8_gemm_TOPS": round(ops8 / (t8[:, 1].mean() * 1e-3) / 1e12, 2),
                                    "speedup_vs_w8a8": round(ms8 / ms_step, 3)})
            del layer8, prep8
    if not args.no_configs and args.workload == "flux_qkv" and not args.format and not args.batch:
        out["configs"] = configs_block(dev, min(args.steps, 20), min(args.warmup, 5), flush)
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
