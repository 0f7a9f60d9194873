"""Seeded synthetic inputs for the W4A4 + low-rank linear layer.

This module only draws random tensors and stores them as bfloat16 bit patterns; it
holds none of the layer's arithmetic. Both the oracle-side tests and the HIP library's
tests/benchmark take their inputs from here, so both sides see the same bytes.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, fixed draw order):

1. activations X: standard normal [M, K] (fp64 -> fp32);
2. outlier channels: ``rng.choice(K, n_outliers, replace=False)``; those columns of X are
   multiplied by ``outlier_scale`` in fp32; X is then rounded to bf16 (nearest-even);
3. weights W: normal(0, 0.02) [N, K] -> fp32 -> bf16;
4. (LoRA workload) A [K, 16] then B [16, N], normal(0, 0.01) -> bf16.

The MLP workload's second layer takes X2 = bf16(GELU(X1 · W1ᵀ)) (exact erf GELU in fp64),
the activation a real fc2 would see, and W2 ~ normal(0, 0.02) [N2 = K1, K2 = N1].

These stand in for FLUX.1 layer activations and weights, which are not available here.
"""
from __future__ import annotations

import numpy as np

__all__ = ["WORKLOADS", "make_layer", "workload", "f32_to_bf16_bits", "bf16_bits_to_f32", "gelu_erf"]


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (input generation only)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16).reshape(f.shape)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def _activations(rng, m, k, n_outliers, outlier_scale):
    x = rng.standard_normal((m, k)).astype(np.float32)
    idx = np.sort(rng.choice(k, n_outliers, replace=False)) if n_outliers else np.zeros(0, np.int64)
    if n_outliers:
        x[:, idx] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x), idx


def _normal_bf16(rng, shape, std):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def make_layer(m: int, k: int, n: int, *, n_outliers: int, outlier_scale: float, seed: int = 0,
               w_std: float = 0.02, lora_rank: int = 0, lora_std: float = 0.01) -> dict:
    """One synthetic layer: X [m, k] and W [n, k] as bf16 bit patterns (+ optional LoRA A, B)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, idx = _activations(rng, m, k, n_outliers, outlier_scale)
    w = _normal_bf16(rng, (n, k), w_std)
    out = dict(x=x, w=w, outlier_idx=idx, M=m, K=k, N=n)
    if lora_rank:
        out["lora_a"] = _normal_bf16(rng, (k, lora_rank), lora_std)
        out["lora_b"] = _normal_bf16(rng, (lora_rank, n), lora_std)
    return out


# name -> (description, rank, format, shapes)
WORKLOADS = {
    "tiny": dict(M=128, K=256, N=256, rank=16, fmt="int4_g64", n_outliers=4, outlier_scale=50.0),
    "flux_qkv": dict(M=4608, K=3072, N=9216, rank=32, fmt="int4_g64", n_outliers=31, outlier_scale=30.0),
    "flux_mlp_fc1": dict(M=4608, K=3072, N=12288, rank=32, fmt="int4_g64", n_outliers=31, outlier_scale=30.0),
    "flux_mlp_fc2": dict(M=4608, K=12288, N=3072, rank=32, fmt="int4_g64"),
    "flux_qkv_lora": dict(M=4608, K=3072, N=9216, rank=32, lora_rank=16, fmt="int4_g64", n_outliers=31,
                          outlier_scale=30.0),
    "mxfp4_sweep": dict(M=16384, K=3072, N=3072, rank=32, fmt="mxfp4_b32", n_outliers=31, outlier_scale=30.0,
                        batches=(1024, 4608, 16384)),
}


def workload(name: str, seed: int = 0) -> dict:
    """Materialise a named workload. 1% outlier channels of K = 3072 is round(30.72) = 31."""
    spec = dict(WORKLOADS[name])
    if name == "flux_mlp_fc2":
        f1 = WORKLOADS["flux_mlp_fc1"]
        rng = np.random.Generator(np.random.PCG64(seed))
        x1, _ = _activations(rng, f1["M"], f1["K"], f1["n_outliers"], f1["outlier_scale"])  # = fc1's X
        w1 = _normal_bf16(rng, (f1["N"], f1["K"]), 0.02)                                   # = fc1's W
        w2 = _normal_bf16(rng, (f1["K"], f1["N"]), 0.02)
        h = bf16_bits_to_f32(x1).astype(np.float64) @ bf16_bits_to_f32(w1).astype(np.float64).T
        x2 = f32_to_bf16_bits(gelu_erf(h).astype(np.float32))
        out = dict(x=x2, w=w2, outlier_idx=np.zeros(0, np.int64), M=f1["M"], K=f1["N"], N=f1["K"])
    else:
        out = make_layer(spec["M"], spec["K"], spec["N"], n_outliers=spec["n_outliers"],
                         outlier_scale=spec["outlier_scale"], seed=seed, lora_rank=spec.get("lora_rank", 0))
    out.update(name=name, rank=spec["rank"], fmt=spec["fmt"])
    if "batches" in spec:
        out["batches"] = spec["batches"]
    return out
