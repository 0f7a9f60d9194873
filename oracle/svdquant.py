"""SVDQuant W4A4 + 16-bit low-rank linear layer, written out step by step (oracle).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never by the product library.

Source: the web summary of "SVDQuant: Absorbing Outliers by Low-Rank Components
for 4-Bit Diffusion Models" (Li et al., arXiv 2411.05007v4). Section names below
refer to that page:

* §3 "Quantization preliminary": signed k-bit integer qmax = 2^(k-1) - 1; FP4 with
  2 exponent bits and 1 mantissa bit has qmax 6; dequantization multiplies the
  low-bit tensor by its scale.
* §4.2: activation outliers are migrated into the weights (smoothing), the
  smoothed weight is split by SVD into a 16-bit low-rank branch L1·L2 and a
  residual R that is quantized to 4 bits.
* §4.3 / Fig. 6: the down projection X̂·L1 shares the activations with the
  quantizer; the up projection is added to the 4-bit GEMM's output.
* App. D "Implementation details": per-group symmetric 4-bit quantization of
  activations and weights, group size 64, 16-bit scales, rank 32; per-channel
  smoothing factor from activation and weight maxima with migration strength α,
  following SmoothQuant.
* §A.1: Proposition 4.1 error bound (used by the tests as an invariant).

The layer computed here is

    Y = Q(X̂) · Q(R)ᵀ + bf16(bf16(X̂) · L1) · L2 (+ bias),   X̂ = X · diag(λ)^-1,
    Ŵ = W · diag(λ),  Ŵᵀ ≈ L1 · L2 (rank r),  R = Ŵ − (L1 · L2)ᵀ.

Readings of points the page leaves open (all listed in the design notes):

* α = 0.5, so λ_j = sqrt(max|X_j| / max|W_j|); λ_j = 1 when either max is 0.
* "16-bit" scales and low-rank factors are bfloat16, rounded to nearest-even.
  Any fp64 value that becomes bf16 is rounded to fp32 first, then to bf16.
* The scale used to quantize is the stored 16-bit scale; codes are
  round-half-to-even of (v · fp32(1/s)) clamped to [-8, 7]; a group whose scale
  is zero or below the smallest normal fp32 (2^-126) gets scale 0 and codes 0.
* The singular values go into L1 (L1 = U_r Σ_r, L2 = V_rᵀ); each singular pair's
  sign is fixed so that the largest-magnitude entry of its L1 column is positive
  (ties: lowest index).
* The residual is formed from the bf16-rounded factors, with the rank-r dot
  product summed in fp64 in increasing rank order, then rounded to fp32.
* The down projection t = bf16(X̂)·L1 is rounded to bf16 (through fp32) before
  the up projection ("16-bit low-rank branch").
* The FP4 variant uses MX-style blocks of 32 along K with a power-of-two scale
  2^e, e the smallest integer with 6·2^e >= max|v| (the power-of-two round-up of
  max|v|/qmax); element codes are E2M1 round-half-to-even of v / 2^e; the sign
  bit of v is kept even when the magnitude rounds to 0.
* The MLP pair (fc1 → GELU → fc2) joined at the producer: fc2's activations are
  X₂ = bf16(GELU(Y₁)) of fc1's bf16 output Y₁, with GELU(y) = y/2 · (1 + erf(y/√2))
  evaluated in fp32 and erf taken from Abramowitz & Stegun 7.1.28 (a rational form
  with |error| ≤ 3e-7, no exponential), so that a GPU kernel can take the same
  fp32 steps and both sides round X₂ (and so decide fc2's codes) identically.
"""
from __future__ import annotations

import numpy as np

GROUP = 64            # App. D: group size 64 along the input channels
QMAX_INT4 = 7         # §3: signed k-bit integer, qmax = 2^(k-1) - 1 with k = 4
MX_BLOCK = 32         # FP4 variant: block of 32 elements share one power-of-two scale
QMAX_FP4 = 6.0        # §3: FP4 with 2 exponent bits and 1 mantissa bit has qmax 6
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # magnitude of code 0..7

QMAX_INT8 = 127       # §3 with k = 8 (the 8-bit SVDQuant setting, App. D)

FMT_INT4_G64 = "int4_g64"
FMT_MXFP4_B32 = "mxfp4_b32"
FMT_W8A8 = "w8a8"     # per-token INT8 activations, per-output-channel INT8 weights, fp32 scales


# ----------------------------------------------------------------------------------------
# 16-bit float helpers (the oracle's own; nothing here is shared with the HIP library)
# ----------------------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_rne(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returned as float32.

    fp64 inputs are first rounded to float32 (the two-step rounding every fp64 -> bf16
    conversion in this module uses)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 values that are already bf16-representable -> uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------------------
# Smoothing (§4.2, App. D)
# ----------------------------------------------------------------------------------------
def column_absmax(a: np.ndarray) -> np.ndarray:
    """max_i |a[i, j]| per column j, in float32 (exact: a maximum of float32 magnitudes)."""
    return np.max(np.abs(np.asarray(a, dtype=np.float32)), axis=0).astype(np.float32)


def smooth_factors(amax_x: np.ndarray, amax_w: np.ndarray, alpha: float = 0.5):
    """Per-channel smoothing factor λ_j = max|X_j|^α / max|W_j|^(1-α) (App. D, after SmoothQuant).

    α = 0.5 is evaluated as fp32(sqrt_f64(max|X_j| / max|W_j|)); other α as
    fp32(pow(max|X_j|, α) / pow(max|W_j|, 1-α)) in fp64. A channel whose activation or
    weight maximum is 0 gets λ_j = 1. Returns (λ, 1/λ) as float32, the reciprocal being
    the IEEE float32 quotient 1.0f / λ_j.
    """
    ax = np.asarray(amax_x, dtype=np.float32).astype(np.float64)
    aw = np.asarray(amax_w, dtype=np.float32).astype(np.float64)
    lam = np.ones(ax.shape, dtype=np.float32)
    ok = (ax > 0) & (aw > 0)
    if alpha == 0.5:
        lam[ok] = np.sqrt(ax[ok] / aw[ok]).astype(np.float32)
    else:
        lam[ok] = (np.power(ax[ok], alpha) / np.power(aw[ok], 1.0 - alpha)).astype(np.float32)
    if not np.all(np.isfinite(lam)) or np.any(lam < np.float32(2.0 ** -126)):
        raise FloatingPointError("smoothing factor is not a finite normal float32")
    inv = (np.float32(1.0) / lam).astype(np.float32)
    return lam, inv


def smooth_activations(x: np.ndarray, inv_lam: np.ndarray) -> np.ndarray:
    """X̂ = X · diag(λ)^-1 as one float32 multiply per element by the stored 1/λ."""
    return (np.asarray(x, dtype=np.float32) * np.asarray(inv_lam, dtype=np.float32)[None, :]).astype(np.float32)


def smooth_weights(w: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """Ŵ = W · diag(λ) in fp64 (exact for bf16 W and float32 λ)."""
    return np.asarray(w, dtype=np.float64) * np.asarray(lam, dtype=np.float64)[None, :]


# ----------------------------------------------------------------------------------------
# Low-rank branch (§4.2, Fig. 4)
# ----------------------------------------------------------------------------------------
def truncated_svd(w_hat: np.ndarray, rank: int):
    """Rank-r truncated SVD of Ŵᵀ [K, N] with the sign convention of the module docstring.

    Returns (U_r [K, r], sigma_r [r], V_r [N, r]) in fp64 and the full singular values."""
    u, s, vt = np.linalg.svd(np.asarray(w_hat, dtype=np.float64).T, full_matrices=False)
    u = u[:, :rank].copy()
    v = vt[:rank, :].T.copy()
    if rank:
        lead = np.argmax(np.abs(u), axis=0)            # first occurrence = lowest index
        sgn = np.sign(u[lead, np.arange(rank)])
        sgn[sgn == 0] = 1.0
        u *= sgn[None, :]
        v *= sgn[None, :]
    return u, s[:rank].copy(), v, s


def lowrank_split(w_hat: np.ndarray, rank: int):
    """L1 = bf16(U_r Σ_r) [K, r] and L2 = bf16(V_rᵀ) [r, N] (float32 arrays holding bf16 values)."""
    u, s, v, _ = truncated_svd(w_hat, rank)
    l1 = bf16_rne((u * s[None, :]).astype(np.float32))
    l2 = bf16_rne(v.T.astype(np.float32))
    return l1, l2


def lowrank_product_t(l1: np.ndarray, l2: np.ndarray) -> np.ndarray:
    """(L1 · L2) [K, N] in fp64, summed over the rank index in increasing order."""
    l1 = np.asarray(l1, dtype=np.float64)
    l2 = np.asarray(l2, dtype=np.float64)
    d = np.zeros((l1.shape[0], l2.shape[1]), dtype=np.float64)
    for i in range(l1.shape[1]):
        d += np.outer(l1[:, i], l2[i, :])
    return d


def residual(w_hat: np.ndarray, l1: np.ndarray, l2: np.ndarray) -> np.ndarray:
    """R = fp32(Ŵ − (L1 L2)ᵀ) [N, K] (§4.2: the part left for the 4-bit branch)."""
    d = lowrank_product_t(l1, l2)
    return (np.asarray(w_hat, dtype=np.float64) - d.T).astype(np.float32)


# ----------------------------------------------------------------------------------------
# 4-bit quantizers (§3, App. D)
# ----------------------------------------------------------------------------------------
def quant_int4_g64(v: np.ndarray):
    """Per-group (64 along K) symmetric INT4 quantization with bf16 scales.

    s = bf16(fp32(max|v| / 7)); q = clamp(rint(fp32(v · fp32(1/s))), -8, 7).
    Returns (codes int8 [rows, K], scales float32-with-bf16-values [rows, K/64])."""
    v = np.asarray(v, dtype=np.float32)
    rows, k = v.shape
    assert k % GROUP == 0
    vg = v.reshape(rows, k // GROUP, GROUP)
    amax = np.max(np.abs(vg), axis=2)
    s = bf16_rne((amax / np.float32(QMAX_INT4)).astype(np.float32))
    s[s < np.float32(2.0 ** -126)] = 0.0
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    inv = np.where(s > 0, np.float32(1.0) / safe, np.float32(0.0)).astype(np.float32)
    y = (vg * inv[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(y), -8, 7).astype(np.int8)
    return q.reshape(rows, k), s.astype(np.float32)


def dequant_int4_g64(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """s ⊙ q in fp64 (§3: dequantization multiplies the low-bit tensor by its scale)."""
    rows, k = q.shape
    return (np.asarray(q, dtype=np.float64).reshape(rows, k // GROUP, GROUP)
            * np.asarray(s, dtype=np.float64)[:, :, None]).reshape(rows, k)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Canonical packing: row-major [rows, K/2] bytes, element 2i in the low nibble,
    two's-complement nibbles."""
    q = np.asarray(q, dtype=np.int16)
    lo = (q[:, 0::2] & 0xF).astype(np.uint8)
    hi = (q[:, 1::2] & 0xF).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def mx_exponent(amax: np.ndarray) -> np.ndarray:
    """e = the smallest integer with 6·2^e >= amax (amax > 0), clamped to [-127, 127];
    e = -127 for amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(a)                   # a = m · 2^ex, m in [0.5, 1)
    e = np.where(m <= 0.75, ex - 3, ex - 2).astype(np.int64)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127)


def e2m1_round(y: np.ndarray) -> np.ndarray:
    """E2M1 code (sign bit | 3-bit magnitude index) of float y, |y| <= 6:
    nearest grid magnitude, ties to the even index (even mantissa bit); sign = signbit(y)."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    d = np.abs(mag[..., None] - E2M1_GRID)          # distance to each of the 8 magnitudes
    best = np.min(d, axis=-1, keepdims=True)
    cand = d == best
    idx = np.where(cand[..., 0::2].any(-1),
                   2 * np.argmax(cand[..., 0::2], axis=-1),   # an even index is among the nearest
                   2 * np.argmax(cand[..., 1::2], axis=-1) + 1)
    sign = np.signbit(y).astype(np.int64)
    return (sign << 3 | idx).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    v = E2M1_GRID[code & 7]
    return np.where(code & 8, -v, v)


def quant_mxfp4_b32(v: np.ndarray):
    """FP4 (E2M1) codes with one power-of-two scale per block of 32 along K.

    Returns (codes uint8 [rows, K] in 0..15, e8m0 uint8 [rows, K/32] = e + 127)."""
    v = np.asarray(v, dtype=np.float32)
    rows, k = v.shape
    assert k % MX_BLOCK == 0
    vb = v.reshape(rows, k // MX_BLOCK, MX_BLOCK)
    e = mx_exponent(np.max(np.abs(vb), axis=2))
    y = np.ldexp(vb.astype(np.float64), (-e)[:, :, None])
    codes = e2m1_round(y)
    return codes.reshape(rows, k), (e + 127).astype(np.uint8)


def dequant_mxfp4_b32(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    rows, k = codes.shape
    val = e2m1_value(codes).reshape(rows, k // MX_BLOCK, MX_BLOCK)
    return np.ldexp(val, (np.asarray(e8m0, dtype=np.int64) - 127)[:, :, None]).reshape(rows, k)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Row-major [rows, K/2] bytes from 4-bit codes 0..15, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


# ----------------------------------------------------------------------------------------
# The two branches and the layer (§4.2, §4.3)
# ----------------------------------------------------------------------------------------
def lowrank_down(x_hat: np.ndarray, l1: np.ndarray) -> np.ndarray:
    """t = bf16(X̂) · L1 in fp64 [M, r] (the down projection that shares X̂ with the quantizer)."""
    return bf16_rne(x_hat).astype(np.float64) @ np.asarray(l1, dtype=np.float64)


def lowrank_up(t: np.ndarray, l2: np.ndarray) -> np.ndarray:
    """Y_l = bf16(fp32(t)) · L2 in fp64 [M, N]."""
    return bf16_rne(np.asarray(t).astype(np.float32)).astype(np.float64) @ np.asarray(l2, dtype=np.float64)


def main_branch_int4(qx, sx, qw, sw) -> np.ndarray:
    """Y_m = Σ_g s_x[m,g]·s_w[n,g]·Σ_{k∈g} q_x[m,k]·q_w[n,k], integer partial sums in fp64."""
    qx = np.asarray(qx, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    sx = np.asarray(sx, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    y = np.zeros((qx.shape[0], qw.shape[0]), dtype=np.float64)
    for g in range(qx.shape[1] // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        p = qx[:, ks] @ qw[:, ks].T
        y += (sx[:, g, None] * sw[None, :, g]) * p
    return y


def main_branch_mxfp4(cx, ex, cw, ew) -> np.ndarray:
    """Y_m = Σ_b 2^(e_x[m,b] + e_w[n,b]) · Σ_{k∈b} val(c_x[m,k])·val(c_w[n,k]) in fp64."""
    vx = e2m1_value(cx)
    vw = e2m1_value(cw)
    ex = np.asarray(ex, dtype=np.int64) - 127
    ew = np.asarray(ew, dtype=np.int64) - 127
    y = np.zeros((vx.shape[0], vw.shape[0]), dtype=np.float64)
    for b in range(vx.shape[1] // MX_BLOCK):
        ks = slice(b * MX_BLOCK, (b + 1) * MX_BLOCK)
        y += np.ldexp(vx[:, ks] @ vw[:, ks].T, ex[:, b, None] + ew[None, :, b])
    return y


def quant_int8_rows(v: np.ndarray):
    """The 8-bit setting (App. D): one symmetric INT8 scale per row — per token for activations,
    per output channel for weights — kept in fp32.

    s = fp32(max|v| / 127); q = clamp(rint(fp32(v · fp32(1/s))), -127, 127); a row whose scale is
    zero or below 2^-126 gets scale 0 and codes 0. Returns (codes int8 [rows, K], scales float32
    [rows])."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1)
    s = (amax / np.float32(QMAX_INT8)).astype(np.float32)
    s[s < np.float32(2.0 ** -126)] = 0.0
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    inv = np.where(s > 0, np.float32(1.0) / safe, np.float32(0.0)).astype(np.float32)
    y = (v * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(y), -QMAX_INT8, QMAX_INT8).astype(np.int8)
    return q, s


def dequant_int8_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[:, None]


def main_branch_w8a8(qx, sx, qw, sw) -> np.ndarray:
    """Y_m = s_x[m]·s_w[n]·Σ_k q_x[m,k]·q_w[n,k], the integer sum exact in int64."""
    p = np.asarray(qx, dtype=np.int64) @ np.asarray(qw, dtype=np.int64).T
    return (np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]) * p.astype(np.float64)


def quantize(v: np.ndarray, fmt: str):
    """(codes, scales) of a [rows, K] float32 tensor in the given low-bit format."""
    if fmt == FMT_INT4_G64:
        return quant_int4_g64(v)
    if fmt == FMT_MXFP4_B32:
        return quant_mxfp4_b32(v)
    if fmt == FMT_W8A8:
        return quant_int8_rows(v)
    raise ValueError(fmt)


def main_branch(cx, sx, cw, sw, fmt: str) -> np.ndarray:
    if fmt == FMT_INT4_G64:
        return main_branch_int4(cx, sx, cw, sw)
    if fmt == FMT_W8A8:
        return main_branch_w8a8(cx, sx, cw, sw)
    return main_branch_mxfp4(cx, sx, cw, sw)


def prepare_weights(w_bits: np.ndarray, lam: np.ndarray, rank: int, fmt: str = FMT_INT4_G64,
                    l1: np.ndarray | None = None, l2: np.ndarray | None = None):
    """Offline weight preparation (§4.2): smooth, split off the rank-r branch, quantize R.

    ``l1``/``l2`` (float32 with bf16 values) replace the SVD when given (e.g. after a LoRA merge)."""
    w = bf16_bits_to_f32(w_bits)
    w_hat = smooth_weights(w, lam)
    if l1 is None:
        l1, l2 = lowrank_split(w_hat, rank)
    r = residual(w_hat, l1, l2)
    cw, sw = quantize(r, fmt)
    return dict(w_hat=w_hat, l1=np.asarray(l1, np.float32), l2=np.asarray(l2, np.float32), r=r,
                cw=cw, sw=sw, fmt=fmt)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """The 4-bit tensor's values in fp64 (§3: the low-bit tensor times its scale)."""
    if fmt == FMT_INT4_G64:
        return dequant_int4_g64(codes, scales)
    if fmt == FMT_W8A8:
        return dequant_int8_rows(codes, scales)
    return dequant_mxfp4_b32(codes, scales)


def split_error(w_hat: np.ndarray, l1: np.ndarray, l2: np.ndarray, cw: np.ndarray, sw: np.ndarray,
                fmt: str) -> float:
    """||Ŵ − (L1 L2)ᵀ − deq(Q(R))||_F in fp64: the part of the smoothed weight that neither the
    16-bit branch nor the 4-bit branch represents."""
    miss = np.asarray(w_hat, np.float64) - lowrank_product_t(l1, l2).T - dequantize(cw, sw, fmt)
    return float(np.sqrt(np.sum(miss * miss)))


def prepare_weights_refined(w_bits: np.ndarray, lam: np.ndarray, rank: int, fmt: str = FMT_INT4_G64,
                            iters: int = 3):
    """§4.2's iterative refinement of the split. The page says only that iterative updates reduce
    the quantization error further and that the result with the smallest error after several
    iterations is kept; the reading taken: alternate the two branches. Iteration 0 is
    ``prepare_weights``; iteration i >= 1 re-fits the low-rank branch to what the current 4-bit
    branch misses, L1·L2 = SVD_r(Ŵ − deq(Q(R_{i-1})))ᵀ, and quantizes R_i = Ŵ − (L1·L2)ᵀ afresh.
    Every iteration is scored by ``split_error``; the one with the smallest error wins (the
    earliest on ties). Returns ``prepare_weights``' dict plus ``errors`` (all iterations) and
    ``iteration`` (the winner)."""
    w_hat = smooth_weights(bf16_bits_to_f32(w_bits), lam)
    target = w_hat
    errors, best = [], None
    for it in range(iters + 1):
        l1, l2 = lowrank_split(target, rank)
        r = residual(w_hat, l1, l2)
        cw, sw = quantize(r, fmt)
        e = split_error(w_hat, l1, l2, cw, sw, fmt)
        errors.append(e)
        if best is None or e < errors[best[0]]:
            best = (it, dict(w_hat=w_hat, l1=np.asarray(l1, np.float32), l2=np.asarray(l2, np.float32), r=r,
                             cw=cw, sw=sw, fmt=fmt))
        target = w_hat - dequantize(cw, sw, fmt)
    out = best[1]
    out.update(errors=errors, iteration=best[0])
    return out


def quantize_activations(x_bits: np.ndarray, inv_lam: np.ndarray, l1: np.ndarray, fmt: str = FMT_INT4_G64):
    """The activation side: X̂, its codes and scales, and the down projection t (fp64)."""
    x_hat = smooth_activations(bf16_bits_to_f32(x_bits), inv_lam)
    cx, sx = quantize(x_hat, fmt)
    t = lowrank_down(x_hat, l1)
    return dict(x_hat=x_hat, cx=cx, sx=sx, t=t)


def linear(x_bits: np.ndarray, inv_lam: np.ndarray, prep: dict, bias_bits: np.ndarray | None = None):
    """The whole layer; returns dict with Y (float32 holding bf16 values) and its parts."""
    act = quantize_activations(x_bits, inv_lam, prep["l1"], prep["fmt"])
    y_m = main_branch(act["cx"], act["sx"], prep["cw"], prep["sw"], prep["fmt"])
    y_l = lowrank_up(act["t"], prep["l2"])
    y = y_m + y_l
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    act.update(y_m=y_m, y_l=y_l, y=bf16_rne(y.astype(np.float32)))
    return act


def linear_unquantized(x: np.ndarray, inv_lam: np.ndarray, r: np.ndarray, l1: np.ndarray, l2: np.ndarray):
    """Special case with quantization and 16-bit rounding switched off:
    X̂·Rᵀ + (X̂·L1)·L2 in fp64 (for r = 0 this is X̂·Ŵᵀ, i.e. X·Wᵀ up to fp32 rounding)."""
    x_hat = smooth_activations(x, inv_lam).astype(np.float64)
    return x_hat @ np.asarray(r, np.float64).T + (x_hat @ np.asarray(l1, np.float64)) @ np.asarray(l2, np.float64)


def prop41_terms(x: np.ndarray, w: np.ndarray, qx: np.ndarray, qw: np.ndarray):
    """Both sides of Proposition 4.1 (§4.1, §A.1): E = ||XWᵀ − Q(X)Q(W)ᵀ||_F and
    ||X||F ||W−Q(W)||F + ||X−Q(X)||F (||W||F + ||W−Q(W)||F)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    qx = np.asarray(qx, np.float64)
    qw = np.asarray(qw, np.float64)
    err = np.linalg.norm(x @ w.T - qx @ qw.T)
    fro = np.linalg.norm
    bound = fro(x) * fro(w - qw) + fro(x - qx) * (fro(w) + fro(w - qw))
    return err, bound


# ---------------------------------------------------------------- MLP producer: GELU → fc2 codes
# Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.28:
#   erf(x) ≈ 1 − (1 + a1 x + a2 x² + a3 x³ + a4 x⁴ + a5 x⁵ + a6 x⁶)^−16 for x ≥ 0, |ε| ≤ 3e−7.
AS7128 = (0.0705230784, 0.0422820123, 0.0092705272, 0.0001520143, 0.0002765672, 0.0000430638)
INV_SQRT2_F32 = np.float32(0.70710678118654752)


def erf32(x) -> np.ndarray:
    """erf in fp32 by A&S 7.1.28, one IEEE fp32 operation at a time: the polynomial by Horner's
    rule from a6 down (multiply, then add), the 16th power by four squarings, 1 − 1/p¹⁶, and the
    sign of x restored (erf is odd)."""
    x = np.asarray(x, dtype=np.float32)
    ax = np.abs(x)
    f = np.float32
    p = np.full_like(ax, f(AS7128[5]))
    with np.errstate(over="ignore", divide="ignore"):  # p overflows to inf for large |x|: erf = ±1
        for a in (AS7128[4], AS7128[3], AS7128[2], AS7128[1], AS7128[0], 1.0):
            p = (p * ax).astype(np.float32)
            p = (p + f(a)).astype(np.float32)
        for _ in range(4):
            p = (p * p).astype(np.float32)
        e = (f(1.0) - (f(1.0) / p).astype(np.float32)).astype(np.float32)
    return np.where(x < 0, -e, e).astype(np.float32)


def gelu32(y) -> np.ndarray:
    """GELU(y) = (y/2)·(1 + erf(y/√2)) in fp32: u = y·fp32(1/√2), e = erf32(u), (0.5·y)·(1 + e)."""
    y = np.asarray(y, dtype=np.float32)
    e = erf32((y * INV_SQRT2_F32).astype(np.float32))
    return ((np.float32(0.5) * y).astype(np.float32) * (np.float32(1.0) + e).astype(np.float32)).astype(np.float32)


def gelu_quantize(y1_bits: np.ndarray, inv_lam2: np.ndarray, l1_2: np.ndarray, fmt: str = FMT_INT4_G64):
    """fc2's activation side computed from fc1's bf16 output Y₁ (bit patterns): X₂ = bf16(GELU(Y₁)),
    then the ordinary activation side of fc2 (smoothing by 1/λ₂, codes and scales, t₂ = bf16(X̂₂)·L1₂).
    Returns the activation dict plus ``x2_bits``."""
    x2_bits = f32_to_bf16_bits(bf16_rne(gelu32(bf16_bits_to_f32(y1_bits))))
    act = quantize_activations(x2_bits, inv_lam2, l1_2, fmt)
    act["x2_bits"] = x2_bits
    return act
