"""Pins for the oracle: checks against what the SVDQuant page and plain mathematics fix.

Each test compares the oracle with something other than itself: hand-derived golden values,
brute force over all codes, closed forms (Eckart-Young), constructed matrices with a known SVD,
torch's bfloat16 conversion, exact rational arithmetic, and the Proposition 4.1 bound.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth
from conftest import read_golden_cases

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_golden():
    with open(__file__.replace("test_oracle_pins.py", "golden/bf16_rne_cases.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for src, dst in rows:
        f32 = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        assert O.f32_to_bf16_bits(O.bf16_rne(f32))[0] == int(dst, 16), src


def test_bf16_matches_torch():
    bits = RNG.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000            # exact ties
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(O.bf16_rne(f)), ref)


# ---------------------------------------------------------------- INT4 group quantizer
def _group(values):
    g = np.zeros((1, 64), dtype=np.float32)
    g[0, :len(values)] = values
    return g


def test_int4_golden():
    for case in read_golden_cases("int4_g64_cases.txt"):
        q, s = O.quant_int4_g64(_group(case["values"]))
        assert s[0, 0] == np.float32(float(case["scale"][0])), case
        want = [int(c) for c in case["codes"]]
        assert q[0, :len(want)].tolist() == want, case
        assert not q[0, len(want):].any()


def _random_groups(n):
    mags = 10.0 ** RNG.uniform(-6, 4, size=(n, 1))
    v = (RNG.standard_normal((n, 64)) * mags).astype(np.float32)
    v[::7, RNG.integers(0, 64)] *= 40                               # outliers
    v[::11, :32] = 0                                                 # sparse groups
    return v


def test_int4_nearest_code_bruteforce():
    """Each code is a nearest point of the 16-point grid s*{-8..7} (slack for the reciprocal)."""
    v = _random_groups(3000)
    q, s = O.quant_int4_g64(v)
    sv = s[:, 0].astype(np.float64)[:, None]
    grid = np.arange(-8, 8, dtype=np.float64)
    err_all = np.abs(v.astype(np.float64)[:, :, None] - sv[:, :, None] * grid[None, None, :])
    best = err_all.min(axis=2)
    mine = np.abs(v.astype(np.float64) - sv * q.astype(np.float64))
    assert np.all(mine <= best + sv * 2.0 ** -20)
    assert np.all(mine <= sv * (0.5 + 2.0 ** -20))


def test_int4_ties_go_to_even():
    """With power-of-two scales the reciprocal is exact, so half-way values are true ties."""
    for e in (-3, 0, 5):
        s = 2.0 ** e
        v = np.array([7, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -6.5], dtype=np.float64) * s
        q, sc = O.quant_int4_g64(_group(v))
        assert sc[0, 0] == s
        assert q[0, :9].tolist() == [7, 0, 2, 2, 4, 0, -2, -2, -6]


def test_int4_scale_is_bf16_of_amax_over_7():
    v = _random_groups(2000)
    _, s = O.quant_int4_g64(v)
    amax = torch.from_numpy(np.abs(v).max(axis=1))
    ref = (amax / torch.tensor(7.0, dtype=torch.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    ref[ref < 2.0 ** -126] = 0
    assert np.array_equal(s[:, 0], ref)


def test_int4_code_range_and_full_scale():
    """Symmetric scaling never reaches -8, and every non-zero group uses +-7."""
    v = _random_groups(5000)
    q, s = O.quant_int4_g64(v)
    assert q.min() >= -7 and q.max() <= 7
    nz = s[:, 0] > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 7)
    assert not q[~nz].any()


def test_int4_representable_roundtrip():
    """R = s*q with bf16 s and a +-7 in each group re-quantizes to the same (q, s) exactly."""
    n = 4000
    s = O.bf16_rne((10.0 ** RNG.uniform(-5, 3, size=n)).astype(np.float32))
    q = RNG.integers(-7, 8, size=(n, 64))
    q[np.arange(n), RNG.integers(0, 64, size=n)] = RNG.choice([-7, 7], size=n)
    v = (q * s[:, None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), q * s[:, None].astype(np.float64))   # exact in fp32
    q2, s2 = O.quant_int4_g64(v)
    assert np.array_equal(s2[:, 0], s)
    assert np.array_equal(q2, q)


# ---------------------------------------------------------------- INT8 rows (8-bit setting)
def test_int8_nearest_code_bruteforce():
    """Each code is a nearest point of the grid s*{-127..127} (slack for the reciprocal)."""
    v = (RNG.standard_normal((500, 256)) * 10.0 ** RNG.uniform(-3, 3, size=(500, 1))).astype(np.float32)
    q, s = O.quant_int8_rows(v)
    sv = s.astype(np.float64)[:, None]
    grid = np.arange(-127, 128, dtype=np.float64)
    best = np.abs(v.astype(np.float64)[:, :, None] - sv[:, :, None] * grid[None, None, :]).min(axis=2)
    mine = np.abs(v.astype(np.float64) - sv * q.astype(np.float64))
    assert np.all(mine <= best + sv * 2.0 ** -16)
    assert np.all(mine <= sv * (0.5 + 2.0 ** -16))


def test_int8_scale_ties_and_range():
    """s = fp32(amax/127) per row; the row maximum maps to +-127; with a power-of-two scale the
    reciprocal is exact and half-way values go to the even code; a zero row gets 0 and 0."""
    v = np.array([[127, 0.5, 1.5, 2.5, -2.5, 126.5, -3.5, 0]], np.float64) * 2.0 ** -4
    q, s = O.quant_int8_rows(v)
    assert s[0] == 2.0 ** -4
    assert q[0].tolist() == [127, 0, 2, 2, -2, 126, -4, 0]
    w = (RNG.standard_normal((300, 96)) * 3).astype(np.float32)
    w[7] = 0
    q, s = O.quant_int8_rows(w)
    amax = torch.from_numpy(np.abs(w).max(axis=1))
    ref = (amax / torch.tensor(127.0, dtype=torch.float32)).numpy()
    ref[ref < 2.0 ** -126] = 0
    assert np.array_equal(s, ref)
    nz = s > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 127) and not q[~nz].any() and q.min() >= -127


def test_int8_representable_roundtrip():
    """v = s*q with a power-of-two s and a +-127 in each row re-quantizes to the same codes."""
    q = RNG.integers(-127, 128, size=(200, 64))
    q[:, 3] = 127
    for e in (-20, -3, 4):
        v = (q * 2.0 ** e).astype(np.float32)
        q2, s2 = O.quant_int8_rows(v)
        assert np.all(s2 == 2.0 ** e) and np.array_equal(q2, q)


def test_main_branch_w8a8_two_formulas():
    """s_x s_w (q_x·q_w) (exact integer dot) equals dequant(X)·dequant(W)ᵀ up to fp64 rounding."""
    x = (RNG.standard_normal((40, 192)) * 2).astype(np.float32)
    w = (RNG.standard_normal((24, 192)) * 0.05).astype(np.float32)
    qx, sx = O.quant_int8_rows(x)
    qw, sw = O.quant_int8_rows(w)
    a = O.main_branch_w8a8(qx, sx, qw, sw)
    b = O.dequant_int8_rows(qx, sx) @ O.dequant_int8_rows(qw, sw).T
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(b).max())
    assert np.array_equal(O.main_branch(qx, sx, qw, sw, O.FMT_W8A8), a)


def test_pack_int4_layout():
    q = np.array([[1, -1, -8, 7, 7, -8, 0, -3]], dtype=np.int8)
    assert O.pack_int4(q).tolist() == [[0xF1, 0x78, 0x87, 0xD0]]


def test_pack_nibbles_golden():
    """Golden bytes of the canonical MXFP4 packing: E2M1 fields unchanged, element 2i in the low
    nibble (negative zero 0x8 and the sign bit of every field survive, no sign extension)."""
    cases, cur = [], None
    import os
    from conftest import GOLDEN
    for line in open(os.path.join(GOLDEN, "pack_nibbles_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"codes": [int(v, 16) for v in vals]}
            cases.append(cur)
        else:
            cur["bytes"] = [int(v, 16) for v in vals]
    assert len(cases) == 3
    for c in cases:
        got = O.pack_nibbles(np.array([c["codes"]], dtype=np.uint8))
        assert got.tolist() == [c["bytes"]], c
        # two rows at once: rows are packed independently
        two = O.pack_nibbles(np.array([c["codes"], c["codes"][::-1]], dtype=np.uint8))
        assert two[0].tolist() == c["bytes"]


def test_linear_bias_hand_worked():
    """A 1 x 64 layer worked by hand: λ = 1, rank 0, x = (7, 0, ..., 0) gives s_x = bf16(7/7) = 1 and
    q_x = (7, 0, ...); weight row 0 = (0.875, 0, ...) gives s_w = 0.125, q_w = 7; row 1 = (-1.75, 0, ...)
    gives s_w = 0.25, q_w = -7; so Y_main = (1·0.125·49, 1·0.25·(-49)) = (6.125, -12.25). The bias
    is added before the single rounding to bf16 (step 2^-5 at 6.125, 2^-4 at 12.25):
      bias (0.5, -0.75)               -> (6.625, -13.0)      exact
      bias (2^-6, 2^-5)               -> (6.125, -12.25)     6.140625 is a tie -> even 6.125;
                                                             -12.21875 is a tie -> even -12.25
      bias (2^-6 + 2^-10, -2^-5 - 2^-9) -> (6.15625, -12.3125)  just past the ties, rounded away
      no bias                         -> (6.125, -12.25)"""
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 7.0
    w = np.zeros((2, 64), np.float32)
    w[0, 0], w[1, 0] = 0.875, -1.75
    lam = np.ones(64, np.float32)
    prep = O.prepare_weights(O.f32_to_bf16_bits(w), lam, 0)
    assert prep["sw"].tolist() == [[0.125], [0.25]] and prep["cw"][:, 0].tolist() == [7, -7]
    xb = O.f32_to_bf16_bits(x)
    cases = [((0.5, -0.75), (6.625, -13.0)),
             ((2.0 ** -6, 2.0 ** -5), (6.125, -12.25)),
             ((2.0 ** -6 + 2.0 ** -10, -2.0 ** -5 - 2.0 ** -9), (6.15625, -12.3125))]
    for bias, want in cases:
        b = O.f32_to_bf16_bits(np.array(bias, np.float32))
        assert O.bf16_bits_to_f32(b).tolist() == list(bias)          # the biases are bf16 values
        y = O.linear(xb, lam, prep, b)["y"]
        assert y[0].tolist() == list(want), (bias, y)
    assert O.linear(xb, lam, prep)["y"][0].tolist() == [6.125, -12.25]


# ---------------------------------------------------------------- FP4 (E2M1) block quantizer
def _block(values):
    b = np.zeros((1, 32), dtype=np.float32)
    b[0, :len(values)] = values
    return b


def test_mxfp4_golden():
    for case in read_golden_cases("mxfp4_b32_cases.txt"):
        c, e8 = O.quant_mxfp4_b32(_block(case["values"]))
        assert int(e8[0, 0]) - 127 == int(case["e"][0]), case
        want = [int(x, 16) for x in case["codes"]]
        assert c[0, :len(want)].tolist() == want, case


def test_mx_exponent_bruteforce():
    amax = np.concatenate([10.0 ** RNG.uniform(-30, 30, size=5000),
                           [6 * 2.0 ** k for k in range(-20, 20)],
                           [np.nextafter(np.float32(6 * 2.0 ** k), np.float32(np.inf)) for k in range(-20, 20)]])
    amax = amax.astype(np.float32).astype(np.float64)
    e = O.mx_exponent(amax)
    for a, ee in zip(amax, e):
        assert math.ldexp(6.0, int(ee)) >= a > math.ldexp(6.0, int(ee) - 1)


def test_e2m1_nearest_even_bruteforce():
    y = np.concatenate([RNG.uniform(-6, 6, size=20000),
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0]])
    codes = O.e2m1_round(y)
    val = O.e2m1_value(codes)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for yy, c, v in zip(y, codes, val):
        d = np.abs(abs(yy) - grid)
        nearest = np.flatnonzero(d == d.min())
        assert (c & 7) in nearest
        if len(nearest) == 2:
            assert (c & 7) % 2 == 0                  # tie -> even mantissa bit
        assert (c >> 3) == (1 if np.signbit(yy) else 0)
        assert abs(v) == grid[c & 7]


def test_mxfp4_never_saturates():
    v = (RNG.standard_normal((2000, 32)) * 10.0 ** RNG.uniform(-8, 8, size=(2000, 1))).astype(np.float32)
    c, e8 = O.quant_mxfp4_b32(v)
    y = np.ldexp(v.astype(np.float64), -(e8.astype(np.int64)[:, :1] - 127))
    assert np.abs(y).max() <= 6.0
    err = np.abs(O.dequant_mxfp4_b32(c, e8) - v)
    step = np.ldexp(1.0, e8.astype(np.int64)[:, :1] - 127)        # half of the largest grid gap (2) * 2^e
    assert np.all(err <= step)


# ---------------------------------------------------------------- smoothing
def test_smoothing_equalizes_maxima():
    """α = 0.5 gives max|X̂_j| = max|Ŵ_j| = sqrt(max|X_j| max|W_j|) (App. D, after SmoothQuant)."""
    d = synth.workload("tiny")
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    xh = np.abs(x.astype(np.float64) / lam.astype(np.float64)).max(axis=0)
    wh = np.abs(w.astype(np.float64) * lam.astype(np.float64)).max(axis=0)
    assert np.allclose(xh, wh, rtol=2e-7)
    assert np.allclose(lam.astype(np.float64) ** 2, x.__abs__().max(0) / np.abs(w).max(0), rtol=3e-7)
    assert np.array_equal(inv, (np.float32(1) / lam).astype(np.float32))


def test_smoothing_preserves_product():
    d = synth.workload("tiny")
    x = O.bf16_bits_to_f32(d["x"]).astype(np.float64)
    w = O.bf16_bits_to_f32(d["w"]).astype(np.float64)
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    xh = O.smooth_activations(x, inv).astype(np.float64)
    wh = O.smooth_weights(w, lam)
    bound = 2.0 ** -22 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(xh @ wh.T - x @ w.T) <= bound)


def test_smoothing_zero_channel():
    lam, inv = O.smooth_factors(np.array([0.0, 4.0, 2.0], np.float32), np.array([1.0, 0.0, 0.5], np.float32))
    assert lam.tolist() == [1.0, 1.0, 2.0] and inv.tolist() == [1.0, 1.0, 0.5]


# ---------------------------------------------------------------- SVD split
def _known_svd(k, n, sig):
    u, _ = np.linalg.qr(RNG.standard_normal((k, len(sig))))
    v, _ = np.linalg.qr(RNG.standard_normal((n, len(sig))))
    return u, v, (u * sig) @ v.T          # Ŵᵀ [k, n]


def test_svd_recovers_known_factors():
    sig = np.array([9.0, 7.0, 5.0, 3.0, 2.0, 1.0, 0.5, 0.25])
    u, v, wt = _known_svd(96, 80, sig)
    ur, sr, vr, s_all = O.truncated_svd(wt.T, 4)
    assert np.allclose(sr, sig[:4], rtol=1e-12)
    assert np.allclose(s_all[:8], sig, rtol=1e-12)
    for i in range(4):
        sgn = np.sign(np.dot(ur[:, i], u[:, i]))
        assert np.allclose(ur[:, i], sgn * u[:, i], atol=1e-10)
        assert np.allclose(vr[:, i], sgn * v[:, i], atol=1e-10)
        j = np.argmax(np.abs(ur[:, i]))
        assert ur[j, i] > 0                                    # sign convention
    l1, l2 = O.lowrank_split(wt.T, 4)
    best = (ur * sr) @ vr.T
    assert np.abs(l1.astype(np.float64) @ l2.astype(np.float64) - best).max() <= 2.0 ** -7 * np.abs(best).max()


def test_eckart_young_tail_energy():
    w = RNG.standard_normal((60, 128))
    for r in (0, 1, 7, 32, 60):
        ur, sr, vr, s_all = O.truncated_svd(w, r)
        err = np.linalg.norm(w.T - (ur * sr) @ vr.T) ** 2
        assert err == pytest.approx(np.sum(s_all[r:] ** 2), rel=1e-10, abs=1e-18)


def test_residual_definition_and_rank_order():
    d = synth.workload("tiny")
    w = O.bf16_bits_to_f32(d["w"])
    lam = np.ones(w.shape[1], np.float32)
    wh = O.smooth_weights(w, lam)
    l1, l2 = O.lowrank_split(wh, 16)
    r = O.residual(wh, l1, l2)
    # every fp64 product of two bf16 values is exact; the sum over 16 terms is within 16 ulp
    recon = r.astype(np.float64) + (l1.astype(np.float64) @ l2.astype(np.float64)).T
    assert np.all(np.abs(recon - wh) <= np.abs(wh) * 2.0 ** -23 + np.abs(r) * 2.0 ** -23 + 1e-15)


def test_residual_is_narrower_than_smoothed_weight():
    """§4.2: the residual has a narrower range and fewer outliers than Ŵ (checked on the tiny layer)."""
    d = synth.workload("tiny")
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, _ = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    prep = O.prepare_weights(d["w"], lam, 16)
    assert np.abs(prep["r"]).max() < np.abs(prep["w_hat"]).max()
    assert np.linalg.norm(prep["r"]) < np.linalg.norm(prep["w_hat"])


def test_split_error_closed_form():
    """What both branches miss: zero when the 4-bit branch represents R exactly (every group is
    q·2^-3 with a 7 in it, rank 0); exactly |δ| after one element moves by δ less than half a
    quantization step (the code rounds the move away)."""
    rng = np.random.default_rng(5)
    q = rng.integers(-7, 8, size=(8, 128)).astype(np.float64)
    q[:, 0] = 7
    q[:, 64] = -7
    q[3, 5] = 2
    lam = np.ones(128, np.float32)
    w = q * 2.0 ** -3
    prep = O.prepare_weights(O.f32_to_bf16_bits(w.astype(np.float32)), lam, 0)
    assert O.split_error(prep["w_hat"], prep["l1"], prep["l2"], prep["cw"], prep["sw"], "int4_g64") == 0.0
    w[3, 5] += 2.0 ** -6
    prep = O.prepare_weights(O.f32_to_bf16_bits(w.astype(np.float32)), lam, 0)
    assert O.split_error(prep["w_hat"], prep["l1"], prep["l2"], prep["cw"], prep["sw"], "int4_g64") == 2.0 ** -6


def test_refine_iteration0_is_the_plain_split():
    d = synth.workload("tiny")
    lam, _ = O.smooth_factors(O.column_absmax(O.bf16_bits_to_f32(d["x"])), O.column_absmax(O.bf16_bits_to_f32(d["w"])))
    for fmt in ("int4_g64", "mxfp4_b32"):
        plain = O.prepare_weights(d["w"], lam, 16, fmt)
        rf = O.prepare_weights_refined(d["w"], lam, 16, fmt, iters=0)
        for k in ("l1", "l2", "cw", "sw"):
            assert np.array_equal(rf[k], plain[k]), k
        assert rf["iteration"] == 0
        assert rf["errors"] == [O.split_error(plain["w_hat"], plain["l1"], plain["l2"], plain["cw"], plain["sw"], fmt)]


def test_refine_keeps_the_smallest_error_and_reduces_it():
    """§4.2: iterative updates reduce the quantization error, and the result with the smallest
    error is kept. The kept arrays reproduce the reported error; on the outlier layer the error
    falls below the plain split's."""
    d = synth.make_layer(96, 256, 192, n_outliers=4, outlier_scale=30.0, seed=21)
    lam, _ = O.smooth_factors(O.column_absmax(O.bf16_bits_to_f32(d["x"])), O.column_absmax(O.bf16_bits_to_f32(d["w"])))
    for fmt in ("int4_g64", "mxfp4_b32"):
        rf = O.prepare_weights_refined(d["w"], lam, 8, fmt, iters=4)
        e = O.split_error(rf["w_hat"], rf["l1"], rf["l2"], rf["cw"], rf["sw"], fmt)
        assert e == rf["errors"][rf["iteration"]] == min(rf["errors"])
        assert min(rf["errors"]) < 0.97 * rf["errors"][0]
        assert rf["errors"].index(min(rf["errors"])) == rf["iteration"]


# ---------------------------------------------------------------- special cases of the layer
def test_rank0_unquantized_is_plain_gemm():
    d = synth.workload("tiny")
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    wh = O.smooth_weights(w, lam)
    z1, z2 = np.zeros((256, 0), np.float32), np.zeros((0, 256), np.float32)
    y = O.linear_unquantized(x, inv, O.residual(wh, z1, z2), z1, z2)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.all(np.abs(y - ref) <= 2.0 ** -21 * (np.abs(x).astype(np.float64) @ np.abs(w).T.astype(np.float64)))


def test_full_rank_unquantized_is_plain_gemm():
    d = synth.make_layer(64, 128, 96, n_outliers=3, outlier_scale=20.0, seed=5)
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    wh = O.smooth_weights(w, lam)
    l1, l2 = O.lowrank_split(wh, 96)
    y = O.linear_unquantized(x, inv, O.residual(wh, l1, l2), l1, l2)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()


def test_main_branch_two_formulas():
    """Σ_g s_x s_w (q_x·q_w) equals the dense product of the dequantized matrices."""
    qx = RNG.integers(-7, 8, size=(40, 256))
    qw = RNG.integers(-7, 8, size=(24, 256))
    sx = O.bf16_rne(RNG.uniform(0.01, 3, size=(40, 4)).astype(np.float32))
    sw = O.bf16_rne(RNG.uniform(0.001, 0.3, size=(24, 4)).astype(np.float32))
    dense = (qx * np.repeat(sx.astype(np.float64), 64, axis=1)) @ (qw * np.repeat(sw.astype(np.float64), 64, axis=1)).T
    assert np.allclose(O.main_branch_int4(qx, sx, qw, sw), dense, rtol=1e-13, atol=1e-13)


def test_main_branch_mxfp4_two_formulas():
    cx = RNG.integers(0, 16, size=(20, 128)).astype(np.uint8)
    cw = RNG.integers(0, 16, size=(12, 128)).astype(np.uint8)
    ex = RNG.integers(110, 140, size=(20, 4)).astype(np.uint8)
    ew = RNG.integers(110, 140, size=(12, 4)).astype(np.uint8)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    val = lambda c: np.where(c & 8, -1.0, 1.0) * grid[c & 7]
    dx = val(cx) * np.repeat(2.0 ** (ex.astype(np.float64) - 127), 32, axis=1)
    dw = val(cw) * np.repeat(2.0 ** (ew.astype(np.float64) - 127), 32, axis=1)
    assert np.allclose(O.main_branch_mxfp4(cx, ex, cw, ew), dx @ dw.T, rtol=1e-13, atol=0)


def test_prop41_bound():
    """Proposition 4.1 (§4.1, §A.1) holds for the oracle's quantizers on the tiny layer and on random data."""
    d = synth.workload("tiny")
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    prep = O.prepare_weights(d["w"], lam, 16)
    act = O.quantize_activations(d["x"], inv, prep["l1"])
    for fmt in (O.FMT_INT4_G64, O.FMT_MXFP4_B32):
        for xx, ww in ((act["x_hat"], prep["r"]), (RNG.standard_normal((50, 128)), RNG.standard_normal((70, 128)))):
            xx = np.asarray(xx, np.float32)
            ww = np.asarray(ww, np.float32)
            cx, sx = O.quantize(xx, fmt)
            cw, sw = O.quantize(ww, fmt)
            deq = O.dequant_int4_g64 if fmt == O.FMT_INT4_G64 else O.dequant_mxfp4_b32
            err, bound = O.prop41_terms(xx, ww, deq(cx, sx), deq(cw, sw))
            assert 0 < err <= bound


# ---------------------------------------------------------------- exact end-to-end case
def _force_full_scale(q, rng, block, val):
    """Put +val into one element and -val into another of every block of each row, so that every
    block's maximum magnitude is val (the scale is then exactly its power-of-two factor)."""
    rows, k = q.shape
    for b in range(k // block):
        pos = rng.permutation(block)[:2]
        q[:, b * block + pos[0]] = val
        q[:, b * block + pos[1]] = -val
    return q


def exact_case(m=64, k=128, n=96, r=2, seed=3):
    """A layer on which every rounding in the method is exact (λ = 1, power-of-two group scales,
    representable activations and residual, one-hot L1). Returns inputs and the exact Y.

    Every group of every row holds a code of +7 and one of -7, so each INT4 scale is exactly
    7·2^e / 7 = 2^e. Exactness of any fp32 summation order: x·8 and resid·64 are integers bounded by
    7·4·8 and 7·2^-4·64, so every partial sum of x·resid is a multiple of 2^-9 below K·6272·2^-9 in
    magnitude; the bound is asserted below 2^24 units (fp32-exact) and, with it, below 2^53 (the fp64
    matmul used here is exact too)."""
    rng = np.random.default_rng(seed)
    g = k // 64
    ex = rng.integers(-3, 3, size=(m, g))
    qx = _force_full_scale(rng.integers(-7, 8, size=(m, k)), rng, 64, 7)
    x = qx * np.repeat(2.0 ** ex, 64, axis=1)
    ew = rng.integers(-6, -3, size=(n, g))
    qw = _force_full_scale(rng.integers(-7, 8, size=(n, k)), rng, 64, 7)
    resid = qw * np.repeat(2.0 ** ew, 64, axis=1)
    sel = rng.choice(k, r, replace=False)
    l1 = np.zeros((k, r))
    l1[sel, np.arange(r)] = 1.0
    l2 = rng.integers(-3, 4, size=(r, n)) * 0.125
    w = resid + (l1 @ l2).T
    bits = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(bits(x)), x) and np.array_equal(O.bf16_bits_to_f32(bits(w)), w)
    # exact result in scaled integers: x*2^3, resid*2^6 and l2*2^3 are integers
    assert k * (7 * 4 * 8) * (7 * 64 // 16) + r * 8 * (7 * 4 * 8) * 3 < 2 ** 24
    xi = x * 8
    ri = resid * 64
    li = l2 * 8
    acc = xi @ ri.T + 8 * (xi[:, sel] @ li)       # integer-valued fp64, exact below 2^53
    y = acc / 512.0
    # cross-check a few entries with rational arithmetic
    for i, j in ((0, 0), (m - 1, n - 1), (m // 2, n // 3)):
        fr = sum(Fraction(float(x[i, kk])) * Fraction(float(resid[j, kk])) for kk in range(k)) + \
            sum(Fraction(float(x[i, sel[t]])) * Fraction(float(l2[t, j])) for t in range(r))
        assert Fraction(float(y[i, j])) == fr
    return dict(x_bits=bits(x), w_bits=bits(w), l1=l1.astype(np.float32), l2=l2.astype(np.float32),
                y_exact=y, rank=r)


def mx_exact_case(m=64, k=128, n=96, r=2, seed=5):
    """The MXFP4 counterpart of ``exact_case``: activations and residual are E2M1 values times a
    power of two per 32-block, with a ±6 in every block (so the block exponent is exactly that power),
    λ = 1 and a one-hot L1. Products of two E2M1 values are multiples of 1/4; with block exponents
    ex in [-3, 0] and ew in [-6, -4] every partial sum is a multiple of 2^-11 bounded by
    K·36·2^-4 (+ the low-rank terms), asserted below 2^24 units, so fp32 accumulation in any order is
    exact and Y must be reproduced bit for bit."""
    rng = np.random.default_rng(seed)
    b = k // 32
    grid = np.concatenate([O.E2M1_GRID, -O.E2M1_GRID[1:]])            # no negative zero
    vx = _force_full_scale(rng.choice(grid, size=(m, k)), rng, 32, 6.0)
    vw = _force_full_scale(rng.choice(grid, size=(n, k)), rng, 32, 6.0)
    ex = rng.integers(-3, 1, size=(m, b))
    ew = rng.integers(-6, -3, size=(n, b))
    x = vx * np.repeat(2.0 ** ex, 32, axis=1)
    resid = vw * np.repeat(2.0 ** ew, 32, axis=1)
    sel = rng.choice(k, r, replace=False)
    l1 = np.zeros((k, r))
    l1[sel, np.arange(r)] = 1.0
    l2 = rng.integers(-3, 4, size=(r, n)) * 0.125
    w = resid + (l1 @ l2).T
    bits = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(bits(x)), x) and np.array_equal(O.bf16_bits_to_f32(bits(w)), w)
    assert (k * 36 * 2.0 ** -4 + r * 6 * 0.375) * 2 ** 11 < 2 ** 24
    y = x @ resid.T + x[:, sel] @ l2                   # dyadic, exact in fp64
    for i, j in ((0, 0), (m - 1, n - 1), (m // 2, n // 3)):
        fr = sum(Fraction(float(x[i, kk])) * Fraction(float(resid[j, kk])) for kk in range(k)) + \
            sum(Fraction(float(x[i, sel[t]])) * Fraction(float(l2[t, j])) for t in range(r))
        assert Fraction(float(y[i, j])) == fr
    return dict(x_bits=bits(x), w_bits=bits(w), l1=l1.astype(np.float32), l2=l2.astype(np.float32),
                y_exact=y, rank=r)


def w8_exact_case(m=64, k=256, n=96, r=2, seed=7):
    """The 8-bit setting's counterpart of ``exact_case``: row m of X is q·2^e_m with integer
    |q| <= 127 and a +127 and a -127 in every row, so the per-token scale is exactly 2^e_m; the
    residual's rows are q·2^-9 built the same way (per-channel scale 2^-9); λ = 1, one-hot L1 and
    L2 in {-1/8, 0, 1/8}, so W stays bf16-representable. In units of 2^(e_m - 9) the main term is
    the integer dot product (at most K·127²) and each low-rank term at most 127·64, so with the sum
    asserted below 2^24 units every fp32 partial sum is exact and Y is reproduced bit for bit."""
    rng = np.random.default_rng(seed)
    ex = rng.integers(-3, 3, size=m)
    qx = _force_full_scale(rng.integers(-127, 128, size=(m, k)), rng, k, 127)
    x = qx * (2.0 ** ex)[:, None]
    qw = _force_full_scale(rng.integers(-127, 128, size=(n, k)), rng, k, 127)
    resid = qw * 2.0 ** -9
    sel = rng.choice(k, r, replace=False)
    l1 = np.zeros((k, r))
    l1[sel, np.arange(r)] = 1.0
    l2 = rng.integers(-1, 2, size=(r, n)) * 0.125
    w = resid + (l1 @ l2).T
    bits = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(bits(x)), x) and np.array_equal(O.bf16_bits_to_f32(bits(w)), w)
    assert k * 127 * 127 + r * 127 * 64 < 2 ** 24
    y = x @ resid.T + x[:, sel] @ l2                   # dyadic, exact in fp64
    for i, j in ((0, 0), (m - 1, n - 1), (m // 2, n // 3)):
        fr = sum(Fraction(float(x[i, kk])) * Fraction(float(resid[j, kk])) for kk in range(k)) + \
            sum(Fraction(float(x[i, sel[t]])) * Fraction(float(l2[t, j])) for t in range(r))
        assert Fraction(float(y[i, j])) == fr
    return dict(x_bits=bits(x), w_bits=bits(w), l1=l1.astype(np.float32), l2=l2.astype(np.float32),
                y_exact=y, rank=r)


def test_exact_case_end_to_end():
    c = exact_case()
    lam = np.ones(128, np.float32)
    prep = O.prepare_weights(c["w_bits"], lam, c["rank"], l1=c["l1"], l2=c["l2"])
    out = O.linear(c["x_bits"], lam, prep)
    assert np.array_equal(out["y_m"] + out["y_l"], c["y_exact"])
    assert np.array_equal(out["y"], O.bf16_rne(c["y_exact"].astype(np.float32)))
    # every group's scale is the exact power of two, and the codes are the constructed integers
    assert np.all(np.log2(out["sx"][out["sx"] > 0]) % 1 == 0)
    assert np.abs(out["cx"]).max() == 7 and np.abs(prep["cw"]).max() == 7


def test_mx_exact_case_end_to_end():
    c = mx_exact_case(m=40, k=160, n=72, r=3)
    lam = np.ones(160, np.float32)
    prep = O.prepare_weights(c["w_bits"], lam, c["rank"], "mxfp4_b32", l1=c["l1"], l2=c["l2"])
    out = O.linear(c["x_bits"], lam, prep)
    assert np.array_equal(out["y_m"] + out["y_l"], c["y_exact"])
    assert np.array_equal(out["y"], O.bf16_rne(c["y_exact"].astype(np.float32)))
    # decoded codes times 2^e give back the constructed values: the block exponent was chosen exactly
    assert np.array_equal(O.dequant_mxfp4_b32(out["cx"], out["sx"]), O.bf16_bits_to_f32(c["x_bits"]))
    assert np.array_equal(O.dequant_mxfp4_b32(prep["cw"], prep["sw"]), prep["r"])


# ---------------------------------------------------------------- LoRA merge (§4.2 / §5.2)

def test_w8_exact_case_end_to_end():
    c = w8_exact_case(m=40, k=256, n=72, r=3)
    lam = np.ones(256, np.float32)
    prep = O.prepare_weights(c["w_bits"], lam, c["rank"], O.FMT_W8A8, l1=c["l1"], l2=c["l2"])
    out = O.linear(c["x_bits"], lam, prep)
    assert np.array_equal(out["y_m"] + out["y_l"], c["y_exact"])
    assert np.array_equal(out["y"], O.bf16_rne(c["y_exact"].astype(np.float32)))
    # the scales are the constructed powers of two and the codes the constructed integers
    x = O.bf16_bits_to_f32(c["x_bits"]).astype(np.float64)
    assert np.all(np.log2(out["sx"]) % 1 == 0) and np.all(prep["sw"] == np.float32(2.0 ** -9))
    assert np.array_equal(out["cx"].astype(np.float64) * out["sx"][:, None], x)
    assert np.abs(out["cx"]).max() == 127 and np.abs(prep["cw"]).max() == 127
def test_lora_merge_adds_exactly_the_lora_term():
    d = synth.make_layer(64, 256, 128, n_outliers=4, outlier_scale=30.0, seed=7, lora_rank=16)
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    base = O.prepare_weights(d["w"], lam, 16)
    a = O.bf16_bits_to_f32(d["lora_a"])
    b = O.bf16_bits_to_f32(d["lora_b"])
    # the residual is not re-quantized: reuse base codes/scales with the widened factors
    merged = dict(base, l1=np.concatenate([base["l1"], a], axis=1), l2=np.concatenate([base["l2"], b], axis=0))
    yb = O.linear(d["x"], inv, base)
    ym = O.linear(d["x"], inv, merged)
    xh = O.smooth_activations(x, inv)
    xb = torch.from_numpy(xh).to(torch.bfloat16).to(torch.float64).numpy()
    tb_a = torch.from_numpy((xb @ a.astype(np.float64)).astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    diff = (ym["y_m"] + ym["y_l"]) - (yb["y_m"] + yb["y_l"])
    assert np.allclose(diff, tb_a @ b.astype(np.float64), rtol=1e-12, atol=1e-15)
    assert np.array_equal(ym["cx"], yb["cx"]) and np.array_equal(ym["sx"], yb["sx"])


# ---------------------------------------------------------------- MLP producer: fp32 GELU
def _phi_gelu(y):
    """Exact GELU in fp64 from math.erf (the textbook definition)."""
    return 0.5 * y * (1.0 + math.erf(y / math.sqrt(2.0)))


def test_erf32_within_the_rational_form_bound():
    """A&S 7.1.28 is within 3e-7 of erf; fp32 evaluation (16th power by squaring) adds ≤ 1.5e-6."""
    x = np.concatenate([np.linspace(-8, 8, 160001), [0.0, 1e-30, 1e-8, 3.0, 5.5, 40.0, 1e30]]).astype(np.float32)
    e = O.erf32(x)
    ref = np.array([math.erf(float(v)) for v in x])
    assert np.abs(e - ref).max() <= 2e-6
    assert np.array_equal(O.erf32(-x), -e)                     # odd, bit for bit
    assert O.erf32(np.float32([0.0]))[0] == 0.0 and O.erf32(np.float32([40.0]))[0] == 1.0


def test_gelu32_matches_the_erf_definition():
    y = np.concatenate([np.linspace(-12, 12, 240001), [0.0, -0.0, 1e-20, 100.0, -100.0]]).astype(np.float32)
    g = O.gelu32(y)
    ref = np.array([_phi_gelu(float(v)) for v in y])
    assert np.all(np.abs(g - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref)))
    assert O.gelu32(np.float32([100.0]))[0] == 100.0 and O.gelu32(np.float32([-100.0]))[0] == 0.0
    assert O.gelu32(np.float32([0.0]))[0] == 0.0


def test_gelu32_rounds_to_the_same_bf16_as_exact_gelu():
    """Brute force over every bf16 value in [-16, 16]. Wherever |GELU(y)| >= 2^-6 (everything
    but the far negative tail, where 1 + erf cancels and only the absolute bound holds),
    bf16(gelu32(y)) is bf16 of the exact GELU unless the exact value lies within the fp32
    evaluation error of a bf16 rounding midpoint; everywhere the bf16 results differ by at most
    one bf16 step or 4e-6."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    y = O.bf16_bits_to_f32(bits)
    y = y[np.isfinite(y) & (np.abs(y) <= 16)]
    got = O.bf16_rne(O.gelu32(y)).astype(np.float64)
    exact = np.array([_phi_gelu(float(v)) for v in y])
    want = O.bf16_rne(exact).astype(np.float64)
    big = np.abs(exact) >= 2.0 ** -6
    differ = (got != want) & big
    mid_dist = np.abs(np.abs(exact) - np.abs((got + want) / 2))
    assert np.all(mid_dist[differ] <= 2e-6 * np.abs(exact[differ]))
    assert differ.sum() <= 8
    step = np.abs(want) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= np.maximum(step, 4e-6))


def test_gelu_quantize_is_fc2_activation_side_of_gelu_output():
    """fc2's codes from fc1's output are the ordinary activation side applied to X₂ = bf16(GELU(Y₁))."""
    rng = np.random.default_rng(5)
    y1 = O.f32_to_bf16_bits(O.bf16_rne(rng.standard_normal((20, 128)).astype(np.float32) * 3))
    inv = (1.0 / rng.uniform(0.5, 2.0, 128)).astype(np.float32)
    l1 = O.bf16_rne(rng.standard_normal((128, 8)).astype(np.float32) * 0.1)
    act = O.gelu_quantize(y1, inv, l1)
    x2 = O.bf16_rne(np.array([[_phi_gelu(float(v)) for v in row] for row in O.bf16_bits_to_f32(y1)]))
    assert np.abs(O.bf16_bits_to_f32(act["x2_bits"]) - x2).max() <= 2.0 ** -8 * np.abs(x2).max()
    direct = O.quantize_activations(act["x2_bits"], inv, l1)
    assert np.array_equal(act["cx"], direct["cx"]) and np.array_equal(act["sx"], direct["sx"])
