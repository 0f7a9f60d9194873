"""GPU parity of the MLP pair fc1 -> GELU -> fc2 (through the C ABI): fc2's activation side
produced by fc2's activation kernel from fc1's output (consumer side) and by fc1's GEMM epilogue
(producer side).

Contract: fc2's activation codes and scales bit-exact against the oracle's activation side of
X2 = bf16(GELU(Y1)) taken from the GPU's own Y1 (fc1's output is within tolerance of the oracle's,
not bit-identical, so its rounding decisions are the GPU's); t2 within the fp32 accumulation
bound; fc1's Y1 and fc2's Y2 within 2^-7 max|Y_ref|."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import w4a4_quantized_gemm_smooth_amd as w4

pytestmark = pytest.mark.gpu
TOL = 2.0 ** -7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    w4.lib()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _pair(m, k, n, n2, r1, r2, seed, bias=True):
    """fc1 [n, k] and fc2 [n2, n] layers with the oracle's preparations; λ₂ from an fp64 GELU of an
    unquantized fc1 output (any calibration would do)."""
    d1 = synth.make_layer(m, k, n, n_outliers=max(1, k // 64), outlier_scale=30.0, seed=seed)
    x1 = O.bf16_bits_to_f32(d1["x"])
    w1 = O.bf16_bits_to_f32(d1["w"])
    lam1, inv1 = O.smooth_factors(O.column_absmax(x1), O.column_absmax(w1))
    ref1 = O.prepare_weights(d1["w"], lam1, r1)
    rng = np.random.default_rng(seed + 1)
    w2_bits = O.f32_to_bf16_bits(O.bf16_rne((rng.standard_normal((n2, n)) * 0.02).astype(np.float32)))
    x2_cal = O.bf16_rne(O.gelu32(O.bf16_rne((x1.astype(np.float64) @ w1.T.astype(np.float64)).astype(np.float32))))
    lam2, inv2 = O.smooth_factors(O.column_absmax(x2_cal), O.column_absmax(O.bf16_bits_to_f32(w2_bits)))
    ref2 = O.prepare_weights(w2_bits, lam2, r2)
    b1 = O.f32_to_bf16_bits(O.bf16_rne(rng.standard_normal(n).astype(np.float32))) if bias else None
    bf = lambda a: O.f32_to_bf16_bits(a) if a is not None and a.size else None
    p1 = w4.prepare_weights(d1["w"], lam1, r1, "int4_g64", bf(ref1["l1"]) if r1 else None, bf(ref1["l2"]) if r1 else None)
    p2 = w4.prepare_weights(w2_bits, lam2, r2, "int4_g64", bf(ref2["l1"]) if r2 else None, bf(ref2["l2"]) if r2 else None)
    fc1 = w4.W4A4Linear(p1, inv1, bias_bits=b1)
    fc2 = w4.W4A4Linear(p2, inv2)
    x = torch.from_numpy(np.ascontiguousarray(d1["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    return dict(d1=d1, inv1=inv1, ref1=ref1, b1=b1, inv2=inv2, ref2=ref2, fc1=fc1, fc2=fc2, x=x, m=m, n=n, n2=n2,
                r2=r2, pair=w4.MLPPair(fc1, fc2))


def _check_fc2_activations(c, y1_bits, a2, rows=None):
    """fc2's codes, scales (bit-exact) and t2 (fp32 bound) against the oracle from the GPU's Y1."""
    m, n, r2 = c["m"], c["n"], c["r2"]
    y1 = y1_bits if rows is None else y1_bits[rows]
    act = O.gelu_quantize(y1, c["inv2"], c["ref2"]["l1"])
    mm = y1.shape[0]
    codes = w4.codes_to_canonical(a2["xq"].cpu().numpy(), m, n, "int4_g64")
    scales = w4.scales_to_canonical(a2["xscale"].cpu().numpy(), m, n, "int4_g64")
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    assert np.array_equal(codes, O.pack_int4(act["cx"])), "fc2 activation codes differ"
    assert np.array_equal(scales, O.f32_to_bf16_bits(act["sx"])), "fc2 activation scales differ"
    mp = (m + 255) // 256 * 256
    xq = a2["xq"].cpu().numpy()
    main = xq[: n // 64 * mp * 32].reshape(n // 64, mp, 32)
    extra = xq[n // 64 * mp * 32:].reshape(n // 64, 2, mp, 8)
    assert not main[:, m:].any() and not extra[:, :, m:].any(), "padding rows of fc2's codes must be zero"
    if r2:
        rp = (r2 + 15) // 16 * 16
        t = a2["xl1"].cpu().numpy()[: mp * rp].reshape(mp, rp)
        tt = t[:m] if rows is None else t[:m][rows]
        terms = np.abs(O.bf16_rne(act["x_hat"]).astype(np.float64)) @ np.abs(c["ref2"]["l1"].astype(np.float64))
        assert np.all(np.abs(tt[:, :r2] - act["t"]) <= 2.0 * n * 2.0 ** -24 * terms + 1e-30), "t2 outside the bound"
        assert not t[m:].any() and not tt[:, r2:].any()
    return act


def _check_y(y, y_ref):
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64)).max()
    assert err <= TOL * np.abs(y_ref).max(), f"max|dY| = {err} > 2^-7 * {np.abs(y_ref).max()}"


@pytest.mark.parametrize("shape", [(300, 256, 640, 384, 20, 20), (64, 128, 256, 128, 0, 16), (1, 64, 128, 64, 16, 0),
                                   (260, 192, 512, 320, 32, 32)])
def test_consumer_side_gelu_quantize(shape):
    """fc2's activation kernel applying the GELU to fc1's Y1 as it reads it."""
    m, k, n, n2, r1, r2 = shape
    print(f"[consumer gelu] M={m} K={k} N={n} N2={n2} r={r1},{r2}", flush=True)
    c = _pair(m, k, n, n2, r1, r2, seed=m + n)
    y2 = torch.empty((m, n2), dtype=torch.bfloat16, device="cuda")
    a2 = c["pair"].unfused(c["x"], y2)
    torch.cuda.synchronize()
    y1_bits = _bits(c["pair"].buffers(m)["y1"])
    _check_y(O.bf16_bits_to_f32(y1_bits), O.linear(c["d1"]["x"], c["inv1"], c["ref1"], c["b1"])["y"])
    act = _check_fc2_activations(c, y1_bits, a2)
    y2_ref = O.linear(act["x2_bits"], c["inv2"], c["ref2"])["y"]
    _check_y(O.bf16_bits_to_f32(_bits(y2)), y2_ref)


@pytest.mark.parametrize("shape", [(300, 256, 640, 384, 20, 20), (64, 128, 256, 128, 0, 16), (1, 64, 128, 64, 16, 0),
                                   (260, 192, 512, 320, 32, 32), (513, 128, 1024, 256, 8, 32)])
def test_producer_side_fusion(shape):
    """fc1's GEMM epilogue emitting fc2's activation side: the same codes and scales as the
    consumer-side path (and as the oracle from the GPU's Y1), t2 within the bound, Y2 within
    tolerance; fc1's Y1 (written for checking) within tolerance of the oracle."""
    m, k, n, n2, r1, r2 = shape
    print(f"[producer fusion] M={m} K={k} N={n} N2={n2} r={r1},{r2}", flush=True)
    c = _pair(m, k, n, n2, r1, r2, seed=m + n + 1)
    y1 = torch.full((m, n), -7.0, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((m, n2), dtype=torch.bfloat16, device="cuda")
    a2 = c["pair"].fused(c["x"], y2, y1_check=y1)
    torch.cuda.synchronize()
    y1_bits = _bits(y1)
    _check_y(O.bf16_bits_to_f32(y1_bits), O.linear(c["d1"]["x"], c["inv1"], c["ref1"], c["b1"])["y"])
    act = _check_fc2_activations(c, y1_bits, a2)
    _check_y(O.bf16_bits_to_f32(_bits(y2)), O.linear(act["x2_bits"], c["inv2"], c["ref2"])["y"])
    # the consumer-side path on the same input decides every code the same way
    codes_f = a2["xq"].clone()
    scales_f = a2["xscale"].clone()
    y2u = torch.empty_like(y2)
    a2u = c["pair"].unfused(c["x"], y2u)
    torch.cuda.synchronize()
    assert torch.equal(a2u["xq"], codes_f) and torch.equal(a2u["xscale"], scales_f)
    _check_y(O.bf16_bits_to_f32(_bits(y2u)), O.bf16_bits_to_f32(_bits(y2)))


def test_producer_side_fusion_without_y1():
    """Y = NULL: the fused GEMM writes no fc1 output at all, and fc2's activations are unchanged."""
    c = _pair(300, 256, 640, 384, 20, 20, seed=77)
    y1 = torch.empty((300, 640), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((300, 384), dtype=torch.bfloat16, device="cuda")
    a2 = c["pair"].fused(c["x"], y2, y1_check=y1)
    torch.cuda.synchronize()
    codes, scales, t = a2["xq"].clone(), a2["xscale"].clone(), a2["xl1"].clone()
    a2b = c["pair"].fused(c["x"], y2, y1_check=None)
    torch.cuda.synchronize()
    assert torch.equal(a2b["xq"], codes) and torch.equal(a2b["xscale"], scales) and torch.equal(a2b["xl1"], t)


def test_consumer_side_strided_producer_output():
    """fc2's activation kernel reading fc1's output through a row stride above K (Y1 a column slice
    of a wider matrix, the extra columns holding values that must not be read): codes, scales and t2
    bit-identical to the contiguous call."""
    m, k, r = 200, 384, 24
    rng = np.random.default_rng(12)
    y_bits = O.f32_to_bf16_bits(O.bf16_rne((rng.standard_normal((m, k)) * 3).astype(np.float32)))
    print(f"[strided Y1] M={m} K={k} ldy={k + 136} r={r}", flush=True)
    y = torch.from_numpy(np.ascontiguousarray(y_bits).view(np.int16)).cuda().view(torch.bfloat16)
    wide = torch.full((m, k + 136), -2.0e4, dtype=torch.bfloat16, device="cuda")
    wide[:, :k] = y
    ys = wide[:, :k]
    inv = torch.from_numpy((rng.uniform(0.5, 2.0, k)).astype(np.float32)).cuda()
    l1t = torch.from_numpy(O.f32_to_bf16_bits(O.bf16_rne((rng.standard_normal((32, k)) * 0.05).astype(np.float32)))
                           .view(np.int16)).cuda()
    sz = w4.buffer_sizes(m, r, k, r)
    outs = []
    for yin in (y, ys):
        xq = torch.zeros(sz["xq"], dtype=torch.uint8, device="cuda")
        xs = torch.zeros(sz["xscale"], dtype=torch.uint8, device="cuda")
        xl1 = torch.zeros(sz["xl1"] // 4, dtype=torch.float32, device="cuda")
        w4.gelu_quantize_act(yin, inv, l1t, r, "int4_g64", xq, xs, xl1)
        torch.cuda.synchronize()
        outs.append((xq.cpu(), xs.cpu(), xl1[: sz["m_pad"] * sz["rank_pad"]].cpu()))
    for name, u, v in zip(("codes", "scales", "t2"), outs[0], outs[1]):
        assert torch.equal(u, v), f"{name} differ with a row stride above K"


def test_gelu_of_every_finite_bf16_input():
    """The device GELU on every finite bf16 pattern (65280 of them, as a 510 x 128 fc1 output) through
    fc2's activation kernel with 1/λ₂ = 1 and L1₂ the 128 x 128 identity (rank 128): then
    t₂ = bf16(X̂₂)·L1₂ is X₂ = bf16(GELU(Y₁)) itself, one exact product per entry, so every GELU value
    is compared with the oracle's. A subnormal X₂ may come back as 0 (bf16 MFMA inputs) and -0 as +0
    (a sum with signed zeros); every other entry must match exactly. Codes and scales of the same X₂
    bit-exact."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    y1_bits = bits[((bits >> 7) & 0xFF) != 0xFF].reshape(510, 128)
    m, k, r = 510, 128, 128
    print(f"[gelu every bf16] M={m} K={k} r={r}", flush=True)
    inv2 = np.ones(k, np.float32)
    l1 = np.eye(k, r, dtype=np.float32)
    act = O.gelu_quantize(y1_bits, inv2, l1)
    x2 = O.bf16_bits_to_f32(act["x2_bits"])
    assert np.array_equal(act["t"], x2.astype(np.float64)), "oracle: t must be X2 for an identity L1"
    sz = w4.buffer_sizes(m, r, k, r)
    y1 = torch.from_numpy(np.ascontiguousarray(y1_bits).view(np.int16)).cuda().view(torch.bfloat16)
    l1t = torch.from_numpy(O.f32_to_bf16_bits(np.ascontiguousarray(l1.T)).view(np.int16)).cuda()
    xq = torch.empty(sz["xq"], dtype=torch.uint8, device="cuda")
    xs = torch.empty(sz["xscale"], dtype=torch.uint8, device="cuda")
    xl1 = torch.empty(sz["xl1"] // 4, dtype=torch.float32, device="cuda")
    w4.gelu_quantize_act(y1, torch.ones(k, dtype=torch.float32, device="cuda"), l1t, r, "int4_g64", xq, xs, xl1)
    torch.cuda.synchronize()
    codes = w4.codes_to_canonical(xq.cpu().numpy(), m, k, "int4_g64")
    scales = w4.scales_to_canonical(xs.cpu().numpy(), m, k, "int4_g64")
    assert np.array_equal(codes, O.pack_int4(act["cx"])), "codes differ"
    assert np.array_equal(scales, O.f32_to_bf16_bits(act["sx"])), "scales differ"
    mp = sz["m_pad"]
    t = xl1.cpu().numpy()[: mp * r].reshape(mp, r)[:m]
    normal = np.abs(x2) >= 2.0 ** -126
    bad = normal & (t != x2)
    assert not bad.any(), f"{bad.sum()} GELU values differ, e.g. input {hex(int(y1_bits[bad][0]))}"
    sub = ~normal
    assert np.all((t[sub] == x2[sub]) | (t[sub] == 0)), "a subnormal GELU value came back neither exact nor 0"


def test_full_size_flux_mlp_fused():
    """FLUX MLP: fc1 4608 x 3072 -> 12288 with fc2's activation side (K 12288, r 32) in its
    epilogue: all fc2 codes and scales bit-exact against the oracle from the GPU's Y1, t2 on
    sampled rows; fc2 (12288 -> 3072) then runs on them."""
    d1 = synth.workload("flux_mlp_fc1")
    d2 = synth.workload("flux_mlp_fc2")
    m, k, n, n2, r = d1["M"], d1["K"], d1["N"], d2["N"], d1["rank"]
    print(f"[flux mlp fused] M={m} K={k} N={n} N2={n2} r={r}", flush=True)
    x1 = O.bf16_bits_to_f32(d1["x"])
    lam1, inv1 = O.smooth_factors(O.column_absmax(x1), O.column_absmax(O.bf16_bits_to_f32(d1["w"])))
    lam2, inv2 = O.smooth_factors(O.column_absmax(O.bf16_bits_to_f32(d2["x"])),
                                  O.column_absmax(O.bf16_bits_to_f32(d2["w"])))
    ref1 = O.prepare_weights(d1["w"], lam1, r)
    ref2 = O.prepare_weights(d2["w"], lam2, r)
    bf = O.f32_to_bf16_bits
    fc1 = w4.W4A4Linear(w4.prepare_weights(d1["w"], lam1, r, "int4_g64", bf(ref1["l1"]), bf(ref1["l2"])), inv1)
    fc2 = w4.W4A4Linear(w4.prepare_weights(d2["w"], lam2, r, "int4_g64", bf(ref2["l1"]), bf(ref2["l2"])), inv2)
    pair = w4.MLPPair(fc1, fc2)
    x = torch.from_numpy(np.ascontiguousarray(d1["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((m, n2), dtype=torch.bfloat16, device="cuda")
    a2 = pair.fused(x, y2, y1_check=y1)
    torch.cuda.synchronize()
    y1_bits = _bits(y1)
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(9).choice(m, 40, replace=False)]))
    _check_y(O.bf16_bits_to_f32(y1_bits)[rows], O.linear(d1["x"][rows], inv1, ref1)["y"])
    c = dict(m=m, n=n, r2=r, inv2=inv2, ref2=ref2)
    # codes and scales of every row; t2 on the sampled rows
    act_all = O.gelu_quantize(y1_bits, inv2, np.zeros((n, 0), np.float32))
    codes = w4.codes_to_canonical(a2["xq"].cpu().numpy(), m, n, "int4_g64")
    scales = w4.scales_to_canonical(a2["xscale"].cpu().numpy(), m, n, "int4_g64")
    assert np.array_equal(codes, O.pack_int4(act_all["cx"]))
    assert np.array_equal(scales, O.f32_to_bf16_bits(act_all["sx"]))
    act = _check_fc2_activations(c, y1_bits, a2, rows=rows)
    _check_y(O.bf16_bits_to_f32(_bits(y2))[rows], O.linear(act["x2_bits"], inv2, ref2)["y"])
