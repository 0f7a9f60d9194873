"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element.

Contract
  * activation codes and scales: bit-exact (canonical form);
  * t = bf16(X̂)·L1: |Δ| <= 2·K·2^-24·Σ_k |bf16(X̂)_k·L1_k| per element (fp32 accumulation bound);
  * Y: max|Y_gpu − Y_ref| <= 2^-7 · max|Y_ref| (bf16 output), the oracle's Y computed in fp64;
  * exact-arithmetic layers: Y bit-exact.
Weights are prepared by the library's host code from the oracle's own low-rank factors, so the
4-bit weight codes are the oracle's (checked bit-exact on the CPU in test_host_prep.py, and again
here at full size). Full-size workloads are checked on all activation codes and on sampled rows
of Y that the oracle computes one by one.
"""
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


# ------------------------------------------------------------------------------- helpers
def _smooth(d):
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    return O.smooth_factors(O.column_absmax(x), O.column_absmax(w))


def oracle_weights(d, rank, fmt, lam):
    return O.prepare_weights(d["w"], lam, rank, fmt)


def gpu_layer(d, lam, inv, rank, fmt, ref_prep, bias=None, x_rows=None, pad_cols=0):
    """Library prep from the oracle's factors, upload, run both kernels; return host copies."""
    l1b = O.f32_to_bf16_bits(ref_prep["l1"]) if rank else None
    l2b = O.f32_to_bf16_bits(ref_prep["l2"]) if rank else None
    prep = w4.prepare_weights(d["w"], lam, rank, fmt, l1b, l2b)
    layer = w4.W4A4Linear(prep, inv, bias_bits=bias)
    xb = d["x"] if x_rows is None else d["x"][:x_rows]
    M, K = xb.shape
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.full((M, prep["N"] + pad_cols), -7.0, dtype=torch.bfloat16, device="cuda")   # canary columns
    a = layer.quantize(x)
    layer.gemm(a, M, y)
    torch.cuda.synchronize()
    out = dict(prep=prep, layer=layer, M=M,
               xq=a["xq"].cpu().numpy(), xscale=a["xscale"].cpu().numpy(),
               y=O.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)))
    if rank:
        rp = prep["rank_pad"]
        out["t"] = a["xl1"].cpu().numpy()[: (M + 255) // 256 * 256 * rp].reshape(-1, rp)[:M]  # t, then scratch
    return out


def check_activation_side(d, inv, ref_prep, fmt, g, rows=None):
    xb = d["x"] if rows is None else d["x"][:rows]
    act = O.quantize_activations(xb, inv, ref_prep["l1"], fmt)
    M, K = xb.shape
    codes = w4.codes_to_canonical(g["xq"], M, K, fmt)
    scales = w4.scales_to_canonical(g["xscale"], M, K, fmt)
    if fmt == "int4_g64":
        assert np.array_equal(codes, O.pack_int4(act["cx"])), "activation codes differ"
        assert np.array_equal(scales, O.f32_to_bf16_bits(act["sx"])), "activation scales differ"
    elif fmt == "w8a8":
        assert np.array_equal(codes, act["cx"]), "activation codes differ"
        assert np.array_equal(scales, act["sx"]), "activation scales differ"
        # padding rows: zero codes, zero scales
        mp = (M + 255) // 256 * 256
        assert not g["xq"].view(np.int8).reshape(K // 32, mp, 32)[:, M:].any()
        assert not g["xscale"].view(np.float32)[M:mp].any()
    else:
        assert np.array_equal(codes, O.pack_nibbles(act["cx"])), "activation codes differ"
        assert np.array_equal(scales, act["sx"]), "activation scales differ"
    r = ref_prep["l1"].shape[1]
    if r:
        terms = np.abs(O.bf16_rne(act["x_hat"]).astype(np.float64)) @ np.abs(ref_prep["l1"].astype(np.float64))
        bound = 2.0 * K * 2.0 ** -24 * terms + 1e-30
        assert np.all(np.abs(g["t"][:, :r] - act["t"]) <= bound), "t outside the fp32 bound"
        assert not g["t"][:, r:].any()
    return act


def check_y(g, y_ref, rows=None):
    y = g["y"][:, : y_ref.shape[1]] if rows is None else g["y"][rows, : y_ref.shape[1]]
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64)).max()
    assert err <= TOL * np.abs(y_ref).max(), f"max|dY| = {err} > 2^-7 * {np.abs(y_ref).max()}"
    return err


def oracle_rows(d, inv, ref_prep, fmt, rows, bias=None):
    """Oracle Y for selected rows only (each row is independent of the others)."""
    sub = O.linear(d["x"][rows], inv, ref_prep, bias)
    return sub["y"]


# ------------------------------------------------------------------------------- small cases
@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_tiny_layer(fmt):
    d = synth.workload("tiny")
    lam, inv = _smooth(d)
    ref = oracle_weights(d, 16, fmt, lam)
    g = gpu_layer(d, lam, inv, 16, fmt, ref, pad_cols=8)
    check_activation_side(d, inv, ref, fmt, g)
    y_ref = O.linear(d["x"], inv, ref)["y"]
    check_y(g, y_ref)
    assert np.all(g["y"][:, 256:] == -7.0), "wrote outside the M x N block"


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
@pytest.mark.parametrize("shape", [(200, 320, 300, 20), (1, 64, 7, 0), (257, 128, 513, 48), (130, 192, 129, 5)])
def test_ragged_shapes_with_bias(fmt, shape):
    m, k, n, r = shape
    d = synth.make_layer(m, k, n, n_outliers=max(1, k // 64), outlier_scale=30.0, seed=100 + m + n)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, fmt, lam)
    bias = synth.f32_to_bf16_bits(np.random.default_rng(m).standard_normal(n).astype(np.float32))
    g = gpu_layer(d, lam, inv, r, fmt, ref, bias=bias, pad_cols=3)
    check_activation_side(d, inv, ref, fmt, g)
    y_ref = O.linear(d["x"], inv, ref, bias)["y"]
    check_y(g, y_ref)
    assert np.all(g["y"][:, n:] == -7.0)


def test_exact_arithmetic_layer_bit_exact():
    """λ = 1, power-of-two scales, representable X̂ and R, one-hot L1: every rounding is exact, so
    the GPU must reproduce the oracle's Y bit for bit."""
    from test_oracle_pins import exact_case
    for (m, k, n, r) in ((64, 128, 96, 2), (300, 256, 260, 16)):
        c = exact_case(m, k, n, r, seed=m)
        lam = np.ones(k, np.float32)
        ref = O.prepare_weights(c["w_bits"], lam, r, l1=c["l1"], l2=c["l2"])
        d = dict(x=c["x_bits"], w=c["w_bits"])
        g = gpu_layer(d, lam, lam, r, "int4_g64", ref)
        y_ref = O.linear(c["x_bits"], lam, ref)["y"]
        assert np.array_equal(g["y"][:, :n], y_ref)
        assert np.array_equal(y_ref, O.bf16_rne(c["y_exact"].astype(np.float32)))


def test_zero_and_tiny_activations():
    """All-zero rows and groups whose scale would be subnormal give zero codes and zero scales."""
    d = synth.make_layer(64, 256, 128, n_outliers=2, outlier_scale=30.0, seed=4)
    x = d["x"].copy()
    x[3] = 0
    x[5, :64] = synth.f32_to_bf16_bits(np.full(64, 1e-39, np.float32))
    d = dict(d, x=x)
    lam, inv = _smooth(d)
    for fmt in ("int4_g64", "mxfp4_b32", "w8a8"):
        ref = oracle_weights(d, 8, fmt, lam)
        g = gpu_layer(d, lam, inv, 8, fmt, ref)
        check_activation_side(d, inv, ref, fmt, g)
        check_y(g, O.linear(d["x"], inv, ref)["y"])


def test_deterministic_and_stream():
    d = synth.make_layer(512, 512, 384, n_outliers=5, outlier_scale=30.0, seed=8)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, 32, "int4_g64", lam)
    g1 = gpu_layer(d, lam, inv, 32, "int4_g64", ref)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g2 = gpu_layer(d, lam, inv, 32, "int4_g64", ref)
    torch.cuda.synchronize()
    for k in ("xq", "xscale", "t", "y"):
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
@pytest.mark.parametrize("case", [
    (2000, 512, 8440, 20, True),   # 8 x 33 = 264 tiles (more than the GPU runs at once), 8 groups
    (2000, 832, 8440, 20, True),   # 13 groups: the last ring round is partial
    (1999, 512, 8443, 0, False),   # N not a multiple of 8: element stores
])
def test_many_tiles_ragged(fmt, case):
    """More 256 x 256 output tiles than the GPU has compute units, with ragged M and N, so the last
    tile row and column are partial (Y checked on sampled rows, every column, and the canary
    columns past N)."""
    m, k, n, r, with_bias = case
    d = synth.make_layer(m, k, n, n_outliers=3, outlier_scale=30.0, seed=m + k + n)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, fmt, lam)
    bias = (synth.f32_to_bf16_bits(np.random.default_rng(n).standard_normal(n).astype(np.float32))
            if with_bias else None)
    print(f"[many tiles] {fmt} M={m} K={k} N={n} r={r} bias={with_bias}", flush=True)
    g = gpu_layer(d, lam, inv, r, fmt, ref, bias=bias, pad_cols=5)
    check_activation_side(d, inv, ref, fmt, g)
    rows = _sample_rows(m, n=40, seed=k)
    check_y(g, O.linear(d["x"][rows], inv, ref, bias)["y"], rows)
    assert np.all(g["y"][:, n:] == -7.0), "wrote outside the M x N block"


# ------------------------------------------------------------------------------- full sizes
_CACHE = {}


def _full(name):
    if name not in _CACHE:
        d = synth.workload(name)
        lam, inv = _smooth(d)
        ref = oracle_weights(d, d["rank"], d["fmt"], lam)
        _CACHE[name] = (d, lam, inv, ref)
    return _CACHE[name]


def _sample_rows(M, n=48, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n, replace=False)]))


@pytest.mark.parametrize("name", ["flux_qkv", "flux_mlp_fc1", "flux_mlp_fc2"])
def test_full_size_int4(name):
    d, lam, inv, ref = _full(name)
    print(f"[{name}] M={d['M']} K={d['K']} N={d['N']} r={d['rank']}", flush=True)
    g = gpu_layer(d, lam, inv, d["rank"], d["fmt"], ref)
    wcodes = w4.codes_to_canonical(g["prep"]["wq"], d["N"], d["K"], d["fmt"])
    assert np.array_equal(wcodes, O.pack_int4(ref["cw"]))
    check_activation_side(d, inv, ref, d["fmt"], g)
    rows = _sample_rows(d["M"])
    check_y(g, oracle_rows(d, inv, ref, d["fmt"], rows), rows)


def test_full_size_w8a8():
    """The 8-bit setting (App. D) on the FLUX QKV shapes: all activation codes and per-token
    scales bit-exact, the weight codes bit-exact, Y on sampled rows."""
    d, lam, inv, _ = _full("flux_qkv")
    key = ("flux_qkv", "w8a8")
    if key not in _CACHE:
        _CACHE[key] = oracle_weights(d, d["rank"], "w8a8", lam)
    ref = _CACHE[key]
    print(f"[flux_qkv w8a8] M={d['M']} K={d['K']} N={d['N']} r={d['rank']}", flush=True)
    g = gpu_layer(d, lam, inv, d["rank"], "w8a8", ref)
    wcodes = w4.codes_to_canonical(g["prep"]["wq"], d["N"], d["K"], "w8a8")
    assert np.array_equal(wcodes, ref["cw"])
    check_activation_side(d, inv, ref, "w8a8", g)
    rows = _sample_rows(d["M"], seed=5)
    check_y(g, oracle_rows(d, inv, ref, "w8a8", rows), rows)


def test_full_size_lora_merge():
    """LoRA merged into the low-rank branch without re-quantizing R (r = 32 + 16 = 48)."""
    d = synth.workload("flux_qkv_lora")
    lam, inv = _smooth(d)
    base = _full("flux_qkv")[3]
    a = O.bf16_bits_to_f32(d["lora_a"])
    b = O.bf16_bits_to_f32(d["lora_b"])
    merged = dict(base, l1=np.concatenate([base["l1"], a], 1), l2=np.concatenate([base["l2"], b], 0))
    l1b, l2b = O.f32_to_bf16_bits(base["l1"]), O.f32_to_bf16_bits(base["l2"])
    prep = w4.prepare_weights(d["w"], lam, 32, "int4_g64", l1b, l2b)
    l1t, l2t, r2 = w4.append_lowrank(prep["l1t"], prep["l2t"], d["K"], d["N"], 32, d["lora_a"], d["lora_b"])
    prep_m = dict(prep, l1t=l1t, l2t=l2t, rank=r2, rank_pad=48)
    layer = w4.W4A4Linear(prep_m, inv)
    x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
    y = layer(x)
    torch.cuda.synchronize()
    M = d["M"]
    t = layer.act_buffers(M)["xl1"].cpu().numpy()[: (M + 255) // 256 * 256 * 48].reshape(-1, 48)[:M]
    yg = O.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))
    rows = _sample_rows(M, seed=3)
    check_y(dict(y=yg), oracle_rows(d, inv, merged, "int4_g64", rows), rows)
    # the LoRA columns of t are bf16(X̂)·A within the fp32 bound
    xh = O.smooth_activations(O.bf16_bits_to_f32(d["x"]), inv)
    xb = O.bf16_rne(xh).astype(np.float64)
    ta = xb @ a.astype(np.float64)
    assert np.all(np.abs(t[:, 32:48] - ta) <= 2 * d["K"] * 2.0 ** -24 * (np.abs(xb) @ np.abs(a.astype(np.float64))) + 1e-30)
    # low-rank-only run: zero 4-bit branch, L1 = A, L2 = B -> Y = bf16(bf16(t_A)·B)
    zprep = dict(prep, wq=np.zeros_like(prep["wq"]), wscale=np.zeros_like(prep["wscale"]))
    z1, z2, _ = w4.append_lowrank(np.zeros(0, np.uint16), np.zeros(0, np.uint16), d["K"], d["N"], 0,
                                  d["lora_a"], d["lora_b"])
    zl = w4.W4A4Linear(dict(zprep, l1t=z1, l2t=z2, rank=16, rank_pad=16), inv)
    yz = O.bf16_bits_to_f32(zl(x).view(torch.int16).cpu().numpy().view(np.uint16))
    want = O.bf16_rne((O.bf16_rne(ta.astype(np.float32)).astype(np.float64) @ b.astype(np.float64)).astype(np.float32))
    assert np.abs(yz - want).max() <= TOL * np.abs(want).max()


def test_unfused_lowrank_ablation():
    """The bench's unfused baseline (rank-0 main branch of this library on the residual codes, the
    low-rank branch as separate library GEMMs) computes the same layer: Y within the same bound."""
    import bench
    d = synth.make_layer(300, 512, 640, n_outliers=5, outlier_scale=30.0, seed=11)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, 32, "int4_g64", lam)
    l1b, l2b = O.f32_to_bf16_bits(ref["l1"]), O.f32_to_bf16_bits(ref["l2"])
    prep = w4.prepare_weights(d["w"], lam, 32, "int4_g64", l1b, l2b)
    dev = torch.device("cuda")
    layer_u = bench.unfused_layer(prep, inv, dev)
    l1s, l2 = bench.unfused_lowrank_factors(prep, inv, dev)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((300, 640), dtype=torch.bfloat16, device=dev)
    bench.unfused_step(layer_u, layer_u.act_buffers(300), x, y, l1s, l2)
    torch.cuda.synchronize()
    check_y(dict(y=O.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))),
            O.linear(d["x"], inv, ref)["y"])


@pytest.mark.parametrize("m", [1024, 4608, 16384])
def test_full_size_mxfp4_sweep(m):
    d, lam, inv, ref = _full("mxfp4_sweep")
    print(f"[mxfp4_sweep] M={m} K={d['K']} N={d['N']}", flush=True)
    g = gpu_layer(d, lam, inv, d["rank"], d["fmt"], ref, x_rows=m)
    check_activation_side(d, inv, ref, d["fmt"], g, rows=m)
    rows = _sample_rows(m, seed=m)
    check_y(g, oracle_rows(d, inv, ref, d["fmt"], rows), rows)


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_max_rank(fmt):
    """The largest supported rank (128: eight 16-rank MFMA steps in both projections)."""
    m, k, n, r = 300, 256, 300, w4.MAX_RANK
    d = synth.make_layer(m, k, n, n_outliers=4, outlier_scale=30.0, seed=128)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, fmt, lam)
    print(f"[max rank] {fmt} M={m} K={k} N={n} r={r}", flush=True)
    g = gpu_layer(d, lam, inv, r, fmt, ref, pad_cols=2)
    check_activation_side(d, inv, ref, fmt, g)
    check_y(g, O.linear(d["x"], inv, ref)["y"])


@pytest.mark.parametrize("r", [48, 128])
def test_mxfp4_large_grid_high_rank(r):
    """MXFP4 on a grid too large for the 128 x 128 kernel (8 x 66 blocks of 128², so the INT8
    GEMM's MXFP4 mode runs) with a rank above 32, whose up projection is added in the epilogue from
    global memory instead of before the main loop; ragged M and N, canary columns past N."""
    m, k, n = 1000, 256, 8440
    d = synth.make_layer(m, k, n, n_outliers=4, outlier_scale=30.0, seed=r)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, "mxfp4_b32", lam)
    print(f"[mxfp4 large grid] M={m} K={k} N={n} r={r}", flush=True)
    g = gpu_layer(d, lam, inv, r, "mxfp4_b32", ref, pad_cols=3)
    check_activation_side(d, inv, ref, "mxfp4_b32", g)
    rows = _sample_rows(m, n=40, seed=r)
    check_y(g, O.linear(d["x"][rows], inv, ref)["y"], rows)
    assert np.all(g["y"][:, n:] == -7.0), "wrote outside the M x N block"


def test_w8a8_largest_k():
    """W8A8 at the largest K whose int32 dot products cannot overflow (127² · 131072 < 2^31), with
    rows of near-full-scale codes so that the exact sums come close to the limit."""
    m, k, n = 40, w4.W8A8_MAX_K, 24
    rng = np.random.default_rng(31)
    x = np.sign(rng.standard_normal((m, k))).astype(np.float32)        # ±1: every code ±127
    w = (np.sign(rng.standard_normal((n, k))) * 0.02).astype(np.float32)
    x[:4] = 1.0                                                        # rows whose products all align
    w[:4] = 0.02
    d = dict(x=synth.f32_to_bf16_bits(x), w=synth.f32_to_bf16_bits(w))
    lam = np.ones(k, np.float32)
    ref = O.prepare_weights(d["w"], lam, 0, "w8a8")
    assert np.abs(ref["cw"]).max() == 127
    print(f"[w8a8 max K] M={m} K={k} N={n}", flush=True)
    g = gpu_layer(d, lam, lam, 0, "w8a8", ref)
    act = check_activation_side(d, lam, ref, "w8a8", g)
    assert np.abs(act["cx"]).min() == 127
    check_y(g, O.linear(d["x"], lam, ref)["y"])
