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


GUARD = 256          # canary bytes before and after every activation buffer
CANARY = 0xA5


def _guarded(nbytes, dev="cuda"):
    """A device buffer of `nbytes` (16-byte aligned) with GUARD canary bytes on each side."""
    n = max(nbytes, 16)
    raw = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=dev)
    return raw, raw[GUARD: GUARD + n]


def _guards_intact(raw, nbytes):
    h = raw.cpu().numpy()
    n = max(nbytes, 16)
    return bool(np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + n:] == CANARY))


def gpu_layer(d, lam, inv, rank, fmt, ref_prep=None, bias=None, x_rows=None, pad_cols=0, prep=None):
    """Library prep from the oracle's factors (or the given `prep`), upload, run both kernels with
    canary-guarded activation buffers and a canary row and columns around Y; return host copies."""
    if prep is None:
        l1b = O.f32_to_bf16_bits(ref_prep["l1"]) if rank else None
        l2b = O.f32_to_bf16_bits(ref_prep["l2"]) if rank else None
        prep = w4.prepare_weights(d["w"], lam, rank, fmt, l1b, l2b)
    layer = w4.W4A4Linear(prep, inv, bias_bits=bias)
    xb = d["x"] if x_rows is None else d["x"][:x_rows]
    M, K = xb.shape
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)
    sz = w4.buffer_sizes(M, prep["N"], K, rank, fmt)
    raw = {k: _guarded(sz[k]) for k in ("xq", "xscale", "xl1")}
    xq, xs, xl1 = raw["xq"][1], raw["xscale"][1], raw["xl1"][1].view(torch.float32) if rank else None
    yfull = torch.full((M + 1, prep["N"] + pad_cols), -7.0, dtype=torch.bfloat16, device="cuda")   # canaries
    y = yfull[:M]
    w4.quantize_act(x, layer.inv_lambda, layer.l1t, rank, fmt, xq, xs, xl1)
    w4.lowrank_linear(xq, xs, xl1, layer.wq, layer.wscale, layer.l2t, layer.bias, y, M, prep["N"], K, rank, fmt)
    torch.cuda.synchronize()
    for k, (r, _) in raw.items():
        if k != "xl1" or rank:
            assert _guards_intact(r, sz[k]), f"{k}: canary bytes around the buffer were overwritten"
    yh = O.bf16_bits_to_f32(yfull.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(yh[M] == -7.0), "wrote past row M of Y"
    out = dict(prep=prep, layer=layer, M=M, xq=xq.cpu().numpy(), xscale=xs.cpu().numpy(), y=yh[:M])
    if rank:
        rp = prep["rank_pad"]
        out["t"] = xl1.cpu().numpy()[: (M + 255) // 256 * 256 * rp].reshape(-1, rp)[:M]  # t, then scratch
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


@pytest.mark.parametrize("shape", [
    (64, 128, 96, 2),
    (300, 256, 260, 16),
    (2000, 1088, 8440, 16),   # 17 groups: two full rounds of the GEMM's 8-slot LDS ring and a partial one,
                              # on 8 x 33 = 264 output tiles (more than the GPU runs at once), ragged M and N
    (300, 256, 260, 32),      # t tile staged in LDS with 128-byte rows (two 16-rank steps per read)
    (520, 1088, 600, 48),     # 192-byte t rows (a two-step and a one-step read), ragged tiles
])
def test_exact_arithmetic_layer_bit_exact(shape):
    """λ = 1, power-of-two scales, representable X̂ and R, one-hot L1: every rounding is exact, so
    the GPU must reproduce the oracle's Y bit for bit."""
    from test_oracle_pins import exact_case
    m, k, n, r = shape
    c = exact_case(m, k, n, r, seed=m)
    lam = np.ones(k, np.float32)
    ref = O.prepare_weights(c["w_bits"], lam, r, l1=c["l1"], l2=c["l2"])
    d = dict(x=c["x_bits"], w=c["w_bits"])
    print(f"[exact int4] M={m} K={k} N={n} r={r}", flush=True)
    g = gpu_layer(d, lam, lam, r, "int4_g64", ref, pad_cols=3)
    y_ref = O.linear(c["x_bits"], lam, ref)["y"]
    assert np.array_equal(y_ref, O.bf16_rne(c["y_exact"].astype(np.float32)))
    assert np.array_equal(g["y"][:, :n], y_ref)
    assert np.all(g["y"][:, n:] == -7.0)


@pytest.mark.parametrize("shape", [
    (96, 128, 160, 0),        # 128 x 128 small-grid kernel, no low-rank branch
    (300, 1088, 260, 16),     # small-grid kernel, 17 groups (the 8-slot ring wraps twice)
    (2000, 1088, 8440, 16),   # large-grid kernel (16 x 66 blocks of 128²), up projection before the loop
    (1000, 256, 8440, 40),    # large-grid kernel, rank > 32: up projection in the epilogue
    (300, 1088, 260, 32),     # small-grid kernel, t tile staged with 128-byte rows
    (2000, 256, 8440, 32),    # large-grid kernel, t tile staged with 128-byte rows
])
def test_mxfp4_exact_arithmetic_layer_bit_exact(shape):
    """MXFP4 counterpart: E2M1 values times a power of two per 32-block with a ±6 in every block
    (so the block exponent and the codes are exact), λ = 1, one-hot L1; the scaled MFMA applies the
    block scales exactly and every fp32 partial sum is exact, so Y is bit-exact."""
    from test_oracle_pins import mx_exact_case
    m, k, n, r = shape
    c = mx_exact_case(m, k, n, r, seed=k + n)
    lam = np.ones(k, np.float32)
    ref = O.prepare_weights(c["w_bits"], lam, r, "mxfp4_b32", l1=c["l1"], l2=c["l2"])
    d = dict(x=c["x_bits"], w=c["w_bits"])
    print(f"[exact mxfp4] M={m} K={k} N={n} r={r}", flush=True)
    g = gpu_layer(d, lam, lam, r, "mxfp4_b32", ref, pad_cols=3)
    check_activation_side(d, lam, ref, "mxfp4_b32", g)
    y_ref = O.linear(c["x_bits"], lam, ref)["y"]
    assert np.array_equal(y_ref, O.bf16_rne(c["y_exact"].astype(np.float32)))
    assert np.array_equal(g["y"][:, :n], y_ref)
    assert np.all(g["y"][:, n:] == -7.0)


@pytest.mark.parametrize("shape", [
    (64, 256, 96, 0),         # no low-rank branch
    (300, 512, 260, 16),      # t tile staged in LDS (64-byte rows)
    (2000, 512, 8440, 32),    # 128-byte t rows, 8 x 33 = 264 output tiles, ragged M and N
    (520, 256, 600, 48),      # rank > 32: t read from global memory in the epilogue
])
def test_w8a8_exact_arithmetic_layer_bit_exact(shape):
    """8-bit setting: per-row powers of two as the per-token and per-channel scales, λ = 1, one-hot
    L1; the int32 products and every fp32 step of the epilogue are exact, so Y is bit-exact."""
    from test_oracle_pins import w8_exact_case
    m, k, n, r = shape
    c = w8_exact_case(m, k, n, r, seed=m + k)
    lam = np.ones(k, np.float32)
    ref = O.prepare_weights(c["w_bits"], lam, r, "w8a8", l1=c["l1"], l2=c["l2"])
    d = dict(x=c["x_bits"], w=c["w_bits"])
    print(f"[exact w8a8] M={m} K={k} N={n} r={r}", flush=True)
    g = gpu_layer(d, lam, lam, r, "w8a8", ref, pad_cols=3)
    check_activation_side(d, lam, ref, "w8a8", g)
    y_ref = O.linear(c["x_bits"], lam, ref)["y"]
    assert np.array_equal(y_ref, O.bf16_rne(c["y_exact"].astype(np.float32)))
    assert np.array_equal(g["y"][:, :n], y_ref)
    assert np.all(g["y"][:, n:] == -7.0)


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
def test_strided_activations(fmt):
    """X as a column slice of a wider matrix (row stride ldx = K + 72 elements, the extra columns
    filled with large values that must not be read): codes, scales, t and Y bit-identical to the
    same rows passed contiguously."""
    m, k, n, r = 333, 448, 264, 20
    d = synth.make_layer(m, k, n, n_outliers=5, outlier_scale=30.0, seed=31)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, fmt, lam)
    bf = lambda a: O.f32_to_bf16_bits(a)
    lay = w4.W4A4Linear(w4.prepare_weights(d["w"], lam, r, fmt, bf(ref["l1"]), bf(ref["l2"])), inv)
    print(f"[strided X] fmt={fmt} M={m} K={k} ldx={k + 72} N={n} r={r}", flush=True)
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    wide = torch.full((m, k + 72), 3.0e4, dtype=torch.bfloat16, device="cuda")
    wide[:, :k] = x
    xs = wide[:, :k]
    assert xs.stride(0) == k + 72 and xs.stride(1) == 1
    outs = []
    for xin in (x, xs):
        sz = w4.buffer_sizes(m, n, k, r, fmt)
        a = dict(xq=torch.zeros(sz["xq"], dtype=torch.uint8, device="cuda"),
                 xscale=torch.zeros(sz["xscale"], dtype=torch.uint8, device="cuda"),
                 xl1=torch.zeros(sz["xl1"] // 4, dtype=torch.float32, device="cuda"))
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        w4.quantize_act(xin, lay.inv_lambda, lay.l1t, r, fmt, a["xq"], a["xscale"], a["xl1"])
        lay.gemm(a, m, y)
        torch.cuda.synchronize()
        mp, rp = sz["m_pad"], sz["rank_pad"]
        outs.append((a["xq"].cpu(), a["xscale"][: sz["xscale"] if fmt != "w8a8" else mp * 4].cpu(),
                     a["xl1"][: mp * rp].cpu(), y.cpu()))
    for name, u, v in zip(("codes", "scales", "t", "y"), outs[0], outs[1]):
        assert torch.equal(u, v), f"{name} differ with a row stride above K"
    y_ref = O.linear(d["x"], inv, ref)["y"]
    yb = O.bf16_bits_to_f32(outs[1][3].view(torch.int16).numpy().view(np.uint16))
    assert np.abs(yb - y_ref).max() <= TOL * np.abs(y_ref).max()


def test_concurrent_host_threads():
    """Two host threads, each with its own stream, layer (INT4 and MXFP4) and buffers, call both
    kernels eight times at once; every result is bit-identical to the same call made alone."""
    import threading
    jobs = []
    for i, fmt in enumerate(("int4_g64", "mxfp4_b32")):
        d = synth.make_layer(300 + 97 * i, 320, 392, n_outliers=4, outlier_scale=30.0, seed=41 + i)
        lam, inv = _smooth(d)
        ref = oracle_weights(d, 16, fmt, lam)
        bf = lambda a: O.f32_to_bf16_bits(a)
        lay = w4.W4A4Linear(w4.prepare_weights(d["w"], lam, 16, fmt, bf(ref["l1"]), bf(ref["l2"])), inv)
        x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
        jobs.append((lay, x, torch.cuda.Stream()))
    print("[threads] int4 + mxfp4 on two streams from two host threads", flush=True)
    alone = [lay(x).cpu() for lay, x, _ in jobs]
    torch.cuda.synchronize()
    got, errors = [[], []], []

    def work(j):
        lay, x, st = jobs[j]
        try:
            with torch.cuda.stream(st):
                for _ in range(8):
                    got[j].append(lay(x, stream=st))
            st.synchronize()
        except Exception as e:  # reported below: a thread's exception does not fail the test by itself
            errors.append(e)
    th = [threading.Thread(target=work, args=(j,)) for j in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for j in range(2):
        assert len(got[j]) == 8
        for y in got[j]:
            assert torch.equal(y.cpu(), alone[j]), f"thread {j}: a concurrent call differs from the call made alone"


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_graph_capture_and_replay(fmt):
    """The layer step (activation side, then the GEMM) captured once in a HIP graph: the library's
    launches allocate nothing and clear nothing, so the graph replays it. Three replays, each on new
    activations copied into the captured input and with eager library calls on other buffers in
    between; every replay bit-exact against the eager step on the same input, and the first against
    the oracle."""
    m, k, n, r = 700, 384, 520, 24
    d = synth.make_layer(m, k, n, n_outliers=4, outlier_scale=30.0, seed=21)
    lam, inv = _smooth(d)
    ref = oracle_weights(d, r, fmt, lam)
    bf = lambda a: O.f32_to_bf16_bits(a)
    lay = w4.W4A4Linear(w4.prepare_weights(d["w"], lam, r, fmt, bf(ref["l1"]), bf(ref["l2"])), inv)
    print(f"[graph replay] fmt={fmt} M={m} K={k} N={n} r={r}", flush=True)
    xs = [synth.make_layer(m, k, n, n_outliers=4, outlier_scale=30.0, seed=21 + i)["x"] for i in range(4)]
    dev_x = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
    x = dev_x(xs[0])
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    a = lay.act_buffers(m)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        lay.quantize(x, side)
        lay.gemm(a, m, y, side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            lay.quantize(x, side)
            lay.gemm(a, m, y, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # eager references on separate buffers (the graph's own buffers belong to the capture)
    other = w4.W4A4Linear(w4.prepare_weights(d["w"], lam, r, fmt, bf(ref["l1"]), bf(ref["l2"])), inv)
    for i, xb in enumerate(xs[1:] + xs[:1]):
        x.copy_(dev_x(xb))
        y_eager = other(dev_x(xb))
        torch.cuda.synchronize()
        g.replay()
        junk = other(dev_x(xs[(i + 2) % 4]))   # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs from the eager step"
        if i == 3:   # xs[0] again: against the oracle
            y_ref = O.linear(xs[0], inv, ref)["y"]
            yb = O.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))
            assert np.abs(yb - y_ref).max() <= 2.0 ** -7 * np.abs(y_ref).max()
        del junk


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
    rows = _sample_rows(m, n=160, seed=k)
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


def _full_y(name):
    """The oracle's Y over every row of a full-size workload (cached: several tests compare to it)."""
    key = (name, "y")
    if key not in _CACHE:
        d, lam, inv, ref = _full(name)
        _CACHE[key] = O.linear(d["x"], inv, ref)["y"]
    return _CACHE[key]


def _sample_rows(M, n=48, seed=0):
    """Random rows plus the first and last row of every 256-row output tile row."""
    rng = np.random.default_rng(seed)
    edges = np.concatenate([np.arange(0, M, 256), np.minimum(np.arange(255, M + 255, 256), M - 1)])
    return np.unique(np.concatenate([[0, M - 1], edges, rng.choice(M, min(n, M), replace=False)]))


@pytest.mark.parametrize("name", ["flux_qkv", "flux_mlp_fc1", "flux_mlp_fc2"])
def test_full_size_int4(name):
    d, lam, inv, ref = _full(name)
    print(f"[{name}] M={d['M']} K={d['K']} N={d['N']} r={d['rank']}", flush=True)
    g = gpu_layer(d, lam, inv, d["rank"], d["fmt"], ref)
    wcodes = w4.codes_to_canonical(g["prep"]["wq"], d["N"], d["K"], d["fmt"])
    assert np.array_equal(wcodes, O.pack_int4(ref["cw"]))
    check_activation_side(d, inv, ref, d["fmt"], g)
    check_y(g, _full_y(name))                                # every row of Y


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
    check_y(g, O.linear(d["x"], inv, ref)["y"])              # every row of Y


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
    check_y(dict(y=yg), O.linear(d["x"], inv, merged)["y"])   # every row of Y
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
    if m <= 4608:   # every row; at M = 16384 sampled rows (the oracle's full Y takes minutes there)
        check_y(g, O.linear(d["x"][:m], inv, ref)["y"])
    else:
        rows = _sample_rows(m, n=200, seed=m)
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
    rows = _sample_rows(m, n=160, seed=r)
    check_y(g, O.linear(d["x"][rows], inv, ref)["y"], rows)
    assert np.all(g["y"][:, n:] == -7.0), "wrote outside the M x N block"


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_largest_operands(fmt):
    """The largest activation operand the kernels' 32-bit offsets allow: rows_pad·K = 2^31 elements
    (INT4, MXFP4; W8A8, whose one-byte codes must stay below 2^31 bytes, one row tile less) at
    K 16384 with a ragged M, ragged N (320) with bias and rank 16. X repeats 512 seeded rows (the
    host holds only those); every row of Y's first and last tiles, the rows around each 8192-row
    boundary and random rows are compared with the oracle, and t on the same rows."""
    K, N, r = 16384, 320, 16
    rows_pad = (1 << 31) // K - (256 if fmt == "w8a8" else 0)
    M = rows_pad - 100
    base = synth.make_layer(512, K, N, n_outliers=16, outlier_scale=30.0, seed=77)
    lam, inv = _smooth(base)
    ref = oracle_weights(base, r, fmt, lam)
    rng = np.random.default_rng(5)
    bias = O.f32_to_bf16_bits(O.bf16_rne(rng.standard_normal(N).astype(np.float32)))
    bf = O.f32_to_bf16_bits
    lay = w4.W4A4Linear(w4.prepare_weights(base["w"], lam, r, fmt, bf(ref["l1"]), bf(ref["l2"])), inv, bias_bits=bias)
    print(f"[largest operands] fmt={fmt} M={M} (rows_pad {rows_pad}) K={K} N={N} r={r}", flush=True)
    xb = torch.from_numpy(np.ascontiguousarray(base["x"]).view(np.int16)).cuda()
    x = xb[torch.arange(M, device="cuda") % 512].view(torch.bfloat16)       # row i = base row i % 512
    y = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    a = lay.act_buffers(M)
    lay.quantize(x)
    lay.gemm(a, M, y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(M - 256, M),
                                     (np.arange(8192, M, 8192)[:, None] + np.arange(-2, 2)).ravel(),
                                     rng.choice(M, 64, replace=False)]))
    rows = rows[(rows >= 0) & (rows < M)]
    sel = torch.from_numpy(rows).cuda()
    yb = O.bf16_bits_to_f32(y[sel].view(torch.int16).cpu().numpy().view(np.uint16))
    xr = base["x"][rows % 512]
    want = O.linear(xr, inv, ref, bias)
    err = np.abs(yb.astype(np.float64) - want["y"].astype(np.float64)).max()
    assert err <= TOL * np.abs(want["y"]).max(), f"max|dY| = {err}"
    rp = (r + 15) // 16 * 16
    t = a["xl1"][: rows_pad * rp].view(rows_pad, rp)[sel].cpu().numpy()
    act = O.quantize_activations(xr, inv, ref["l1"], fmt)
    terms = np.abs(O.bf16_rne(act["x_hat"]).astype(np.float64)) @ np.abs(ref["l1"].astype(np.float64))
    assert np.all(np.abs(t[:, :r] - act["t"]) <= 2.0 * K * 2.0 ** -24 * terms + 1e-30), "t outside the fp32 bound"
    del x, xb, y, a
    lay._act.clear()
    torch.cuda.empty_cache()


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


# ------------------------------------------------------------ the layer the library prepares itself
def _check_weight_codes(prep, ref, N, K, fmt):
    """The library's weight codes and scales, canonicalized, against the oracle's quantization."""
    codes = w4.codes_to_canonical(prep["wq"], N, K, fmt)
    scales = w4.scales_to_canonical(prep["wscale"], N, K, fmt)
    if fmt == "int4_g64":
        assert np.array_equal(codes, O.pack_int4(ref["cw"])) and np.array_equal(scales, O.f32_to_bf16_bits(ref["sw"]))
    elif fmt == "mxfp4_b32":
        assert np.array_equal(codes, O.pack_nibbles(ref["cw"])) and np.array_equal(scales, ref["sw"])
    else:
        assert np.array_equal(codes, ref["cw"]) and np.array_equal(scales, ref["sw"])


@pytest.mark.parametrize("name,fmt", [("tiny", "int4_g64"), ("flux_qkv", "int4_g64"), ("tiny", "mxfp4_b32"),
                                      ("tiny", "w8a8")])
@pytest.mark.parametrize("refine", [0, 2])
def test_library_prepared_layer(name, fmt, refine):
    """The layer exactly as the bench builds it: λ from the library's own channel maxima, the
    library's own rank-r SVD (and, with `refine`, its iterative refinement of the split, §4.2),
    then both kernels. λ and 1/λ are bit-exact; the weight codes and scales are bit-exact against
    the oracle's quantization of the residual left by the library's factors; the activation side is
    bit-exact; every row of Y is within 2^-7·max|Y_ref| of the oracle's layer built from the same
    factors; and the whole layer is as close to the unquantized X·Wᵀ as the oracle's own
    (LAPACK-SVD) layer, within 5% (the SVD is a different algorithm, so its factors are not
    elementwise comparable)."""
    d = synth.workload(name)
    r, K, N = d["rank"], d["K"], d["N"]
    ax, aw = w4.column_absmax(d["x"]), w4.column_absmax(d["w"])
    lam, inv = w4.smooth_factors(ax, aw)
    lo, io = _smooth(d)
    assert np.array_equal(lam, lo) and np.array_equal(inv, io), "λ or 1/λ differ from the oracle's"
    prep = w4.prepare_weights(d["w"], lam, r, fmt, refine_iters=refine)
    if refine:
        assert prep["errors"][prep["iteration"]] == min(prep["errors"])
    l1, l2 = O.bf16_bits_to_f32(prep["l1"]), O.bf16_bits_to_f32(prep["l2"])
    ref = O.prepare_weights(d["w"], lam, r, fmt, l1=l1, l2=l2)
    _check_weight_codes(prep, ref, N, K, fmt)
    print(f"[library prep] {name} {fmt} M={d['M']} K={K} N={N} r={r} refine={refine}", flush=True)
    g = gpu_layer(d, lam, inv, r, fmt, prep=prep, pad_cols=3)
    check_activation_side(d, inv, ref, fmt, g)
    check_y(g, O.linear(d["x"], inv, ref)["y"])
    # end to end against the unquantized layer: ||Y - X·Wᵀ||_F vs the oracle's own layer
    x64 = O.bf16_bits_to_f32(d["x"]).astype(np.float64)
    exact = x64 @ O.bf16_bits_to_f32(d["w"]).astype(np.float64).T
    y_lapack = _full_y(name) if name != "tiny" else O.linear(d["x"], inv, O.prepare_weights(d["w"], lam, r, fmt))["y"]
    e_lib = np.linalg.norm(g["y"][:, :N].astype(np.float64) - exact)
    e_ref = np.linalg.norm(y_lapack.astype(np.float64) - exact)
    assert e_lib <= 1.05 * e_ref, f"library-prepared layer error {e_lib} vs oracle layer {e_ref}"
