"""CPU tests of libw4a4's host half against the oracle, ABI validation and the exported symbols.

No GPU is needed: these call only host functions, and device entry points only with arguments
that the library must reject before launching anything.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
import w4a4_quantized_gemm_smooth_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")


def test_library_exports_every_declared_symbol():
    decl = set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", open(HEADER).read()))
    assert len(decl) == 16, sorted(decl)
    L = w4.lib()
    missing = [n for n in decl if not hasattr(L, n)]
    assert not missing, missing
    assert L.w4a4_abi_version() == 2


def test_single_hip_runtime_in_process():
    """libw4a4 binds to the HIP runtime torch loaded (device pointers and streams are shared)."""
    w4.lib()
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths


def test_buffer_sizes():
    s = w4.buffer_sizes(4608, 9216, 3072, 32, w4.FMT_INT4_G64)
    assert (s["m_pad"], s["n_pad"], s["rank_pad"]) == (4608, 9216, 32)
    assert s["wq"] == 9216 * 2304 and s["wscale"] == 48 * 9216 * 2 and s["xl1"] >= 4608 * 32 * 4
    s = w4.buffer_sizes(1000, 300, 128, 20, w4.FMT_MXFP4_B32)
    assert (s["m_pad"], s["n_pad"], s["rank_pad"]) == (1024, 512, 32)
    assert s["wscale"] == 4 * 512 and s["xscale"] == 4 * 1024 and s["l1t"] == 32 * 128 * 2
    s = w4.buffer_sizes(4608, 9216, 3072, 32, w4.FMT_W8A8)
    assert s["wq"] == 9216 * 3072 and s["wscale"] == 9216 * 4 and s["xq"] == 4608 * 3072
    assert s["xscale"] >= 4608 * 4 * 2 and s["xscale"] % (4608 * 4) == 0   # scales + partial maxima


@pytest.mark.parametrize("args,status", [
    ((0, 10, 64, 0, 0), 1), ((10, 0, 64, 0, 0), 1), ((10, 10, 96, 0, 0), 1), ((10, 10, 0, 0, 0), 1),
    ((10, 10, 64, 11, 0), 1), ((10, 200, 64, 65, 0), 1), ((10, 10, 64, -1, 0), 1), ((300, 300, 256, 129, 0), 1),
    ((10, 10, 64, 0, 7), 2), ((10, 10, w4.W8A8_MAX_K + 64, 0, 2), 1),
])
def test_buffer_sizes_rejects(args, status):
    s = w4._Sizes()
    assert w4.lib().w4a4_buffer_sizes(*args, ctypes.byref(s)) == status


def test_column_absmax_and_smooth_factors_match_oracle():
    d = synth.workload("tiny")
    ax, aw = w4.column_absmax(d["x"]), w4.column_absmax(d["w"])
    assert np.array_equal(ax, O.column_absmax(O.bf16_bits_to_f32(d["x"])))
    assert np.array_equal(aw, O.column_absmax(O.bf16_bits_to_f32(d["w"])))
    lam, inv = w4.smooth_factors(ax, aw)
    lo, io = O.smooth_factors(ax, aw)
    assert np.array_equal(lam, lo) and np.array_equal(inv, io)
    ax[3] = 0.0
    lam, _ = w4.smooth_factors(ax, aw)
    assert lam[3] == 1.0
    lam3, _ = w4.smooth_factors(ax, aw, alpha=0.3)
    lo3, _ = O.smooth_factors(ax, aw, alpha=0.3)
    assert np.all(np.abs(lam3.view(np.int32) - lo3.view(np.int32)) <= 1)


def test_smooth_factors_rejects():
    a = np.ones(4, np.float32)
    lam, inv = np.empty(4, np.float32), np.empty(4, np.float32)
    L = w4.lib()
    p = lambda x: ctypes.c_void_p(x.ctypes.data)
    assert L.w4a4_smooth_factors(p(a), p(a), 4, 1.5, p(lam), p(inv)) == 1
    assert L.w4a4_smooth_factors(None, p(a), 4, 0.5, p(lam), p(inv)) == 1
    big = np.full(4, 3e38, np.float32)
    tiny = np.full(4, 1e-45, np.float32)
    assert L.w4a4_smooth_factors(p(big), p(tiny), 4, 0.5, p(lam), p(inv)) == 3  # λ overflows fp32


def _oracle_prep(d, rank, fmt):
    x = O.bf16_bits_to_f32(d["x"])
    w = O.bf16_bits_to_f32(d["w"])
    lam, inv = O.smooth_factors(O.column_absmax(x), O.column_absmax(w))
    return lam, inv, O.prepare_weights(d["w"], lam, rank, fmt)


@pytest.mark.parametrize("shape", [(128, 256, 256, 16), (70, 320, 200, 8), (33, 64, 300, 0), (20, 192, 130, 48)])
@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_weight_codes_bit_exact_given_oracle_factors(shape, fmt):
    m, k, n, r = shape
    d = synth.make_layer(m, k, n, n_outliers=max(1, k // 64), outlier_scale=40.0, seed=11 + k + n)
    lam, inv, ref = _oracle_prep(d, r, fmt)
    l1b, l2b = O.f32_to_bf16_bits(ref["l1"]), O.f32_to_bf16_bits(ref["l2"])
    prep = w4.prepare_weights(d["w"], lam, r, fmt, l1b if r else None, l2b if r else None)
    codes = w4.codes_to_canonical(prep["wq"], n, k, fmt)
    scales = w4.scales_to_canonical(prep["wscale"], n, k, fmt)
    if fmt == "int4_g64":
        assert np.array_equal(codes, O.pack_int4(ref["cw"]))
        assert np.array_equal(scales, O.f32_to_bf16_bits(ref["sw"]))
    elif fmt == "w8a8":
        assert np.array_equal(codes, ref["cw"]) and np.array_equal(scales, ref["sw"])
    else:
        assert np.array_equal(codes, O.pack_nibbles(ref["cw"]))
        assert np.array_equal(scales, ref["sw"])
    if r:
        rp = prep["rank_pad"]
        l1t = prep["l1t"].reshape(rp, k)
        l2t = prep["l2t"].reshape(prep["n_pad"], rp)
        assert np.array_equal(l1t[:r].T, l1b) and not l1t[r:].any()
        assert np.array_equal(l2t[:n, :r].T, l2b) and not l2t[:, r:].any() and not l2t[n:].any()
    # padding rows are zero codes with zero scales
    np_ = prep["n_pad"]
    if fmt == "int4_g64":   # main parts, then the extra parts of both halves
        main = prep["wq"][: k // 64 * np_ * 32].reshape(k // 64, np_, 32)
        extra = prep["wq"][k // 64 * np_ * 32:].reshape(k // 64, 2, np_, 8)
        assert not main[:, n:].any() and not extra[:, :, n:].any()
    else:
        wq = prep["wq"].reshape(k // (32 if fmt == "w8a8" else 64), np_, 32)
        assert not wq[:, n:].any()


def _decode_int4(main, extra0, extra1):
    """Decode the INT4 layout of include/w4a4.h for rows of one group: the FP6 E2M3 images (fields
    sign<<5 | |q| at bit 6f) of the four 16-code runs; half h's main part holds dwords d0 d1 d2 of
    run 2h and d0 of run 2h+1, its extra part d1 d2 of run 2h+1."""
    dw = lambda a: (a.reshape(a.shape[0], -1, 4).astype(np.uint64) *
                    (np.uint64(1) << np.arange(0, 32, 8, dtype=np.uint64))).sum(-1)
    m, x = dw(main), [dw(extra0), dw(extra1)]
    out = np.zeros((main.shape[0], 64), np.int16)
    for h in range(2):
        runs = [m[:, 4 * h: 4 * h + 3], np.stack([m[:, 4 * h + 3], x[h][:, 0], x[h][:, 1]], 1)]
        for j, run in enumerate(runs):
            img = [int(a) | (int(b) << 32) | (int(c) << 64) for a, b, c in run]
            for f in range(16):
                fld = np.array([(v >> (6 * f)) & 63 for v in img], np.int16)
                assert not (fld & 0b011000).any(), "exponent bits of an FP6 carrier must be zero"
                out[:, 32 * h + 16 * j + f] = np.where(fld & 32, -(fld & 7), fld & 7)
        assert all((v >> 96) == 0 for v in img)
    return out


def test_padding_and_layout_of_weight_codes():
    """Library layout: INT4 FP6 images, main parts [G][n_pad][32] then extra parts [G][2][n_pad][8];
    MXFP4 plain E2M1 nibbles [G][n_pad][32]."""
    d = synth.make_layer(8, 64, 3, n_outliers=1, outlier_scale=10.0, seed=3)
    lam = np.ones(64, np.float32)
    prep = w4.prepare_weights(d["w"], lam, 0, "int4_g64")
    q, s = O.quant_int4_g64(O.bf16_bits_to_f32(d["w"]))
    assert prep["wq"].size == 256 * 48
    main = prep["wq"][: 256 * 32].reshape(256, 32)
    extra = prep["wq"][256 * 32:].reshape(2, 256, 8)
    assert np.array_equal(_decode_int4(main[:3], extra[0, :3], extra[1, :3]), q)
    assert not main[3:].any() and not extra[:, 3:].any()
    assert (np.abs(q) >= 6).any() and (q < 0).any()      # the case exercises signs and large codes
    prep = w4.prepare_weights(d["w"], lam, 0, "mxfp4_b32")
    qm, _ = O.quant_mxfp4_b32(O.bf16_bits_to_f32(d["w"]))
    raw = prep["wq"].reshape(1, 256, 32)[0, :3]
    assert np.array_equal(raw & 0xF, qm[:, 0::2]) and np.array_equal(raw >> 4, qm[:, 1::2])
    # W8A8: [K/32][n_pad][32] int8 codes, fp32 per-row scales [n_pad]
    prep = w4.prepare_weights(d["w"], lam, 0, "w8a8")
    q8, s8 = O.quant_int8_rows(O.bf16_bits_to_f32(d["w"]))
    raw = prep["wq"].view(np.int8).reshape(2, 256, 32)
    assert np.array_equal(np.concatenate([raw[0, :3], raw[1, :3]], axis=1), q8) and not raw[:, 3:].any()
    sc = prep["wscale"].view(np.float32)
    assert np.array_equal(sc[:3], s8) and not sc[3:].any()


def _lowrank_err(w_hat, l1_bits, l2_bits):
    approx = O.bf16_bits_to_f32(l1_bits).astype(np.float64) @ O.bf16_bits_to_f32(l2_bits).astype(np.float64)
    return np.linalg.norm(w_hat.T - approx) ** 2


@pytest.mark.parametrize("shape", [(256, 256, 16), (640, 384, 32), (128, 130, 96)])
def test_own_svd_quality(shape):
    """The library's own truncated SVD meets the quality contract of the oracle's LAPACK SVD: the
    rank-r tail energy within 1e-3, each well-separated singular component (gaps > 5% on both sides)
    equal to the oracle's up to the bf16 rounding of the factors, and the same end-to-end error.

    (Singular values are compared through the bf16 factors the ABI returns, so the bound is the
    bf16 rounding of one dominant entry, 2^-8, not the fp64 accuracy of the SVD itself.)"""
    k, n, r = shape
    d = synth.make_layer(128, k, n, n_outliers=max(1, k // 100), outlier_scale=30.0, seed=21 + k)
    lam, inv, ref = _oracle_prep(d, r, "int4_g64")
    prep = w4.prepare_weights(d["w"], lam, r, "int4_g64")
    e_lib = _lowrank_err(ref["w_hat"], prep["l1"], prep["l2"])
    e_ref = _lowrank_err(ref["w_hat"], O.f32_to_bf16_bits(ref["l1"]), O.f32_to_bf16_bits(ref["l2"]))
    assert e_lib <= (1 + 1e-3) * e_ref + 1e-12
    _, s_ref, _, s_all = O.truncated_svd(ref["w_hat"], r)
    l1 = O.bf16_bits_to_f32(prep["l1"]).astype(np.float64)
    l2 = O.bf16_bits_to_f32(prep["l2"]).astype(np.float64)
    gap = np.abs(np.diff(s_all[: r + 1])) / s_all[:r]
    sep = (gap > 0.05) & np.concatenate([[True], gap[:-1] > 0.05])
    assert np.allclose(np.linalg.norm(l1, axis=0)[sep], s_ref[sep], rtol=2.0 ** -8)
    for i in np.flatnonzero(sep):
        mine = np.outer(l1[:, i], l2[i])
        theirs = np.outer(ref["l1"][:, i].astype(np.float64), ref["l2"][i].astype(np.float64))
        assert np.linalg.norm(mine - theirs) <= 2.0 ** -7 * s_ref[i]
    # end-to-end layer error against the unquantized X·Wᵀ, with its own factors vs the oracle's
    x, w = O.bf16_bits_to_f32(d["x"]).astype(np.float64), O.bf16_bits_to_f32(d["w"]).astype(np.float64)
    exact = x @ w.T
    y_ref = O.linear(d["x"], inv, ref)["y"]
    own = O.prepare_weights(d["w"], lam, r, "int4_g64", l1=O.bf16_bits_to_f32(prep["l1"]), l2=O.bf16_bits_to_f32(prep["l2"]))
    y_own = O.linear(d["x"], inv, own)["y"]
    assert np.linalg.norm(y_own - exact) <= 1.05 * np.linalg.norm(y_ref - exact)


def test_own_svd_deterministic():
    d = synth.make_layer(16, 256, 256, n_outliers=3, outlier_scale=30.0, seed=2)
    lam = np.ones(256, np.float32)
    a = w4.prepare_weights(d["w"], lam, 16)
    b = w4.prepare_weights(d["w"], lam, 16)
    assert all(np.array_equal(a[k], b[k]) for k in ("wq", "wscale", "l1t", "l2t"))


def _split_error_of(prep, w_bits, lam, fmt):
    """The oracle's split error of a library preparation (codes and scales decoded canonically)."""
    n, k = w_bits.shape
    canon = w4.codes_to_canonical(prep["wq"], n, k, fmt)
    w_hat = O.smooth_weights(O.bf16_bits_to_f32(w_bits), lam)
    l1 = O.bf16_bits_to_f32(prep["l1"])
    l2 = O.bf16_bits_to_f32(prep["l2"])
    if fmt == "w8a8":
        return O.split_error(w_hat, l1, l2, canon, w4.scales_to_canonical(prep["wscale"], n, k, fmt), fmt)
    lo, hi = canon & 0xF, canon >> 4
    nib = np.empty((n, k), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = lo, hi
    sc = w4.scales_to_canonical(prep["wscale"], n, k, fmt)
    if fmt == "int4_g64":
        codes = np.where(nib >= 8, nib.astype(np.int16) - 16, nib.astype(np.int16))
        scales = O.bf16_bits_to_f32(sc)
    else:
        codes, scales = nib, sc
    return O.split_error(w_hat, l1, l2, codes, scales, fmt)


@pytest.mark.parametrize("fmt", ["int4_g64", "mxfp4_b32", "w8a8"])
def test_refined_split(fmt):
    """Iterative refinement (§4.2): iteration 0 is the plain preparation byte for byte; the kept
    iteration's arrays reproduce its reported score (recomputed by the oracle) and have the
    smallest score; the refinement lowers the error, as the oracle's own refinement does."""
    d = synth.make_layer(96, 256, 192, n_outliers=4, outlier_scale=30.0, seed=21)
    lam, _ = O.smooth_factors(O.column_absmax(O.bf16_bits_to_f32(d["x"])), O.column_absmax(O.bf16_bits_to_f32(d["w"])))
    plain = w4.prepare_weights(d["w"], lam, 8, fmt)
    r0 = w4._prepare_weights_refined(d["w"], lam, 8, fmt, 0)
    for key in ("wq", "wscale", "l1t", "l2t", "l1", "l2"):
        assert np.array_equal(r0[key], plain[key]), key
    assert r0["errors"][0] == pytest.approx(_split_error_of(plain, d["w"], lam, fmt), rel=1e-12)
    rf = w4.prepare_weights(d["w"], lam, 8, fmt, refine_iters=4)
    e = rf["errors"]
    assert len(e) == 5 and e[rf["iteration"]] == min(e) and e.index(min(e)) == rf["iteration"]
    assert _split_error_of(rf, d["w"], lam, fmt) == pytest.approx(e[rf["iteration"]], rel=1e-12)
    assert min(e) < 0.97 * e[0]
    ref = O.prepare_weights_refined(d["w"], lam, 8, fmt, iters=4)
    assert e[0] == pytest.approx(ref["errors"][0], rel=2e-3)          # own SVD vs LAPACK
    assert min(e) == pytest.approx(min(ref["errors"]), rel=2e-2)
    with pytest.raises(w4.W4A4Error):
        w4._prepare_weights_refined(d["w"], lam, 8, fmt, 65)


def test_append_lowrank():
    d = synth.make_layer(16, 128, 200, n_outliers=2, outlier_scale=30.0, seed=9, lora_rank=16)
    lam = np.ones(128, np.float32)
    base = w4.prepare_weights(d["w"], lam, 8)
    l1t, l2t, r2 = w4.append_lowrank(base["l1t"], base["l2t"], 128, 200, 8, d["lora_a"], d["lora_b"])
    assert r2 == 24
    l1t = l1t.reshape(32, 128)
    l2t = l2t.reshape(256, 32)
    assert np.array_equal(l1t[:8].T, base["l1"]) and np.array_equal(l1t[8:24].T, d["lora_a"]) and not l1t[24:].any()
    assert np.array_equal(l2t[:200, :8].T, base["l2"]) and np.array_equal(l2t[:200, 8:24].T, d["lora_b"])
    assert not l2t[:, 24:].any() and not l2t[200:].any()


def test_prepare_rejects():
    L = w4.lib()
    w = np.zeros((8, 64), np.uint16)
    lam = np.ones(64, np.float32)
    buf = np.zeros(1 << 16, np.uint8)
    p = lambda x: ctypes.c_void_p(x.ctypes.data)
    assert L.w4a4_prepare_weights(p(w), 8, 64, p(lam), 0, 0, None, None, None, p(buf), None, None, None, None) == 1
    assert L.w4a4_prepare_weights(p(w), 8, 64, p(lam), 9, 0, None, None, p(buf), p(buf), p(buf), p(buf), None, None) == 1
    assert L.w4a4_prepare_weights(p(w), 8, 64, p(lam), 2, 0, p(w), None, p(buf), p(buf), p(buf), p(buf), None, None) == 1
    assert L.w4a4_prepare_weights(p(w), 8, 60, p(lam), 0, 0, None, None, p(buf), p(buf), None, None, None, None) == 1
    assert L.w4a4_prepare_weights(p(w), 8, 64, p(lam), 0, 3, None, None, p(buf), p(buf), None, None, None, None) == 2
    bad = lam.copy()
    bad[5] = 0.0
    assert L.w4a4_prepare_weights(p(w), 8, 64, p(bad), 0, 0, None, None, p(buf), p(buf), None, None, None, None) == 1


def test_device_entry_points_validate_before_launch():
    """Invalid arguments are rejected on the host; nothing reaches the GPU (none is present here)."""
    L = w4.lib()
    al = np.zeros(1 << 12, np.uint8)
    base = al.ctypes.data + (-al.ctypes.data) % 256
    P = lambda off=0: ctypes.c_void_p(base + off)
    # quantize_act: null X, bad K, ldx < K, ldx misaligned, misaligned pointer, rank without l1t, bad fmt
    assert L.w4a4_quantize_act(None, 4, 64, 64, P(), None, 0, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(), 4, 96, 96, P(), None, 0, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(), 4, 64, 32, P(), None, 0, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(), 4, 64, 68, P(), None, 0, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(2), 4, 64, 64, P(), None, 0, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(), 4, 64, 64, P(), None, 16, 0, P(), P(), None, None) == 1
    assert L.w4a4_quantize_act(P(), 4, 64, 64, P(), None, 0, 5, P(), P(), None, None) == 2
    # lowrank_linear: ldy < N, null Y, rank > N, misaligned codes, rank without l2t, odd Y
    assert L.w4a4_lowrank_linear(P(), P(), None, P(), P(), None, None, P(), 8, 4, 16, 64, 0, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(), P(), None, P(), P(), None, None, None, 16, 4, 16, 64, 0, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(), P(), P(), P(), P(), P(), None, P(), 16, 4, 16, 64, 17, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(8), P(), None, P(), P(), None, None, P(), 16, 4, 16, 64, 0, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(), P(), P(), P(), P(), None, None, P(), 16, 4, 16, 64, 8, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(), P(), None, P(), P(), None, None, P(1), 16, 4, 16, 64, 0, 0, None) == 1
    assert L.w4a4_lowrank_linear(P(), P(), None, P(), P(), None, None, P(), 16, 4, 16, 64, 0, 9, None) == 2


def test_mlp_pair_entry_points_validate_before_launch():
    """The GELU paths accept INT4 only, ranks <= 32 for the fused GEMM, and whole 64-groups."""
    L = w4.lib()
    al = np.zeros(1 << 12, np.uint8)
    base = al.ctypes.data + (-al.ctypes.data) % 256
    P = lambda off=0: ctypes.c_void_p(base + off)
    assert L.w4a4_gelu_quantize_act(P(), 4, 64, 64, P(), None, 0, 1, P(), P(), None, None) == 2   # MXFP4
    assert L.w4a4_gelu_quantize_act(P(), 4, 64, 32, P(), None, 0, 0, P(), P(), None, None) == 1   # ldy < K
    assert L.w4a4_gelu_quantize_act(None, 4, 64, 64, P(), None, 0, 0, P(), P(), None, None) == 1
    args = lambda **kw: dict(dict(xq=P(), xs=P(), xl1=None, wq=P(), ws=P(), l2t=None, bias=None, M=4, N=128, K=64,
                                  rank=0, fmt=0, il2=P(), l1t2=None, rank2=0, xq2=P(), xs2=P(), xl12=None, Y=None,
                                  ldy=0), **kw)
    call = lambda a: L.w4a4_lowrank_linear_gelu_quant(*a.values(), None)
    assert call(args(fmt=1)) == 2
    assert call(args(rank=33, N=256, K=64, xl1=P(), l2t=P())) in (1, 2)
    assert call(args(rank2=33, l1t2=P(), xl12=P())) == 2
    assert call(args(N=96)) == 1                     # fc2's K = N must be whole 64-groups
    assert call(args(il2=None)) == 1
    assert call(args(rank2=8)) == 1                  # rank2 without L1_2 / t2 buffers
    assert call(args(Y=P(1), ldy=128)) == 1          # misaligned Y
    assert w4.gelu_quant_xl1_bytes(300, 640, 20) == 512 * 32 * 4 * (1 + 3)
    assert w4.gelu_quant_xl1_bytes(300, 256, 20) == 512 * 32 * 4
    assert w4.gelu_quant_xl1_bytes(300, 256, 0) == 0


def test_binding_validates_tensors_before_the_library():
    """The Python binding rejects tensors whose dtype, layout, shape, size or device would make a
    kernel read or write out of bounds; none of these calls reaches libw4a4."""
    import torch
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    M, K, N, r = 300, 256, 320, 16
    sz = w4.buffer_sizes(M, N, K, r)
    cpu = torch.device("cpu")
    buf = lambda n, dt=u8: torch.zeros(max(n, 16) // torch.tensor([], dtype=dt).element_size(), dtype=dt)
    xq, xs, xl1 = buf(sz["xq"]), buf(sz["xscale"]), buf(sz["xl1"], f32)
    wq, ws, l1t, l2t = buf(sz["wq"]), buf(sz["wscale"]), buf(sz["l1t"], torch.int16), buf(sz["l2t"], torch.int16)
    inv = buf(4 * K, f32)
    x = torch.zeros((M, K), dtype=bf)
    y = torch.zeros((M, N), dtype=bf)
    with pytest.raises(ValueError, match="bfloat16"):
        w4.quantize_act(x.float(), inv, l1t, r, 0, xq, xs, xl1)
    with pytest.raises(ValueError, match="unit stride"):
        w4.quantize_act(torch.zeros((K, M), dtype=bf).t(), inv, l1t, r, 0, xq, xs, xl1)
    with pytest.raises(ValueError, match="GPU"):                       # a host tensor
        w4.quantize_act(x, inv, l1t, r, 0, xq, xs, xl1)
    with pytest.raises(ValueError, match="needs at least"):            # Y with too few rows
        w4.lowrank_linear(xq, xs, xl1, wq, ws, l2t, None, y[: M - 1], M, N, K, r, 0)
    with pytest.raises(ValueError, match="needs at least"):            # Y with too few columns
        w4.lowrank_linear(xq, xs, xl1, wq, ws, l2t, None, y[:, : N - 1], M, N, K, r, 0)
    with pytest.raises(ValueError, match="bytes, needs"):              # weight codes sized for a smaller N
        w4.lowrank_linear(xq, xs, xl1, wq[: sz["wq"] // 2], ws, l2t, None, y, M, N, K, r, 0)
    with pytest.raises(ValueError, match="bytes, needs"):              # bias shorter than N
        w4.lowrank_linear(xq, xs, xl1, wq, ws, l2t, buf(2 * N - 2, torch.int16), y, M, N, K, r, 0)
    with pytest.raises(ValueError, match="contiguous"):
        w4.lowrank_linear(xq, xs, xl1, wq, ws, l2t.view(-1, 2).t(), None, y, M, N, K, r, 0)
    with pytest.raises(TypeError):
        w4.lowrank_linear(xq, xs, xl1, None, ws, l2t, None, y, M, N, K, r, 0)
    # a layer object checks x against its K before anything else
    layer = object.__new__(w4.W4A4Linear)
    layer.K, layer.device = K, cpu
    with pytest.raises(ValueError, match="needs \\[M, 256\\]"):
        layer.quantize(torch.zeros((M, K + 64), dtype=bf))


def test_non_finite_inputs_are_rejected():
    """Inf / NaN in any host input gives W4A4_ERR_NUMERIC and leaves the outputs untouched."""
    L = w4.lib()
    p = lambda a: ctypes.c_void_p(a.ctypes.data)
    rng = np.random.default_rng(9)
    N, K = 8, 64
    w = synth.f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    lam = np.ones(K, np.float32)
    sz = w4.buffer_sizes(1, N, K, 0)
    for bad in (0x7F80, 0xFF80, 0x7FC1):            # +Inf, -Inf, NaN (bf16 bit patterns)
        wb = w.copy()
        wb[3, 17] = bad
        out = np.full(K, -1.0, np.float32)
        assert L.w4a4_column_absmax(p(wb), N, K, K, p(out)) == 3
        assert np.all(out == -1.0)
        wq = np.full(sz["wq"], 0xAB, np.uint8)
        ws = np.full(sz["wscale"], 0xAB, np.uint8)
        assert L.w4a4_prepare_weights(p(wb), N, K, p(lam), 0, 0, None, None, p(wq), p(ws),
                                      None, None, None, None) == 3
        assert np.all(wq == 0xAB) and np.all(ws == 0xAB)
    # a non-finite channel maximum
    ax = np.ones(K, np.float32)
    lo, io = np.zeros(K, np.float32), np.zeros(K, np.float32)
    for v in (np.inf, np.nan):
        a2 = ax.copy()
        a2[5] = v
        assert L.w4a4_smooth_factors(p(a2), p(ax), K, ctypes.c_float(0.5), p(lo), p(io)) == 3
        assert L.w4a4_smooth_factors(p(ax), p(a2), K, ctypes.c_float(0.5), p(lo), p(io)) == 3
        assert not lo.any() and not io.any()
    # non-finite factors given to the preparation, or to the LoRA merge
    r = 2
    l1 = synth.f32_to_bf16_bits(rng.standard_normal((K, r)).astype(np.float32))
    l2 = synth.f32_to_bf16_bits(rng.standard_normal((r, N)).astype(np.float32))
    l1[7, 1] = 0x7FC0
    s2 = w4.buffer_sizes(1, N, K, r)
    bufs = [np.zeros(s2[k], np.uint8) for k in ("wq", "wscale", "l1t", "l2t")]
    assert L.w4a4_prepare_weights(p(w), N, K, p(lam), r, 0, p(l1), p(l2), *[p(b) for b in bufs], None, None) == 3
    l1t = np.zeros(s2["l1t"] // 2, np.uint16)
    l2t = np.zeros(s2["l2t"] // 2, np.uint16)
    so = w4.buffer_sizes(1, N, K, 2 * r)
    o1, o2 = np.zeros(so["l1t"] // 2, np.uint16), np.zeros(so["l2t"] // 2, np.uint16)
    assert L.w4a4_append_lowrank(p(l1t), p(l2t), K, N, r, p(l1), p(l2), r, p(o1), p(o2)) == 3
    assert w4.lib().w4a4_status_str(5) == b"host memory allocation failed"


def test_shape_checks_do_not_overflow():
    """Row counts close to INT_MAX are rejected instead of wrapping when padded to 256."""
    s = w4._Sizes()
    big = 2 ** 31 - 1
    assert w4.lib().w4a4_buffer_sizes(big, 64, 64, 0, 0, ctypes.byref(s)) == 1
    assert w4.lib().w4a4_buffer_sizes(64, big - 100, 64, 0, 0, ctypes.byref(s)) == 1


def test_host_half_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The host half (w4a4_host.cpp, plain C++) built with ASan + UBSan and driven through its C ABI by
    a small program (tests/host_sanitize_main.cpp): the preparations, refinement, LoRA merge, canonical
    layouts and argument checks run clean (any report aborts the program)."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_sanitize")
    src = os.path.join(ROOT, "w4a4_quantized_gemm_smooth_amd", "csrc", "w4a4_host.cpp")
    drv = os.path.join(ROOT, "tests", "host_sanitize_main.cpp")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "w4a4_quantized_gemm_smooth_amd", "csrc"),
           src, drv, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "host half OK" in run.stdout


def test_noalloc_entry_point_rejects_before_touching_the_gpu():
    """The no-allocation MLP call checks its arguments, and that the partial planes fit its fixed
    scratch, before anything else (no GPU is present here)."""
    L = w4.lib()
    al = np.zeros(1 << 12, np.uint8)
    base = al.ctypes.data + (-al.ctypes.data) % 256
    P = lambda off=0: ctypes.c_void_p(base + off)
    f = L.w4a4_lowrank_linear_gelu_quant_noalloc
    # planes: ceil(N / 256) * m_pad * rank2_pad * 4 bytes > 32 MiB -> W4A4_ERR_TOO_LARGE (6)
    M, N = 16384, 4096                      # 16 tiles * 16384 * 32 * 4 = 32 MiB + ... > limit at rank2 32
    assert 16 * 16384 * 32 * 4 >= w4.NOALLOC_SCRATCH_BYTES
    assert f(P(), P(), None, P(), P(), None, None, M + 256, N, 64, 0, 0, P(), P(), 32, P(), P(), P(), None, 0, None) == 6
    assert f(P(), P(), None, P(), P(), None, None, 4, 128, 64, 0, 1, P(), None, 0, P(), P(), None, None, 0, None) == 2
    assert f(P(), P(), None, P(), P(), None, None, 4, 96, 64, 0, 0, P(), None, 0, P(), P(), None, None, 0, None) == 1
    assert f(P(), P(), None, P(), P(), None, None, 4, 128, 64, 0, 0, P(), None, 8, P(), P(), None, None, 0, None) == 1
    assert L.w4a4_status_str(6) == b"problem exceeds the no-allocation call's fixed scratch"
