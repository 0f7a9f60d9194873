"""Python binding of libw4a4: the SVDQuant W4A4 + 16-bit low-rank linear layer on MI355X.

Argument marshalling only. Every step of the layer runs in libw4a4 (host C++ for the offline
weight preparation, HIP kernels for the activation quantizer and the fused GEMM). torch is used
for device memory and streams; numpy arrays carry host buffers.

    import w4a4_quantized_gemm_smooth_amd as w4
    lam, inv = w4.smooth_factors(w4.column_absmax(x_bits), w4.column_absmax(w_bits))
    layer = w4.W4A4Linear.from_weights(w_bits, lam, inv, rank=32)        # host prep + upload
    y = layer(x_bf16_cuda)                                               # two kernels

The library fails loudly when it is missing: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "FMT_INT4_G64", "FMT_MXFP4_B32", "GROUP", "ROW_ALIGN", "MAX_RANK", "W4A4Error", "lib", "lib_path",
    "buffer_sizes", "column_absmax", "smooth_factors", "prepare_weights", "append_lowrank",
    "codes_to_canonical", "scales_to_canonical", "quantize_act", "lowrank_linear", "W4A4Linear",
    "FMT_W8A8", "gelu_quantize_act", "lowrank_linear_gelu_quant", "gelu_quant_xl1_bytes", "MLPPair",
    "lowrank_linear_gelu_quant_noalloc", "NOALLOC_SCRATCH_BYTES",
]

FMT_INT4_G64 = 0
FMT_MXFP4_B32 = 1
FMT_W8A8 = 2
GROUP = 64
MX_BLOCK = 32
ROW_ALIGN = 256
RANK_ALIGN = 16
MAX_RANK = 128
W8A8_MAX_K = 131072
NOALLOC_SCRATCH_BYTES = 32 << 20
_FMT_NAMES = {"int4_g64": FMT_INT4_G64, "mxfp4_b32": FMT_MXFP4_B32, "w8a8": FMT_W8A8}

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libw4a4.so")
_lib = None


class W4A4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().w4a4_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: status {status} ({msg})")


class _Sizes(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_size_t), ("wscale", ctypes.c_size_t), ("l1t", ctypes.c_size_t),
                ("l2t", ctypes.c_size_t), ("xq", ctypes.c_size_t), ("xscale", ctypes.c_size_t),
                ("xl1", ctypes.c_size_t), ("m_pad", ctypes.c_int), ("n_pad", ctypes.c_int),
                ("rank_pad", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """Load libw4a4.so (built by ``python -m w4a4_quantized_gemm_smooth_amd.build``).

    torch is imported first so that the library binds to the HIP runtime torch already loaded
    (one runtime per process; device pointers and streams are shared with torch)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads the process's HIP runtime before libw4a4)
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is missing: build it with "
                              "`python -m w4a4_quantized_gemm_smooth_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(lib_path)
        P, I, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.w4a4_abi_version.restype = I
        L.w4a4_status_str.restype = ctypes.c_char_p
        L.w4a4_status_str.argtypes = [I]
        sigs = {
            "w4a4_buffer_sizes": [I, I, I, I, I, ctypes.POINTER(_Sizes)],
            "w4a4_column_absmax": [P, I, I, I, P],
            "w4a4_smooth_factors": [P, P, I, F, P, P],
            "w4a4_prepare_weights": [P, I, I, P, I, I, P, P, P, P, P, P, P, P],
            "w4a4_prepare_weights_refined": [P, I, I, P, I, I, I, P, P, P, P, P, P, P, P],
            "w4a4_append_lowrank": [P, P, I, I, I, P, P, I, P, P],
            "w4a4_codes_to_canonical": [P, I, I, I, P],
            "w4a4_scales_to_canonical": [P, I, I, I, P],
            "w4a4_quantize_act": [P, I, I, I, P, P, I, I, P, P, P, P],
            "w4a4_lowrank_linear": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P],
            "w4a4_gelu_quantize_act": [P, I, I, I, P, P, I, I, P, P, P, P],
            "w4a4_lowrank_linear_gelu_quant": [P, P, P, P, P, P, P, I, I, I, I, I, P, P, I, P, P, P, P, I, P],
            "w4a4_lowrank_linear_gelu_quant_noalloc": [P, P, P, P, P, P, P, I, I, I, I, I, P, P, I, P, P, P, P, I, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I
        L.w4a4_gelu_quant_xl1_bytes.argtypes = [I, I, I]
        L.w4a4_gelu_quant_xl1_bytes.restype = S
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise W4A4Error(fn, status)


def _fmt(fmt) -> int:
    return _FMT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def _hptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------------- host side
def buffer_sizes(M: int, N: int, K: int, rank: int, fmt=FMT_INT4_G64) -> dict:
    s = _Sizes()
    _check("w4a4_buffer_sizes", lib().w4a4_buffer_sizes(M, N, K, rank, _fmt(fmt), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in _Sizes._fields_}


def column_absmax(a_bits: np.ndarray) -> np.ndarray:
    a = _c(a_bits, np.uint16)
    out = np.empty(a.shape[1], np.float32)
    _check("w4a4_column_absmax", lib().w4a4_column_absmax(_hptr(a), a.shape[0], a.shape[1], a.shape[1], _hptr(out)))
    return out


def smooth_factors(amax_x: np.ndarray, amax_w: np.ndarray, alpha: float = 0.5):
    ax = _c(amax_x, np.float32)
    aw = _c(amax_w, np.float32)
    lam = np.empty_like(ax)
    inv = np.empty_like(ax)
    _check("w4a4_smooth_factors", lib().w4a4_smooth_factors(_hptr(ax), _hptr(aw), ax.size, alpha, _hptr(lam), _hptr(inv)))
    return lam, inv


def prepare_weights(w_bits: np.ndarray, lam: np.ndarray, rank: int, fmt=FMT_INT4_G64, l1_bits=None, l2_bits=None,
                    refine_iters: int = 0):
    """Host weight preparation. Returns numpy arrays in library layout plus the bf16 factors used.
    With ``refine_iters`` > 0 the split is refined iteratively (w4a4_prepare_weights_refined) and the
    result also holds the score of every iteration (``errors``) and the one kept (``iteration``)."""
    if refine_iters:
        return _prepare_weights_refined(w_bits, lam, rank, fmt, refine_iters)
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    f = _fmt(fmt)
    sz = buffer_sizes(1, n, k, rank, f)
    lam = _c(lam, np.float32)
    wq = np.empty(sz["wq"], np.uint8)
    ws = np.empty(sz["wscale"], np.uint8)
    l1t = np.empty(max(sz["l1t"] // 2, 1), np.uint16)
    l2t = np.empty(max(sz["l2t"] // 2, 1), np.uint16)
    l1o = np.empty((k, rank), np.uint16)
    l2o = np.empty((rank, n), np.uint16)
    l1i = None if l1_bits is None else _c(l1_bits, np.uint16)
    l2i = None if l2_bits is None else _c(l2_bits, np.uint16)
    _check("w4a4_prepare_weights", lib().w4a4_prepare_weights(
        _hptr(w), n, k, _hptr(lam), rank, f, _hptr(l1i), _hptr(l2i), _hptr(wq), _hptr(ws),
        _hptr(l1t), _hptr(l2t), _hptr(l1o), _hptr(l2o)))
    return dict(wq=wq, wscale=ws, l1t=l1t[: sz["l1t"] // 2], l2t=l2t[: sz["l2t"] // 2], l1=l1o, l2=l2o,
                N=n, K=k, rank=rank, fmt=f, n_pad=sz["n_pad"], rank_pad=sz["rank_pad"])


def _prepare_weights_refined(w_bits, lam, rank, fmt, iters):
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    f = _fmt(fmt)
    sz = buffer_sizes(1, n, k, rank, f)
    lam = _c(lam, np.float32)
    wq = np.empty(sz["wq"], np.uint8)
    ws = np.empty(sz["wscale"], np.uint8)
    l1t = np.empty(max(sz["l1t"] // 2, 1), np.uint16)
    l2t = np.empty(max(sz["l2t"] // 2, 1), np.uint16)
    l1o = np.empty((k, rank), np.uint16)
    l2o = np.empty((rank, n), np.uint16)
    errs = np.empty(iters + 1, np.float64)
    best = ctypes.c_int(-1)
    _check("w4a4_prepare_weights_refined", lib().w4a4_prepare_weights_refined(
        _hptr(w), n, k, _hptr(lam), rank, f, int(iters), _hptr(wq), _hptr(ws), _hptr(l1t), _hptr(l2t),
        _hptr(l1o), _hptr(l2o), _hptr(errs), ctypes.addressof(best)))
    return dict(wq=wq, wscale=ws, l1t=l1t[: sz["l1t"] // 2], l2t=l2t[: sz["l2t"] // 2], l1=l1o, l2=l2o,
                N=n, K=k, rank=rank, fmt=f, n_pad=sz["n_pad"], rank_pad=sz["rank_pad"], errors=errs.tolist(),
                iteration=best.value)


def append_lowrank(l1t: np.ndarray, l2t: np.ndarray, K: int, N: int, rank: int, a_bits: np.ndarray, b_bits: np.ndarray):
    """LoRA merge on the library-layout factors; returns (l1t', l2t', rank')."""
    a = _c(a_bits, np.uint16)
    b = _c(b_bits, np.uint16)
    ra = a.shape[1]
    sz = buffer_sizes(1, N, K, rank + ra)
    o1 = np.empty(sz["l1t"] // 2, np.uint16)
    o2 = np.empty(sz["l2t"] // 2, np.uint16)
    _check("w4a4_append_lowrank", lib().w4a4_append_lowrank(
        _hptr(_c(l1t, np.uint16)), _hptr(_c(l2t, np.uint16)), K, N, rank, _hptr(a), _hptr(b), ra, _hptr(o1), _hptr(o2)))
    return o1, o2, rank + ra


def codes_to_canonical(q: np.ndarray, rows: int, K: int, fmt=FMT_INT4_G64) -> np.ndarray:
    """[rows][K/2] packed nibbles (INT4, MXFP4) or [rows][K] int8 (W8A8)."""
    w8 = _fmt(fmt) == FMT_W8A8
    out = np.empty((rows, K), np.int8) if w8 else np.empty((rows, K // 2), np.uint8)
    src = np.ascontiguousarray(q).view(np.uint8)
    _check("w4a4_codes_to_canonical", lib().w4a4_codes_to_canonical(_hptr(src), rows, K, _fmt(fmt), _hptr(out)))
    return out


def scales_to_canonical(s: np.ndarray, rows: int, K: int, fmt=FMT_INT4_G64) -> np.ndarray:
    """INT4 [rows][K/64] bf16 bits; MXFP4 [rows][K/32] E8M0 bytes; W8A8 [rows] fp32."""
    f = _fmt(fmt)
    if f == FMT_W8A8:
        out = np.empty(rows, np.float32)
    elif f == FMT_INT4_G64:
        out = np.empty((rows, K // GROUP), np.uint16)
    else:
        out = np.empty((rows, K // MX_BLOCK), np.uint8)
    src = np.ascontiguousarray(s).view(np.uint8)  # raw bytes of the library buffer
    _check("w4a4_scales_to_canonical", lib().w4a4_scales_to_canonical(_hptr(src), rows, K, f, _hptr(out)))
    return out


# --------------------------------------------------------------------------------- device side
def _dptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_matrix(name, t, rows, cols, device=None):
    """A bf16 matrix the kernels read or write by rows: 2-D, unit stride along a row, at least
    ``rows`` x ``cols`` (the kernels address row i at i * stride(0)), on ``device`` if given."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16 (got {t.dtype})")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along its last dimension")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} is {tuple(t.shape)}, needs at least ({rows}, {cols})")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device or 'a GPU'} (got {t.device})")


def _check_buffer(name, t, nbytes, device):
    """A library-layout device buffer of at least ``nbytes`` bytes (None allowed when 0 are needed)."""
    import torch
    if nbytes == 0 and t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor of {nbytes} bytes")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_activation_args(x, inv_lambda, l1t, rank, fmt, xq, xscale, xl1):
    """Shapes, dtypes, devices and sizes of an activation-side call, checked before the launch."""
    M, K = x.shape if hasattr(x, "shape") and len(x.shape) == 2 else (0, 0)
    _check_matrix("x", x, M, K)
    dev = x.device
    sz = buffer_sizes(M, max(rank, 1), K, rank, fmt)
    _check_buffer("inv_lambda", inv_lambda, 4 * K, dev)
    _check_buffer("l1t", l1t, sz["l1t"], dev)
    _check_buffer("xq", xq, sz["xq"], dev)
    _check_buffer("xscale", xscale, sz["xscale"], dev)
    _check_buffer("xl1", xl1, sz["xl1"], dev)


def _check_gemm_args(xq, xscale, xl1, wq, wscale, l2t, bias, y, M, N, K, rank, fmt):
    """Shapes, dtypes, devices and sizes of a GEMM call, checked before the launch."""
    import torch
    if not isinstance(xq, torch.Tensor):
        raise TypeError("xq must be a torch tensor")
    dev = xq.device
    sz = buffer_sizes(M, N, K, rank, fmt)
    # the GEMM reads the scales and t only, not the activation kernel's scratch behind them
    xs_bytes = sz["m_pad"] * 4 if _fmt(fmt) == FMT_W8A8 else sz["xscale"]
    t_bytes = sz["m_pad"] * sz["rank_pad"] * 4
    for name, t, n in (("xq", xq, sz["xq"]), ("xscale", xscale, xs_bytes), ("xl1", xl1, t_bytes),
                       ("wq", wq, sz["wq"]), ("wscale", wscale, sz["wscale"]), ("l2t", l2t, sz["l2t"])):
        _check_buffer(name, t, n, dev)
    if bias is not None:
        _check_buffer("bias", bias, 2 * N, dev)
    if y is not None:
        _check_matrix("y", y, M, N, dev)


def quantize_act(x, inv_lambda, l1t, rank, fmt, xq, xscale, xl1, stream=None):
    """Launch the activation kernel on `stream` (torch stream; default: current). x: [M, K] bf16
    (row stride x.stride(0)); other tensors are library-layout device buffers."""
    M, K = x.shape
    _check_activation_args(x, inv_lambda, l1t, rank, fmt, xq, xscale, xl1)
    _check("w4a4_quantize_act", lib().w4a4_quantize_act(
        _dptr(x), M, K, x.stride(0), _dptr(inv_lambda), _dptr(l1t), rank, _fmt(fmt), _dptr(xq), _dptr(xscale),
        _dptr(xl1), _stream(stream)))


def lowrank_linear(xq, xscale, xl1, wq, wscale, l2t, bias, y, M, N, K, rank, fmt, stream=None):
    """Launch the fused 4-bit GEMM + low-rank epilogue; y: [M, >=N] bf16 (row stride y.stride(0))."""
    _check_gemm_args(xq, xscale, xl1, wq, wscale, l2t, bias, y, M, N, K, rank, fmt)
    _check("w4a4_lowrank_linear", lib().w4a4_lowrank_linear(
        _dptr(xq), _dptr(xscale), _dptr(xl1), _dptr(wq), _dptr(wscale), _dptr(l2t), _dptr(bias), _dptr(y),
        y.stride(0), M, N, K, rank, _fmt(fmt), _stream(stream)))


def gelu_quantize_act(y, inv_lambda, l1t, rank, fmt, xq, xscale, xl1, stream=None):
    """The activation kernel on X = bf16(GELU(y)) of a producer's bf16 output y [M, K] (INT4)."""
    M, K = y.shape
    _check_activation_args(y, inv_lambda, l1t, rank, fmt, xq, xscale, xl1)
    _check("w4a4_gelu_quantize_act", lib().w4a4_gelu_quantize_act(
        _dptr(y), M, K, y.stride(0), _dptr(inv_lambda), _dptr(l1t), rank, _fmt(fmt), _dptr(xq), _dptr(xscale),
        _dptr(xl1), _stream(stream)))


def lowrank_linear_gelu_quant(xq, xscale, xl1, wq, wscale, l2t, bias, M, N, K, rank, fmt, inv_lambda2, l1t2, rank2,
                              xq2, xscale2, xl1_2, y=None, stream=None):
    """fc1's GEMM with fc2's activation side (GELU, smoothing, INT4 codes, t2) in its epilogue;
    y (optional, [M, >=N] bf16) receives fc1's output for checking."""
    _check_gemm_args(xq, xscale, xl1, wq, wscale, l2t, bias, y, M, N, K, rank, fmt)
    dev = xq.device
    s2 = buffer_sizes(M, max(rank2, 1), N, rank2, FMT_INT4_G64)
    _check_buffer("inv_lambda2", inv_lambda2, 4 * N, dev)
    _check_buffer("l1t2", l1t2, s2["l1t"], dev)
    _check_buffer("xq2", xq2, s2["xq"], dev)
    _check_buffer("xscale2", xscale2, s2["xscale"], dev)
    _check_buffer("xl1_2", xl1_2, gelu_quant_xl1_bytes(M, N, rank2), dev)
    _check("w4a4_lowrank_linear_gelu_quant", lib().w4a4_lowrank_linear_gelu_quant(
        _dptr(xq), _dptr(xscale), _dptr(xl1), _dptr(wq), _dptr(wscale), _dptr(l2t), _dptr(bias), M, N, K, rank,
        _fmt(fmt), _dptr(inv_lambda2), _dptr(l1t2), rank2, _dptr(xq2), _dptr(xscale2), _dptr(xl1_2), _dptr(y),
        0 if y is None else y.stride(0), _stream(stream)))


def lowrank_linear_gelu_quant_noalloc(xq, xscale, xl1, wq, wscale, l2t, bias, M, N, K, rank, fmt, inv_lambda2, l1t2,
                                      rank2, xq2, xscale2, t2, y=None, stream=None):
    """As ``lowrank_linear_gelu_quant``, but t2 holds only fc2's t ([m_pad, rank2_pad] fp32) and the
    library keeps the partial planes in its fixed per-GPU scratch (no allocation anywhere; calls that
    overlap on one GPU race)."""
    _check_gemm_args(xq, xscale, xl1, wq, wscale, l2t, bias, y, M, N, K, rank, fmt)
    dev = xq.device
    s2 = buffer_sizes(M, max(rank2, 1), N, rank2, FMT_INT4_G64)
    _check_buffer("inv_lambda2", inv_lambda2, 4 * N, dev)
    _check_buffer("l1t2", l1t2, s2["l1t"], dev)
    _check_buffer("xq2", xq2, s2["xq"], dev)
    _check_buffer("xscale2", xscale2, s2["xscale"], dev)
    _check_buffer("t2", t2, s2["m_pad"] * s2["rank_pad"] * 4, dev)
    _check("w4a4_lowrank_linear_gelu_quant_noalloc", lib().w4a4_lowrank_linear_gelu_quant_noalloc(
        _dptr(xq), _dptr(xscale), _dptr(xl1), _dptr(wq), _dptr(wscale), _dptr(l2t), _dptr(bias), M, N, K, rank,
        _fmt(fmt), _dptr(inv_lambda2), _dptr(l1t2), rank2, _dptr(xq2), _dptr(xscale2), _dptr(t2), _dptr(y),
        0 if y is None else y.stride(0), _stream(stream)))


def gelu_quant_xl1_bytes(M: int, N: int, rank2: int) -> int:
    return int(lib().w4a4_gelu_quant_xl1_bytes(M, N, rank2))


class W4A4Linear:
    """A prepared layer resident in HBM: codes, scales and low-rank factors of one weight.

    ``__call__(x)`` runs the two kernels (quantize_act, lowrank_linear) on the current stream;
    activation buffers are cached per batch size M."""

    def __init__(self, prep: dict, inv_lambda: np.ndarray, device="cuda", bias_bits=None):
        import torch
        self.N, self.K, self.rank, self.fmt = prep["N"], prep["K"], prep["rank"], prep["fmt"]
        dev = torch.device(device)
        up = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
        self.wq = up(prep["wq"], np.uint8)
        self.wscale = up(prep["wscale"], np.uint8)
        self.l1t = up(prep["l1t"], np.int16) if self.rank else None
        self.l2t = up(prep["l2t"], np.int16) if self.rank else None
        self.inv_lambda = up(np.asarray(inv_lambda, np.float32), np.float32)
        self.bias = None if bias_bits is None else up(np.asarray(bias_bits, np.uint16), np.int16)
        self.device = self.wq.device   # with its index ("cuda" -> "cuda:0")
        self._act = {}

    @classmethod
    def from_weights(cls, w_bits, lam, inv_lambda, rank, fmt=FMT_INT4_G64, l1_bits=None, l2_bits=None, **kw):
        return cls(prepare_weights(w_bits, lam, rank, fmt, l1_bits, l2_bits), inv_lambda, **kw)

    def act_buffers(self, M: int):
        import torch
        if M not in self._act:
            sz = buffer_sizes(M, self.N, self.K, self.rank, self.fmt)
            e = lambda n, dt: torch.empty(max(n, 16), dtype=dt, device=self.device)
            self._act[M] = dict(xq=e(sz["xq"], torch.uint8), xscale=e(sz["xscale"], torch.uint8),
                                xl1=e(sz["xl1"] // 4, torch.float32) if self.rank else None)
        return self._act[M]

    def quantize(self, x, stream=None):
        if len(x.shape) != 2 or x.shape[1] != self.K:
            raise ValueError(f"x has shape {tuple(x.shape)}, the layer needs [M, {self.K}]")
        _check_matrix("x", x, 1, self.K, self.device)
        a = self.act_buffers(x.shape[0])
        quantize_act(x, self.inv_lambda, self.l1t, self.rank, self.fmt, a["xq"], a["xscale"], a["xl1"], stream)
        return a

    def gemm(self, a, M, y, stream=None):
        lowrank_linear(a["xq"], a["xscale"], a["xl1"], self.wq, self.wscale, self.l2t, self.bias, y, M, self.N,
                       self.K, self.rank, self.fmt, stream)
        return y

    def __call__(self, x, y=None, stream=None):
        import torch
        M = x.shape[0]
        if y is None:
            y = torch.empty((M, self.N), dtype=torch.bfloat16, device=self.device)
        a = self.quantize(x, stream)
        return self.gemm(a, M, y, stream)


class MLPPair:
    """fc1 -> GELU -> fc2, both prepared W4A4 layers resident in HBM (fc2's K = fc1's N).

    ``fused(x)``: fc1's activation kernel, then fc1's GEMM with fc2's activation side in its
    epilogue (no fc1 output in HBM), then fc2's GEMM. ``unfused(x)``: fc1's two kernels writing
    Y1, fc2's activation kernel applying the GELU to Y1 as it reads it, fc2's GEMM."""

    def __init__(self, fc1: W4A4Linear, fc2: W4A4Linear):
        assert fc2.K == fc1.N, "fc2's K must be fc1's N"
        self.fc1, self.fc2 = fc1, fc2
        self._buf = {}

    def buffers(self, M: int):
        import torch
        if M not in self._buf:
            dev = self.fc1.device
            b = dict(y1=torch.empty((M, self.fc1.N), dtype=torch.bfloat16, device=dev))
            b["act2"] = self.fc2.act_buffers(M)
            n = gelu_quant_xl1_bytes(M, self.fc1.N, self.fc2.rank) // 4
            b["xl1_2_fused"] = torch.empty(max(n, 16), dtype=torch.float32, device=dev) if self.fc2.rank else None
            self._buf[M] = b
        return self._buf[M]

    def fused(self, x, y2, y1_check=None, stream=None):
        M = x.shape[0]
        b = self.buffers(M)
        a1 = self.fc1.quantize(x, stream)
        f1, f2, a2 = self.fc1, self.fc2, b["act2"]
        lowrank_linear_gelu_quant(a1["xq"], a1["xscale"], a1["xl1"], f1.wq, f1.wscale, f1.l2t, f1.bias, M, f1.N, f1.K,
                                  f1.rank, f1.fmt, f2.inv_lambda, f2.l1t, f2.rank, a2["xq"], a2["xscale"],
                                  b["xl1_2_fused"], y1_check, stream)
        a2f = dict(a2, xl1=b["xl1_2_fused"])
        f2.gemm(a2f, M, y2, stream)
        return a2f

    def unfused(self, x, y2, stream=None):
        M = x.shape[0]
        b = self.buffers(M)
        self.fc1(x, b["y1"], stream)
        f2, a2 = self.fc2, b["act2"]
        gelu_quantize_act(b["y1"], f2.inv_lambda, f2.l1t, f2.rank, f2.fmt, a2["xq"], a2["xscale"], a2["xl1"], stream)
        f2.gemm(a2, M, y2, stream)
        return a2
