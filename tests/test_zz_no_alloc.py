"""The no-allocation entry point (w4a4_lowrank_linear_gelu_quant_noalloc) against the entry point
it is a variant of (w4a4_lowrank_linear_gelu_quant), both through the C ABI, on two calls in a row:
the second with a smaller batch, so the fixed scratch is reused with another plane layout. The two
paths run the same kernels on the same inputs, so fc2's codes, scales, t2 and fc1's Y1 must agree
bit for bit."""
import numpy as np
import pytest
import torch

import w4a4_quantized_gemm_smooth_amd as w4
from test_gpu_mlp import _pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    w4.lib()


def _fc2_buffers(m, n, r2):
    sz = w4.buffer_sizes(m, max(r2, 1), n, r2)
    e = lambda nbytes, dt: torch.full((max(nbytes, 16) // torch.tensor([], dtype=dt).element_size(),), 7,
                                      dtype=dt, device="cuda")
    return sz, e(sz["xq"], torch.uint8), e(sz["xscale"], torch.uint8)


def _call(c, m, noalloc):
    """fc1's activation kernel on the first m rows, then fc1's GEMM with fc2's activation side in its
    epilogue through one of the two entry points; returns host copies of what it wrote."""
    f1, f2, n, r2 = c["fc1"], c["fc2"], c["n"], c["r2"]
    x = c["x"][:m]
    a1 = f1.quantize(x)
    sz, xq2, xs2 = _fc2_buffers(m, n, r2)
    mp, rp2 = sz["m_pad"], sz["rank_pad"]
    y1 = torch.full((m, n), -3.0, dtype=torch.bfloat16, device="cuda")
    if noalloc:
        t2 = torch.full((mp * rp2,), 5.0, dtype=torch.float32, device="cuda")   # t2 only: no scratch planes
        w4.lowrank_linear_gelu_quant_noalloc(a1["xq"], a1["xscale"], a1["xl1"], f1.wq, f1.wscale, f1.l2t, f1.bias,
                                             m, n, f1.K, f1.rank, f1.fmt, f2.inv_lambda, f2.l1t, r2, xq2, xs2, t2, y1)
    else:
        t2 = torch.full((w4.gelu_quant_xl1_bytes(m, n, r2) // 4,), 5.0, dtype=torch.float32, device="cuda")
        w4.lowrank_linear_gelu_quant(a1["xq"], a1["xscale"], a1["xl1"], f1.wq, f1.wscale, f1.l2t, f1.bias,
                                     m, n, f1.K, f1.rank, f1.fmt, f2.inv_lambda, f2.l1t, r2, xq2, xs2, t2, y1)
    torch.cuda.synchronize()
    return dict(xq2=xq2.cpu().numpy(), xs2=xs2.cpu().numpy(), t2=t2[: mp * rp2].cpu().numpy(),
                y1=y1.view(torch.int16).cpu().numpy())


def test_noalloc_matches_the_allocating_entry_point_on_two_calls():
    # fc1 700 x 320 -> 1280 (5 column tiles, so 5 partial t2 planes), fc2 rank 20
    c = _pair(700, 320, 1280, 256, 16, 20, seed=61)
    for m in (700, 300):                   # the second call is smaller: other m_pad, other plane layout
        print(f"[no-alloc] M={m} N={c['n']} rank2={c['r2']}", flush=True)
        got = _call(c, m, noalloc=True)
        want = _call(c, m, noalloc=False)
        for k in ("xq2", "xs2", "t2", "y1"):
            assert np.array_equal(got[k], want[k]), f"M={m}: {k} differs from w4a4_lowrank_linear_gelu_quant"
        assert not np.any(got["t2"] == 5.0), "t2 not fully written"
