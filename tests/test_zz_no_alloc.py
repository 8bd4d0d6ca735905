"""w12_gemm_noalloc, the entry point for callers that cannot allocate: called
through the C ABI, its output equals w12_gemm_ws's bit for bit (same kernels,
same tiling, same summation order) and the fp64 oracle's within the GEMM
tolerance -- on two calls in a row, the second on a smaller input, both with
K split over workgroups so the library's fixed scratch carries the partial
sums (the first also with an exception list)."""
import ctypes

import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import assert_gemm_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _raw(shape, sigma, seed, p_zero=0.001):
    return inputs.inject_zeros(inputs.gaussian_bf16(shape, sigma, seed), p_zero, seed + 1)


def _noalloc_raw(x, wt, y):
    """The C call itself, with every pointer marshalled here."""
    eo, ee = wt.exc_ptrs()
    return w12.lib().w12_gemm_noalloc(
        x.data_ptr(), x.shape[0], x.stride(0), wt.p0.data_ptr(), wt.p1.data_ptr(),
        wt.p2.data_ptr(), wt.meta.data_ptr(), eo, ee, wt.N, wt.K, y.data_ptr(), y.stride(0),
        w12.OUT_F32 if y.dtype == torch.float32 else w12.OUT_BF16,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (M, N, K, seed, with exception list): the second call is smaller; both
# default tilings split K (checked below).
CALLS = [(16, 1024, 5120, 61, True), (9, 512, 2560, 62, False)]


def test_noalloc_matches_gemm_ws_twice(oracle):
    require_gpu()
    for M, N, K, seed, exc in CALLS:
        print("noalloc: M=%d N=%d K=%d exceptions=%s" % (M, N, K, exc), flush=True)
        assert w12.w12_default_tiling(M, N, K, True).splitk > 1
        bits = _raw((N, K), 0.02, seed)
        if exc:
            wt, bad = w12.pack(to_dev(bits), exceptions=True)
            assert bad > 0 and wt.exc_offsets is not None
            w_ref = bits
        else:
            first, _ = w12.pack(to_dev(bits))
            w_ref = first_bits = w12.w12_unpack(first).view(torch.int16).cpu().numpy().view(np.uint16)
            wt, bad = w12.pack(to_dev(first_bits))
            assert bad == 0
        xb = inputs.gaussian_bf16((M, K), 1.0, seed + 100)
        x = to_dev(xb)
        y_ws = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        w12.w12_gemm(x, wt, y=y_ws)                      # w12_gemm_ws
        assert _noalloc_raw(x, wt, y_na) == 0
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), "w12_gemm_noalloc differs from w12_gemm_ws"
        yh = y_na.cpu().numpy()
        assert_gemm_close(yh, oracle.gemm_bf16_f64(xb, w_ref), oracle.tolerance(xb, w_ref),
                          "noalloc M=%d N=%d K=%d" % (M, N, K))
        # BF16 output through the binding: the rounding of the same sums
        y_b = w12.w12_gemm_noalloc(x, wt, torch.bfloat16)
        y_wb = w12.w12_gemm(x, wt, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y_b.view(torch.int16), y_wb.view(torch.int16))
