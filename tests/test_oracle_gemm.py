"""Pins for the oracle's fp64 GEMM y = x . W^T (the plain definition of the
decode GEMM the pages describe: AI Radar summary of SpecPilot, English
edition, "Reasons"; HotRepo digest of StargazerX0/SpecPilot, project
introduction, batch 1-32), against exact integer arithmetic, special cases
and an independently rounded sum."""
import math

import numpy as np
import pytest

from lossless_bit_weight_amd.inputs import f32_to_bf16_bits, gaussian_bf16


def _bf16_of(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_exact_on_small_integers(oracle):
    """Small integer operands make every partial sum exact in fp64, so the
    result must equal Python's exact integer arithmetic bit for bit, and a
    transposed or shifted operand would show."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 256
    xi = rng.integers(-16, 17, size=(M, K))
    wi = rng.integers(-16, 17, size=(N, K))
    y = oracle.gemm_bf16_f64(_bf16_of(xi), _bf16_of(wi))
    exact = [[sum(int(a) * int(b) for a, b in zip(xi[m], wi[n])) for n in range(N)]
             for m in range(M)]
    assert np.array_equal(y, np.array(exact, dtype=np.float64))


def test_one_hot_rows_select_weight_columns(oracle):
    """x = e_k picks column k of W exactly."""
    w = gaussian_bf16((9, 384), 0.02, 5)
    ks = [0, 1, 127, 128, 200, 383]
    x = np.zeros((len(ks), 384), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80
    y = oracle.gemm_bf16_f64(x, w)
    wf = oracle.bf16_bits_to_f64(w)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], wf[:, k])


def test_zero_and_linearity(oracle):
    w = gaussian_bf16((6, 256), 0.02, 8)
    x = gaussian_bf16((3, 256), 1.0, 9)
    assert not oracle.gemm_bf16_f64(np.zeros_like(x), w).any()
    # doubling x is exact in bf16 and in every fp64 partial sum
    x2 = _bf16_of(2.0 * oracle.bf16_bits_to_f64(x).astype(np.float32))
    assert np.array_equal(oracle.gemm_bf16_f64(x2, w), 2.0 * oracle.gemm_bf16_f64(x, w))


def test_against_correctly_rounded_sum(oracle):
    """Compare with math.fsum (correctly rounded) within the textbook bound
    for recursive summation, |err| <= (K-1) u sum|terms|, u = 2^-53."""
    M, N, K = 3, 5, 640
    x = gaussian_bf16((M, K), 1.0, 21)
    w = gaussian_bf16((N, K), 0.02, 22)
    y = oracle.gemm_bf16_f64(x, w)
    xf, wf = oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w)
    for m in range(M):
        for n in range(N):
            terms = xf[m] * wf[n]
            ref = math.fsum(terms.tolist())
            bound = (K - 1) * 2.0 ** -53 * float(np.abs(terms).sum())
            assert abs(y[m, n] - ref) <= bound


def test_matches_library_matmul(oracle):
    """numpy's fp64 matmul is another correct evaluation of the same sum."""
    x = gaussian_bf16((4, 1024), 1.0, 31)
    w = gaussian_bf16((33, 1024), 0.02, 32)
    y = oracle.gemm_bf16_f64(x, w)
    ref = oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_w12_container_gemm_equals_plain_gemm(oracle):
    """Decode-in-the-loop GEMM from the container equals the plain GEMM on
    the unpacked weights, bit for bit, for any thread count."""
    from lossless_bit_weight_amd.inputs import TINY
    p0, p1, p2, meta, _ = oracle.pack(TINY.weights_raw())
    w = oracle.unpack(p0, p1, p2, meta, TINY.N, TINY.K)
    x = TINY.activations(3)
    ref = oracle.gemm_bf16_f64(x, w)
    for t in (1, 3, 8):
        assert np.array_equal(oracle.gemm_w12_f64(x, p0, p1, p2, meta, TINY.N, t), ref)


def test_ieee_specials_propagate(oracle):
    w = np.zeros((3, 128), np.uint16)
    w[0, 5] = 0x7F80          # +Inf
    w[1, 6] = 0x7FC0          # NaN
    w[2, :] = 0x3F80          # 1.0
    x = np.zeros((2, 128), np.uint16)
    x[0, 5] = 0xBF80          # -1 at the Inf column
    x[0, 6] = 0x3F80
    y = oracle.gemm_bf16_f64(x, w)
    assert y[0, 0] == -math.inf
    assert math.isnan(y[0, 1])
    assert y[0, 2] == 0.0
    assert math.isnan(y[1, 0])          # 0 * Inf
    assert math.isnan(y[1, 1])


def test_tolerance_rule(oracle):
    x = _bf16_of([[3.0, 4.0] + [0.0] * 126])
    w = _bf16_of([[1.0] + [0.0] * 127, [0.0] * 128])
    tol = oracle.tolerance(x, w)
    assert tol.shape == (1, 2)
    assert tol[0, 0] == pytest.approx(1e-3 * 5.0 * 1.0 + 1e-6)
    assert tol[0, 1] == pytest.approx(1e-6)
