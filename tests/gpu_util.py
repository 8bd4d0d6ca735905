"""Helpers for the GPU tests: host <-> device copies of BF16 bit patterns and
the GEMM acceptance rule.  Imported by tests only."""
from __future__ import annotations

import numpy as np
import torch


def require_gpu() -> None:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns -> int16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def assert_gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, tol: np.ndarray, what: str) -> None:
    """|y_gpu - y_ref| <= 1e-3 ||x_m|| ||w_n|| + 1e-6 element by element
    (tol holds that bound); NaN must match NaN and infinities must match."""
    y_gpu = y_gpu.astype(np.float64)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y_gpu), nan_ref), what + ": NaN positions differ"
    inf_ref = np.isinf(y_ref)
    assert np.array_equal(y_gpu[inf_ref], y_ref[inf_ref]), what + ": Inf mismatch"
    fin = ~(nan_ref | inf_ref)
    err = np.abs(y_gpu[fin] - y_ref[fin])
    bound = tol[fin]
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError("%s: %d elements out of tolerance; worst err %.3e bound %.3e"
                             % (what, int(bad.sum()), err[i], bound[i]))
