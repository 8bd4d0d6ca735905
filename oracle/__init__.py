"""CPU oracle for the W12 lossless 12-bit weight format (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never touches it, and the two share no code: this
wrapper loads ``libw12_oracle.so``, built from the plain C file
``w12_oracle.c`` next to it, and marshals numpy arrays into it.

Every function below is a thin argument adapter; the arithmetic lives in the
C file, which follows the format definition element by element (see its
header).  The fp64 GEMM computes the plain definition y = x . W^T of the
decode GEMM that the pages describe (AI Radar summary of SpecPilot, English
edition, "Reasons": BF16 rebuilt bit by bit inside the GEMM; HotRepo digest
of StargazerX0/SpecPilot, project introduction: decoded bit-exactly inside
the GEMM at batch 1-32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w12_oracle.c")
_LIB = os.path.join(_HERE, "libw12_oracle.so")

GROUP = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no -ffast-math) and return the .so path."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
             _SRC, "-o", tmp, "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.w12o_beta_for_emax.argtypes = [i32]
    lib.w12o_beta_for_emax.restype = i32
    lib.w12o_encodable.argtypes = [ctypes.c_uint16, i32]
    lib.w12o_encodable.restype = i32
    lib.w12o_encode.argtypes = [ctypes.c_uint16, i32, ctypes.POINTER(ctypes.c_int)]
    lib.w12o_encode.restype = ctypes.c_uint16
    lib.w12o_decode.argtypes = [ctypes.c_uint16, i32]
    lib.w12o_decode.restype = ctypes.c_uint16
    lib.w12o_encode_many.argtypes = [p, i64, i32, p, p]
    lib.w12o_encode_many.restype = None
    lib.w12o_decode_many.argtypes = [p, i64, i32, p]
    lib.w12o_decode_many.restype = None
    lib.w12o_pack.argtypes = [p, i64, i64, p, p, p, p]
    lib.w12o_pack.restype = i64
    lib.w12o_unpack.argtypes = [p, p, p, p, i64, i64, p]
    lib.w12o_unpack.restype = i32
    lib.w12o_bf16_tile.argtypes = [p, i64, i64, p]
    lib.w12o_bf16_tile.restype = i32
    lib.w12o_gemm_bf16_f64.argtypes = [p, i64, i64, p, i64, p]
    lib.w12o_gemm_bf16_f64.restype = i32
    lib.w12o_gemm_w12_f64.argtypes = [p, i64, i64, p, p, p, p, i64, p, i32]
    lib.w12o_exceptions.argtypes = [p, i64, i64, p, p]
    lib.w12o_exceptions.restype = i64
    lib.w12o_apply_exceptions.argtypes = [p, i64, i64, p, p]
    lib.w12o_apply_exceptions.restype = i32
    lib.w12o_gemm_w12_f64.restype = i32
    lib.w12o_b_base_for_emax.argtypes = [i32]
    lib.w12o_b_base_for_emax.restype = i32
    lib.w12o_b_encodable.argtypes = [ctypes.c_uint16, i32]
    lib.w12o_b_encodable.restype = i32
    lib.w12o_b_encode.argtypes = [ctypes.c_uint16, i32, ctypes.POINTER(ctypes.c_int)]
    lib.w12o_b_encode.restype = ctypes.c_uint16
    lib.w12o_b_decode.argtypes = [ctypes.c_uint16, i32]
    lib.w12o_b_decode.restype = ctypes.c_uint16
    lib.w12o_b_encode_many.argtypes = [p, i64, i32, p, p]
    lib.w12o_b_encode_many.restype = None
    lib.w12o_b_decode_many.argtypes = [p, i64, i32, p]
    lib.w12o_b_decode_many.restype = None
    lib.w12o_pack_fmt.argtypes = [i32, p, i64, i64, p, p, p, p]
    lib.w12o_pack_fmt.restype = i64
    lib.w12o_unpack_fmt.argtypes = [i32, p, p, p, p, i64, i64, p]
    lib.w12o_unpack_fmt.restype = i32
    lib.w12o_exceptions_fmt.argtypes = [i32, p, i64, i64, p, p]
    lib.w12o_exceptions_fmt.restype = i64
    lib.w12o_gemm_w12_f64_fmt.argtypes = [i32, p, i64, i64, p, p, p, p, i64, p, i32]
    lib.w12o_gemm_w12_f64_fmt.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected BF16 bit patterns as uint16, got %s" % a.dtype)
    return a


# Allocations: "v1" = W12-v1 (3-bit offset of E[7:1] from an even base, low
# byte verbatim); "b" = W12-b (4-bit offset of E from a base of any value).
FORMATS = {"v1": 0, "b": 1}


def _fmt(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError("unknown W12 format %r" % (fmt,))
    return FORMATS[fmt]


# ---- element level ---------------------------------------------------------

def beta_for_emax(emax: int) -> int:
    return int(_load().w12o_beta_for_emax(int(emax)))


def encodable(v: int, beta: int) -> bool:
    return bool(_load().w12o_encodable(int(v), int(beta)))


def encode(v: int, beta: int) -> tuple[int, bool]:
    ok = ctypes.c_int(0)
    code = _load().w12o_encode(int(v), int(beta), ctypes.byref(ok))
    return int(code), bool(ok.value)


def decode(code: int, beta: int) -> int:
    return int(_load().w12o_decode(int(code), int(beta)))


def encode_many(v: np.ndarray, beta: int):
    """Vector form of encode: returns (codes uint16, ok bool)."""
    v = _u16(v)
    code = np.empty(v.shape, np.uint16)
    ok = np.empty(v.shape, np.uint8)
    _load().w12o_encode_many(_ptr(v), v.size, int(beta), _ptr(code), _ptr(ok))
    return code, ok.astype(bool)


def decode_many(code: np.ndarray, beta: int) -> np.ndarray:
    code = _u16(code)
    v = np.empty(code.shape, np.uint16)
    _load().w12o_decode_many(_ptr(code), code.size, int(beta), _ptr(v))
    return v


# W12-b element level (base b, code = c << 8 | s << 7 | m)

def b_base_for_emax(emax: int) -> int:
    return int(_load().w12o_b_base_for_emax(int(emax)))


def b_encodable(v: int, b: int) -> bool:
    return bool(_load().w12o_b_encodable(int(v), int(b)))


def b_encode(v: int, b: int) -> tuple[int, bool]:
    ok = ctypes.c_int(0)
    code = _load().w12o_b_encode(int(v), int(b), ctypes.byref(ok))
    return int(code), bool(ok.value)


def b_decode(code: int, b: int) -> int:
    return int(_load().w12o_b_decode(int(code), int(b)))


def b_encode_many(v: np.ndarray, b: int):
    v = _u16(v)
    code = np.empty(v.shape, np.uint16)
    ok = np.empty(v.shape, np.uint8)
    _load().w12o_b_encode_many(_ptr(v), v.size, int(b), _ptr(code), _ptr(ok))
    return code, ok.astype(bool)


def b_decode_many(code: np.ndarray, b: int) -> np.ndarray:
    code = _u16(code)
    v = np.empty(code.shape, np.uint16)
    _load().w12o_b_decode_many(_ptr(code), code.size, int(b), _ptr(v))
    return v


# ---- tensor level ----------------------------------------------------------

def padded_rows(N: int) -> int:
    """Rows of the container: N rounded up to a multiple of 16 (tile height)."""
    return (N + 15) // 16 * 16


def plane_bytes(N: int, K: int) -> int:
    return padded_rows(N) * K // 2


def meta_bytes(N: int, K: int) -> int:
    return padded_rows(N) * (K // GROUP)


def meta_of(meta: np.ndarray, N: int, K: int) -> np.ndarray:
    """View a flat meta array as [N, K/128] (row n, group g), undoing the
    16-row tiling: byte ((n // 16) * (K/128) + g) * 16 + n % 16."""
    G = K // GROUP
    m = np.asarray(meta, dtype=np.uint8).reshape(-1, G, 16)      # [tile, g, row]
    return m.transpose(0, 2, 1).reshape(-1, G)[:N]


def pack(w: np.ndarray, fmt: str = "v1"):
    """BF16 bits [N, K] -> (p0, p1, p2, meta, bad_groups).

    p0/p1/p2 are flat uint8 arrays of plane_bytes(N, K); meta is a flat uint8
    array of meta_bytes(N, K) (tiled layout, see w12_oracle.c).  fmt selects
    the allocation ("v1" or "b")."""
    w = _u16(w)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    p0 = np.zeros(plane_bytes(N, K), np.uint8)
    p1 = np.zeros(plane_bytes(N, K), np.uint8)
    p2 = np.zeros(plane_bytes(N, K), np.uint8)
    meta = np.zeros(meta_bytes(N, K), np.uint8)
    bad = _load().w12o_pack_fmt(_fmt(fmt), _ptr(w), N, K, _ptr(p0), _ptr(p1), _ptr(p2),
                                _ptr(meta))
    if bad < 0:
        raise ValueError("oracle pack rejected shape %r" % ((N, K),))
    return p0, p1, p2, meta, int(bad)


def unpack(p0, p1, p2, meta, N: int, K: int, fmt: str = "v1") -> np.ndarray:
    arrs = [np.ascontiguousarray(a, dtype=np.uint8).reshape(-1) for a in (p0, p1, p2, meta)]
    for a, n in zip(arrs, (plane_bytes(N, K),) * 3 + (meta_bytes(N, K),)):
        if a.size != n:
            raise ValueError("container size mismatch")
    w = np.empty((N, K), np.uint16)
    if _load().w12o_unpack_fmt(_fmt(fmt), *(_ptr(a) for a in arrs), N, K, _ptr(w)) != 0:
        raise ValueError("oracle unpack rejected shape %r" % ((N, K),))
    return w


def exceptions(w: np.ndarray, fmt: str = "v1"):
    """BF16 bits [N, K] -> (offsets, entries): the exception list of the
    elements that fall below their group's window (see w12_oracle.c).
    offsets: uint32[(padded_rows(N)/16) * (K/128) + 1], one per (tile, group)
    block in block order, then the total; entries: uint32[count, 2] with
    word 0 = (row in tile) << 24 | k and word 1 = base << 16 | the original
    BF16 word."""
    w = _u16(w)
    N, K = w.shape
    lib = _load()
    f = _fmt(fmt)
    count = lib.w12o_exceptions_fmt(f, _ptr(w), N, K, None, None)
    if count < 0:
        raise ValueError("oracle exceptions rejected shape %r" % ((N, K),))
    offsets = np.zeros(padded_rows(N) // 16 * (K // 128) + 1, np.uint32)
    entries = np.zeros((count, 2), np.uint32)
    lib.w12o_exceptions_fmt(f, _ptr(w), N, K, _ptr(offsets), _ptr(entries) if count else None)
    return offsets, entries


def apply_exceptions(w: np.ndarray, offsets: np.ndarray, entries: np.ndarray) -> np.ndarray:
    """A copy of the unpacked BF16 weight [N, K] with the exceptions written in."""
    out = np.array(_u16(w), copy=True)
    N, K = out.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.uint32)
    entries = np.ascontiguousarray(entries, dtype=np.uint32).reshape(-1, 2)
    if offsets.size != padded_rows(N) // 16 * (K // 128) + 1 or entries.shape[0] < int(offsets[-1]):
        raise ValueError("exception list size mismatch")
    if _load().w12o_apply_exceptions(_ptr(out), N, K, _ptr(offsets),
                                     _ptr(entries) if entries.size else None) != 0:
        raise ValueError("exception entry outside the weight")
    return out


def bf16_tile(w: np.ndarray) -> np.ndarray:
    """Row-major BF16 [N, K] -> the control layout (flat, padded_rows(N)*K words)."""
    w = _u16(w)
    N, K = w.shape
    out = np.empty(padded_rows(N) * K, np.uint16)
    if _load().w12o_bf16_tile(_ptr(w), N, K, _ptr(out)) != 0:
        raise ValueError("oracle bf16_tile rejected shape %r" % ((N, K),))
    return out


def gemm_bf16_f64(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w[n, k] in fp64 (x, w: BF16 bits)."""
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("K mismatch")
    y = np.empty((M, N), np.float64)
    _load().w12o_gemm_bf16_f64(_ptr(x), M, K, _ptr(w), N, _ptr(y))
    return y


def gemm_w12_f64(x: np.ndarray, p0, p1, p2, meta, N: int, nthreads: int = 1,
                 fmt: str = "v1") -> np.ndarray:
    """Decode the container row by row and form y = x . W^T in fp64."""
    x = _u16(x)
    M, K = x.shape
    arrs = [np.ascontiguousarray(a, dtype=np.uint8).reshape(-1) for a in (p0, p1, p2, meta)]
    for a, n in zip(arrs, (plane_bytes(N, K),) * 3 + (meta_bytes(N, K),)):
        if a.size != n:
            raise ValueError("container size mismatch")
    y = np.empty((M, N), np.float64)
    rc = _load().w12o_gemm_w12_f64_fmt(_fmt(fmt), _ptr(x), M, K, *(_ptr(a) for a in arrs), N,
                                       _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle gemm rejected shape")
    return y


def tolerance(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-element GEMM pass bound 1e-3 * ||x_m||_2 * ||w_n||_2 + 1e-6.

    This is the acceptance rule for floating-point GEMM outputs;
    norms are taken in fp64 over the BF16 values (NaN/Inf rows give NaN/Inf
    bounds and are compared separately by the tests)."""
    xf = bf16_bits_to_f64(x)
    wf = bf16_bits_to_f64(w)
    nx = np.sqrt(np.sum(xf * xf, axis=1))
    nw = np.sqrt(np.sum(wf * wf, axis=1))
    return 1e-3 * np.outer(nx, nw) + 1e-6


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float64."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
