"""Python binding of libw12.so (include/w12.h): argument marshalling only.

Every function here hands torch tensors' device pointers and torch's current
HIP stream to the C ABI; all arithmetic runs in the library's HIP kernels.
There is no fallback: if the library is missing or the tensors are not on
the GPU, the call raises.

BF16 tensors may be passed as torch.bfloat16, torch.int16 or torch.uint16
(the bit pattern is what crosses the boundary).
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw12.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "w12.h")

GROUP = 128
MAX_M = 128
OUT_BF16 = 0
OUT_F32 = 1

STATUS = {
    0: "W12_OK", -1: "W12_ERR_NULL", -2: "W12_ERR_SHAPE", -3: "W12_ERR_ALIGN",
    -4: "W12_ERR_DTYPE", -6: "W12_ERR_UNSUPPORTED", -7: "W12_ERR_HIP",
    -8: "W12_ERR_WORKSPACE", -9: "W12_ERR_SCRATCH",
}


class W12Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status),
                                          w12_status_string(status)))


class W12UnencodableError(ValueError):
    """Raised by pack(..., strict=True) when some group cannot round-trip."""


class Tiling(ctypes.Structure):
    """w12_tiling_t: kind (0 GEMV, 1 MFMA), r, kw, depth, x_direct, splitk
    (0 or 1 = K not split across workgroups), waves (0 or 4 = 256-thread
    workgroups, 8 = 512 threads, 16 = 1024 threads)."""
    _fields_ = [("kind", ctypes.c_int32), ("r", ctypes.c_int32), ("kw", ctypes.c_int32),
                ("depth", ctypes.c_int32), ("x_direct", ctypes.c_int32),
                ("splitk", ctypes.c_int32), ("waves", ctypes.c_int32)]

    def astuple(self):
        return (self.kind, self.r, self.kw, self.depth, self.x_direct, self.splitk, self.waves)

    def __repr__(self):
        return ("Tiling(kind=%d, r=%d, kw=%d, depth=%d, x_direct=%d, splitk=%d, waves=%d)"
                % self.astuple())


# Every tiling the library instantiates: (kind, r, kw, depth, x_direct); any
# of them may add a sixth entry, the split-K factor (1..64).  The 512-thread
# MFMA tilings (x in LDS, r = 1, depth 2) also carry the wave count 8.  x_direct needs a
# ring of at most 192 registers: depth * (16 * r + 4 * M) for the GEMV
# (M <= 4), depth * 16 * (r + A tiles) for the MFMA (1 tile up to M = 16, 2
# above); see x_direct_fits.
_PAIRS = ((1, 2), (1, 4), (1, 8), (2, 2), (2, 4))
GEMV_TILINGS = [(0, r, kw, d, xd) for (r, d) in _PAIRS for kw in (1, 2, 4) for xd in (0, 1)]
MFMA_TILINGS = [(1, r, kw, d, xd) for (r, d) in _PAIRS for kw in (1, 2, 4) for xd in (0, 1)]
MFMA8_TILINGS = [(1, 1, kw, 2, 0, 1, 8) for kw in (1, 2, 4, 8)]
# 1024-thread workgroups: the same, 16 and 32 rows, two to eight K-waves.
MFMA16_TILINGS = [(1, 1, kw, 2, 0, 1, 16) for kw in (2, 4, 8)]


def x_direct_fits(M: int, r: int, depth: int, kind: int = 0) -> bool:
    if kind == 1:
        return depth * 16 * (r + (1 if M <= 16 else 2)) <= 192
    return M <= 4 and depth * (16 * r + 4 * M) <= 192


def _tiling_arg(tiling):
    if tiling is None:
        return None
    if not isinstance(tiling, Tiling):
        tiling = Tiling(*tiling)
    return ctypes.byref(tiling)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw12.so (after torch, so the library binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libw12.so is not built (%s); run `python -m lossless_bit_weight_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.w12_abi_version.argtypes = []
    L.w12_abi_version.restype = i32
    L.w12_status_string.argtypes = [i32]
    L.w12_status_string.restype = ctypes.c_char_p
    L.w12_padded_rows.argtypes = [i64]
    L.w12_padded_rows.restype = i64
    L.w12_bf16_tiled_bytes.argtypes = [i64, i64]
    L.w12_bf16_tiled_bytes.restype = ctypes.c_size_t
    L.w12_bf16_tile.argtypes = [p, i64, i64, p, p]
    L.w12_bf16_tile.restype = i32
    L.w12_plane_bytes.argtypes = [i64, i64]
    L.w12_plane_bytes.restype = ctypes.c_size_t
    L.w12_meta_bytes.argtypes = [i64, i64]
    L.w12_meta_bytes.restype = ctypes.c_size_t
    L.w12_pack.argtypes = [p, i64, i64, p, p, p, p, p, p]
    L.w12_pack.restype = i32
    L.w12_unpack.argtypes = [p, p, p, p, p, p, i64, i64, p, p]
    L.w12_unpack.restype = i32
    L.w12_exceptions_workspace_bytes.argtypes = [i64, i64]
    L.w12_exceptions_workspace_bytes.restype = ctypes.c_size_t
    L.w12_exceptions.argtypes = [p, i64, i64, p, ctypes.c_size_t, p, p, i64, p, p]
    L.w12_exceptions.restype = i32
    L.w12_gemm.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, i64, p, i64, i32, p]
    L.w12_gemm.restype = i32
    L.bf16_gemm.argtypes = [p, i64, i64, p, i64, i64, p, i64, i32, p]
    L.bf16_gemm.restype = i32
    sz = ctypes.c_size_t
    L.w12_gemm_ex.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, i64, p, i64, i32, p, p, sz, p]
    L.w12_gemm_ex.restype = i32
    L.bf16_gemm_ex.argtypes = [p, i64, i64, p, i64, i64, p, i64, i32, p, p, sz, p]
    L.bf16_gemm_ex.restype = i32
    L.w12_gemm_ws.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, i64, p, i64, i32, p, sz, p]
    L.w12_gemm_ws.restype = i32
    L.bf16_gemm_ws.argtypes = [p, i64, i64, p, i64, i64, p, i64, i32, p, sz, p]
    L.bf16_gemm_ws.restype = i32
    L.w12_gemm_noalloc.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, i64, p, i64, i32, p]
    L.w12_gemm_noalloc.restype = i32
    L.w12_gemm_workspace_bytes.argtypes = [i64, i64, i64, p, ctypes.POINTER(sz)]
    L.w12_gemm_workspace_bytes.restype = i32
    L.w12_default_tiling.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Tiling)]
    L.w12_default_tiling.restype = i32
    L.w12_read_probe.argtypes = [p, ctypes.c_size_t, p, p]
    L.w12_read_probe.restype = i32
    L.w12_gemm_variant.argtypes = [i64, i64, i64, i32, i32]
    L.w12_gemm_variant.restype = ctypes.c_char_p
    L.w12_tiling_variant.argtypes = [i64, i64, i64, ctypes.POINTER(Tiling), i32]
    L.w12_tiling_variant.restype = ctypes.c_char_p
    # W12-b entry points: the W12-v1 signatures
    for name in ("pack", "unpack", "exceptions", "gemm", "gemm_ws", "gemm_ex"):
        fb, fv = getattr(L, "w12b_" + name), getattr(L, "w12_" + name)
        fb.argtypes, fb.restype = fv.argtypes, fv.restype
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/w12.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


# ---- marshalling helpers ---------------------------------------------------

# Bit allocations: "v1" (W12-v1) and "b" (W12-b, arbitrary base); the W12-b
# calls carry a "w12b_" prefix and the W12-v1 signatures.
FORMATS = ("v1", "b")


def _fmt_fn(fmt: str, name: str):
    """(library function, its name) of the W12-v1 call `name` ("w12_...") for
    containers of allocation `fmt`."""
    if fmt not in FORMATS:
        raise ValueError("unknown W12 format %r" % (fmt,))
    full = name if fmt == "v1" else "w12b_" + name[len("w12_"):]
    return getattr(lib(), full), full


_BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _dev_ptr(t: torch.Tensor, what: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % what)
    return t.data_ptr()


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise W12Error(status, what)


def _bf16_2d(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype not in _BF16_TYPES:
        raise TypeError("%s must hold BF16 bits (bfloat16/int16/uint16), got %s" % (what, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % what)
    return t


# ---- the C ABI, by name ----------------------------------------------------

def w12_abi_version() -> int:
    return int(lib().w12_abi_version())


def w12_status_string(status: int) -> str:
    return lib().w12_status_string(int(status)).decode()


def w12_padded_rows(N: int) -> int:
    return int(lib().w12_padded_rows(int(N)))


def w12_bf16_tiled_bytes(N: int, K: int) -> int:
    return int(lib().w12_bf16_tiled_bytes(int(N), int(K)))


def w12_plane_bytes(N: int, K: int) -> int:
    return int(lib().w12_plane_bytes(int(N), int(K)))


def w12_meta_bytes(N: int, K: int) -> int:
    return int(lib().w12_meta_bytes(int(N), int(K)))


def w12_default_tiling(M: int, N: int, K: int, allow_splitk: bool = True) -> Tiling:
    t = Tiling()
    _check(lib().w12_default_tiling(int(M), int(N), int(K), int(bool(allow_splitk)), ctypes.byref(t)),
           "w12_default_tiling")
    return t


def w12_gemm_variant(M: int, N: int, K: int, is_w12: bool | int = True,
                     allow_splitk: bool = True) -> str | None:
    """Variant name; is_w12: False/0 = BF16 control, True/1 = W12-v1, 2 = W12-b,
    3 = W12-v1 with an exception list."""
    fetch = int(is_w12) if (not isinstance(is_w12, bool) and int(is_w12) in (2, 3)) else int(bool(is_w12))
    r = lib().w12_gemm_variant(int(M), int(N), int(K), fetch, int(bool(allow_splitk)))
    return None if r is None else r.decode()


def w12_tiling_variant(M: int, N: int, K: int, tiling, is_w12: bool | int = True) -> str | None:
    """Variant name an explicit tiling launches (None if rejected)."""
    fetch = 2 if (not isinstance(is_w12, bool) and int(is_w12) == 2) else int(bool(is_w12))
    r = lib().w12_tiling_variant(int(M), int(N), int(K), _tiling_arg(tiling), fetch)
    return None if r is None else r.decode()


def w12_gemm_workspace_bytes(M: int, N: int, K: int, tiling=None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().w12_gemm_workspace_bytes(int(M), int(N), int(K), _tiling_arg(tiling),
                                          ctypes.byref(n)), "w12_gemm_workspace_bytes")
    return int(n.value)


# One zero-filled split-K workspace per (device, stream): launches on one
# stream run in order, so they can share it (each leaves its counters at
# zero); launches on another stream get their own.  The first split-K call on
# a stream allocates it, so make that call before capturing the stream in a
# graph.
_workspaces: dict = {}


def workspace(nbytes: int) -> torch.Tensor:
    """The binding's split-K workspace for the current device and stream,
    grown (and zero-filled anew) to at least `nbytes`."""
    dev = torch.cuda.current_device()
    key = (dev, torch.cuda.current_stream().cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 1 << 20), dtype=torch.uint8, device="cuda:%d" % dev)
        _workspaces[key] = ws
    return ws


@dataclass
class W12Weight:
    """A packed [N, K] weight: three flat uint8 planes of w12_plane_bytes(N, K)
    and a flat uint8 meta array of w12_meta_bytes(N, K) (tiled layout), plus
    an optional exception list (int32 tensors: (Np/16)*(K/128) + 1 block
    offsets and [count, 2] entries) that makes every group lossless."""
    p0: torch.Tensor
    p1: torch.Tensor
    p2: torch.Tensor
    meta: torch.Tensor
    N: int
    K: int
    exc_offsets: torch.Tensor | None = None
    exc_entries: torch.Tensor | None = None
    fmt: str = "v1"     # "v1" (W12-v1) or "b" (W12-b)

    @property
    def nbytes(self) -> int:
        n = 3 * self.p0.numel() + self.meta.numel()
        if self.exc_offsets is not None:
            n += 4 * (self.exc_offsets.numel() + self.exc_entries.numel())
        return n

    def exc_ptrs(self) -> tuple:
        if self.exc_offsets is None:
            return None, None
        return _dev_ptr(self.exc_offsets, "exc_offsets"), _dev_ptr(self.exc_entries, "exc_entries")


@dataclass
class BF16Tiled:
    """An [N, K] BF16 weight in the control layout (flat, padded rows)."""
    w: torch.Tensor
    N: int
    K: int

    @property
    def nbytes(self) -> int:
        return 2 * self.w.numel()


def empty_weight(N: int, K: int, device="cuda", fmt: str = "v1") -> W12Weight:
    pb, mb = w12_plane_bytes(N, K), w12_meta_bytes(N, K)
    if pb == 0:
        raise W12Error(-2, "empty_weight(%d, %d)" % (N, K))
    if fmt not in FORMATS:
        raise ValueError("unknown W12 format %r" % (fmt,))
    mk = lambda: torch.empty(pb, dtype=torch.uint8, device=device)
    return W12Weight(mk(), mk(), mk(), torch.empty(mb, dtype=torch.uint8, device=device), N, K,
                     fmt=fmt)


def w12_bf16_tile(w: torch.Tensor) -> BF16Tiled:
    """Arrange a row-major BF16 [N, K] weight in the control layout."""
    w = _bf16_2d(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    N, K = w.shape
    nb = w12_bf16_tiled_bytes(N, K)
    if nb == 0:
        raise W12Error(-2, "w12_bf16_tile(%d, %d)" % (N, K))
    out = torch.empty(nb // 2, dtype=torch.bfloat16, device=w.device)
    _check(lib().w12_bf16_tile(_dev_ptr(w, "w"), N, K, _dev_ptr(out, "w_tiled"), _stream()),
           "w12_bf16_tile")
    return BF16Tiled(out, N, K)


def w12_pack(w: torch.Tensor, out: W12Weight | None = None,
             bad_groups: torch.Tensor | None = None, fmt: str = "v1") -> W12Weight:
    """Pack BF16 [N, K] (contiguous) into W12 (fmt "v1": w12_pack, "b":
    w12b_pack).  If `bad_groups` (int32/uint32 GPU tensor with one element)
    is given, the count of unencodable groups is added to it on the
    stream."""
    w = _bf16_2d(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    N, K = w.shape
    if out is None:
        out = empty_weight(N, K, w.device, fmt)
    out.fmt = fmt
    bad_ptr = None
    if bad_groups is not None:
        if bad_groups.dtype not in (torch.int32, torch.uint32) or bad_groups.numel() < 1:
            raise TypeError("bad_groups must be a 32-bit integer GPU tensor")
        bad_ptr = _dev_ptr(bad_groups, "bad_groups")
    fn, name = _fmt_fn(fmt, "w12_pack")
    _check(fn(_dev_ptr(w, "w"), N, K, _dev_ptr(out.p0, "p0"), _dev_ptr(out.p1, "p1"),
              _dev_ptr(out.p2, "p2"), _dev_ptr(out.meta, "meta"), bad_ptr, _stream()), name)
    return out


def w12_exceptions(w: torch.Tensor, fmt: str = "v1") -> tuple[torch.Tensor, torch.Tensor]:
    """The exception list of BF16 [N, K] (contiguous): (tile offsets,
    entries [count, 2]) as int32 tensors.  Counts first, reads the count
    (a stream synchronisation), then writes the entries."""
    w = _bf16_2d(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    N, K = w.shape
    wsb = int(lib().w12_exceptions_workspace_bytes(N, K))
    if wsb == 0:
        raise W12Error(-2, "w12_exceptions(%d, %d)" % (N, K))
    ws = torch.empty(wsb // 4, dtype=torch.int32, device=w.device)
    off = torch.empty(w12_padded_rows(N) // 16 * (K // GROUP) + 1, dtype=torch.int32,
                      device=w.device)
    total = torch.zeros(1, dtype=torch.int32, device=w.device)
    args = (_dev_ptr(w, "w"), N, K, _dev_ptr(ws, "workspace"), wsb, _dev_ptr(off, "exc_offsets"))
    fn, name = _fmt_fn(fmt, "w12_exceptions")
    _check(fn(*args, None, 0, _dev_ptr(total, "total"), _stream()), name)
    count = int(total.item())
    ent = torch.empty((max(count, 1), 2), dtype=torch.int32, device=w.device)
    if count:
        _check(fn(*args, _dev_ptr(ent, "exc_entries"), count, _dev_ptr(total, "total"), _stream()),
               name)
    return off, ent


def pack(w: torch.Tensor, strict: bool = False, exceptions: bool = False,
         fmt: str = "v1") -> tuple[W12Weight, int]:
    """Pack and return (container, number of unencodable groups).  Reading the
    count synchronises the stream; with strict=True a non-zero count raises;
    with exceptions=True a container with unencodable groups also gets its
    exception list, which makes it lossless.  fmt: "v1" or "b"."""
    bad = torch.zeros(1, dtype=torch.int32, device=w.device)
    out = w12_pack(w, bad_groups=bad, fmt=fmt)
    n_bad = int(bad.item())
    if strict and n_bad:
        raise W12UnencodableError("%d of %d groups cannot be stored losslessly"
                                  % (n_bad, w.numel() // GROUP))
    if exceptions and n_bad:
        out.exc_offsets, out.exc_entries = w12_exceptions(w, fmt)
    return out, n_bad


def w12_unpack(wt: W12Weight, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode a container back to BF16 [N, K] (torch.bfloat16)."""
    if out is None:
        out = torch.empty((wt.N, wt.K), dtype=torch.bfloat16, device=wt.p0.device)
    _bf16_2d(out, "out")
    fn, name = _fmt_fn(wt.fmt, "w12_unpack")
    _check(fn(_dev_ptr(wt.p0, "p0"), _dev_ptr(wt.p1, "p1"), _dev_ptr(wt.p2, "p2"),
              _dev_ptr(wt.meta, "meta"), *wt.exc_ptrs(), wt.N, wt.K, _dev_ptr(out, "out"),
              _stream()), name)
    return out


def _out_tensor(M: int, N: int, out_dtype: torch.dtype, device) -> tuple[torch.Tensor, int]:
    if out_dtype == torch.float32:
        return torch.empty((M, N), dtype=torch.float32, device=device), OUT_F32
    if out_dtype == torch.bfloat16:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device), OUT_BF16
    raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")


def _y_args(y: torch.Tensor) -> tuple[int, int]:
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with unit column stride")
    if y.dtype == torch.float32:
        return y.stride(0), OUT_F32
    if y.dtype in _BF16_TYPES:
        return y.stride(0), OUT_BF16
    raise TypeError("y must be float32 or BF16")


def _x_args(x: torch.Tensor) -> tuple[int, int]:
    x = _bf16_2d(x, "x")
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    return x.shape[0], x.stride(0)


def _ws_args(M: int, N: int, K: int, tiling, split_k: bool, ws: torch.Tensor | None):
    """(pointer, bytes) of the workspace a call needs, or (None, 0)."""
    if tiling is None and not split_k:
        return None, 0
    need = w12_gemm_workspace_bytes(M, N, K, tiling)
    if need == 0:
        return None, 0
    if ws is None:
        ws = workspace(need)
    elif ws.numel() * ws.element_size() < need:
        raise ValueError("workspace holds %d bytes, this call needs %d"
                         % (ws.numel() * ws.element_size(), need))
    return _dev_ptr(ws, "workspace"), ws.numel() * ws.element_size()


def w12_gemm(x: torch.Tensor, wt: W12Weight, out_dtype: torch.dtype = torch.float32,
             y: torch.Tensor | None = None, tiling=None, split_k: bool = True,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = sum_k x[m, k] W[n, k] with W rebuilt from the container.
    Default: w12_gemm_ws (K may be split over workgroups, using `workspace`
    or the binding's own); split_k=False: w12_gemm.  `tiling` (a Tiling or a
    (kind, r, kw, depth, x_direct[, splitk[, waves]]) tuple) selects
    w12_gemm_ex."""
    M, ldx = _x_args(x)
    if y is None:
        y, _ = _out_tensor(M, wt.N, out_dtype, x.device)
    ldy, yt = _y_args(y)
    args = (_dev_ptr(x, "x"), M, ldx, _dev_ptr(wt.p0, "p0"), _dev_ptr(wt.p1, "p1"),
            _dev_ptr(wt.p2, "p2"), _dev_ptr(wt.meta, "meta"), *wt.exc_ptrs(), wt.N, wt.K,
            _dev_ptr(y, "y"), ldy, yt)
    wsp, wsb = _ws_args(M, wt.N, wt.K, tiling, split_k, workspace)
    if tiling is not None:
        fn, name = _fmt_fn(wt.fmt, "w12_gemm_ex")
        _check(fn(*args, _tiling_arg(tiling), wsp, wsb, _stream()), name)
    elif split_k:
        fn, name = _fmt_fn(wt.fmt, "w12_gemm_ws")
        _check(fn(*args, wsp, wsb, _stream()), name)
    else:
        fn, name = _fmt_fn(wt.fmt, "w12_gemm")
        _check(fn(*args, _stream()), name)
    return y


def w12_gemm_noalloc(x: torch.Tensor, wt: W12Weight, out_dtype: torch.dtype = torch.float32,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """w12_gemm_noalloc: the w12_gemm_ws operation with its split-K scratch
    in the library's fixed device array (no workspace, no allocation by the
    library; y is allocated here only if not given).  W12-v1 containers."""
    if wt.fmt != "v1":
        raise ValueError("w12_gemm_noalloc takes W12-v1 containers")
    M, ldx = _x_args(x)
    if y is None:
        y, _ = _out_tensor(M, wt.N, out_dtype, x.device)
    ldy, yt = _y_args(y)
    _check(lib().w12_gemm_noalloc(_dev_ptr(x, "x"), M, ldx, _dev_ptr(wt.p0, "p0"),
                                  _dev_ptr(wt.p1, "p1"), _dev_ptr(wt.p2, "p2"),
                                  _dev_ptr(wt.meta, "meta"), *wt.exc_ptrs(), wt.N, wt.K,
                                  _dev_ptr(y, "y"), ldy, yt, _stream()), "w12_gemm_noalloc")
    return y


def bf16_gemm(x: torch.Tensor, wt: BF16Tiled, out_dtype: torch.dtype = torch.float32,
              y: torch.Tensor | None = None, tiling=None, split_k: bool = True,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The same-tiling control: y = x . W^T with W read as BF16 words from the
    control layout (see w12_bf16_tile).  Arguments as w12_gemm."""
    M, ldx = _x_args(x)
    if not isinstance(wt, BF16Tiled):
        raise TypeError("bf16_gemm takes a BF16Tiled weight (w12_bf16_tile)")
    if y is None:
        y, _ = _out_tensor(M, wt.N, out_dtype, x.device)
    ldy, yt = _y_args(y)
    args = (_dev_ptr(x, "x"), M, ldx, _dev_ptr(wt.w, "w_tiled"), wt.N, wt.K, _dev_ptr(y, "y"), ldy, yt)
    wsp, wsb = _ws_args(M, wt.N, wt.K, tiling, split_k, workspace)
    if tiling is not None:
        _check(lib().bf16_gemm_ex(*args, _tiling_arg(tiling), wsp, wsb, _stream()), "bf16_gemm_ex")
    elif split_k:
        _check(lib().bf16_gemm_ws(*args, wsp, wsb, _stream()), "bf16_gemm_ws")
    else:
        _check(lib().bf16_gemm(*args, _stream()), "bf16_gemm")
    return y


def w12_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Measurement aid: stream all bytes of `buf` (a contiguous GPU tensor,
    16-byte aligned, size a multiple of 16) through the library's plain read
    kernel; `sink` is a GPU tensor of at least 4 bytes that is written only
    in the rare case described in include/w12.h."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().w12_read_probe(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink"), _stream()),
           "w12_read_probe")
