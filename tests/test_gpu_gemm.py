"""GPU parity for w12_gemm and the bf16_gemm control.

Reference: the oracle's fp64 y = x . W^T on the oracle's own pack/unpack of
the same raw weights (the GEMM the pages describe rebuilds W bit-exactly
inside the kernel: HotRepo digest of StargazerX0/SpecPilot, project
introduction, batch 1-32).  Pass rule for fp32 outputs, per element:
|y_gpu - y_ref| <= 1e-3 ||x_m||_2 ||w_n||_2 + 1e-6.  BF16 outputs must equal
the round-to-nearest-even of the same kernel's fp32 output bit for bit, and
w12_gemm must equal bf16_gemm on the unpacked weights bit for bit (same
kernels, same summation order; only the weight fetch differs).

The binding's default GEMM is the split-K capable w12_gemm_ws; the checks
below also run the plain w12_gemm (split_k=False) on every case.
"""
import os

import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import assert_gemm_close, require_gpu, to_dev, to_host_u16

pytestmark = pytest.mark.gpu

M_SWEEP = [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32]


class Prepared:
    """Raw weights on the host; the GPU container packed from them and its
    unpacked BF16 tensor (the control's operand)."""

    def __init__(self, raw: np.ndarray):
        require_gpu()
        self.raw = raw
        self.N, self.K = raw.shape
        self.wt = w12.w12_pack(to_dev(raw))
        self.w_bf16 = w12.w12_unpack(self.wt)
        self.w_tiled = w12.w12_bf16_tile(self.w_bf16)
        torch.cuda.synchronize()

    def container(self, fmt: str):
        """The projected weight as a container of allocation fmt (W12-v1's
        projection holds no exponent W12-b cannot store for these inputs)."""
        if fmt == "v1":
            return self.wt
        if not hasattr(self, "wt_b"):
            self.wt_b, bad = w12.pack(self.w_bf16, fmt="b")
            assert bad == 0
        return self.wt_b

    def ref_rows(self, oracle, rows):
        """Oracle projection of the raw rows (groups never span rows)."""
        sub = np.ascontiguousarray(self.raw[rows])
        p0, p1, p2, meta, _ = oracle.pack(sub)
        return oracle.unpack(p0, p1, p2, meta, sub.shape[0], self.K)


_cache = {}


def prepared(name_or_shape) -> Prepared:
    if name_or_shape not in _cache:
        if isinstance(name_or_shape, str):
            raw = inputs.CASES[name_or_shape].weights_raw()
        else:
            N, K = name_or_shape
            raw = inputs.gaussian_bf16((N, K), 0.02, 7 * N + K)
        _cache[name_or_shape] = Prepared(raw)
    return _cache[name_or_shape]


def _sample_rows(N, n=384, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, N))) | set(range(max(0, N - 64), N))
    rows |= set(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(rows))


def _run_both(x_bits, P: Prepared, out=torch.float32):
    xd = to_dev(x_bits)
    y12 = w12.w12_gemm(xd, P.wt, out)
    y16 = w12.bf16_gemm(xd, P.w_tiled, out)
    torch.cuda.synchronize()
    return y12, y16


def _check(oracle, P: Prepared, x_bits, rows, what):
    print("gemm parity:", what, flush=True)
    y12, y16 = _run_both(x_bits, P)
    xd = to_dev(x_bits)
    n12 = w12.w12_gemm(xd, P.wt, split_k=False)
    n16 = w12.bf16_gemm(xd, P.w_tiled, split_k=False)
    torch.cuda.synchronize()
    w_ref = P.ref_rows(oracle, rows)
    y_ref = oracle.gemm_bf16_f64(x_bits, w_ref)
    tol = oracle.tolerance(x_bits, w_ref)
    for a, b, kind in ((y12, y16, "w12_gemm_ws"), (n12, n16, "w12_gemm")):
        ah, bh = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(ah.view(np.uint32), bh.view(np.uint32)), what + ": w12 != bf16 bitwise"
        assert_gemm_close(ah[:, rows], y_ref, tol, "%s %s" % (what, kind))
    return y12


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_tiny_every_m(oracle, M):
    P = prepared("tiny")
    x = inputs.TINY.activations(M)
    _check(oracle, P, x, np.arange(P.N), "tiny M=%d" % M)


@pytest.mark.parametrize("shape", [(1000, 640), (37, 128), (4099, 384), (130, 1152), (17, 2560)])
@pytest.mark.parametrize("M", [1, 3, 8, 9, 16, 17, 32])
def test_ragged_shapes(oracle, shape, M):
    P = prepared(shape)
    x = inputs.gaussian_bf16((M, shape[1]), 1.0, 11 * M + shape[1])
    _check(oracle, P, x, np.arange(P.N), "ragged %s M=%d" % (shape, M))


@pytest.mark.parametrize("name", ["qkv", "gate_up", "down", "o"])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32])
def test_workloads_sampled(oracle, name, M):
    case = inputs.CASES[name]
    P = prepared(name)
    x = case.activations(M)
    _check(oracle, P, x, _sample_rows(P.N, seed=M), "%s M=%d" % (name, M))


@pytest.mark.parametrize("shape", [(896, 5120), (1536, 5120), (1024, 17408), (896, 2176),
                                   (4352, 5120), (5120, 640), (5120, 2176)])
@pytest.mark.parametrize("M", [2, 4, 9, 12, 16, 24, 32])
def test_shard_shapes_default(oracle, shape, M):
    """One GPU's share of the QKV, gate+up, O and down weights under 8-way
    tensor parallelism and nearby small weights, with the default tilings
    (one tile per wave and K split across workgroups on <= 256 tiles; x read
    directly with two K-waves on short rows; x in LDS from 4 rows on the
    gate+up share)."""
    P = prepared(shape)
    x = inputs.gaussian_bf16((M, shape[1]), 1.0, 13 * M + shape[0])
    _check(oracle, P, x, _sample_rows(P.N, seed=M), "shard %s M=%d" % (shape, M))


@pytest.mark.parametrize("shape", [(301, 640), (45, 5120), (77, 17408), (1000, 1152)])
@pytest.mark.parametrize("M", [33, 48, 64, 65, 100, 128])
def test_large_m_default(oracle, shape, M):
    """M = 33-128: x padded to 64 or 128 rows, staged in LDS for 512-thread
    workgroups, with and without split K; W12 and BF16 bitwise equal."""
    P = prepared(shape)
    x = inputs.gaussian_bf16((M, shape[1]), 1.0, 17 * M + shape[0])
    _check(oracle, P, x, np.arange(P.N), "large M %s M=%d" % (shape, M))


@pytest.mark.parametrize("shape", [(7168, 5120), (5120, 17408), (4100, 5120)])
@pytest.mark.parametrize("M", [64, 100, 128])
def test_large_m_split_default(oracle, shape, M):
    """Weights of >= 256 tiles above 32 rows: the default takes one K-wave
    and K split into four to six slices, which the last workgroup of each
    row block finishes from its lanes' registers (full QKV and down shapes,
    and a ragged 257-tile weight)."""
    t = w12.w12_default_tiling(M, *shape)
    assert (t.kw, t.waves) == (1, 8) and t.splitk >= 4
    P = prepared(shape)
    x = inputs.gaussian_bf16((M, shape[1]), 1.0, 29 * M + shape[0])
    _check(oracle, P, x, _sample_rows(P.N, n=256, seed=M), "large M split %s M=%d" % (shape, M))


@pytest.mark.parametrize("tiling", [(1, 1, 1, 2, 0, 1, 8), (1, 1, 2, 2, 0, 1, 8),
                                    (1, 1, 1, 2, 0, 3, 8), (1, 1, 2, 2, 0, 7, 8),
                                    (1, 1, 1, 2, 0, 64, 8), (1, 2, 1, 2, 0, 1, 8),
                                    (1, 2, 1, 2, 0, 3, 8)],
                         ids=lambda t: "r%d_kw%d_s%d_w%d" % (t[1], t[2], t[5], t[6]))
def test_large_m_tilings(oracle, tiling):
    """Every 64- and 128-row tiling that is built, ragged shapes, split K
    down to one group per slice; a tiling that is not built for a shape is
    rejected (a chunk beyond 128 KB of LDS)."""
    for shape in ((301, 640), (33, 2688), (77, 17408)):
        P = prepared(shape)
        w_ref = P.ref_rows(oracle, np.arange(P.N))
        for M in (40, 64, 97, 128):
            what = "large M tiling %s %s M=%d" % (tiling, shape, M)
            print(what, flush=True)
            x = inputs.gaussian_bf16((M, shape[1]), 1.0, 3 * M + shape[1])
            xd = to_dev(x)
            try:
                y12 = w12.w12_gemm(xd, P.wt, tiling=tiling)
            except w12.W12Error as e:
                # only a chunk beyond 128 KB of LDS is rejected here
                mt = 64 if M <= 64 else 128
                assert e.status == -6 and mt * 128 * tiling[2] * 2 > 32768, what
                continue
            y16 = w12.bf16_gemm(xd, P.w_tiled, tiling=tiling)
            torch.cuda.synchronize()
            y12h, y16h = y12.cpu().numpy(), y16.cpu().numpy()
            assert np.array_equal(y12h.view(np.uint32), y16h.view(np.uint32)), what
            assert_gemm_close(y12h, oracle.gemm_bf16_f64(x, w_ref), oracle.tolerance(x, w_ref), what)


@pytest.mark.parametrize("M", [1, 5, 8, 16, 32, 64, 128])
def test_bf16_output_is_rounded_fp32(M):
    P = prepared("tiny")
    xd = to_dev(inputs.TINY.activations(M))
    for fn, w in ((w12.w12_gemm, P.wt), (w12.bf16_gemm, P.w_tiled)):
        yf = fn(xd, w, torch.float32)
        yb = fn(xd, w, torch.bfloat16)
        torch.cuda.synchronize()
        expect = yf.cpu().to(torch.bfloat16).view(torch.int16)
        assert torch.equal(yb.cpu().view(torch.int16), expect)


@pytest.mark.parametrize("M", [1, 8, 16, 32, 64, 128])
def test_strided_x_and_y(oracle, M):
    P = prepared((1000, 640))
    x_full = inputs.gaussian_bf16((M, 640 + 64), 1.0, 5 + M)
    xd = to_dev(x_full)[:, :640]
    y_full = torch.full((M, 1000 + 24), -7.0, dtype=torch.float32, device="cuda")
    y = y_full[:, :1000]
    w12.w12_gemm(xd, P.wt, y=y)
    torch.cuda.synchronize()
    x = np.ascontiguousarray(x_full[:, :640])
    w_ref = P.ref_rows(oracle, np.arange(1000))
    assert_gemm_close(y.cpu().numpy(), oracle.gemm_bf16_f64(x, w_ref),
                      oracle.tolerance(x, w_ref), "strided M=%d" % M)
    assert torch.all(y_full[:, 1000:] == -7.0)


@pytest.mark.parametrize("name,M", [("qkv", M) for M in (1, 4, 8, 16, 32, 64, 128)]
                         + [("gate_up", 128), ("down", 100)])
def test_one_hot_rows_rebuild_weights_exactly(oracle, name, M):
    """x rows = unit vectors: y[m, :] is column k_m of W, bit for bit, i.e.
    the in-register reassembly reproduces the BF16 weights exactly (every
    kernel family the defaults reach, two tiles per wave at gate+up M =
    128 included)."""
    P = prepared(name)
    K = P.K
    ks = np.random.default_rng(M).choice(K, size=M, replace=False)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80
    y12, y16 = _run_both(x, P)
    rows = np.arange(P.N)
    w_ref = P.ref_rows(oracle, rows)
    expect = oracle.bf16_bits_to_f64(w_ref[:, ks].T).astype(np.float32)
    assert np.array_equal(y12.cpu().numpy().view(np.uint32) & 0x7FFFFFFF,
                          expect.view(np.uint32) & 0x7FFFFFFF)
    assert np.array_equal(y12.cpu().numpy(), expect)


def test_ieee_specials(oracle):
    require_gpu()
    K = 256
    w = np.zeros((6, K), np.uint16)
    w[0, 5] = 0x7F80            # +Inf
    w[1, 6] = 0x7FC0            # NaN
    w[2, :] = 0x3F80
    w[3, 7] = 0xFF80            # -Inf
    P = Prepared(w)
    x = np.zeros((2, K), np.uint16)
    x[0, 5] = 0xBF80
    x[0, 6] = 0x3F80
    x[0, 7] = 0x3F80
    for out in (torch.float32, torch.bfloat16):
        y12, y16 = _run_both(x, P, out)
        yh = y12.float().cpu().numpy().astype(np.float64)
        ref = oracle.gemm_bf16_f64(x, w)
        assert np.array_equal(np.isnan(yh), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(yh[fin], ref[fin])


def _tiling_id(t):
    return "k%d_r%d_kw%d_d%d_x%d" % t[:5] + ("_w%d" % t[6] if len(t) > 6 else "")


@pytest.mark.parametrize("fmt", ["v1", "b"])
@pytest.mark.parametrize("tiling", w12.GEMV_TILINGS + w12.MFMA_TILINGS + w12.MFMA8_TILINGS +
                         w12.MFMA16_TILINGS, ids=_tiling_id)
def test_every_tiling(oracle, tiling, fmt):
    """Every instantiated variant, single-chunk and chunked x, ragged rows and
    a K tail, against the oracle; W12 (both allocations) and BF16 bitwise
    equal per tiling."""
    Ms = ([1, 2, 4] if tiling[4] else [1, 3, 8]) if tiling[0] == 0 else [9, 16, 17, 32]
    for shape in ((301, 640), (33, 2688), (45, 5120), (77, 17408)):
        P = prepared(shape)
        rows = np.arange(P.N)
        w_ref = P.ref_rows(oracle, rows)
        for M in Ms:
            what = "tiling %s %s %s M=%d" % (fmt, tiling, shape, M)
            print(what, flush=True)
            x = inputs.gaussian_bf16((M, shape[1]), 1.0, 3 * M + shape[1])
            xd = to_dev(x)
            try:
                y12 = w12.w12_gemm(xd, P.container(fmt), tiling=tiling)
            except w12.W12Error as e:
                # only a chunked x buffer that would not fit LDS is rejected
                rows = M if tiling[0] == 0 else (16 if M <= 16 else 32)
                if tiling[4]:
                    assert e.status == -6 and not w12.x_direct_fits(M, tiling[1], tiling[3],
                                                                     tiling[0]), what
                else:
                    assert e.status == -6 and rows * shape[1] * 2 > 40 * 1024, what
                continue
            y16 = w12.bf16_gemm(xd, P.w_tiled, tiling=tiling)
            torch.cuda.synchronize()
            y12h, y16h = y12.cpu().numpy(), y16.cpu().numpy()
            assert np.array_equal(y12h.view(np.uint32), y16h.view(np.uint32)), what
            assert_gemm_close(y12h, oracle.gemm_bf16_f64(x, w_ref), oracle.tolerance(x, w_ref), what)


# (kind, r, kw, depth, x_direct[, waves])
SPLIT_BASES = [(0, 1, 4, 2, 0), (0, 2, 1, 2, 0), (0, 1, 2, 4, 1),
               (1, 1, 1, 2, 0), (1, 2, 4, 2, 0), (1, 1, 2, 4, 0), (1, 1, 2, 2, 1), (1, 2, 1, 2, 1),
               (1, 1, 2, 2, 0, 8), (1, 1, 8, 2, 0, 8), (1, 1, 4, 2, 0, 16), (1, 1, 8, 2, 0, 16)]


@pytest.mark.parametrize("base", SPLIT_BASES,
                         ids=lambda t: "k%d_r%d_kw%d_d%d_x%d" % t[:5] + ("_w%d" % t[5] if len(t) > 5 else ""))
@pytest.mark.parametrize("splitk", [2, 3, 7, 64])
@pytest.mark.parametrize("fmt", ["v1", "b"])
def test_split_k(oracle, base, splitk, fmt):
    """K split over workgroups: ragged slices (G not a multiple of the
    factor), one group per slice (64 > G), chunked x inside a slice (K =
    17408 at 32 rows); W12 and BF16 bitwise equal, oracle tolerance."""
    tiling = base[:5] + (splitk,) + base[5:]
    Ms = ([1, 2, 4] if base[4] else [1, 3, 8]) if base[0] == 0 else [9, 16, 17, 32]
    for shape in ((301, 640), (33, 2688), (45, 5120), (77, 17408)):
        P = prepared(shape)
        rows = np.arange(P.N)
        w_ref = P.ref_rows(oracle, rows)
        for M in Ms:
            what = "split tiling %s %s %s M=%d" % (fmt, tiling, shape, M)
            print(what, flush=True)
            if base[4] and not w12.x_direct_fits(M, base[1], base[3], base[0]):
                continue
            x = inputs.gaussian_bf16((M, shape[1]), 1.0, 5 * M + shape[1])
            xd = to_dev(x)
            try:
                y12 = w12.w12_gemm(xd, P.container(fmt), tiling=tiling)
            except w12.W12Error as e:
                assert e.status == -6, what   # a chunked x buffer too large for LDS
                continue
            y16 = w12.bf16_gemm(xd, P.w_tiled, tiling=tiling)
            torch.cuda.synchronize()
            y12h, y16h = y12.cpu().numpy(), y16.cpu().numpy()
            assert np.array_equal(y12h.view(np.uint32), y16h.view(np.uint32)), what
            assert_gemm_close(y12h, oracle.gemm_bf16_f64(x, w_ref), oracle.tolerance(x, w_ref), what)


def test_split_k_counters_reset(oracle):
    """Every split-K launch leaves its row-block counters at zero and no
    two-slice exchange slot tagged, so the next launch on the same workspace
    writes all of y again (y is prefilled with NaN) and is correct, whatever
    the previous launch's shape, slice count or kernel: two-slice launches
    follow launches that stored many slices of partial sums over the same
    bytes, and launches with many row blocks follow ones with few."""
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    seq = [((130, 1152), 16, (1, 1, 1, 2, 0, 8)),   # 3 row blocks, 5 slices
           ((4099, 384), 1, (0, 1, 4, 2, 0, 3)),    # 257 row blocks
           ((1000, 640), 16, (1, 1, 1, 2, 0, 8)),
           ((1000, 640), 16, (1, 1, 1, 2, 0, 2)),   # two slices: exchange slots
           ((1000, 640), 16, (1, 1, 1, 2, 0, 8)),
           ((300, 2560), 64, (1, 1, 1, 2, 0, 4, 8)),   # 64-row tiles, 4 slices
           ((1000, 640), 32, (1, 1, 2, 2, 0, 2, 8)),   # two slices, 32 rows
           ((300, 2560), 128, (1, 1, 1, 2, 0, 5, 8)),
           ((1000, 640), 9, (1, 1, 4, 2, 1, 2)),       # two slices, x direct
           ((4099, 384), 3, (0, 1, 4, 2, 0, 2))]       # two slices, GEMV
    for i, (shape, M, tiling) in enumerate(seq):
        P = prepared(shape)
        x = inputs.gaussian_bf16((M, shape[1]), 1.0, 100 + i)
        y = torch.full((M, shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        w12.w12_gemm(to_dev(x), P.wt, y=y, tiling=tiling, workspace=ws)
        torch.cuda.synchronize()
        assert w12.w12_gemm_workspace_bytes(M, shape[0], shape[1], tiling) > 65536
        assert int(ws[:65536].count_nonzero()) == 0, "counters not reset (%s %s)" % (tiling, shape)
        hi = ws[65536:].view(torch.int32)[1::2]
        assert int((hi == -1).sum()) == 0, "a tagged slot left behind (%s %s)" % (tiling, shape)
        w_ref = P.ref_rows(oracle, np.arange(P.N))
        assert_gemm_close(y.cpu().numpy(), oracle.gemm_bf16_f64(x, w_ref),
                          oracle.tolerance(x, w_ref), "counters %s %s" % (tiling, shape))


def test_split_k_bf16_output():
    P = prepared((1000, 640))
    xd = to_dev(inputs.gaussian_bf16((16, 640), 1.0, 9))
    for tiling in ((0, 1, 4, 2, 0, 3), (1, 1, 2, 2, 0, 5)):
        M = 4 if tiling[0] == 0 else 16
        yf = w12.w12_gemm(xd[:M], P.wt, torch.float32, tiling=tiling)
        yb = w12.w12_gemm(xd[:M], P.wt, torch.bfloat16, tiling=tiling)
        torch.cuda.synchronize()
        assert torch.equal(yb.cpu().view(torch.int16), yf.cpu().to(torch.bfloat16).view(torch.int16))


def test_ex_null_tiling_follows_workspace(oracle):
    """w12_gemm_ex with no tiling takes the w12_gemm_ws default when given a
    workspace and the w12_gemm default without one (bitwise the same calls)."""
    import ctypes
    P = prepared((77, 17408))
    M = 16
    x = inputs.gaussian_bf16((M, 17408), 1.0, 77)
    xd = to_dev(x)
    ref_ws = w12.w12_gemm(xd, P.wt)                    # w12_gemm_ws
    ref_plain = w12.w12_gemm(xd, P.wt, split_k=False)  # w12_gemm
    L = w12.lib()
    need = w12.w12_gemm_workspace_bytes(M, P.N, P.K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for wsp, wsb in ((ws.data_ptr(), need), (None, 0)):
        y = torch.empty((M, P.N), dtype=torch.float32, device="cuda")
        st = L.w12_gemm_ex(xd.data_ptr(), M, 17408, P.wt.p0.data_ptr(), P.wt.p1.data_ptr(),
                           P.wt.p2.data_ptr(), P.wt.meta.data_ptr(), None, None, P.N, P.K,
                           y.data_ptr(), P.N, 1, None, wsp, wsb, stream)
        assert st == 0
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref_ws) and torch.equal(outs[1], ref_plain)


def test_two_streams_split_k():
    """Split-K GEMMs issued on two streams at once: each stream gets its own
    workspace from the binding, and every result equals the one computed
    alone on the default stream, bit for bit."""
    P = prepared((301, 17408))
    xs = [to_dev(inputs.gaussian_bf16((16, 17408), 1.0, 900 + i)) for i in range(8)]
    ref = []
    for x in xs:
        ref.append(w12.w12_gemm(x, P.wt))
    torch.cuda.synchronize()
    ref = [r.cpu() for r in ref]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None] * len(xs)
    for rep in range(3):
        for i, x in enumerate(xs):
            with torch.cuda.stream(streams[i % 2]):
                outs[i] = w12.w12_gemm(x, P.wt)
        torch.cuda.synchronize()
        for i in range(len(xs)):
            assert torch.equal(outs[i].cpu().view(torch.int32), ref[i].view(torch.int32)), (rep, i)
    assert w12.w12_default_tiling(16, 301, 17408).splitk > 1


@pytest.mark.parametrize("name,M", [("tiny", 1), ("qkv", 1), ("gate_up", 16), ("down", 32)])
def test_headline_configs_every_row(oracle, name, M):
    """The four benchmark configurations at their own M, every output row
    against the oracle's container GEMM (decode + fp64, threaded), in the
    default tiling the benchmark times."""
    case = inputs.CASES[name]
    P = prepared(name)
    x = case.activations(M)
    print("gemm parity every row:", name, M, flush=True)
    y12, y16 = _run_both(x, P)
    yh = y12.cpu().numpy()
    assert np.array_equal(yh.view(np.uint32), y16.cpu().numpy().view(np.uint32))
    p0, p1, p2, meta, _ = oracle.pack(P.raw)
    y_ref = oracle.gemm_w12_f64(x, p0, p1, p2, meta, P.N, nthreads=min(16, os.cpu_count() or 1))
    w_ref = oracle.unpack(p0, p1, p2, meta, P.N, P.K)
    assert_gemm_close(yh, y_ref, oracle.tolerance(x, w_ref), "%s M=%d every row" % (name, M))


# Short rows (1-6 groups): every wave's groups fit the ring's last windows,
# so each count of groups left takes its own tail of the main loop.
SHORT_TILINGS = [(1, 1, 1, 2, 1), (1, 1, 2, 2, 1), (1, 1, 4, 2, 1), (1, 2, 2, 2, 1),
                 (1, 1, 2, 2, 0), (1, 1, 4, 2, 0), (1, 1, 2, 2, 0, 1, 8), (1, 1, 4, 2, 0, 1, 16),
                 (0, 1, 2, 4, 1), (0, 1, 4, 2, 1)]


@pytest.mark.parametrize("tiling", SHORT_TILINGS, ids=lambda t: "x".join(map(str, t)))
def test_short_rows_every_tail(oracle, tiling):
    """K = 128 .. 768 (1 to 6 groups) with one, two and four K-waves: W12 and
    BF16 bitwise equal and within the oracle tolerance.  (Regression: the
    BF16 control with two K-waves and x read directly returned stale sums
    when the wait states after its last MFMAs were missing.)"""
    Ms = [1, 2, 4] if tiling[0] == 0 else [1, 2, 4, 16, 32]
    for K in (128, 256, 384, 512, 768):
        P = prepared((48, K))
        rows = np.arange(P.N)
        w_ref = P.ref_rows(oracle, rows)
        for M in Ms:
            what = "short rows %s K=%d M=%d" % (tiling, K, M)
            print(what, flush=True)
            if tiling[4] and not w12.x_direct_fits(M, tiling[1], tiling[3], tiling[0]):
                continue
            x = inputs.gaussian_bf16((M, K), 1.0, 7 * M + K)
            xd = to_dev(x)
            try:
                y12 = w12.w12_gemm(xd, P.container("v1"), tiling=tiling)
            except w12.W12Error as e:
                assert e.status == -6, what
                continue
            y16 = w12.bf16_gemm(xd, P.w_tiled, tiling=tiling)
            torch.cuda.synchronize()
            y12h, y16h = y12.cpu().numpy(), y16.cpu().numpy()
            assert np.array_equal(y12h.view(np.uint32), y16h.view(np.uint32)), what
            assert_gemm_close(y12h, oracle.gemm_bf16_f64(x, w_ref), oracle.tolerance(x, w_ref), what)
