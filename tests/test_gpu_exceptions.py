"""GPU parity for the exception list (the escape path that keeps every group
lossless): offsets and entries identical to the oracle's, unpack restoring
the original words bit for bit, and GEMMs on raw (unprojected) weights that
reproduce the original weights -- one-hot rows give the original BF16 values
exactly -- on every kernel family (the pages call W12 lossless: AI Radar
summary of SpecPilot, English edition, "Reasons")."""
import ctypes

import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import assert_gemm_close, require_gpu, to_dev, to_host_u16

pytestmark = pytest.mark.gpu


def _raw(shape, sigma, seed, p_zero=0.01):
    return inputs.inject_zeros(inputs.gaussian_bf16(shape, sigma, seed), p_zero, seed + 1)


def _specials(N=48, K=384, seed=5):
    """Gaussian rows plus NaN, +-Inf, subnormals, +-0 and out-of-window values
    next to large ones in the same groups."""
    w = _raw((N, K), 0.02, seed)
    rng = np.random.default_rng(seed)
    w[0, 3] = 0x7FC1        # NaN with payload (E = 255 -> beta 120)
    w[0, 4] = 0x3F80        # 1.0, far below that window -> exception
    w[1, 130] = 0xFF80      # -Inf
    w[1, 131] = 0x8001      # negative subnormal (E = 0: stored, not an exception)
    w[2, 7] = 0x4780        # 65536
    w[2, 8:40] = 0x0100     # E = 2, smallest exponent outside {0, 1}
    w[3, :] = rng.integers(0, 65536, K).astype(np.uint16)   # arbitrary words
    return w


CASES = [("tiny", lambda: inputs.TINY.weights_raw()),
         ("ragged 37x384", lambda: _raw((37, 384), 0.015, 7)),
         ("wide 130x1152", lambda: _raw((130, 1152), 1.0, 8)),
         ("specials", _specials),
         ("qkv", lambda: inputs.QKV.weights_raw())]


def _pack_exc(bits):
    require_gpu()
    wt, bad = w12.pack(to_dev(bits), exceptions=True)
    torch.cuda.synchronize()
    return wt, bad


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_list_and_lossless_unpack(oracle, name, make):
    bits = make()
    print("exceptions:", name, bits.shape, flush=True)
    wt, bad = _pack_exc(bits)
    off, ent = oracle.exceptions(bits)
    assert bad > 0 and len(ent) > 0
    assert np.array_equal(wt.exc_offsets.cpu().numpy().view(np.uint32), off), name + ": offsets"
    got = wt.exc_entries.cpu().numpy().view(np.uint32)[:len(ent)]
    assert np.array_equal(got, ent), name + ": entries"
    assert np.array_equal(to_host_u16(w12.w12_unpack(wt)), bits), name + ": unpack not lossless"


def test_capacity_short_and_count_only(oracle):
    bits = _raw((130, 1152), 1.0, 8)
    off, ent = oracle.exceptions(bits)
    n = len(ent)
    assert n > 40
    L = w12.lib()
    N, K = bits.shape
    wd = to_dev(bits)
    wsb = L.w12_exceptions_workspace_bytes(N, K)
    ws = torch.empty(wsb // 4, dtype=torch.int32, device="cuda")
    offs = torch.full((off.size,), -1, dtype=torch.int32, device="cuda")
    cap = n // 2
    guard = 64
    entries = torch.full((cap + guard, 2), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    total = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.w12_exceptions(wd.data_ptr(), N, K, ws.data_ptr(), wsb, offs.data_ptr(),
                            entries.data_ptr(), cap, total.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(total.item()) == n
    assert np.array_equal(offs.cpu().numpy().view(np.uint32), off)
    e = entries.cpu().numpy().view(np.uint32)
    assert np.array_equal(e[:cap], ent[:cap])
    assert np.all(e[cap:] == 0x5A5A5A5A), "wrote past the capacity"
    # count only
    total.zero_()
    assert L.w12_exceptions(wd.data_ptr(), N, K, ws.data_ptr(), wsb, offs.data_ptr(), None, 0,
                            total.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(total.item()) == n


GEMM_SHAPES = [(1000, 640), (45, 5120), (77, 17408), (130, 1152)]
TILINGS = [None, "plain", (0, 1, 4, 2, 0), (0, 2, 1, 2, 1), (1, 2, 4, 2, 1), (1, 1, 2, 2, 0),
           (1, 1, 1, 2, 0, 3), (0, 1, 4, 4, 0, 5), (1, 2, 4, 2, 1, 2),
           (1, 1, 1, 2, 0, 1, 8), (1, 1, 2, 2, 0, 3, 8), (1, 1, 8, 2, 0, 64, 8)]


def _gemm(x, wt, tiling):
    if tiling is None:
        return w12.w12_gemm(x, wt)
    if tiling == "plain":
        return w12.w12_gemm(x, wt, split_k=False)
    return w12.w12_gemm(x, wt, tiling=tiling)


def _control(x, bt, tiling):
    """The BF16 control on the raw weights with the same tiling."""
    if tiling is None:
        return w12.bf16_gemm(x, bt)
    if tiling == "plain":
        return w12.bf16_gemm(x, bt, split_k=False)
    return w12.bf16_gemm(x, bt, tiling=tiling)


def _ms(tiling):
    if tiling is None or tiling == "plain":
        return [1, 3, 8, 16, 32, 64, 128]
    if tiling[0] == 0:
        return [1, 2] if tiling[4] else [1, 4, 8]
    return [5, 16] if tiling[4] else [9, 32]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "%dx%d" % s)
@pytest.mark.parametrize("tiling", TILINGS, ids=lambda t: str(t))
def test_gemm_on_raw_weights(oracle, shape, tiling):
    """With its list the container multiplies as the raw weights: the oracle's
    GEMM of the raw weights within the tolerance (and the BF16 control on the
    raw weights with the same tiling within the same bound)."""
    N, K = shape
    bits = _raw(shape, 0.02, 17 * N + K)
    wt, bad = _pack_exc(bits)
    assert bad > 0
    bt = w12.w12_bf16_tile(to_dev(bits))
    for M in _ms(tiling):
        what = "exc gemm %s %s M=%d" % (shape, tiling, M)
        print(what, flush=True)
        x = inputs.gaussian_bf16((M, K), 1.0, M + K)
        try:
            y = _gemm(to_dev(x), wt, tiling)
        except w12.W12Error as e:
            assert e.status == -6, what
            continue
        yc = _control(to_dev(x), bt, tiling)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        ref = oracle.gemm_bf16_f64(x, bits)
        tol = oracle.tolerance(x, bits)
        assert_gemm_close(yh, ref, tol, what)
        assert_gemm_close(yc.cpu().numpy(), ref, tol, what + " (control)")


@pytest.mark.parametrize("M", [1, 2, 16, 32])
def test_specials_with_list(oracle, M):
    """NaN payloads, infinities, subnormals, arbitrary words and elements far
    below their group's window: the GEMM of the raw weights (NaN and infinity
    where the oracle has them, the rest within the tolerance), like the BF16
    control on them."""
    bits = _specials()
    wt, _ = _pack_exc(bits)
    bt = w12.w12_bf16_tile(to_dev(bits))
    x = inputs.gaussian_bf16((M, bits.shape[1]), 1.0, 97 + M)
    y = w12.w12_gemm(to_dev(x), wt)
    yc = w12.bf16_gemm(to_dev(x), bt)
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16_f64(x, bits)
    tol = oracle.tolerance(x, bits)
    assert_gemm_close(y.cpu().numpy(), ref, tol, "specials M=%d" % M)
    assert_gemm_close(yc.cpu().numpy(), ref, tol, "specials M=%d (control)" % M)


@pytest.mark.parametrize("tiling", [None, "plain", (0, 1, 4, 2, 0), (1, 2, 4, 2, 1),
                                    (1, 1, 2, 2, 0), (1, 1, 1, 2, 0, 3), (1, 1, 1, 2, 0, 1, 8),
                                    (1, 1, 4, 2, 0, 2, 8)], ids=lambda t: str(t))
def test_one_hot_rows_give_original_words(oracle, tiling):
    """x rows = unit vectors at columns that hold exceptions: y[m, n] is the
    original weight w[n, k_m] exactly (the clamp is taken back exactly and the
    original added), for every exception of those columns."""
    bits = _raw((1000, 640), 0.02, 23)
    wt, _ = _pack_exc(bits)
    off, ent = oracle.exceptions(bits)
    ks = np.unique(ent[:, 0] & 0xFFFFFF)
    for M in ([1, 4] if tiling not in (None, "plain") and tiling[0] == 0 else [8, 32, 64]):
        pick = ks[np.random.default_rng(M).choice(ks.size, size=min(M, ks.size), replace=False)]
        x = np.zeros((pick.size, 640), np.uint16)
        x[np.arange(pick.size), pick] = 0x3F80
        try:
            y = _gemm(to_dev(x), wt, tiling)
        except w12.W12Error as e:
            assert e.status == -6
            continue
        torch.cuda.synchronize()
        expect = oracle.bf16_bits_to_f64(bits[:, pick].T).astype(np.float32)
        yh = y.cpu().numpy()
        # an fp32 sum that starts at +0 turns a -0 weight into +0; every
        # other value, the exception originals included, must match bit for bit
        assert np.array_equal(yh, expect), "one-hot %s M=%d" % (tiling, M)
        nz = expect != 0
        assert np.array_equal(yh[nz].view(np.uint32), expect[nz].view(np.uint32)), \
            "one-hot %s M=%d" % (tiling, M)


@pytest.mark.parametrize("M", [1, 5, 16, 32])
def test_bf16_output_and_strides_with_list(oracle, M):
    """BF16 y equals the round-to-nearest-even of the same call's fp32 y, and
    strided x / y views give the oracle's result, with corrections applied."""
    K = 640
    bits = _raw((300, K), 0.02, 41)
    wt, _ = _pack_exc(bits)
    x_full = inputs.gaussian_bf16((M, K + 64), 1.0, 43 + M)
    xd = to_dev(x_full)[:, :K]
    yf = w12.w12_gemm(xd, wt, torch.float32)
    yb = w12.w12_gemm(xd, wt, torch.bfloat16)
    y_full = torch.full((M, 300 + 20), -3.0, dtype=torch.float32, device="cuda")
    w12.w12_gemm(xd, wt, y=y_full[:, :300])
    torch.cuda.synchronize()
    assert torch.equal(yb.cpu().view(torch.int16), yf.cpu().to(torch.bfloat16).view(torch.int16))
    assert torch.equal(y_full[:, :300].cpu(), yf.cpu())
    assert torch.all(y_full[:, 300:] == -3.0)
    x = np.ascontiguousarray(x_full[:, :K])
    assert_gemm_close(yf.cpu().numpy(), oracle.gemm_bf16_f64(x, bits), oracle.tolerance(x, bits),
                      "strided with list M=%d" % M)


def test_shared_workspace_mixed_containers(oracle):
    """One split-K workspace serving, in turn, containers with and without an
    exception list and of different shapes; each result matches the oracle."""
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    seq = [((77, 17408), True, 8), ((1000, 640), False, 1), ((77, 17408), False, 32),
           ((130, 1152), True, 16), ((77, 17408), True, 1)]
    for i, (shape, with_list, M) in enumerate(seq):
        N, K = shape
        bits = _raw(shape, 0.02, 60 + i)
        if with_list:
            wt, _ = _pack_exc(bits)
            ref_w = bits
        else:
            wt = w12.w12_pack(to_dev(bits))
            ref_w = to_host_u16(w12.w12_unpack(wt))
        x = inputs.gaussian_bf16((M, K), 1.0, 70 + i)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        w12.w12_gemm(to_dev(x), wt, y=y, tiling=(1 if M > 1 else 0, 1, 2, 2, 0, 3), workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:65536].count_nonzero()) == 0
        assert_gemm_close(y.cpu().numpy(), oracle.gemm_bf16_f64(x, ref_w),
                          oracle.tolerance(x, ref_w), "mixed %d %s" % (i, shape))


# x staged in LDS (one to five chunks), every split mode: one slice, the
# two-slice exchange, the counted finish of three or more
STAGED_TILINGS = [(0, 1, 2, 2, 0), (0, 1, 4, 4, 0, 5), (1, 1, 1, 2, 0), (1, 1, 4, 2, 0, 2),
                  (1, 2, 2, 2, 0), (1, 2, 4, 2, 0, 3), (1, 1, 2, 4, 0),
                  (1, 1, 1, 2, 0, 1, 8), (1, 1, 4, 2, 0, 1, 8), (1, 1, 4, 2, 0, 2, 8),
                  (1, 1, 2, 2, 0, 3, 8), (1, 1, 8, 2, 0, 1, 8), (1, 1, 4, 2, 0, 1, 16),
                  (1, 1, 2, 2, 0, 3, 16)]


@pytest.mark.parametrize("tiling", STAGED_TILINGS, ids=lambda t: str(t))
def test_dense_lists_staged_x(oracle, tiling):
    """Weights of unit scale (so that most groups are flagged and a tile's
    slice holds hundreds of entries, past the 64 the correction wave loads
    at once) and a sparse one, with x staged in LDS: the oracle's GEMM of
    the raw weights within the tolerance, and the BF16 control on the same
    weights with the same tiling within the same bound."""
    for shape, sigma in (((96, 5120), 1.0), ((70, 2304), 0.02)):
        N, K = shape
        bits = _raw(shape, sigma, 5 * N + K)
        wt, bad = _pack_exc(bits)
        assert bad > 0
        bt = w12.w12_bf16_tile(to_dev(bits))
        for M in ([1, 3] if tiling[0] == 0 else [5, 16, 32]):
            what = "dense exc gemm %s %s M=%d" % (shape, tiling, M)
            print(what, flush=True)
            x = inputs.gaussian_bf16((M, K), 1.0, 3 * M + K)
            try:
                y = _gemm(to_dev(x), wt, tiling)
            except w12.W12Error as e:
                assert e.status == -6, what
                continue
            yc = _control(to_dev(x), bt, tiling)
            torch.cuda.synchronize()
            ref = oracle.gemm_bf16_f64(x, bits)
            tol = oracle.tolerance(x, bits)
            assert_gemm_close(y.cpu().numpy(), ref, tol, what)
            assert_gemm_close(yc.cpu().numpy(), ref, tol, what + " (control)")


@pytest.mark.parametrize("M", [1, 4, 6, 8, 16, 32, 64])
def test_raw_qkv_default_with_list(oracle, M):
    """The full-size raw QKV weight (7168x5120, 11 174 listed weights) with
    its exception list through the default tiling the benchmark times at each
    row count -- the correction wave at M = 1-4, in-loop corrections from 6
    rows (chosen because a list is present), the post-loop walk at 64 --
    against the oracle's GEMM of the raw weights on sampled rows (the first
    and last 64 and 384 more), and the BF16 control on the raw weights with
    the same tiling within the same bound."""
    bits = inputs.QKV.weights_raw()
    wt, bad = _pack_exc(bits)
    assert bad > 0
    bt = w12.w12_bf16_tile(to_dev(bits))
    rng = np.random.default_rng(M)
    N, K = bits.shape
    rows = np.array(sorted(set(range(64)) | set(range(N - 64, N)) |
                           set(rng.choice(N, size=384, replace=False).tolist())))
    x = inputs.QKV.activations(M)
    what = "raw qkv default M=%d (%s)" % (M, w12.w12_gemm_variant(M, N, K, 3))
    print(what, flush=True)
    y = w12.w12_gemm(to_dev(x), wt)
    yc = w12.bf16_gemm(to_dev(x), bt)
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16_f64(x, bits[rows])
    tol = oracle.tolerance(x, bits[rows])
    assert_gemm_close(y.cpu().numpy()[:, rows], ref, tol, what)
    assert_gemm_close(yc.cpu().numpy()[:, rows], ref, tol, what + " (control)")
