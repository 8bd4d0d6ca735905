"""GPU parity for W12-b, the arbitrary-base bit allocation: pack, unpack and
the exception list byte-identical to the oracle's W12-b (including every
code of every base), and the W12-b GEMMs within the oracle tolerance and
bitwise equal to the BF16 control of the same tiling, on projected and on
raw weights (the pages call W12 lossless and rebuilt bit-exactly in the
GEMM: AI Radar summary of SpecPilot, English edition, "Reasons")."""
import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import assert_gemm_close, require_gpu, to_dev, to_host_u16, to_host_u8

pytestmark = pytest.mark.gpu


def _check_pack(oracle, bits: np.ndarray, what: str):
    require_gpu()
    N, K = bits.shape
    print("w12b pack parity:", what, N, K, flush=True)
    bad_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    wt = w12.w12_pack(to_dev(bits), bad_groups=bad_t, fmt="b")
    torch.cuda.synchronize()
    r0, r1, r2, rmeta, rbad = oracle.pack(bits, fmt="b")
    assert np.array_equal(to_host_u8(wt.p0), r0), what + ": P0"
    assert np.array_equal(to_host_u8(wt.p1), r1), what + ": P1"
    assert np.array_equal(to_host_u8(wt.p2), r2), what + ": P2"
    assert np.array_equal(to_host_u8(wt.meta), rmeta), what + ": meta"
    assert int(bad_t.item()) == rbad, what + ": unencodable count"
    back = to_host_u16(w12.w12_unpack(wt))
    assert np.array_equal(back, oracle.unpack(r0, r1, r2, rmeta, N, K, fmt="b")), what + ": unpack"
    return wt, back, rbad


def _all_codes_tensor():
    """Every BF16 word each W12-b base stores: for base b (0..240), its 4096
    words in 32 groups of 128, each holding 8 words of the top exponent
    b + 15 so that the packer derives base b.  241 rows x 4096 columns."""
    allw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (allw.astype(np.int32) >> 7) & 0xFF
    rows = []
    for b in range(241):
        stored = (e == 0) | ((e >= b + 1) & (e <= b + 15))
        top = allw[stored & (e == b + 15)]
        rest = allw[stored & (e != b + 15)]
        assert top.size == 256 and rest.size == 3840
        groups = [np.concatenate([top[8 * g:8 * g + 8], rest[120 * g:120 * g + 120]])
                  for g in range(32)]
        rows.append(np.concatenate(groups))
    return np.stack(rows)


def test_every_code_of_every_base(oracle):
    bits = _all_codes_tensor()
    wt, back, bad = _check_pack(oracle, bits, "all codes")
    assert bad == 0
    assert np.array_equal(back, bits)
    assert np.array_equal(oracle.meta_of(to_host_u8(wt.meta), 241, 4096)[:, 0],
                          np.arange(241, dtype=np.uint8))


@pytest.mark.parametrize("name", ["tiny", "qkv", "down"])
def test_workload_pack_parity(oracle, name):
    raw = inputs.CASES[name].weights_raw()
    wt, clamped, bad = _check_pack(oracle, raw, name)
    assert bad > 0
    wt2, back2, bad2 = _check_pack(oracle, clamped, name + " clamped")
    assert bad2 == 0 and np.array_equal(back2, clamped)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (1000, 640)])
def test_random_bits(oracle, N, K):
    rng = np.random.default_rng(N * 5 + K)
    _check_pack(oracle, rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16),
                "random bits %dx%d" % (N, K))


def _raw(shape, sigma, seed):
    return inputs.inject_zeros(inputs.gaussian_bf16(shape, sigma, seed), 0.01, seed + 1)


@pytest.mark.parametrize("shape,sigma,seed", [((1024, 512), 0.02, 101), ((130, 1152), 1.0, 8),
                                              ((7168, 5120), 0.02, 201)])
def test_exception_list_and_lossless_unpack(oracle, shape, sigma, seed):
    bits = _raw(shape, sigma, seed)
    print("w12b exceptions:", shape, flush=True)
    wt, bad = w12.pack(to_dev(bits), exceptions=True, fmt="b")
    torch.cuda.synchronize()
    off, ent = oracle.exceptions(bits, fmt="b")
    assert bad > 0 and len(ent) > 0
    assert np.array_equal(wt.exc_offsets.cpu().numpy().view(np.uint32), off)
    assert np.array_equal(wt.exc_entries.cpu().numpy().view(np.uint32)[:len(ent)], ent)
    assert np.array_equal(to_host_u16(w12.w12_unpack(wt)), bits)


_cache = {}


def _prepared(shape):
    """W12-b container and BF16 control of one projected weight."""
    if shape not in _cache:
        require_gpu()
        raw = inputs.gaussian_bf16(shape, 0.02, 3 * shape[0] + shape[1])
        p0, p1, p2, meta, _ = oracle_mod().pack(raw, fmt="b")
        w = oracle_mod().unpack(p0, p1, p2, meta, *shape, fmt="b")
        wt, bad = w12.pack(to_dev(w), fmt="b")
        assert bad == 0
        tiled = w12.w12_bf16_tile(to_dev(w))
        torch.cuda.synchronize()
        _cache[shape] = (w, wt, tiled)
    return _cache[shape]


def oracle_mod():
    import oracle
    return oracle


TILINGS = [None, "plain", (0, 1, 2, 4, 1), (0, 1, 4, 2, 0), (1, 2, 4, 2, 1), (1, 1, 4, 2, 1, 3),
           (1, 1, 2, 2, 0), (1, 1, 1, 2, 0, 3), (1, 1, 4, 2, 0, 1, 8), (1, 1, 2, 2, 0, 3, 8)]


def _gemm(x, wt, tiling):
    if tiling is None:
        return w12.w12_gemm(x, wt)
    if tiling == "plain":
        return w12.w12_gemm(x, wt, split_k=False)
    return w12.w12_gemm(x, wt, tiling=tiling)


def _bf16(x, tiled, tiling):
    if tiling is None:
        return w12.bf16_gemm(x, tiled)
    if tiling == "plain":
        return w12.bf16_gemm(x, tiled, split_k=False)
    return w12.bf16_gemm(x, tiled, tiling=tiling)


def _ms(tiling):
    if tiling is None or tiling == "plain":
        return [1, 2, 9, 16, 32, 128]
    if tiling[0] == 0:
        return [1, 3] if tiling[4] else [1, 8]
    return [4, 16] if tiling[4] else [9, 32]


@pytest.mark.parametrize("shape", [(301, 640), (45, 5120), (77, 17408), (1000, 1152)],
                         ids=lambda s: "%dx%d" % s)
@pytest.mark.parametrize("tiling", TILINGS, ids=lambda t: str(t))
def test_gemm_parity(oracle, shape, tiling):
    """W12-b GEMM within tolerance of the oracle and bitwise equal to the
    BF16 control of the same tiling."""
    w, wt, tiled = _prepared(shape)
    for M in _ms(tiling):
        what = "w12b gemm %s %s M=%d" % (shape, tiling, M)
        print(what, flush=True)
        x = inputs.gaussian_bf16((M, shape[1]), 1.0, 7 * M + shape[1])
        xd = to_dev(x)
        try:
            y = _gemm(xd, wt, tiling)
        except w12.W12Error as e:
            assert e.status == -6, what    # a tiling not built for this shape
            continue
        y16 = _bf16(xd, tiled, tiling)
        torch.cuda.synchronize()
        yh, y16h = y.cpu().numpy(), y16.cpu().numpy()
        assert np.array_equal(yh.view(np.uint32), y16h.view(np.uint32)), what + ": != bf16"
        assert_gemm_close(yh, oracle.gemm_bf16_f64(x, w), oracle.tolerance(x, w), what)


@pytest.mark.parametrize("name", ["qkv", "gate_up"])
@pytest.mark.parametrize("M", [1, 4, 16, 32])
def test_workloads_sampled(oracle, name, M):
    case = inputs.CASES[name]
    raw = case.weights_raw()
    require_gpu()
    wt, _ = w12.pack(to_dev(raw), fmt="b")
    w = to_host_u16(w12.w12_unpack(wt))
    x = case.activations(M)
    y = w12.w12_gemm(to_dev(x), wt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(64), rng.choice(case.N, 256, replace=False)]))
    ref = oracle.gemm_bf16_f64(x, np.ascontiguousarray(w[rows]))
    assert_gemm_close(y.cpu().numpy()[:, rows], ref, oracle.tolerance(x, w[rows]),
                      "w12b %s M=%d" % (name, M))


@pytest.mark.parametrize("tiling", [None, "plain", (0, 1, 4, 2, 0), (1, 2, 4, 2, 1),
                                    (1, 1, 2, 2, 0, 3, 8), (1, 1, 1, 2, 0, 1, 8)],
                         ids=lambda t: str(t))
def test_raw_weights_with_list(oracle, tiling):
    """On raw weights the W12-b container plus its exception list gives the
    GEMM of the original weights; one-hot rows at listed columns return the
    original words exactly."""
    bits = _raw((1000, 640), 0.02, 23)
    wt, bad = w12.pack(to_dev(bits), exceptions=True, fmt="b")
    torch.cuda.synchronize()
    assert bad > 0
    for M in ([1, 8] if tiling not in (None, "plain") and tiling[0] == 0 else [8, 32, 100]):
        x = inputs.gaussian_bf16((M, 640), 1.0, M + 640)
        try:
            y = _gemm(to_dev(x), wt, tiling)
        except w12.W12Error as e:
            assert e.status == -6
            continue
        torch.cuda.synchronize()
        assert_gemm_close(y.cpu().numpy(), oracle.gemm_bf16_f64(x, bits),
                          oracle.tolerance(x, bits), "w12b raw %s M=%d" % (tiling, M))
        off, ent = oracle.exceptions(bits, fmt="b")
        ks = np.unique(ent[:, 0] & 0xFFFFFF)
        pick = ks[np.random.default_rng(M).choice(ks.size, size=min(M, ks.size), replace=False)]
        xo = np.zeros((pick.size, 640), np.uint16)
        xo[np.arange(pick.size), pick] = 0x3F80
        yo = _gemm(to_dev(xo), wt, tiling)
        torch.cuda.synchronize()
        expect = oracle.bf16_bits_to_f64(bits[:, pick].T).astype(np.float32)
        got = yo.cpu().numpy()
        nz = expect != 0
        assert np.array_equal(got, expect)
        assert np.array_equal(got[nz].view(np.uint32), expect[nz].view(np.uint32))
