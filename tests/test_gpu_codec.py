"""GPU parity for w12_pack / w12_unpack: byte-identical planes, meta and
unencodable count against the CPU oracle, bit-identical unpack, on every
workload shape and on edge tensors (lossless per the pages: AI Radar summary
of SpecPilot, English edition, "Reasons")."""
import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import require_gpu, to_dev, to_host_u16, to_host_u8

pytestmark = pytest.mark.gpu


def _gpu_pack(bits: np.ndarray):
    require_gpu()
    wd = to_dev(bits)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    wt = w12.w12_pack(wd, bad_groups=bad)
    torch.cuda.synchronize()
    return wt, int(bad.item())


def _check_pack(oracle, bits: np.ndarray, what: str):
    N, K = bits.shape
    print("pack parity:", what, N, K, flush=True)
    wt, bad = _gpu_pack(bits)
    r0, r1, r2, rmeta, rbad = oracle.pack(bits)
    assert np.array_equal(to_host_u8(wt.p0), r0), what + ": P0"
    assert np.array_equal(to_host_u8(wt.p1), r1), what + ": P1"
    assert np.array_equal(to_host_u8(wt.p2), r2), what + ": P2"
    assert np.array_equal(to_host_u8(wt.meta), rmeta), what + ": meta"
    assert bad == rbad, what + ": unencodable count"
    back = to_host_u16(w12.w12_unpack(wt))
    assert np.array_equal(back, oracle.unpack(r0, r1, r2, rmeta, N, K)), what + ": unpack"
    return wt, back, rbad


def _all_codes_tensor():
    """Every BF16 word each base can store: for base b, the 4096 stored words
    in 32 groups, each group holding 8 words of the top binade 2b+15 so that
    the packer derives base b.  121 rows x 4096 columns."""
    allw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (allw.astype(np.int32) >> 7) & 0xFF
    rows = []
    for b in range(121):
        stored = (e <= 1) | ((e >= 2 * b + 2) & (e <= 2 * b + 15))
        top = allw[stored & (e == 2 * b + 15)]
        rest = allw[stored & (e != 2 * b + 15)]
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
    assert np.array_equal(oracle.meta_of(to_host_u8(wt.meta), 121, 4096)[:, 0],
                          np.arange(121, dtype=np.uint8))


@pytest.mark.parametrize("name", ["tiny", "qkv", "gate_up", "down"])
def test_workload_pack_parity(oracle, name):
    case = inputs.CASES[name]
    raw = case.weights_raw()
    wt, clamped, bad = _check_pack(oracle, raw, name)
    # the raw Gaussian draw has unencodable groups; the projection has none
    assert bad > 0
    wt2, back2, bad2 = _check_pack(oracle, clamped, name + " clamped")
    assert bad2 == 0
    assert np.array_equal(back2, clamped)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (5, 1152), (1000, 640)])
def test_edge_shapes(oracle, N, K):
    rng = np.random.default_rng(N * 7 + K)
    bits = rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16)
    _check_pack(oracle, bits, "random bits %dx%d" % (N, K))
    g = inputs.gaussian_bf16((N, K), 0.02, N + K)
    _check_pack(oracle, g, "gaussian %dx%d" % (N, K))


def test_special_values(oracle):
    rows = np.zeros((4, 256), np.uint16)
    rows[0, :6] = [0x0000, 0x8000, 0x0001, 0x807F, 0x0080, 0x80FF]
    rows[1, :] = 0x7F00
    rows[1, :6] = [0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x7F81, 0x7900]
    rows[2, :2] = [0x7F7F, 0xFF7F]
    rows[3, :] = 0x3F80
    rows[3, 5] = 0x0100           # E = 2 next to 1.0 (E = 127): flagged
    wt, back, bad = _check_pack(oracle, rows, "specials")
    assert bad == 1
    assert np.array_equal(back[:3], rows[:3])


def test_pack_without_counter(oracle):
    require_gpu()
    raw = inputs.TINY.weights_raw()
    wt = w12.w12_pack(to_dev(raw))
    torch.cuda.synchronize()
    r0, r1, r2, rmeta, _ = oracle.pack(raw)
    assert np.array_equal(to_host_u8(wt.meta), rmeta)
    assert np.array_equal(to_host_u8(wt.p2), r2)


def test_strict_pack_raises():
    require_gpu()
    raw = inputs.TINY.weights_raw()
    with pytest.raises(w12.W12UnencodableError):
        w12.pack(to_dev(raw), strict=True)


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (1000, 640), (7168, 5120)])
def test_bf16_control_layout(oracle, N, K):
    """w12_bf16_tile is the oracle's control-layout permutation, word for word."""
    require_gpu()
    rng = np.random.default_rng(N + K)
    bits = rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16)
    t = w12.w12_bf16_tile(to_dev(bits))
    torch.cuda.synchronize()
    assert np.array_equal(to_host_u16(t.w), oracle.bf16_tile(bits))


def test_readme_example():
    """The usage example of the README, as written there."""
    require_gpu()
    torch.manual_seed(0)
    w = torch.randn(7168, 5120, device="cuda").to(torch.bfloat16)
    wt, flagged = w12.pack(w, exceptions=True)
    x = torch.randn(4, 5120, device="cuda").to(torch.bfloat16)
    y = w12.w12_gemm(x, wt)
    assert torch.equal(w12.w12_unpack(wt).view(torch.int16), w.view(torch.int16))
    wt_b, _ = w12.pack(w, exceptions=True, fmt="b")
    assert torch.equal(w12.w12_unpack(wt_b).view(torch.int16), w.view(torch.int16))
    ref = x.float() @ w.float().t()
    assert flagged > 0 and y.shape == (4, 7168)
    assert torch.allclose(y, ref, rtol=0, atol=1e-3 * float(x.float().norm(dim=1).max())
                          * float(w.float().norm(dim=1).max()) + 1e-6)


def test_layout_worked_example2_on_gpu():
    """The hand-derived second layout example (tests/golden/
    w12_layout_example2.txt) packed by the GPU: the same non-zero plane and
    meta bytes, flag count, unpacked words and exception list."""
    from tests.test_oracle_codec import layout_example2_weight
    w, rec = layout_example2_weight()
    wt, bad = _gpu_pack(w)
    for name, plane in (("p0", wt.p0), ("p1", wt.p1), ("p2", wt.p2)):
        h = to_host_u8(plane)
        assert {int(i): int(h[i]) for i in np.flatnonzero(h)} == rec[name], name
    hm = to_host_u8(wt.meta)
    assert {int(i): int(hm[i]) for i in np.flatnonzero(hm)} == rec["meta"]
    assert bad == rec["bad"][0]
    want = w.copy()
    for n, k, v in rec["unpacked"]:
        want[n, k] = v
    assert np.array_equal(to_host_u16(w12.w12_unpack(wt)), want)
    off, ent = w12.w12_exceptions(to_dev(w))
    assert list(off.cpu().numpy()) == rec["offsets"]
    assert [tuple(int(v) for v in e) for e in ent.cpu().numpy().view(np.uint32)] == rec["entry"]
