"""Pins for the oracle's W12-b allocation (the arbitrary-base alternative:
a 4-bit offset of the exponent from a per-group base of any value).

As for W12-v1, the pages fix that W12 spends 12 bits per BF16 weight in
three 4-bit planes and is lossless (AI Radar summary of SpecPilot, English
edition, "Reasons"; HotRepo digest of StargazerX0/SpecPilot, project
introduction); the bit allocation is this project's reading.  Each test
checks the allocation by brute force, counting or a hand-derived example,
not by restating the oracle's formulas.
"""
import os

import numpy as np
import pytest

from lossless_bit_weight_amd import inputs

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
EXP = (ALL_BF16.astype(np.int32) >> 7) & 0xFF


def test_exhaustive_bijection_every_base(oracle):
    """For every base 0..240 exactly 2^12 BF16 patterns are stored exactly,
    their codes are a bijection onto 0..4095 whose decode is the inverse, and
    the stored exponents are {0} and one run of 15 consecutive exponents
    starting right above the base."""
    for b in range(241):
        code, ok = oracle.b_encode_many(ALL_BF16, b)
        assert code.max() < 4096
        assert int(ok.sum()) == 4096, b
        enc = code[ok]
        assert np.array_equal(np.sort(enc), np.arange(4096, dtype=np.uint16)), b
        assert np.array_equal(oracle.b_decode_many(enc, b), ALL_BF16[ok]), b
        stored = sorted(set(EXP[ok].tolist()))
        assert stored == [0] + list(range(b + 1, b + 16)), b
        for e in stored:
            assert int(ok[EXP == e].sum()) == 256


def test_base_rule_bruteforce(oracle):
    """The base is the smallest one for which the group's largest element
    survives the round trip (every base tried), and it never exceeds 240."""
    rng = np.random.default_rng(17)
    for emax in range(256):
        for _ in range(3):
            v = (int(rng.integers(0, 2)) << 15) | (emax << 7) | int(rng.integers(0, 128))
            smallest = next(b for b in range(256)
                            if oracle.b_decode(oracle.b_encode(v, b)[0], b) == v)
            assert oracle.b_base_for_emax(emax) == smallest
        assert 0 <= oracle.b_base_for_emax(emax) <= 240


def test_one_more_exponent_than_v1(oracle):
    """Counting: W12-b stores 15 normal exponents per group at any offset,
    W12-v1 14 plus the binade E = 1, at even offsets only -- so for every
    largest exponent >= 16 the W12-b window reaches at least as low."""
    for emax in range(16, 256):
        b = oracle.b_base_for_emax(emax)
        beta = oracle.beta_for_emax(emax)
        assert b + 1 <= 2 * beta + 2
        assert emax - (b + 1) == 14          # the window ends at emax


def test_clamp_is_window_floor(oracle):
    """An element below the window decodes to +-2^(b+1-127), the smallest
    stored normal magnitude, with its sign."""
    for b in (1, 5, 57, 112, 240):
        code, ok = oracle.b_encode_many(ALL_BF16, b)
        dec = oracle.b_decode_many(code, b)
        below = (~ok) & (EXP >= 1) & (EXP <= b)
        assert below.any()
        mag = np.float64(2.0) ** (b + 1 - 127)
        got = oracle.bf16_bits_to_f64(dec[below])
        sign = np.where(ALL_BF16[below] >= 0x8000, -1.0, 1.0)
        assert np.array_equal(got, sign * mag)
    code, ok = oracle.b_encode_many(ALL_BF16, 0)
    assert ok[EXP <= 15].all()


def _read_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "w12b_layout_example.txt")
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = [int(t, 16) for t in v.split()]
    return rec


@pytest.mark.parametrize("variant,k7", [("GAP", 0x3800), ("IN", 0x3980)])
def test_layout_worked_example(oracle, variant, k7):
    """Hand-derived worked example: plane bytes, meta byte, flagged count
    and unpacked words of one W12-b group."""
    g = _read_golden()
    w = np.zeros((1, 128), np.uint16)
    w[0, :8] = [0x3F80, 0xBF00, 0x3C01, 0x8000, 0x3A5B, 0x0001, 0xB9C7, k7]
    p0, p1, p2, meta, bad = oracle.pack(w, fmt="b")
    for name, plane in (("p0", p0), ("p1", p1), ("p2", p2)):
        assert list(plane[:4]) == g[variant + "." + name]
        assert not plane[4:].any()
    assert list(meta[:1]) == g[variant + ".meta"]
    assert not meta[1:].any()
    assert bad == g[variant + ".bad"][0]
    out = oracle.unpack(p0, p1, p2, meta, 1, 128, fmt="b")
    assert list(out[0, :8]) == g[variant + ".unpacked"]
    assert not out[0, 8:].any()


def test_special_values_round_trip(oracle):
    """+-0, subnormals, +-Inf and NaN payloads survive with compatible
    neighbours; the base of an Inf/NaN group is 240."""
    rows = [[0x0000, 0x8000, 0x0001, 0x807F] + [0] * 124,
            [0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x7F81, 0x7900] + [0x7F00] * 122,
            [0x0080, 0x8100] + [0x0000] * 126]
    w = np.array(rows, dtype=np.uint16)
    p0, p1, p2, meta, bad = oracle.pack(w, fmt="b")
    assert bad == 0
    assert np.array_equal(oracle.unpack(p0, p1, p2, meta, 3, 128, fmt="b"), w)
    assert list(oracle.meta_of(meta, 3, 128)[:, 0]) == [0, 240, 0]


def test_fewer_unencodable_groups_than_v1(oracle):
    """On raw Gaussian weights (sigma 0.02 and 0.015) W12-b flags fewer
    groups than W12-v1: its window has one more exponent and starts right
    below the group maximum whatever its parity."""
    for sigma, seed in ((0.02, 3), (0.015, 4)):
        w = inputs.gaussian_bf16((512, 1024), sigma, seed)
        bad_v1 = oracle.pack(w)[4]
        bad_b = oracle.pack(w, fmt="b")[4]
        assert 0 < bad_b < bad_v1


@pytest.mark.parametrize("shape,sigma,seed", [((1024, 512), 0.02, 101), ((37, 384), 0.015, 7),
                                              ((130, 1152), 1.0, 8), ((16, 128), 1e-30, 9)])
def test_list_is_exactly_the_lossy_set(oracle, shape, sigma, seed):
    """Brute force: the W12-b exception list holds exactly the elements the
    clamped container does not reproduce, with their original words and
    their group's base, and writing them back restores the weight."""
    w = inputs.inject_zeros(inputs.gaussian_bf16(shape, sigma, seed), 0.01, seed + 1)
    p0, p1, p2, meta, bad = oracle.pack(w, fmt="b")
    back = oracle.unpack(p0, p1, p2, meta, *shape, fmt="b")
    lossy = set(zip(*np.nonzero(back != w)))
    bases = oracle.meta_of(meta, *shape)
    off, ent = oracle.exceptions(w, fmt="b")
    G = shape[1] // 128
    listed = {}
    for t in range(len(off) - 1):
        for i in range(off[t], off[t + 1]):
            c, k = int(ent[i, 0]) >> 24, int(ent[i, 0]) & 0xFFFFFF
            assert k // 128 == t % G
            listed[(16 * (t // G) + c, k)] = int(ent[i, 1])
    assert set(listed) == lossy
    assert all(w[n, k] == v & 0xFFFF for (n, k), v in listed.items())
    assert all(v >> 16 == bases[n, k // 128] for (n, k), v in listed.items())
    assert np.array_equal(oracle.apply_exceptions(back, off, ent), w)
    # a group is counted as flagged exactly when it holds a listed element
    flagged = {(n, k // 128) for (n, k) in listed}
    assert bad == len(flagged)


def test_projection_is_a_fixed_point(oracle):
    """unpack(pack(.)) projects onto the stored set: packing the projection
    flags nothing and reproduces the same planes and bases."""
    w_raw = inputs.TINY.weights_raw()
    p0, p1, p2, meta, bad = oracle.pack(w_raw, fmt="b")
    w = oracle.unpack(p0, p1, p2, meta, inputs.TINY.N, inputs.TINY.K, fmt="b")
    q0, q1, q2, qmeta, bad2 = oracle.pack(w, fmt="b")
    assert bad2 == 0
    assert np.array_equal(q0, p0) and np.array_equal(q1, p1) and np.array_equal(q2, p2)
    assert np.array_equal(qmeta, meta)


def test_container_gemm_matches_plain_gemm(oracle):
    """The oracle's decode-in-GEMM over a W12-b container equals the plain
    fp64 GEMM over the unpacked weight (same definition, two routes)."""
    w = inputs.gaussian_bf16((40, 256), 0.02, 5)
    x = inputs.gaussian_bf16((3, 256), 1.0, 6)
    p0, p1, p2, meta, _ = oracle.pack(w, fmt="b")
    wu = oracle.unpack(p0, p1, p2, meta, 40, 256, fmt="b")
    y1 = oracle.gemm_w12_f64(x, p0, p1, p2, meta, 40, fmt="b")
    y2 = oracle.gemm_bf16_f64(x, wu)
    assert np.array_equal(y1, y2)
