"""Pins for the oracle's W12 codec, independent of the oracle's own formulas.

The pages fix three things about W12 (AI Radar summary of SpecPilot, English
edition, "Reasons"; HotRepo digest of StargazerX0/SpecPilot, project
introduction): it is 12 bits per BF16 weight in three 4-bit planes, it is
lossless, and the GEMM rebuilds the BF16 bits exactly.  Each test below
checks one of those facts (or a consequence that a plausible slip in the
oracle would break) by brute force, counting, or a hand-derived example.
"""
import os

import numpy as np
import pytest

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
EXP = (ALL_BF16.astype(np.int32) >> 7) & 0xFF


@pytest.mark.parametrize("beta", list(range(0, 121)))
def test_exhaustive_bijection_per_beta(oracle, beta):
    """For every base, exactly 2^12 BF16 patterns are stored exactly, and the
    12-bit codes of those patterns are a bijection onto 0..4095 whose decode
    gives the pattern back (lossless 12-bit code, brute force over all
    65536 BF16 words)."""
    code, ok = oracle.encode_many(ALL_BF16, beta)
    assert code.max() < 4096                          # 12 bits per weight
    assert int(ok.sum()) == 4096                      # a 12-bit code's capacity, used fully
    enc = code[ok]
    assert np.array_equal(np.sort(enc), np.arange(4096, dtype=np.uint16))
    assert np.array_equal(oracle.decode_many(enc, beta), ALL_BF16[ok])
    # Every code decodes to a stored pattern: decode is the inverse map.
    dec_all = oracle.decode_many(np.arange(4096, dtype=np.uint16), beta)
    assert len(np.unique(dec_all)) == 4096
    assert set(dec_all.tolist()) == set(ALL_BF16[ok].tolist())
    # The stored set is sign-symmetric and closed under every mantissa for a
    # given exponent (only the exponent decides encodability).
    stored_exps = set(EXP[ok].tolist())
    assert len(stored_exps) == 16
    for e in stored_exps:
        assert int(ok[EXP == e].sum()) == 256
    # Zero, the subnormals and the smallest normal binade are always stored.
    assert {0, 1} <= stored_exps
    # The stored normal exponents above 1 form one contiguous run of 14.
    upper = sorted(e for e in stored_exps if e > 1)
    assert upper == list(range(upper[0], upper[0] + 14))


def test_beta_rule_bruteforce(oracle):
    """The group base is the smallest base for which the group's largest
    element survives the round trip (checked by trying every base), and the
    oracle's base keeps every smaller stored exponent down to its floor."""
    rng = np.random.default_rng(7)
    for emax in range(256):
        for _ in range(3):
            s = int(rng.integers(0, 2))
            m = int(rng.integers(0, 128))
            v = (s << 15) | (emax << 7) | m
            smallest = next(b for b in range(0, 128)
                            if oracle.decode(oracle.encode(v, b)[0], b) == v)
            assert oracle.beta_for_emax(emax) == smallest
        beta = oracle.beta_for_emax(emax)
        assert 0 <= beta <= 120
        # no byte carry: the largest rebuilt exponent field fits 7 bits
        assert beta + 7 <= 127


def test_clamp_is_window_floor(oracle):
    """An element below its group's window is written as the smallest stored
    normal magnitude of that window, with its sign (documented clamp)."""
    for beta in (0, 1, 5, 56, 120):
        code, ok = oracle.encode_many(ALL_BF16, beta)
        dec = oracle.decode_many(code, beta)
        stored = ALL_BF16[ok]
        stored_exp = EXP[ok]
        floor_mag = int(stored[(stored_exp > 1) & (stored < 0x8000)].min())
        below = (~ok) & (EXP > 1) & (EXP < (floor_mag >> 7))
        if beta == 0:
            assert not below.any()
            continue
        assert below.any()
        expect = (ALL_BF16[below] & 0x8000) | floor_mag
        assert np.array_equal(dec[below], expect.astype(np.uint16))


def _read_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "w12_layout_example.txt")
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
    """Hand-derived worked example: plane bytes in split-nibble order, meta
    byte, unencodable flag and count, and the unpacked words."""
    g = _read_golden()
    w = np.zeros((1, 128), np.uint16)
    w[0, :8] = [0x3F80, 0xBF00, 0x3C01, 0x8000, 0x3A5B, 0x0001, 0xB9C7, k7]
    p0, p1, p2, meta, bad = oracle.pack(w)
    for name, plane in (("p0", p0), ("p1", p1), ("p2", p2)):
        assert plane.shape == (1024,)           # one 16-row tile x one group
        assert list(plane[:4]) == g[variant + "." + name]
        assert not plane[4:].any()
    assert meta.shape == (16,)
    assert list(meta[:1]) == g[variant + ".meta"]
    assert not meta[1:].any()                   # padding rows
    assert bad == g[variant + ".bad"][0]
    out = oracle.unpack(p0, p1, p2, meta, 1, 128)
    assert list(out[0, :8]) == g[variant + ".unpacked"]
    assert not out[0, 8:].any()


def test_tile_addressing(oracle):
    """Where each weight lands in the tiled layout: a single marked weight at
    (n, k) shows up as one nibble at the byte the layout rule gives, and the
    meta byte of its (row, group) is the only non-zero meta byte."""
    N, K = 37, 384
    for (n, k) in [(0, 0), (0, 4), (0, 9), (5, 31), (15, 32), (3, 45), (16, 0), (17, 130),
                   (36, 383), (20, 200)]:
        w = np.zeros((N, K), np.uint16)
        w[n, k] = 0x3F8F                      # 1.0 with mantissa low nibble 0xF
        p0, p1, p2, meta, _ = oracle.pack(w)
        G = K // 128
        r = k % 128
        b, q, e = r // 32, (r % 32) // 8, r % 8
        byte = ((n // 16) * G + k // 128) * 1024 + (16 * q + n % 16) * 16 + 4 * b + e % 4
        shift = 0 if e < 4 else 4
        nz = np.flatnonzero(p0)
        assert list(nz) == [byte] and p0[byte] == 0xF << shift, (n, k)
        mz = np.flatnonzero(meta)
        assert list(mz) == [((n // 16) * G + k // 128) * 16 + n % 16], (n, k)
        assert oracle.meta_of(meta, N, K)[n, k // 128] == meta[mz[0]]


def test_container_bytes_are_three_quarters(oracle):
    """Packed planes are exactly 0.75x the BF16 bytes (12 of 16 bits) when N
    is a multiple of the 16-row tile (else 0.75x the padded rows), plus one
    metadata byte per 128-weight group."""
    for N, K in ((16, 128), (48, 256), (1024, 512), (16, 17408), (7168, 5120)):
        assert 3 * oracle.plane_bytes(N, K) == 0.75 * (2 * N * K)
        assert oracle.meta_bytes(N, K) == N * K // 128
    for N, K in ((1, 128), (3, 256), (7, 17408)):
        p0, p1, p2, meta, _ = oracle.pack(np.zeros((N, K), np.uint16))
        Np = (N + 15) // 16 * 16
        assert p0.nbytes + p1.nbytes + p2.nbytes == 0.75 * (2 * Np * K)
        assert meta.nbytes == Np * K // 128


def _groups_random(rng, rows, gap_rows):
    """BF16 rows of one group each; rows in gap_rows get one element pushed
    far below the row maximum."""
    w = rng.standard_normal((rows, 128)).astype(np.float32) * np.float32(0.02)
    from lossless_bit_weight_amd.inputs import f32_to_bf16_bits
    b = f32_to_bf16_bits(w)
    for r in gap_rows:
        b[r, int(rng.integers(0, 128))] = np.uint16(0x3000 | int(rng.integers(0, 128)))
    return b


def test_flag_iff_not_lossless(oracle):
    """A group is flagged exactly when its round trip is not the identity,
    and the count equals the number of flagged groups."""
    rng = np.random.default_rng(11)
    b = _groups_random(rng, 400, gap_rows=range(0, 400, 7))
    p0, p1, p2, meta, bad = oracle.pack(b)
    back = oracle.unpack(p0, p1, p2, meta, 400, 128)
    changed = np.any(back != b, axis=1)
    flagged = (oracle.meta_of(meta, 400, 128)[:, 0] & 0x80) != 0
    assert np.array_equal(changed, flagged)
    assert bad == int(flagged.sum())
    assert flagged[::7].all()


def test_clamped_tensor_round_trips(oracle):
    """unpack(pack(.)) projects onto the stored set: packing the projection
    raises no flag and reproduces it bit for bit, with identical planes."""
    from lossless_bit_weight_amd.inputs import TINY
    w_raw = TINY.weights_raw()
    p0, p1, p2, meta, bad = oracle.pack(w_raw)
    w = oracle.unpack(p0, p1, p2, meta, TINY.N, TINY.K)
    q0, q1, q2, qmeta, bad2 = oracle.pack(w)
    assert bad2 == 0
    assert np.array_equal(oracle.unpack(q0, q1, q2, qmeta, TINY.N, TINY.K), w)
    assert np.array_equal(q0, p0) and np.array_equal(q1, p1) and np.array_equal(q2, p2)
    assert np.array_equal(qmeta, meta & 0x7F)
    # Elements already stored exactly are untouched by the projection.
    same = w == w_raw
    assert same.mean() > 0.999


def test_special_values_round_trip(oracle):
    """+-0, subnormals, the smallest normals, +-Inf and NaN payloads survive
    when they share a group with compatible neighbours."""
    rows = []
    rows.append([0x0000, 0x8000, 0x0001, 0x807F, 0x0080, 0x80FF] + [0] * 122)
    rows.append([0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x7F81, 0x7900] + [0x7F00] * 122)
    rows.append([0x7F7F, 0xFF7F] + [0x0000] * 126)
    w = np.array(rows, dtype=np.uint16)
    p0, p1, p2, meta, bad = oracle.pack(w)
    assert bad == 0
    assert np.array_equal(oracle.unpack(p0, p1, p2, meta, 3, 128), w)
    assert list(oracle.meta_of(meta, 3, 128)[:, 0]) == [0, 120, 120]


def test_bf16_control_layout_is_the_same_permutation(oracle):
    """The BF16 control order places word (n, k) where the W12 planes place
    its nibbles: word index = 2 * (plane byte) + (nibble is high), read per
    1 KB sub-block -- checked by packing single marked weights."""
    N, K = 21, 256
    rng = np.random.default_rng(4)
    w = rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16)
    t = oracle.bf16_tile(w)
    assert t.shape == (oracle.padded_rows(N) * K,)
    assert sorted(t[t != 0].tolist()) == sorted(w[w != 0].tolist())
    for (n, k) in [(0, 0), (0, 7), (0, 8), (0, 32), (1, 0), (15, 127), (16, 128), (20, 255)]:
        marked = np.zeros((N, K), np.uint16)
        marked[n, k] = 0x3F81
        p0, _, _, _, _ = oracle.pack(marked)
        byte = int(np.flatnonzero(p0)[0])
        block, inblock = divmod(byte, 1024)
        lane, within = divmod(inblock, 16)
        b, j = divmod(within, 4)
        e = j + (4 if p0[byte] >= 16 else 0)
        assert t[block * 2048 + b * 512 + lane * 8 + e] == w[n, k], (n, k)


def read_layout_example2():
    """Records of tests/golden/w12_layout_example2.txt (hand-derived)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "w12_layout_example2.txt")
    rec = {"planted": [], "p0": {}, "p1": {}, "p2": {}, "meta": {}, "unpacked": [], "entry": []}
    with open(path) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            v = [int(s, 0) for s in t[1:]]
            if t[0] in ("p0", "p1", "p2", "meta"):
                rec[t[0]][v[0]] = v[1]
            elif t[0] in ("planted", "unpacked", "entry"):
                rec[t[0]].append(tuple(v))
            else:
                rec[t[0]] = v
    return rec


def layout_example2_weight():
    rec = read_layout_example2()
    w = np.zeros((21, 256), np.uint16)
    for n, k, v in rec["planted"]:
        w[n, k] = v
    return w, rec


def test_layout_worked_example2(oracle):
    """Second hand-derived example: a second tile and group, rows c > 0,
    quarters q > 0, dwords b > 0, high nibbles, a flagged group with two
    elements below its window, and the exception list they produce."""
    w, rec = layout_example2_weight()
    p0, p1, p2, meta, bad = oracle.pack(w)
    for name, plane in (("p0", p0), ("p1", p1), ("p2", p2)):
        assert plane.shape == (4096,)
        nz = {int(i): int(plane[i]) for i in np.flatnonzero(plane)}
        assert nz == rec[name], name
    assert meta.shape == (64,)
    assert {int(i): int(meta[i]) for i in np.flatnonzero(meta)} == rec["meta"]
    assert bad == rec["bad"][0]
    out = oracle.unpack(p0, p1, p2, meta, 21, 256)
    want = w.copy()
    for n, k, v in rec["unpacked"]:
        want[n, k] = v
    assert np.array_equal(out, want)
    off, ent = oracle.exceptions(w)
    assert list(off) == rec["offsets"]
    assert [tuple(int(v) for v in e) for e in ent] == rec["entry"]
