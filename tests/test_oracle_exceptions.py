"""Pins of the oracle's exception list (the escape path that makes every
group lossless): a hand-derived example, the set of listed positions equal to
the set where the plain container is lossy, and exact reconstruction."""
import os

import numpy as np
import pytest

from lossless_bit_weight_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w12_exceptions_example.txt")


def _golden():
    planted, offsets, entries = [], None, []
    with open(GOLDEN) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "planted":
                planted.append((int(t[1]), int(t[2]), int(t[3], 16)))
            elif t[0] == "offsets":
                offsets = [int(v) for v in t[1:]]
            elif t[0] == "entry":
                entries.append((int(t[1], 16), int(t[2], 16)))
    return planted, offsets, entries


def test_hand_derived_example(oracle):
    planted, offsets, entries = _golden()
    w = np.full((32, 256), 0x3F80, np.uint16)
    for n, k, v in planted:
        w[n, k] = v
    off, ent = oracle.exceptions(w)
    assert off.tolist() == offsets
    assert [tuple(e) for e in ent.tolist()] == entries


def _lossy_positions(oracle, w):
    p0, p1, p2, meta, _ = oracle.pack(w)
    back = oracle.unpack(p0, p1, p2, meta, *w.shape)
    return back, set(zip(*np.nonzero(back != w)))


@pytest.mark.parametrize("shape,sigma,seed", [((1024, 512), 0.02, 101), ((37, 384), 0.015, 7),
                                              ((130, 1152), 1.0, 8), ((16, 128), 1e-30, 9)])
def test_list_is_exactly_the_lossy_set(oracle, shape, sigma, seed):
    """Brute force: the listed positions are exactly the elements the clamped
    container does not reproduce, each with its original word, and writing
    them back restores the weight bit for bit."""
    w = inputs.inject_zeros(inputs.gaussian_bf16(shape, sigma, seed), 0.01, seed + 1)
    back, lossy = _lossy_positions(oracle, w)
    p0, p1, p2, meta, _ = oracle.pack(w)
    betas = oracle.meta_of(meta, *shape) & 0x7F
    off, ent = oracle.exceptions(w)
    N, K = shape
    G = K // 128
    assert len(off) == (N + 15) // 16 * G + 1
    listed = {}
    for t in range(len(off) - 1):
        for i in range(off[t], off[t + 1]):
            c, k = int(ent[i, 0]) >> 24, int(ent[i, 0]) & 0xFFFFFF
            assert k // 128 == t % G          # the entry lies in its block's group
            listed[(16 * (t // G) + c, k)] = int(ent[i, 1])
    assert set(listed) == lossy
    assert all(w[n, k] == v & 0xFFFF for (n, k), v in listed.items())
    # the base in each entry is the one the container holds for that group
    assert all(v >> 16 == betas[n, k // 128] for (n, k), v in listed.items())
    assert np.array_equal(oracle.apply_exceptions(back, off, ent), w)
    assert off[-1] == len(ent) and np.all(np.diff(off.astype(np.int64)) >= 0)


def test_storage_order_inside_tiles(oracle):
    w = inputs.gaussian_bf16((256, 1024), 0.02, 31)
    off, ent = oracle.exceptions(w)
    assert len(ent) > 40
    G = 1024 // 128
    for T in range(len(off) // G):
        keys = []
        for i in range(off[T * G], off[(T + 1) * G]):
            c, k = int(ent[i, 0]) >> 24, int(ent[i, 0]) & 0xFFFFFF
            r = k % 128
            keys.append((k // 128, 16 * ((r % 32) // 8) + c, r // 32, r % 8))
        assert keys == sorted(keys) and len(set(keys)) == len(keys)


def test_clamped_inputs_have_no_exceptions(oracle):
    w = inputs.TINY.weights_raw()
    p0, p1, p2, meta, bad = oracle.pack(w)
    assert bad > 0
    back = oracle.unpack(p0, p1, p2, meta, *w.shape)
    off, ent = oracle.exceptions(back)
    assert len(ent) == 0 and not off.any()


def test_long_k_rejected(oracle):
    lib = oracle._load()
    assert lib.w12o_exceptions(None, 0, 1 << 24, None, None) == -1
    assert lib.w12o_exceptions(None, 0, (1 << 24) - 128, None, None) == 0


def test_apply_rejects_an_entry_outside_its_block(oracle):
    """An entry listed under a block whose group does not hold its k is
    refused, not written."""
    w = np.full((16, 256), 0x3F80, np.uint16)
    w[3, 200] = 0x3000                      # group 1, below the window
    off, ent = oracle.exceptions(w)
    assert off.tolist() == [0, 0, 1]
    with pytest.raises(ValueError):
        oracle.apply_exceptions(w, np.array([0, 1, 1], np.uint32), ent)
