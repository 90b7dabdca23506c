"""Pins of the oracle's 3-bit packing (CPU only)."""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    onehot, patterns = [], {}
    for line in open(os.path.join(GOLD, "pack_g32_onehot.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, body = line.split(" : ")
        if head.startswith("all"):
            patterns[head] = bytes.fromhex(body.replace(" ", ""))
            continue
        val, idx = map(int, head.split())
        want = np.zeros(12, np.uint8)
        for item in body.split():
            b, h = item.split("=")
            want[int(b)] = int(h, 16)
        onehot.append((val, idx, want))
    return onehot, patterns


ONEHOT, PATTERNS = _golden()


@pytest.mark.parametrize("val,idx,want", ONEHOT)
def test_pack_g32_onehot_golden(val, idx, want):
    e = np.zeros(32, np.uint8)
    e[idx] = val
    assert np.array_equal(oracle.pack_g32(e), want)


@pytest.mark.parametrize("name,val", [("all7", 7), ("all0", 0), ("all4", 4), ("all3", 3)])
def test_pack_g32_patterns_golden(name, val):
    e = np.full(32, val, np.uint8)
    assert oracle.pack_g32(e).tobytes() == PATTERNS[name]


def test_pack_g32_every_position_every_value_round_trip():
    for i in range(32):
        for v in range(8):
            e = np.zeros(32, np.uint8)
            e[i] = v
            assert np.array_equal(oracle.unpack_g32(oracle.pack_g32(e)), e)


def test_pack_g32_bits_are_a_bijection():
    pos = oracle.G32_BIT_POSITIONS
    assert sorted(pos.ravel().tolist()) == list(range(96))


def test_pack_g32_random_round_trip_and_linearity():
    rng = np.random.default_rng(0)
    e = rng.integers(0, 8, size=(200000, 32)).astype(np.uint8)
    g = oracle.pack_g32(e)
    assert g.shape == (200000, 12)
    assert np.array_equal(oracle.unpack_g32(g), e)
    # packing is bitwise linear: OR of disjoint one-hot packings equals the packing
    e2 = e[:1000]
    acc = np.zeros((1000, 12), np.uint8)
    for i in range(32):
        one = np.zeros_like(e2)
        one[:, i] = e2[:, i]
        acc |= oracle.pack_g32(one)
    assert np.array_equal(acc, oracle.pack_g32(e2))


def test_rows_and_tiles_round_trip():
    rng = np.random.default_rng(1)
    for d in (128, 256):
        u = rng.integers(0, 8, size=(77, d)).astype(np.uint8)
        r = oracle.pack_rows(u)
        assert r.shape == (77, 3 * d // 8)
        assert np.array_equal(oracle.unpack_rows(r, d), u)
        t = oracle.pack_vtiles(u)
        assert t.shape == (3, d, 12)
        assert np.array_equal(oracle.unpack_vtiles(t, 77), u)
        # the slots of tokens 77..95 in the last tile hold code 0
        full = oracle.unpack_vtiles(t, 96)
        assert np.all(full[77:] == 0)
        # tile tau, dim j holds the 32 codes of tokens 32 tau .. 32 tau + 31 in dim j
        assert np.array_equal(oracle.unpack_g32(t[1, 5]), u[32:64, 5])
        # row group g holds dims 32 g .. 32 g + 31
        assert np.array_equal(oracle.unpack_g32(r[10, 12:24]), u[10, 32:64])
