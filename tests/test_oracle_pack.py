"""Pins of the oracle's b-bit packing (CPU only): hand-typed golden tables for
b = 2, 3, 4, round trips and the bit bijection."""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name="pack_g32_onehot.txt", nbytes=12):
    onehot, patterns = [], {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, body = line.split(" : ")
        if head.startswith("all"):
            patterns[head] = bytes.fromhex(body.replace(" ", ""))
            continue
        val, idx = map(int, head.split())
        want = np.zeros(nbytes, np.uint8)
        for item in body.split():
            b, h = item.split("=")
            want[int(b)] = int(h, 16)
        onehot.append((val, idx, want))
    return onehot, patterns


ONEHOT, PATTERNS = _golden()
GOLDEN_B = {2: _golden("pack_g32_onehot_b2.txt", 8), 4: _golden("pack_g32_onehot_b4.txt", 16)}


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


@pytest.mark.parametrize("bits,val,idx,want", [(b, *row) for b in (2, 4) for row in GOLDEN_B[b][0]])
def test_pack_b_onehot_golden(bits, val, idx, want):
    e = np.zeros(32, np.uint8)
    e[idx] = val
    assert np.array_equal(oracle.pack_g32(e, bits), want)
    assert np.array_equal(oracle.unpack_g32(want, bits), e)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_b_patterns_golden(bits):
    for name, want in GOLDEN_B[bits][1].items():
        e = np.full(32, int(name[3:]), np.uint8)
        assert oracle.pack_g32(e, bits).tobytes() == want


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_b_bijection_round_trip_and_range(bits):
    pos = oracle.group_bit_positions(bits)
    assert pos.shape == (32, bits)
    assert sorted(pos.ravel().tolist()) == list(range(32 * bits))
    assert oracle.group_bytes(bits) == 4 * bits
    rng = np.random.default_rng(bits)
    e = rng.integers(0, 2 ** bits, size=(20000, 32)).astype(np.uint8)
    g = oracle.pack_g32(e, bits)
    assert g.shape == (20000, 4 * bits)
    assert np.array_equal(oracle.unpack_g32(g, bits), e)
    with pytest.raises(ValueError):
        oracle.pack_g32(np.full(32, 2 ** bits, np.uint8), bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_b_byte_lanes(bits):
    # byte j of unpacked word k holds code 4 k + j: word k of the group masked to the
    # field of codes 4 k .. 4 k + 3 gives them in byte lanes
    rng = np.random.default_rng(7)
    e = rng.integers(0, 2 ** bits, size=32).astype(np.uint8)
    words = np.frombuffer(oracle.pack_g32(e, bits).tobytes(), dtype="<u4")
    mask = (2 ** bits - 1) * 0x01010101
    per_word = 32 // bits
    for k in range(8):
        w, f = divmod(k, per_word // 4)
        lanes = (int(words[w]) >> (bits * f)) & mask
        assert [(lanes >> (8 * j)) & 0xFF for j in range(4)] == list(e[4 * k:4 * k + 4])


@pytest.mark.parametrize("bits", [2, 4])
def test_rows_and_tiles_round_trip_b(bits):
    rng = np.random.default_rng(3)
    d = 128
    u = rng.integers(0, 2 ** bits, size=(45, d)).astype(np.uint8)
    r = oracle.pack_rows(u, bits)
    assert r.shape == (45, bits * d // 8)
    assert np.array_equal(oracle.unpack_rows(r, d, bits), u)
    t = oracle.pack_vtiles(u, bits)
    assert t.shape == (2, d, 4 * bits)
    assert np.array_equal(oracle.unpack_vtiles(t, 45, bits), u)
    assert np.array_equal(oracle.unpack_g32(t[1, 9], bits)[:13], u[32:45, 9])
    assert np.all(oracle.unpack_g32(t[1, 9], bits)[13:] == 0)
