"""Pins of the oracle's storage formats and quantiser (CPU only)."""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle


def spec(**kw):
    base = dict(d=128, block=32, quant="sym", scale_dtype="f32", eps=1e-6, rotation="sign")
    base.update(kw)
    return SimpleNamespace(**base)


def rne_fraction(y, s, lo, hi):
    """Round-half-even of the exact rational y/s, clipped (brute force)."""
    if s == 0:
        return 0
    q = Fraction(float(y)) / Fraction(float(s))
    f = q.numerator // q.denominator
    rem = q - f
    if rem > Fraction(1, 2):
        f += 1
    elif rem == Fraction(1, 2):
        f += f % 2
    return max(lo, min(hi, f))


@pytest.mark.parametrize("s", [np.float32(1.0), np.float32(0.337), np.float32(np.float16(0.0123)),
                               np.float32(3.3333333e-7), np.float32(17.25)])
def test_rne_codes_brute_force_near_thresholds(s):
    # every float32 within 40 ulps of each rounding threshold (k + 1/2) s, plus the
    # thresholds themselves where representable, against exact rational rounding
    ys = []
    for k in range(-5, 5):
        t = np.float32((k + 0.5) * np.float64(s))
        for n in range(-40, 41):
            ys.append(np.nextafter(t, np.float32(np.inf) if n > 0 else np.float32(-np.inf)) if n else t)
            t2 = t
            for _ in range(abs(n)):
                t2 = np.nextafter(t2, np.float32(np.inf) if n > 0 else np.float32(-np.inf))
            ys.append(t2)
    ys = np.array(ys, dtype=np.float32)
    for lo, hi in ((-3, 3), (0, 7)):
        got = oracle.rne_codes(ys[None, :], np.array([s], np.float32), lo, hi)[0]
        want = np.array([rne_fraction(y, s, lo, hi) for y in ys])
        assert np.array_equal(got, want)


def test_rne_codes_exact_ties_go_even():
    s = np.float32(0.75)
    y = np.array([[(k + 0.5) * 0.75 for k in range(-4, 4)]], dtype=np.float32)
    got = oracle.rne_codes(y, np.array([s]), -3, 3)[0]
    # -3.5 -> -3 (clip of -4), -2.5 -> -2, -1.5 -> -2, -0.5 -> 0, 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 3 (clip of 4)
    assert list(got) == [-3, -2, -2, 0, 0, 2, 2, 3]


def test_rne_codes_random_against_fraction():
    rng = np.random.default_rng(11)
    s = np.float32(0.0421)
    y = (rng.standard_normal(3000) * 0.1).astype(np.float32)
    got = oracle.rne_codes(y[None], np.array([s]), -3, 3)[0]
    want = [rne_fraction(v, s, -3, 3) for v in y]
    assert list(got) == want


def test_f16_store_ieee_cases():
    vals = np.array([65504.0, 65519.0, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 1 + 2.0 ** -11,
                     1 + 3 * 2.0 ** -11], dtype=np.float32)
    want = np.array([65504.0, 65504.0, np.inf, 2.0 ** -24, 0.0, 2.0 ** -23, 1.0, 1 + 2.0 ** -9])
    assert np.array_equal(oracle.f16_store(vals).astype(np.float64), want)


def test_e4m3_decode_all_patterns_match_torch():
    bits = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(bits)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_below_464():
    rng = np.random.default_rng(5)
    # every representable value, every midpoint and its float32 neighbours, plus random
    reps = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (reps[:-1] + reps[1:]) / 2
    pts = [reps, mids]
    for v in mids.astype(np.float32):
        pts.append(np.array([np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1e9))]))
    pts.append(np.exp(rng.uniform(np.log(1e-5), np.log(460), 200000)))
    x = np.concatenate(pts).astype(np.float32)
    x = x[x < 464]
    x = np.concatenate([x, -x])
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturation_rule():
    x = np.array([448, 460, 463.9, 464, 480, 1000, np.inf, -1000, -np.inf, np.nan], np.float32)
    got = oracle.e4m3_encode(x)
    assert list(got[:7]) == [0x7E] * 7
    assert list(got[7:9]) == [0xFE, 0xFE]
    assert got[9] == 0x7F


def test_sym_unit_vector_codes_are_pm3_with_hadamard_signs():
    # U = H (D = I): U e_j has every entry +-1/sqrt(d); each block max codes to +-3
    d = 128
    sp = spec()
    h = scipy.linalg.hadamard(d)
    for j in (0, 5, 77):
        x = np.zeros(d, np.float32)
        x[j] = 1.0
        y = oracle.rotate_f32(x, "sign", np.ones(d, np.float32))
        u, _ = oracle.quantize_f32(y, sp)
        c = u.astype(int) - 4
        assert np.array_equal(c, 3 * h[:, j])


def test_sym_constant_vector():
    d = 128
    sp = spec()
    x = np.full(d, 0.25, np.float32)
    y = oracle.rotate_f32(x, "sign", np.ones(d, np.float32))
    u, meta = oracle.quantize_f32(y, sp)
    c = u.astype(int) - 4
    want = np.zeros(d, int)
    want[0] = 3
    assert np.array_equal(c, want)
    # blocks of zeros get the eps scale: RN32(RN32(0 + eps) / 3)
    assert meta[1] == np.float32(np.float32(1e-6) / np.float32(3))


@pytest.mark.parametrize("sdt", ["f32", "f16"])
def test_sym_block_max_and_error_bound(sdt):
    rng = np.random.default_rng(9)
    sp = spec(scale_dtype=sdt)
    y = (rng.standard_normal((500, 128)) * rng.lognormal(0, 1, (500, 1))).astype(np.float32)
    u, meta = oracle.quantize_f32(y, sp)
    c = (u.astype(int) - 4).reshape(500, 4, 32)
    yb = y.reshape(500, 4, 32)
    s = np.asarray(meta).astype(np.float64)
    # the element at the block maximum codes to +-3
    arg = np.abs(yb).argmax(-1)
    cm = np.take_along_axis(c, arg[..., None], -1)[..., 0]
    ym = np.take_along_axis(yb, arg[..., None], -1)[..., 0]
    assert np.all(cm == 3 * np.sign(ym))
    # no clipping happens: |y - s c| <= s / 2 for every element
    err = np.abs(yb - s[..., None] * c)
    assert np.all(err <= s[..., None] / 2)
    # scale formula
    s32 = (np.abs(yb).max(-1) + np.float32(1e-6)) / np.float32(3)
    if sdt == "f32":
        assert np.array_equal(meta, s32)
    else:
        assert np.array_equal(meta, s32.astype(np.float16))


def test_sym_scale_equivariance_eps0():
    # with eps = 0, Q(2^k x) has the same codes and scales times 2^k exactly: the
    # exact form of "reconstruction error scales with the amplitude squared"
    rng = np.random.default_rng(12)
    sp = spec(eps=0.0)
    y = rng.standard_normal((200, 128)).astype(np.float32)
    u0, m0 = oracle.quantize_f32(y, sp)
    for k in (-6, -1, 3, 10):
        u1, m1 = oracle.quantize_f32(y * np.float32(2.0 ** k), sp)
        assert np.array_equal(u0, u1)
        assert np.array_equal(m1, m0 * np.float32(2.0 ** k))
        e0 = oracle.dequantize(u0, m0, sp) - y
        e1 = oracle.dequantize(u1, m1, sp) - y * 2.0 ** k
        assert np.allclose(np.mean(e1 ** 2), np.mean(e0 ** 2) * 4.0 ** k, rtol=1e-12)


def test_sym_zero_block_eps0_all_codes_zero():
    sp = spec(eps=0.0)
    y = np.zeros((1, 128), np.float32)
    u, meta = oracle.quantize_f32(y, sp)
    assert np.all(u == 4) and np.all(meta == 0)


def test_asym_small_example_by_hand():
    # block of 64 values 0, 1, ..., 63 (all exact): min 0, max 63
    # s = RN32(63 / 7) = 9 -> E4M3 9 = 1.125 * 8 exactly; z = 0
    # u_j = rne(j / 9) for j = 0..63: 4/9 -> 0, 5/9 -> 1, 13/9 -> 1, 14/9 -> 2, 63/9 -> 7
    sp = spec(quant="asym", block=64, scale_dtype="e4m3", eps=0.0)
    y = np.tile(np.arange(64, dtype=np.float32), 2)[None]
    u, meta = oracle.quantize_f32(y, sp)
    assert meta.shape == (1, 2, 2)
    assert oracle.e4m3_decode(meta[0, 0, 0]) == 9.0 and oracle.e4m3_decode(meta[0, 0, 1]) == 0.0
    want = [rne_fraction(j, 9.0, 0, 7) for j in range(64)]
    assert list(u[0, :64]) == want
    assert u[0, 4] == 0 and u[0, 5] == 1 and u[0, 13] == 1 and u[0, 14] == 2 and u[0, 40] == 4
    assert u[0, 63] == 7


def asym_pin_block():
    """A hand-worked 128-value vector for the asymmetric quantiser (block 64, E4M3
    scale and zero-point), the news item's third paragraph: unsigned codes with a
    scale and a zero-point per 64-element sub-block, both in FP8.

    Block 0: minimum -1.03125 (not an E4M3 value: it stores as -1.0), maximum
    7.28125, so max - min = 8.3125 and (max - min) / 7 = 1.1875 exactly, the midpoint
    of the E4M3 neighbours 1.125 (mantissa 001) and 1.25 (mantissa 010): the tie goes
    to the even mantissa, s = 1.25.  Taking the stored zero-point -1.0 in place of the
    minimum would give 8.28125 / 7 = 1.183 -> 1.125 instead.
    Codes u = rne(RN32(y + 1.0) / 1.25), clipped to 0..7:
      -1.03125 -> t = -0.03125 -> 0;   7.28125 -> t = 8.28125, 6.625 -> 7;
      2.125 -> t = 3.125, 2.5 (tie) -> 2;   3.375 -> t = 4.375, 3.5 (tie) -> 4;
      -0.375 -> t = 0.625, 0.5 (tie) -> 0;   7.125 -> t = 8.125, 6.5 (tie) -> 6;
      -0.375 + 2^-25 -> t = 0.625 + 2^-25 is halfway between two float32 values and
        rounds to even, t = 0.625, so 0.5 (tie) -> 0; without the float32 rounding of
        y - z the quotient would exceed 0.5 and give 1;
      ramp y = -1 + j / 8 (j = 0..56) -> t = j / 8, u = rne(j / 10):
        j 0-5 -> 0 (j = 5 a tie), 6-14 -> 1, 15-25 -> 2 (15, 25 ties), 26-34 -> 3,
        35-45 -> 4 (35, 45 ties), 46-54 -> 5, 55-56 -> 6 (55 a tie).
    With the raw minimum as the zero-point every tie above moves (e.g. 2.125 -> 3).
    Block 1: 64 x (-0.3): max - min = 0, so s = 0 and every code is 0; z = E4M3(-0.3)
    = -0.3125 (neighbours 0.28125 and 0.3125 in the binade of spacing 1/32).
    E4M3 bytes: 1.25 = 0 0111 010 = 0x3A, -1.0 = 1 0111 000 = 0xB8, 0 = 0x00,
    -0.3125 = 1 0101 010 = 0xAA.
    """
    special = np.array([-1.03125, 7.28125, 2.125, 3.375, -0.375, 7.125,
                        np.float32(-0.375) + np.float32(2.0 ** -25)], np.float32)
    ramp = (np.float32(-1.0) + np.float32(0.125) * np.arange(57, dtype=np.float32)).astype(np.float32)
    y = np.empty(128, np.float32)
    y[:64] = np.concatenate([special, ramp])
    y[64:] = np.float32(-0.3)
    codes0 = [0, 7, 2, 4, 0, 6, 0] + [0] * 6 + [1] * 9 + [2] * 11 + [3] * 9 + [4] * 11 + [5] * 9 + [6] * 2
    codes = codes0 + [0] * 64
    meta = [[0x3A, 0xB8], [0x00, 0xAA]]
    return y, codes, meta


def test_asym_zero_point_block_by_hand():
    y, codes, meta_want = asym_pin_block()
    assert float(y[6]) == -0.375 + 2.0 ** -25        # exact in float32
    sp = spec(quant="asym", block=64, scale_dtype="e4m3", eps=0.0, rotation="none")
    u, meta = oracle.quantize_f32(y[None], sp)
    assert meta.tolist() == [meta_want]
    assert u[0].tolist() == codes
    # reconstruction uses the stored pair: s u + z
    xh = oracle.dequantize(u, meta, sp)[0]
    assert xh[0] == -1.0 and xh[1] == 7.75 and xh[2] == 1.5 and np.all(xh[64:] == -0.3125)


def test_asym_codes_range_and_reconstruction():
    rng = np.random.default_rng(13)
    sp = spec(quant="asym", block=64, scale_dtype="e4m3", eps=0.0)
    y = (rng.standard_normal((300, 128)) * 0.7 + 0.2).astype(np.float32)
    u, meta = oracle.quantize_f32(y, sp)
    assert u.max() <= 7
    s = oracle.e4m3_decode(meta[..., 0]).astype(np.float64)
    z = oracle.e4m3_decode(meta[..., 1]).astype(np.float64)
    xh = oracle.dequantize(u, meta, sp).reshape(300, 2, 64)
    assert np.allclose(xh, u.reshape(300, 2, 64) * s[..., None] + z[..., None])
    # z is the block minimum to E4M3 precision
    mn = y.reshape(300, 2, 64).min(-1)
    assert np.all(np.abs(z - mn) <= np.abs(mn) * 2.0 ** -4 + 2.0 ** -10)


# ---- code widths b = 2 and 4 (the idea card's quantiser with b symbolic:
# s = (max |x| + eps) / (2^(b-1) - 1), codes clipped to +-(2^(b-1) - 1))

@pytest.mark.parametrize("lo,hi", [(-1, 1), (0, 3), (-7, 7), (0, 15)])
def test_rne_codes_brute_force_other_widths(lo, hi):
    s = np.float32(0.3125)
    ys = []
    for k in range(lo - 2, hi + 2):
        t = np.float32((k + 0.5) * np.float64(s))
        ys.append(t)
        for n in (1, 2, 7):
            up, dn = t, t
            for _ in range(n):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            ys += [up, dn]
    ys = np.array(ys, dtype=np.float32)
    got = oracle.rne_codes(ys[None, :], np.array([s], np.float32), lo, hi)[0]
    assert list(got) == [rne_fraction(y, s, lo, hi) for y in ys]


@pytest.mark.parametrize("bits,lev", [(2, 1), (4, 7)])
def test_sym_unit_vector_codes_b(bits, lev):
    d = 128
    sp = spec(bits=bits)
    h = scipy.linalg.hadamard(d)
    for j in (0, 33, 127):
        x = np.zeros(d, np.float32)
        x[j] = 1.0
        y = oracle.rotate_f32(x, "sign", np.ones(d, np.float32))
        u, meta = oracle.quantize_f32(y, sp)
        assert np.array_equal(u.astype(int) - 2 ** (bits - 1), lev * h[:, j])
        # s = RN32(RN32(1/sqrt(d) + eps) / lev)
        want = (np.float32(oracle.c_norm_f32(d)) + np.float32(1e-6)) / np.float32(lev)
        assert np.all(meta == want)


@pytest.mark.parametrize("bits", [2, 4])
def test_sym_block_max_and_error_bound_b(bits):
    lev = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(20 + bits)
    sp = spec(bits=bits, scale_dtype="f16")
    y = (rng.standard_normal((400, 128)) * rng.lognormal(0, 1, (400, 1))).astype(np.float32)
    u, meta = oracle.quantize_f32(y, sp)
    assert u.min() >= 1 and u.max() <= 2 ** bits - 1
    c = (u.astype(int) - 2 ** (bits - 1)).reshape(400, 4, 32)
    yb = y.reshape(400, 4, 32)
    s = np.asarray(meta).astype(np.float64)
    arg = np.abs(yb).argmax(-1)
    cm = np.take_along_axis(c, arg[..., None], -1)[..., 0]
    ym = np.take_along_axis(yb, arg[..., None], -1)[..., 0]
    assert np.all(cm == lev * np.sign(ym))
    assert np.all(np.abs(yb - s[..., None] * c) <= s[..., None] / 2)
    s32 = (np.abs(yb).max(-1) + np.float32(1e-6)) / np.float32(lev)
    assert np.array_equal(meta, s32.astype(np.float16))
    # meta_values: x_hat = s (u - 2^(b-1))
    xh = oracle.dequantize(u, meta, sp).reshape(400, 4, 32)
    assert np.array_equal(xh, s[..., None] * c)


def test_asym_small_example_by_hand_b4():
    # block of 64 values 0..63: s = RN32(63 / 15) = 4.2 -> E4M3 4.0 (the neighbours
    # are 4.0 and 4.5); z = 0; u_j = rne(j / 4) clipped to 15: 2/4 -> 0 (tie, even),
    # 6/4 -> 2, 10/4 -> 2, 59/4 -> 15 (14.75), 63/4 -> 16 -> clip 15
    sp = spec(quant="asym", block=64, scale_dtype="e4m3", eps=0.0, bits=4)
    y = np.tile(np.arange(64, dtype=np.float32), 2)[None]
    u, meta = oracle.quantize_f32(y, sp)
    assert oracle.e4m3_decode(meta[0, 0, 0]) == 4.0 and oracle.e4m3_decode(meta[0, 0, 1]) == 0.0
    assert list(u[0, :64]) == [rne_fraction(j, 4.0, 0, 15) for j in range(64)]
    assert (u[0, 2], u[0, 6], u[0, 10], u[0, 59], u[0, 63]) == (0, 2, 2, 15, 15)


def test_asym_small_example_by_hand_b2():
    # s = RN32(63 / 3) = 21 -> E4M3: 21 lies halfway between 20 (mantissa 010) and
    # 22 (mantissa 011), ties to even -> 20; u_j = rne(j / 20) clipped to 3:
    # 10 -> 0 (tie), 29 -> 1, 30 -> 2 (tie), 31 -> 2, 50 -> 2 (tie), 63 -> 3
    sp = spec(quant="asym", block=64, scale_dtype="e4m3", eps=0.0, bits=2)
    y = np.tile(np.arange(64, dtype=np.float32), 2)[None]
    u, meta = oracle.quantize_f32(y, sp)
    assert oracle.e4m3_decode(meta[0, 0, 0]) == 20.0
    assert list(u[0, :64]) == [rne_fraction(j, 20.0, 0, 3) for j in range(64)]
    assert (u[0, 10], u[0, 29], u[0, 30], u[0, 31], u[0, 50], u[0, 63]) == (0, 1, 2, 2, 2, 3)


def test_more_bits_less_error():
    # same rotated data: reconstruction error falls with b (one code step is 2 s / ...)
    rng = np.random.default_rng(31)
    y = (rng.standard_normal((300, 128)) * 0.5).astype(np.float32)
    errs = []
    for bits in (2, 3, 4):
        sp = spec(bits=bits)
        u, meta = oracle.quantize_f32(y, sp)
        errs.append(np.mean((oracle.dequantize(u, meta, sp) - y) ** 2))
    assert errs[0] > 2 * errs[1] > 4 * errs[2]


def test_bits_validation():
    with pytest.raises(ValueError):
        oracle.quantize_f32(np.zeros((1, 128), np.float32), spec(bits=5))
