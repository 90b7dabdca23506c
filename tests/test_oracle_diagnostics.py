"""Pins of the oracle's rotation-free variant and quality diagnostics (CPU only):
textbook Gini values, closed forms of block maxima under the Hadamard transform, and
zero attention error when the codes are exact."""
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.linalg

import oracle


def spec(**kw):
    base = dict(d=128, block=32, quant="sym", scale_dtype="f32", eps=0.0, rotation="none")
    base.update(kw)
    return SimpleNamespace(**base)


def test_gini_closed_forms():
    assert oracle.gini(np.full(50, 3.0)) == 0.0
    n = 40
    assert abs(oracle.gini(np.eye(1, n)[0]) - (n - 1) / n) < 1e-15
    # {1, 2, 3, 4}: sum over ordered pairs of |a_i - a_j| = 20, 2 n^2 mean = 80
    assert abs(oracle.gini([1.0, 2.0, 3.0, 4.0]) - 0.25) < 1e-15
    # sign and scale do not matter
    assert abs(oracle.gini([-1.0, 2.0, -3.0, 4.0]) - 0.25) < 1e-15
    assert abs(oracle.gini(np.array([1.0, 2.0, 3.0, 4.0]) * 7.5) - 0.25) < 1e-15


def test_gini_textbook_distributions():
    rng = np.random.default_rng(3)
    # Uniform(0, 1): G = 1/3; exponential: G = 1/2; half-normal: G = sqrt(2) - 1
    assert abs(oracle.gini(rng.random(400000)) - 1.0 / 3.0) < 3e-3
    assert abs(oracle.gini(rng.exponential(size=400000)) - 0.5) < 3e-3
    assert abs(oracle.gini(rng.standard_normal(400000)) - (np.sqrt(2.0) - 1.0)) < 3e-3


def test_block_max_of_hadamard_spike_and_constant():
    d, m = 128, 32
    ones = np.ones(d, np.float32)
    # H e_j has every entry +-1/sqrt(d): every block maximum is 1/sqrt(d)
    x = np.zeros(d, np.float32)
    x[9] = 2.0
    st = oracle.block_max_stats(oracle.rotate_f32(x, "sign", ones).astype(np.float64), m)
    assert abs(st["worst"] - 2.0 / np.sqrt(d)) < 1e-6 and abs(st["mean"] - 2.0 / np.sqrt(d)) < 1e-6
    assert abs(st["worst_over_rms"] - 1.0) < 1e-6
    # H of a constant vector c is a single spike sqrt(d) c at index 0
    st = oracle.block_max_stats(oracle.rotate_f32(np.full(d, 0.5, np.float32), "sign", ones), m)
    assert abs(st["worst"] - 0.5 * np.sqrt(d)) < 1e-5
    assert abs(st["mean"] - 0.5 * np.sqrt(d) / (d // m)) < 1e-5
    assert abs(st["worst_over_rms"] - np.sqrt(d)) < 1e-4


def test_rotation_none_is_identity():
    d = 128
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, d)).astype(np.float32)
    assert np.array_equal(oracle.rotate_f32(x, "none", None), x)
    assert np.array_equal(oracle.rotation_matrix("none", None, d), np.eye(d))
    # Hadamard only: the sign rotation with D = I is scipy's Hadamard matrix / sqrt(d)
    assert np.allclose(oracle.rotation_matrix("sign", np.ones(d), d), scipy.linalg.hadamard(d) / np.sqrt(d))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_attention_rel_rmse_zero_on_the_code_grid(bits):
    # rows whose blocks hold multiples of 0.5 in -L .. L with +-L present: with eps = 0
    # the scale is exactly 0.5, every value is a code, and the cache is lossless
    lev = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(bits)
    sp = spec(bits=bits)
    t, d, m = 70, 128, 32
    k = rng.integers(-lev, lev + 1, size=(t, d)).astype(np.float32)
    v = rng.integers(-lev, lev + 1, size=(t, d)).astype(np.float32)
    k[:, ::m] = lev
    v[:, ::m] = -lev
    k *= 0.5
    v *= 0.5
    q = rng.standard_normal((4, d)).astype(np.float32)
    assert oracle.attention_rel_rmse(q, k, v, sp, np.ones(d, np.float32)) < 1e-12


def test_attention_rel_rmse_scale_invariant():
    # exact power-of-two scaling of k and v by 2^j and q by 2^-j keeps the logits and
    # scales every code's scale by 2^j (eps = 0): the relative error is unchanged
    rng = np.random.default_rng(8)
    sp = spec(rotation="sign")
    p32 = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    k = rng.standard_normal((90, 128)).astype(np.float32)
    v = rng.standard_normal((90, 128)).astype(np.float32)
    q = rng.standard_normal((2, 128)).astype(np.float32)
    e0 = oracle.attention_rel_rmse(q, k, v, sp, p32)
    e1 = oracle.attention_rel_rmse(q / np.float32(8), k * np.float32(8), v * np.float32(8), sp, p32)
    assert e0 > 1e-3 and abs(e1 - e0) < 1e-12 * max(1.0, e0) * 1e3


def test_channel_gini_closed_forms():
    # equal channel RMS -> 0; one live channel of d -> (d - 1) / d
    x = np.zeros((10, 8))
    x[:, 3] = np.arange(10)
    assert abs(oracle.channel_gini(x) - 7.0 / 8.0) < 1e-15
    assert oracle.channel_gini(np.ones((5, 8)) * np.array([1, -1] * 4)) == 0.0


def test_rotation_disperses_outliers():
    # keys with a few large channels: the transform flattens the per-channel magnitudes
    # (the OIQ report, Section 6.1) and lowers the worst block maximum relative to the
    # RMS (the idea card's Verification); the elementwise magnitudes become those of a
    # Gaussian (Gini of |N(0,1)| = sqrt(2) - 1)
    import okv_synth
    wl = okv_synth.workload("mha_b4h32_t128k").with_(batch=1, hkv=1, hq=1)
    k, _ = okv_synth.kv_tokens(wl, 0, 2048)
    k = okv_synth.host_f32(k)[0, :, 0]
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    y = oracle.rotate_f32(k, "sign", p32)
    assert oracle.channel_gini(k) > 0.4 and oracle.channel_gini(y) < 0.05
    assert abs(oracle.gini(y) - (np.sqrt(2.0) - 1.0)) < 0.02
    assert oracle.block_max_stats(y, 32)["worst_over_rms"] < 0.5 * oracle.block_max_stats(k, 32)["worst_over_rms"]
