"""Pins of the oracle's rotation against textbook facts (CPU only)."""
import os

import numpy as np
import pytest
import scipy.linalg

import okv_synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy(d):
    # the OIQ report, Section 3.1: H_d is the normalised Hadamard matrix
    h = oracle.hadamard(d)
    ref = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.array_equal(h, ref)
    # idea card, Mathematical statement: H^T H = I; OIQ 3.1: self-inverse
    assert np.abs(h.T @ h - np.eye(d)).max() < 1e-14
    assert np.abs(h @ h - np.eye(d)).max() < 1e-14


@pytest.mark.parametrize("d", [4, 16, 128, 256])
def test_fwht_f32_close_to_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, d)).astype(np.float32)
    y = oracle.fwht_f32(x).astype(np.float64)
    ref = x.astype(np.float64) @ (scipy.linalg.hadamard(d) / np.sqrt(d)).T
    # each output is log2(d) float32 sums plus one multiply: error bound in units of |x|_2
    bound = (np.log2(d) + 2) * 2.0 ** -24 * np.linalg.norm(x, axis=1, keepdims=True) * np.sqrt(d)
    assert np.all(np.abs(y - ref) <= bound)


def test_fwht_f32_integer_inputs_exact():
    # with small integers every butterfly sum is exact; only the final c_d multiply rounds
    rng = np.random.default_rng(7)
    d = 128
    x = rng.integers(-1000, 1000, size=(20, d)).astype(np.float32)
    raw = x.astype(np.float64) @ scipy.linalg.hadamard(d).T      # exact integers
    y = oracle.fwht_f32(x)
    c = np.float32(1.0 / np.sqrt(128.0))
    assert c.view(np.uint32) == 0x3DB504F3
    assert np.array_equal(y, raw.astype(np.float32) * c)


def test_fwht_f32_stage_order_golden():
    # hand-derived float32 example that distinguishes the ascending stage order
    lines = dict(l.split(" : ") for l in open(os.path.join(GOLD, "fwht_order_d4.txt"))
                 if not l.startswith("#") and l.strip())
    x = np.array([int(t, 16) for t in lines["input"].split()], dtype=np.uint32).view(np.float32)
    want = np.array([int(t, 16) for t in lines["output"].split()], dtype=np.uint32)
    got = oracle.fwht_f32(x).view(np.uint32)
    assert np.array_equal(got, want)


def test_identity_and_ones_special_cases():
    d = 128
    u = oracle.rotation_matrix("sign", np.ones(d), d)
    # U e_j = column j of H/sqrt(d): every entry +-c_d
    h = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.allclose(u, h, atol=0, rtol=0)
    ones = np.ones(d, np.float32)
    y = oracle.rotate_f32(ones, "sign", np.ones(d, np.float32))
    e0 = np.zeros(d)
    e0[0] = np.sqrt(d)
    assert np.abs(y - e0).max() < 1e-6
    # FWHT of a constant vector is exact in float32 except the normalisation
    assert np.all(y[1:] == 0)


@pytest.mark.parametrize("name", ["tiny_d128_t256", "so4_d256_b32_t8k"])
def test_rotation_orthogonality_and_dot_invariance(name):
    wl = okv_synth.workload(name)
    p = okv_synth.rotation_params(wl)
    d = wl.d
    u = oracle.rotation_matrix(wl.rotation, p, d)
    # idea card, Mathematical statement: U^T U = I, (Uq).(Uk) = q.k
    assert np.abs(u.T @ u - np.eye(d)).max() < 1e-13
    rng = np.random.default_rng(1)
    q = rng.standard_normal((64, d))
    k = rng.standard_normal((64, d))
    lhs = np.sum((q @ u.T) * (k @ u.T), axis=1)
    rhs = np.sum(q * k, axis=1)
    assert np.abs(lhs - rhs).max() < 1e-12 * np.abs(rhs).max() + 1e-12
    if wl.rotation == "sign":
        assert np.array_equal(p * p, np.ones(d))          # D^2 = I
    else:
        r = p.reshape(d // 4, 4, 4)
        gram = np.einsum("bij,bik->bjk", r, r)
        assert np.abs(gram - np.eye(4)).max() < 1e-14     # R^T R = I
        assert np.abs(np.linalg.det(r) - 1.0).max() < 1e-13   # det R = +1


@pytest.mark.parametrize("name", ["tiny_d128_t256", "so4_d256_b32_t8k"])
def test_rotate_f32_matches_matrix(name):
    wl = okv_synth.workload(name)
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    u = oracle.rotation_matrix(wl.rotation, p32.astype(np.float64), wl.d)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((100, wl.d)) * 5).astype(np.float32)
    y = oracle.rotate_f32(x, wl.rotation, p32).astype(np.float64)
    ref = x.astype(np.float64) @ u.T
    scale = np.linalg.norm(x, axis=1, keepdims=True)
    assert np.all(np.abs(y - ref) <= 64 * 2.0 ** -24 * scale)


def test_so4_identity_quaternions():
    # qL = qR = 1 gives R = I: the SO(4) stage must then leave the transform alone
    d = 16
    r = np.tile(np.eye(4, dtype=np.float32), (d // 4, 1, 1))
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, d)).astype(np.float32)
    assert np.array_equal(oracle.rotate_f32(x, "so4", r), oracle.fwht_f32(x))


def test_so4_product_rounding_separate():
    # y_r = ((R_r0 x0 + R_r1 x1) + R_r2 x2) + R_r3 x3, each product and sum rounded
    # separately.  Hand-derived case: after the transform the vector is
    # [-1, 1 + 2^-12, 0, 0]; with R_00 = 1, R_01 = 1 + 2^-12 the product
    # (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 rounds (tie, to even) to 1 + 2^-11, so
    # y_0 = 2^-11, whereas a fused multiply-add would keep 2^-11 + 2^-24.
    e = 2.0 ** -13
    x = np.array([e, -1 - e, e, -1 - e], dtype=np.float32)
    assert np.array_equal(oracle.fwht_f32(x), np.array([-1, 1 + 2.0 ** -12, 0, 0], np.float32))
    r = np.zeros((1, 4, 4), np.float32)
    r[0] = np.eye(4, dtype=np.float32)
    r[0, 0, :] = [1.0, 1.0 + 2.0 ** -12, 0.0, 0.0]
    y = oracle.rotate_f32(x, "so4", r)
    assert y[0] == np.float32(2.0 ** -11)
    assert y[1] == np.float32(1 + 2.0 ** -12)
