"""Pins of the oracle's SO(4) calibration (CPU only): quaternion rotations against
closed forms, the block error against hand values, recovery of a planted rotation,
and a non-increasing error trace."""
import numpy as np
import pytest

import okv_synth
import oracle


def test_quaternion_rotation_closed_forms():
    t = 0.37
    a = np.array([np.cos(t), np.sin(t), 0.0, 0.0])
    # x -> a x conj(a): fixes 1 and i, turns the (j, k) plane by 2t
    r = oracle.quat_rotation(a, a)
    want = np.eye(4)
    want[2:, 2:] = [[np.cos(2 * t), -np.sin(2 * t)], [np.sin(2 * t), np.cos(2 * t)]]
    assert np.allclose(r, want, atol=1e-15)
    # x -> a x (b = 1): the (1, i) and (j, k) planes both turn by t (isoclinic)
    r = oracle.quat_rotation(a, [1.0, 0.0, 0.0, 0.0])
    c, s = np.cos(t), np.sin(t)
    assert np.allclose(r, [[c, -s, 0, 0], [s, c, 0, 0], [0, 0, c, -s], [0, 0, s, c]], atol=1e-15)
    # i j = k, j i = -k (Hamilton)
    assert np.allclose(oracle.quat_mul([0, 1, 0, 0], [0, 0, 1, 0]), [0, 0, 0, 1])
    assert np.allclose(oracle.quat_mul([0, 0, 1, 0], [0, 1, 0, 0]), [0, 0, 0, -1])
    rng = np.random.default_rng(1)
    r = oracle.quat_rotation(rng.standard_normal(4), rng.standard_normal(4))
    assert np.allclose(r.T @ r, np.eye(4), atol=1e-14) and abs(np.linalg.det(r) - 1) < 1e-14


def test_block_error_by_hand():
    # one vector, B = I, H x = y with y = (1, 1/6, 0, ...) in block 0 (eps = 0, L = 3):
    # s = 1/3, y / s = (3, 1/2) -> codes (3, 0) (half to even), error (1/6)^2
    d = 128
    y = np.zeros((1, d))
    y[0, 0], y[0, 1] = 1.0, 1.0 / 6.0
    x = y @ oracle.hadamard(d)            # H is symmetric and orthogonal: H x = y
    rot = np.tile(np.eye(4), (d // 4, 1, 1))
    e = oracle.so4_block_errors(x, rot, 32, 0.0)
    assert abs(e[0] - 1.0 / 36.0) < 1e-13 and np.all(e[1:] < 1e-30)   # H round trip: ~1e-16
    # b = 2 (L = 1): s = 1, y / s = (1, 1/6) -> codes (1, 0): the same error
    assert abs(oracle.so4_block_errors(x, rot, 32, 0.0, bits=2)[0] - 1.0 / 36.0) < 1e-13


def test_planted_rotation_is_recovered():
    # In every quantisation block only group 8 b + 1 carries data, and there H x is
    # R_b^T g with g on the 3-bit grid (every vector has an entry at +-3 s0): with
    # R_b among the candidates (index 2) the search finds it and the error drops to 0
    # (the empty groups only hold the ~1e-17 residue of the transform round trip).
    d, m, n = 128, 32, 200
    rng = np.random.default_rng(5)
    planted = [oracle.quat_rotation(rng.standard_normal(4), rng.standard_normal(4)) for _ in range(d // m)]
    g = rng.integers(-3, 4, size=(n, d // m, 4)).astype(np.float64)
    g[:, :, 0] = 3.0 * np.where(rng.random((n, d // m)) < 0.5, -1.0, 1.0)
    hx = np.zeros((n, d))
    for b in range(d // m):
        grp = 8 * b + 1
        hx[:, 4 * grp:4 * grp + 4] = (g[:, b] * 0.25) @ planted[b]     # rows of R^T (s0 g)
    x = hx @ oracle.hadamard(d)
    cands = okv_synth.so4_candidates(d, 1, 4)
    for b in range(d // m):
        cands[0, 8 * b + 1, 2] = planted[b]
    rot0 = np.tile(np.eye(4), (d // 4, 1, 1))
    assert oracle.so4_total_error(x, rot0, m, 0.0) > 1.0
    rot, trace, choice = oracle.calibrate_so4(x, rot0, cands, m, 0.0)
    assert trace[-1] < 1e-20
    for b in range(d // m):
        assert choice[0, 8 * b + 1] == 2 and np.allclose(rot[8 * b + 1], planted[b], atol=1e-15)


def test_trace_never_increases_and_total_splits():
    wl = okv_synth.workload("so4_d256_b32_t8k").with_(batch=1, hkv=1, hq=1)
    k, _ = okv_synth.kv_tokens(wl, 0, 256)
    x = okv_synth.host_f32(k)[0, :, 0]
    rot0 = okv_synth.rotation_params(wl)
    cands = okv_synth.so4_candidates(256, 2, 6)
    rot, trace, _ = oracle.calibrate_so4(x, rot0, cands, 32, 1e-6)
    assert np.all(np.diff(trace) <= 0) and trace[-1] < trace[0]
    assert abs(oracle.so4_total_error(x, rot, 32, 1e-6) - trace[-1]) < 1e-9 * trace[-1]
    assert np.allclose(np.einsum("gij,gkj->gik", rot, rot), np.eye(4), atol=1e-12)
