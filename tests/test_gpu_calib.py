"""GPU parity of the SO(4) calibration (okv_so4_eval, okv_so4_calibrate) against the
oracle's coordinate search.  Errors within 1e-5 relative (float32 against float64);
the search makes the same choices; planted rotations are recovered.  Every call goes
through the C ABI."""
import numpy as np
import pytest
import torch

import okv_synth
import oracle
from okv_parity import say

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def keys(name, t):
    wl = okv_synth.workload(name).with_(batch=1, hkv=1, hq=1)
    k, _ = okv_synth.kv_tokens(wl, 0, t)
    return wl, okv_synth.host_f32(k)[0, :, 0]


@pytest.mark.parametrize("d,block,bits", [(256, 32, 3), (128, 64, 3), (128, 32, 4), (256, 128, 2)])
def test_so4_eval_matches_oracle(d, block, bits):
    _need_gpu()
    import decode_attention_okv_amd as okv
    wl, x = keys("so4_d256_b32_t8k" if d == 256 else "mha_b4h32_t128k", 1500)
    x = x[:, :d]
    rot = okv_synth.rotation_params(wl.with_(d=d, rotation="so4"))
    cand = okv_synth.so4_candidates(d, 1, 12)[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    hx = x.astype(np.float64) @ oracle.hadamard(d).T
    for group in (0, 5, d // 4 - 1):
        say("okv_so4_eval", d, block, bits, "group", group)
        got = okv.so4_eval(xd, rot, cand[group], group, block=block, bits=bits, eps=1e-6)
        want = [oracle.okv_calib._block_error(hx, rot, block, 4 * group // block, 1e-6, bits,
                                              (group, cand[group, c] @ rot[group])) for c in range(12)]
        assert np.allclose(got, want, rtol=1e-5, atol=0), (group, got, want)


def test_so4_calibrate_recovers_planted_rotations():
    _need_gpu()
    import decode_attention_okv_amd as okv
    d, m, n = 128, 32, 3000
    rng = np.random.default_rng(5)
    planted = [oracle.quat_rotation(rng.standard_normal(4), rng.standard_normal(4)) for _ in range(d // m)]
    g = rng.integers(-3, 4, size=(n, d // m, 4)).astype(np.float64)
    g[:, :, 0] = 3.0 * np.where(rng.random((n, d // m)) < 0.5, -1.0, 1.0)
    hx = np.zeros((n, d))
    for b in range(d // m):
        grp = 8 * b + 1
        hx[:, 4 * grp:4 * grp + 4] = (g[:, b] * 0.25) @ planted[b]
    x = (hx @ oracle.hadamard(d)).astype(np.float32)
    cand = okv_synth.so4_candidates(d, 1, 4)
    for b in range(d // m):
        cand[0, 8 * b + 1, 2] = planted[b]
    rot0 = np.tile(np.eye(4), (d // 4, 1, 1))
    say("okv_so4_calibrate planted")
    rot, trace = okv.so4_calibrate(torch.from_numpy(x).cuda(), rot0, cand, block=m, bits=3, eps=0.0)
    say("planted trace", trace)
    assert trace[0] > 1.0 and trace[-1] < 1e-6 * trace[0]
    for b in range(d // m):
        assert np.allclose(rot[8 * b + 1], planted[b], atol=1e-6)


def test_so4_calibrate_applies_non_identity_candidate_zero():
    """Candidate 0 need not be the identity: the planted rotations sit at candidate 0
    of their groups (no identity among those candidates), win, and are applied, as the
    oracle's search applies every winner."""
    _need_gpu()
    import decode_attention_okv_amd as okv
    d, m, n = 128, 32, 2000
    rng = np.random.default_rng(11)
    planted = [oracle.quat_rotation(rng.standard_normal(4), rng.standard_normal(4)) for _ in range(d // m)]
    g = rng.integers(-3, 4, size=(n, d // m, 4)).astype(np.float64)
    g[:, :, 0] = 3.0 * np.where(rng.random((n, d // m)) < 0.5, -1.0, 1.0)
    hx = np.zeros((n, d))
    for b in range(d // m):
        grp = 8 * b + 2
        hx[:, 4 * grp:4 * grp + 4] = (g[:, b] * 0.25) @ planted[b]
    x = (hx @ oracle.hadamard(d)).astype(np.float32)
    cand = okv_synth.so4_candidates(d, 1, 4)
    for b in range(d // m):
        cand[0, 8 * b + 2, 0] = planted[b]
    rot0 = np.tile(np.eye(4), (d // 4, 1, 1))
    say("okv_so4_calibrate non-identity candidate 0")
    rot, trace = okv.so4_calibrate(torch.from_numpy(x).cuda(), rot0, cand, block=m, bits=3, eps=0.0)
    rot_o, trace_o, choice = oracle.calibrate_so4(x, rot0, cand, m, 0.0, 3)
    for b in range(d // m):
        assert choice[0, 8 * b + 2] == 0
        assert np.allclose(rot_o[8 * b + 2], planted[b], atol=1e-12)
    assert np.allclose(rot, rot_o, atol=1e-6)
    assert np.allclose(trace, trace_o, rtol=2e-5, atol=1e-9 * trace_o[0])


# The search runs step k of every quantisation block in one launch: block 4 (one group
# per block, 32 blocks at once), block = head_dim (one block of 32 or 64 groups), a
# vector count that leaves a partial chunk, and 70 candidates (two candidate tiles).
@pytest.mark.parametrize("name,d,block,bits,n,n_cand", [
    ("so4_d256_b32_t8k", 256, 32, 3, 1024, 8),
    ("mha_b4h32_t128k", 128, 32, 4, 1024, 8),
    ("mha_b4h32_t128k", 128, 4, 3, 1000, 8),
    ("mha_b4h32_t128k", 128, 128, 3, 777, 70),
    ("so4_d256_b32_t8k", 256, 256, 3, 1000, 8),
])
def test_so4_calibrate_matches_oracle(name, d, block, bits, n, n_cand):
    _need_gpu()
    import decode_attention_okv_amd as okv
    wl, x = keys(name, n)
    rot0 = okv_synth.rotation_params(wl.with_(rotation="so4"))
    cand = okv_synth.so4_candidates(d, 2, n_cand)
    say("okv_so4_calibrate", name, "block", block, "bits", bits, "n", n, "candidates", n_cand)
    rot, trace = okv.so4_calibrate(torch.from_numpy(np.ascontiguousarray(x)).cuda(), rot0, cand,
                                   block=block, bits=bits, eps=1e-6)
    rot_o, trace_o, _ = oracle.calibrate_so4(x, rot0, cand, block, 1e-6, bits)
    say("trace gpu", trace, "oracle", trace_o)
    assert np.allclose(trace, trace_o, rtol=2e-5), (trace, trace_o)
    assert np.allclose(rot, rot_o, atol=1e-5)
    assert trace[-1] < trace[0]
