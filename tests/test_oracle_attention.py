"""Pins of the oracle's read path (CPU only)."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import okv_synth
import oracle


def make_unit(name, t, seed=0):
    wl = okv_synth.workload(name).with_(batch=1, tokens=t)
    k, v = okv_synth.kv_tokens(wl, 0, t)
    k = okv_synth.host_f32(k)[0, :, 0]
    v = okv_synth.host_f32(v)[0, :, 0]
    q = okv_synth.host_f32(okv_synth.queries(wl, step=seed))[0, :wl.group]
    p64 = okv_synth.rotation_params(wl)
    p32 = p64.astype(np.float32)
    u = oracle.rotation_matrix(wl.rotation, p32.astype(np.float64), wl.d)
    return wl, k, v, q, p32, u


@pytest.mark.parametrize("name", ["tiny_d128_t256", "so4_d256_b32_t8k"])
def test_unquantised_rotated_attention_equals_plain(name):
    # the OIQ report, Section 2.3 / idea card, Mathematical statement: rotating q and k
    # by U and the output back by U^T leaves attention unchanged (fp64, tiny inputs)
    wl, k, v, q, _, _ = make_unit(name, 40)
    u = oracle.rotation_matrix(wl.rotation, okv_synth.rotation_params(wl), wl.d)
    y_plain = oracle.attend_exact(q, k, v)
    y_rot = oracle.attend_exact(q @ u.T, k @ u.T, v @ u.T) @ u
    assert np.abs(y_rot - y_plain).max() <= 1e-12 * np.abs(y_plain).max()


def test_attend_exact_matches_torch_sdpa():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 64))
    k = rng.standard_normal((33, 64))
    v = rng.standard_normal((33, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    assert np.abs(oracle.attend_exact(q, k, v) - ref).max() < 1e-13


@pytest.mark.parametrize("name", ["tiny_d128_t256", "so4_d256_b32_t8k",
                                  "gqa_b16h64kv8_t128k_asym"])
def test_attend_unit_equals_sdpa_on_unrotated_dequantised_cache(name):
    # independent route: dequantise, rotate the keys and values back with U^T, and run
    # torch's scaled-dot-product attention in float64 on the ORIGINAL query
    wl, k, v, q, p32, u = make_unit(name, 100)
    c = oracle.write_unit(k, v, wl, p32)
    y = oracle.attend_unit(q, c["k_codes"], c["k_meta"], c["v_codes"], c["v_meta"], 100, wl, u)
    k_hat = oracle.dequantize(c["k_u"], c["k_meta"], wl) @ u      # rows of U^T k_hat_rot
    v_hat = oracle.dequantize(c["v_u"], c["v_meta"], wl) @ u
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None], torch.from_numpy(k_hat)[None],
        torch.from_numpy(v_hat)[None])[0].numpy()
    assert np.abs(y - ref).max() < 1e-11 * np.abs(ref).max()


@pytest.mark.parametrize("name", ["tiny_d128_t256", "gqa_b16h64kv8_t128k_asym"])
def test_single_token_returns_rotated_back_value(name):
    # T = 1: the softmax weight is 1, so y = U^T v_hat_rot
    wl, k, v, q, p32, u = make_unit(name, 1)
    c = oracle.write_unit(k, v, wl, p32)
    y = oracle.attend_unit(q, c["k_codes"], c["k_meta"], c["v_codes"], c["v_meta"], 1, wl, u)
    want = oracle.dequantize(c["v_u"], c["v_meta"], wl)[0] @ u
    assert np.abs(y - want[None]).max() < 1e-13


def test_zero_query_gives_mean_value():
    wl, k, v, q, p32, u = make_unit("tiny_d128_t256", 70)
    c = oracle.write_unit(k, v, wl, p32)
    y = oracle.attend_unit(np.zeros_like(q), c["k_codes"], c["k_meta"], c["v_codes"],
                           c["v_meta"], 70, wl, u)
    want = oracle.dequantize(c["v_u"], c["v_meta"], wl).mean(0) @ u
    assert np.abs(y - want[None]).max() < 1e-13


def test_quantised_attention_close_to_exact_and_rotation_helps():
    # diagnostics on the synthetic outlier model (direction only, as the idea card's
    # Verification reports): Hadamard rotation lowers the worst block maximum relative
    # to the vector norm and the attention error of 3-bit storage
    wl, k, v, q, p32, u = make_unit("mha_b4h32_t128k", 512)
    y_ref = oracle.attend_exact(q, k, v)
    c = oracle.write_unit(k, v, wl, p32)
    y_rot = oracle.attend_unit(q, c["k_codes"], c["k_meta"], c["v_codes"], c["v_meta"], 512, wl, u)
    ident = SimpleNamespace(**{**wl.__dict__})
    ku, km = oracle.quantize_f32(k, ident)
    vu, vm = oracle.quantize_f32(v, ident)
    y_norot = oracle.attend_exact(q, oracle.dequantize(ku, km, ident), oracle.dequantize(vu, vm, ident))
    e_rot = np.sqrt(np.mean((y_rot - y_ref) ** 2)) / np.sqrt(np.mean(y_ref ** 2))
    e_norot = np.sqrt(np.mean((y_norot - y_ref) ** 2)) / np.sqrt(np.mean(y_ref ** 2))
    assert e_rot < e_norot
    assert e_rot < 0.5


@pytest.mark.parametrize("name,t,n", [("tiny_d128_t256", 100, 100), ("tiny_d128_t256", 100, 37),
                                      ("so4_d256_b32_t8k", 70, 70), ("gqa_b16h64kv8_t128k_asym", 90, 21)])
def test_attend_prefill_equals_causal_sdpa_on_unrotated_dequantised_cache(name, t, n):
    # independent route for the prefill rows: torch's float64 scaled-dot-product
    # attention with a causal mask (query at position p sees tokens 0..p) on the
    # dequantised cache rotated back with U^T and the original queries
    wl, k, v, _, p32, u = make_unit(name, t)
    rng = np.random.default_rng(5)
    g = wl.group
    q = rng.standard_normal((n, g, wl.d))
    pos = np.arange(t - n, t)
    c = oracle.write_unit(k, v, wl, p32)
    y = oracle.attend_prefill_unit(q, pos, c["k_codes"], c["k_meta"], c["v_codes"], c["v_meta"], wl, u)
    k_hat = torch.from_numpy(oracle.dequantize(c["k_u"], c["k_meta"], wl) @ u)
    v_hat = torch.from_numpy(oracle.dequantize(c["v_u"], c["v_meta"], wl) @ u)
    mask = torch.from_numpy(np.arange(t)[None, :] <= pos[:, None])          # (n, t)
    for h in range(g):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], k_hat[None], v_hat[None], attn_mask=mask[None])[0].numpy()
        assert np.abs(y[:, h] - ref).max() < 1e-11 * np.abs(ref).max()


def test_attend_prefill_first_position_is_its_own_value():
    # closed form: the query at position 0 sees one token, so its output is that
    # token's dequantised value rotated back (softmax of a single logit is 1)
    wl, k, v, _, p32, u = make_unit("tiny_d128_t256", 8)
    c = oracle.write_unit(k, v, wl, p32)
    q = np.random.default_rng(1).standard_normal((3, 1, wl.d)) * 7.0
    y = oracle.attend_prefill_unit(q, [0, 0, 0], c["k_codes"], c["k_meta"], c["v_codes"], c["v_meta"], wl, u)
    v0 = oracle.dequantize(c["v_u"][:1], c["v_meta"][:1], wl)[0] @ u
    assert np.abs(y[:, 0] - v0).max() <= 1e-13 * np.abs(v0).max()


def test_attend_unit_lengths_equals_attend_unit_per_length():
    # several cache lengths from one decoded cache: each equals the one-length read
    # path over the first t tokens, and the shortest equals torch SDPA on the
    # un-rotated dequantised prefix
    import torch
    rng = np.random.default_rng(41)
    sp = SimpleNamespace(d=128, block=32, quant="sym", scale_dtype="f16", eps=1e-6, rotation="sign")
    p32 = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    u = oracle.rotation_matrix("sign", p32.astype(np.float64), 128)
    k = rng.standard_normal((77, 128)).astype(np.float32)
    v = rng.standard_normal((77, 128)).astype(np.float32)
    ref = oracle.write_unit(k, v, sp, p32)
    qs = [(t, rng.standard_normal((3, 128)).astype(np.float32)) for t in (1, 31, 32, 33, 77)]
    got = oracle.attend_unit_lengths(qs, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], sp, u)
    for (t, q), y in zip(qs, got):
        want = oracle.attend_unit(q, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], t, sp, u)
        assert np.array_equal(y, want)
    t, q = qs[2]
    kx = oracle.dequantize(ref["k_u"][:t], ref["k_meta"][:t], sp) @ u          # U^T k_hat, as rows
    vx = oracle.dequantize(ref["v_u"][:t], ref["v_meta"][:t], sp) @ u
    sd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None], torch.from_numpy(kx)[None], torch.from_numpy(vx)[None])[0]
    assert np.allclose(got[2], sd.numpy(), atol=1e-10)


def test_zero_tokens_closed_form():
    """Tokens whose key and value are zero vectors (zero codes with a zero scale) have
    logit 0 and add only exp(-m) to the denominator: the closed form the largest-slice
    GPU test uses equals the oracle's attention with those rows spelled out, also when
    every real logit is negative (then m = 0 comes from the zero tokens)."""
    from okv_parity import zero_token_attention
    rng = np.random.default_rng(5)
    for shift in (0.0, -40.0):
        q = rng.standard_normal((3, 16))
        k = rng.standard_normal((7, 16)) * 3
        v = rng.standard_normal((7, 16))
        n0 = 11
        k_all = np.concatenate([k, np.zeros((n0, 16))])
        v_all = np.concatenate([v, np.zeros((n0, 16))])
        # a negative shift of every real logit: add a constant key component
        qs = np.concatenate([q, np.ones((3, 1))], axis=1)
        ks = np.concatenate([k_all, np.concatenate([np.full((7, 1), shift * np.sqrt(17)), np.zeros((n0, 1))])], axis=1)
        vs = np.concatenate([v_all, np.zeros((7 + n0, 1))], axis=1)
        want = oracle.attend_exact(qs, ks, vs)
        got = zero_token_attention(qs, ks[:7], vs[:7], n0)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
        # filler tokens with a constant value vector (a zero scale and a zero-point z)
        vz = rng.standard_normal(17)
        vs_z = vs.copy()
        vs_z[7:] = vz
        want = oracle.attend_exact(qs, ks, vs_z)
        got = zero_token_attention(qs, ks[:7], vs[:7], n0, v_zero=vz)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
