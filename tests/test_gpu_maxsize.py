"""The largest (sequence, KV head) slice the library accepts: 89,478,336 cached tokens at
d = 128 and b = 3, whose packed codes take 4.29e9 bytes, just below the 4 GiB limit of
the kernels' 32-bit buffer offsets.

The cache buffers start all zero: a token with zero codes and a zero scale (and zero
zero-point) dequantises to the zero vector, so it has logit 0 and adds nothing to P.V.
The last 97 positions (a ragged start inside a 32-token value tile) are written with
okv_write; the decode at full length then reads every byte of the slice.  Expected:
  - the written rows, scales and value codes byte for byte as the oracle writes those
    97 tokens, and the tile slots before them still zero;
  - y = U^T (sum_t p_t v_t) / (sum_t p_t + N0 exp(-m)) over the 97 written tokens, with
    p_t = exp(L_t - m), m = max(0, max_t L_t) and N0 zero tokens (the softmax over all
    tokens written out; the closed form is pinned against the oracle's attention with
    explicit zero rows in test_oracle_attention.py), within 2e-3 of the output RMS.
Both decode kernels run: the per-head one (one query head) and the grouped one (eight
query heads, blocks of 64; symmetric and asymmetric codes)."""
import numpy as np
import pytest
import torch

import okv_synth
import oracle
from okv_parity import free_gpu, make_cache, out_error, params_of, say, zero_token_attention

pytestmark = pytest.mark.gpu

TOL = 2e-3
CAP = 89478336           # (CAP + 128) x 48 < 2^32: the largest slice at d = 128, b = 3
N_REAL = 97


@pytest.mark.parametrize("hq,block,quant,meta,kernel", [
    (1, 32, "sym", "f16", "per_head"),
    (8, 64, "sym", "f16", "grouped"),
    (8, 64, "asym", "e4m3", "grouped"),
])
def test_largest_slice(hq, block, quant, meta, kernel):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=hq, hkv=1, block=block, quant=quant,
                                                    scale_dtype=meta)
    p32, u = params_of(wl)
    say("largest slice", hq, block, quant, meta, kernel, "capacity", CAP)
    cache = make_cache(wl, CAP, p32)
    assert cache.k_codes.numel() == CAP * 48 and cache.k_codes.numel() + 128 * 48 < 2 ** 32
    for buf in (cache.k_codes, cache.v_codes, cache.k_meta, cache.v_meta):
        buf.zero_()
    cache.set_decode_kernel(kernel)
    pos0 = CAP - N_REAL
    cache.set_length(pos0)
    k, v = okv_synth.kv_tokens(wl, pos0, N_REAL, device="cuda")
    say("okv_write", N_REAL, "tokens at", pos0)
    cache.write(k, v)
    assert cache.length == CAP
    q = okv_synth.queries(wl, 0, device="cuda")
    say("okv_decode_attn", cache.decode_kernel(), "splits", cache.splits())
    out = cache.decode_attn(q)
    torch.cuda.synchronize()
    assert cache.decode_kernel() == kernel

    ref = oracle.write_unit(okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0]), wl, p32)
    # key rows and metadata of the written positions, byte for byte
    assert np.array_equal(cache.k_codes[0, 0, pos0:].cpu().numpy(), ref["k_codes"])
    for key in ("k_meta", "v_meta"):
        got = getattr(cache, key)[0, 0, pos0:].cpu().numpy()
        assert np.array_equal(got.view(np.uint8), np.asarray(ref[key]).view(np.uint8)), key
    # value codes: the tiles holding the written positions; earlier slots stay zero
    t0 = pos0 // 32
    tiles = cache.v_codes[0, 0, t0:].cpu().numpy()
    codes = oracle.unpack_vtiles(tiles, tiles.shape[0] * 32, oracle.bits_of(wl))
    off = pos0 - 32 * t0
    assert np.array_equal(codes[off:off + N_REAL], ref["v_u"])
    assert not codes[:off].any()
    # decode output against the closed form over the written tokens and the zero ones
    k_hat = oracle.dequantize(ref["k_u"], ref["k_meta"], wl)
    v_hat = oracle.dequantize(ref["v_u"], ref["v_meta"], wl)
    q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T
    y_ref = zero_token_attention(q1, k_hat, v_hat, CAP - N_REAL) @ u
    err, worst = out_error(out.cpu().numpy()[0], y_ref)
    say(f"largest slice {kernel} {quant}: max_err/rms={err:.3e} worst_head={worst:.3e}")
    assert err <= TOL, err
    cache.close()
    del cache, out
    free_gpu()


def test_largest_slice_prefill():
    """Causal prefill attention of the 97 written rows over the same largest slice: each
    row sees the 89,478,239 zero tokens before the written ones and the written ones up
    to its own position (every workgroup streams the whole prefix)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=2, hkv=1)
    p32, u = params_of(wl)
    say("largest slice prefill, capacity", CAP)
    cache = make_cache(wl, CAP, p32)
    for buf in (cache.k_codes, cache.v_codes, cache.k_meta, cache.v_meta):
        buf.zero_()
    pos0 = CAP - N_REAL
    cache.set_length(pos0)
    k, v = okv_synth.kv_tokens(wl, pos0, N_REAL, device="cuda")
    cache.write(k, v)
    q = okv_synth.query_rows(wl, pos0, N_REAL, device="cuda")
    say("okv_prefill_attn", N_REAL, "rows over", CAP, "tokens")
    out = cache.prefill_attn(q)
    torch.cuda.synchronize()
    ref = oracle.write_unit(okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0]), wl, p32)
    k_hat = oracle.dequantize(ref["k_u"], ref["k_meta"], wl)
    v_hat = oracle.dequantize(ref["v_u"], ref["v_meta"], wl)
    q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T          # (rows, heads, d)
    y_ref = np.stack([zero_token_attention(q1[r], k_hat[:r + 1], v_hat[:r + 1], pos0) @ u
                      for r in range(N_REAL)])
    err, worst = out_error(out.cpu().numpy()[0], y_ref)
    say(f"largest slice prefill: max_err/rms={err:.3e} worst_head={worst:.3e}")
    assert err <= TOL, err
    cache.close()
    del cache, out
    free_gpu()


@pytest.mark.parametrize("call", ["decode", "prefill"])
def test_largest_slice_asym_zero_points(call):
    """Asymmetric codes at the largest slice (blocks of 64): the filler tokens keep zero
    key metadata (key = zero vector) but their value metadata is the E4M3 pair (scale 0,
    zero-point -0.5), so each has the constant value -0.5 in every rotated dim.  Their
    89 million weighted zero-points must add up to N0 exp(-m) (-0.5) per dim: a plain
    float32 running sum of those terms would saturate.  Decode (grouped kernel) or
    causal prefill of the 97 written rows, against the closed form."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hq = 8 if call == "decode" else 2
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=hq, hkv=1, block=64, quant="asym",
                                                    scale_dtype="e4m3")
    p32, u = params_of(wl)
    z0 = -0.5
    zb = int(oracle.e4m3_encode(np.array([z0], np.float32))[0])
    assert float(oracle.e4m3_decode(np.array([zb], np.uint8))[0]) == z0
    say("largest slice asym zero-points", call, "capacity", CAP)
    cache = make_cache(wl, CAP, p32)
    for buf in (cache.k_codes, cache.v_codes, cache.k_meta):
        buf.zero_()
    cache.v_meta[..., 0].zero_()          # scale bytes
    cache.v_meta[..., 1].fill_(zb)        # zero-point bytes
    pos0 = CAP - N_REAL
    cache.set_length(pos0)
    k, v = okv_synth.kv_tokens(wl, pos0, N_REAL, device="cuda")
    cache.write(k, v)
    ref = oracle.write_unit(okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0]), wl, p32)
    k_hat = oracle.dequantize(ref["k_u"], ref["k_meta"], wl)
    v_hat = oracle.dequantize(ref["v_u"], ref["v_meta"], wl)
    vz = np.full(wl.d, z0)
    if call == "decode":
        cache.set_decode_kernel("grouped")
        q = okv_synth.queries(wl, 0, device="cuda")
        out = cache.decode_attn(q)
        torch.cuda.synchronize()
        q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T
        y_ref = zero_token_attention(q1, k_hat, v_hat, pos0, v_zero=vz) @ u
        got = out.cpu().numpy()[0]
    else:
        q = okv_synth.query_rows(wl, pos0, N_REAL, device="cuda")
        out = cache.prefill_attn(q)
        torch.cuda.synchronize()
        q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T
        y_ref = np.stack([zero_token_attention(q1[r], k_hat[:r + 1], v_hat[:r + 1], pos0, v_zero=vz) @ u
                          for r in range(N_REAL)])
        got = out.cpu().numpy()[0]
    err, worst = out_error(got, y_ref)
    say(f"largest slice asym zero-points {call}: max_err/rms={err:.3e} worst_head={worst:.3e}")
    assert err <= TOL, err
    cache.close()
    del cache, out
    free_gpu()


@pytest.mark.parametrize("call", ["decode", "prefill"])
def test_largest_slice_constant_values(call):
    """Symmetric codes at the largest slice with filler tokens of zero key codes and scale
    but value scale 0.7 (float16): each filler value is code 0 dequantised, the same
    negative non-power-of-two number in every rotated dim, so the 89 million P.V terms of
    a dim share a sign and none is exact in a short float.  The P.V sums must keep that
    mass: a single float32 running sum over 1.4 million 64-token tiles would drift by
    about a tenth.  Decode (grouped kernel, eight query heads) or causal prefill of the
    97 written rows, against the closed form."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hq = 8 if call == "decode" else 2
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=hq, hkv=1)
    p32, u = params_of(wl)
    scale = np.float16(0.7)
    nblk = wl.d // wl.block
    vz = oracle.dequantize(np.zeros((1, wl.d), np.uint8), np.full((1, nblk), scale), wl)[0].astype(np.float64)
    assert np.all(vz == vz[0]) and vz[0] < 0
    say("largest slice constant values", call, "capacity", CAP, "filler value", vz[0])
    cache = make_cache(wl, CAP, p32)
    for buf in (cache.k_codes, cache.v_codes, cache.k_meta):
        buf.zero_()
    cache.v_meta.fill_(float(scale))
    pos0 = CAP - N_REAL
    cache.set_length(pos0)
    k, v = okv_synth.kv_tokens(wl, pos0, N_REAL, device="cuda")
    cache.write(k, v)
    ref = oracle.write_unit(okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0]), wl, p32)
    k_hat = oracle.dequantize(ref["k_u"], ref["k_meta"], wl)
    v_hat = oracle.dequantize(ref["v_u"], ref["v_meta"], wl)
    if call == "decode":
        cache.set_decode_kernel("grouped")
        q = okv_synth.queries(wl, 0, device="cuda")
        out = cache.decode_attn(q)
        torch.cuda.synchronize()
        q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T
        y_ref = zero_token_attention(q1, k_hat, v_hat, pos0, v_zero=vz) @ u
    else:
        q = okv_synth.query_rows(wl, pos0, N_REAL, device="cuda")
        out = cache.prefill_attn(q)
        torch.cuda.synchronize()
        q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T
        y_ref = np.stack([zero_token_attention(q1[r], k_hat[:r + 1], v_hat[:r + 1], pos0, v_zero=vz) @ u
                          for r in range(N_REAL)])
    err, worst = out_error(out.cpu().numpy()[0], y_ref)
    say(f"largest slice constant values {call}: max_err/rms={err:.3e} worst_head={worst:.3e}")
    assert err <= TOL, err
    cache.close()
    del cache, out
    free_gpu()
