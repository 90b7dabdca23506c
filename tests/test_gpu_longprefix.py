"""Prefill attention over a prefix long enough that the kernel folds its P.V sums into the
output rows several times (once per 65,536 tokens), with the running maximum moving
between folds and after the last one.

The cache (one sequence, one KV head, two query heads, b = 3; d = 128 with sign flips,
d = 256 with the SO(4) rotation, or d = 128 asymmetric with E4M3 metadata per 64 values)
holds 270,016 tokens.  Its buffers start with zero key codes and scales and a value
scale of 0.7 for every block (asymmetric: value scale 0 and zero-point -2.75): such a
filler token has key zero (logit 0) and one value, the same negative number in every
rotated dim.  Two runs of tokens are written over it with
okv_write, their keys scaled by 3 so that their logits reach well above the filler's:
  - 64 tokens at position 100,000, between the first fold (65,536) and the second,
    where the running maximum of every row jumps;
  - the last 97 positions (a ragged start inside a value tile), the prefill rows.
Expected, for each row at position p: softmax attention over the filler tokens before
p, the middle tokens and the written end tokens up to p, written out in float64 with
the closed form for the filler (pinned against the oracle's attention with explicit
filler rows in test_oracle_attention.py), within 2e-3 of the output RMS.  The decode
kernel runs on the same cache against the same closed form over all 270,016 tokens.

The filler tokens' weights lie 2^-13 to 2^-21 below the rows' running maxima, so this is
also the case of many equal small weights: taken as float16 subnormals in the P operand
they came out 4.2e-2 (and 9e-3 at 60K tokens, with no fold) off the reference before the
prefill kernel formed its probabilities 2^7 times larger."""
import numpy as np
import pytest
import torch

import okv_synth
import oracle
from okv_parity import free_gpu, make_cache, out_error, params_of, say, zero_token_attention

pytestmark = pytest.mark.gpu

TOL = 2e-3
T = 270_016          # a multiple of 32 (the cache capacity unit)
MID, N_MID = 100_000, 64
N_END = 97
KSCALE = 3.0


@pytest.mark.parametrize("shape", ["gqa_h32kv8_t32k", "so4_d256_b32_t8k", "gqa_b16h64kv8_t128k_asym"])
def test_prefill_folds_with_moving_maximum(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = okv_synth.workload(shape).with_(batch=1, hq=2, hkv=1)
    p32, u = params_of(wl)
    if wl.quant == "asym":
        z0 = -2.75
        zb = int(oracle.e4m3_encode(np.array([z0], np.float32))[0])
        assert float(oracle.e4m3_decode(np.array([zb], np.uint8))[0]) == z0
        vz = np.full(wl.d, z0)
    else:
        scale = np.float16(0.7)
        nblk = wl.d // wl.block
        vz = oracle.dequantize(np.zeros((1, wl.d), np.uint8), np.full((1, nblk), scale), wl)[0].astype(np.float64)
    say("long prefix with folds:", shape, "d", wl.d, "tokens", T, "middle run at", MID, "filler value", vz[0])
    cache = make_cache(wl, T, p32)
    for buf in (cache.k_codes, cache.v_codes, cache.k_meta):
        buf.zero_()
    if wl.quant == "asym":
        cache.v_meta[..., 0].zero_()          # scale bytes
        cache.v_meta[..., 1].fill_(zb)        # zero-point bytes
    else:
        cache.v_meta.fill_(float(scale))

    hats = []
    pos_end = T - N_END
    for pos, n in ((MID, N_MID), (pos_end, N_END)):
        cache.set_length(pos)
        k, v = okv_synth.kv_tokens(wl, pos, n, device="cuda")
        k = (k.float() * KSCALE).to(k.dtype)
        cache.write(k, v)
        ref = oracle.write_unit(okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0]), wl, p32)
        hats.append((oracle.dequantize(ref["k_u"], ref["k_meta"], wl), oracle.dequantize(ref["v_u"], ref["v_meta"], wl)))
    assert cache.length == T
    (k_mid, v_mid), (k_end, v_end) = hats
    n_filler = T - N_MID - N_END

    q = okv_synth.query_rows(wl, pos_end, N_END, device="cuda")
    say("okv_prefill_attn", N_END, "rows over", T, "tokens")
    out = cache.prefill_attn(q)
    torch.cuda.synchronize()
    q1 = okv_synth.host_f32(q)[0].astype(np.float64) @ u.T            # (rows, heads, d)
    y_ref = np.stack([
        zero_token_attention(q1[r], np.concatenate([k_mid, k_end[:r + 1]]),
                             np.concatenate([v_mid, v_end[:r + 1]]), n_filler, v_zero=vz) @ u
        for r in range(N_END)])
    err, worst = out_error(out.cpu().numpy()[0], y_ref)
    # the middle run must matter: without it the rows' outputs differ by far more than TOL
    y_wo = np.stack([zero_token_attention(q1[r], k_end[:r + 1], v_end[:r + 1], n_filler + N_MID, v_zero=vz) @ u
                     for r in range(N_END)])
    sens, _ = out_error(y_wo, y_ref)
    say(f"long prefix prefill: max_err/rms={err:.3e} worst_head={worst:.3e} (middle run moves it by {sens:.2e})")
    assert sens > 100 * TOL
    assert err <= TOL, err

    qd = okv_synth.queries(wl, 0, device="cuda")
    outd = cache.decode_attn(qd)
    torch.cuda.synchronize()
    q1d = okv_synth.host_f32(qd)[0].astype(np.float64) @ u.T
    yd_ref = zero_token_attention(q1d, np.concatenate([k_mid, k_end]), np.concatenate([v_mid, v_end]),
                                  n_filler, v_zero=vz) @ u
    errd, worstd = out_error(outd.cpu().numpy()[0], yd_ref)
    say(f"long prefix decode ({cache.decode_kernel()}): max_err/rms={errd:.3e} worst_head={worstd:.3e}")
    assert errd <= TOL, errd
    cache.close()
    del cache, out, outd
    free_gpu()
