"""GPU parity of okv_prefill_attn (causal attention of the last n cached positions)
against the oracle's attend_prefill_unit.  Output bound per call: max |y - y_ref| <=
2e-3 * RMS(y_ref).  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import okv_synth
import oracle
from okv_parity import free_gpu, make_cache, out_error, params_of, round_up, say, unit_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-3


def run_prefill(wl, t, chunks, n_q):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p32, u = params_of(wl)
    cache = make_cache(wl, round_up(t + 1, 32), p32)
    k, v = okv_synth.kv_tokens(wl, 0, t, device="cuda")
    pos = 0
    for n in chunks:
        cache.write(k[:, pos:pos + n].contiguous(), v[:, pos:pos + n].contiguous())
        pos += n
    q = okv_synth.query_rows(wl, t - n_q, n_q, device="cuda")
    say(wl.name, "okv_prefill_attn", "T", t, "n_q", n_q, "d", wl.d, "G", wl.group, wl.quant, wl.block)
    out = cache.prefill_attn(q)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()                       # [B][n][Hq][d]
    q_h = okv_synth.host_f32(q)
    y_ref = np.zeros_like(out_h, dtype=np.float64)
    positions = np.arange(t - n_q, t)
    g = wl.group
    for b in range(wl.batch):
        for h in range(wl.hkv):
            kh, vh = unit_inputs(k, v, b, h)
            ref = oracle.write_unit(kh, vh, wl, p32)
            y_ref[b, :, h * g:(h + 1) * g] = oracle.attend_prefill_unit(
                q_h[b, :, h * g:(h + 1) * g], positions, ref["k_codes"], ref["k_meta"], ref["v_codes"],
                ref["v_meta"], wl, u)
    err, worst = out_error(out_h, y_ref)
    say(wl.name, f"prefill n_q={n_q} max_err/rms={err:.3e} worst={worst:.3e}")
    cache.close()
    free_gpu()
    assert err <= TOL, err


CASES = [
    # name, overrides, tokens, write chunks, query rows
    ("tiny_d128_t256", dict(), 256, [256], 256),
    ("tiny_d128_t256", dict(), 200, [150, 50], 50),
    ("tiny_d128_t256", dict(), 97, [97], 1),
    ("gqa_h32kv8_t32k", dict(hq=8, hkv=2), 300, [236, 64], 64),
    ("gqa_h32kv8_t32k", dict(hq=8, hkv=2), 130, [130], 130),
    ("mha_b4h32_t128k", dict(batch=2, hq=2, hkv=2), 333, [333], 333),
    ("gqa_b16h64kv8_t128k_asym", dict(batch=1, hq=16, hkv=2), 190, [123, 67], 67),
    ("so4_d256_b32_t8k", dict(batch=1, hq=4, hkv=1), 160, [160], 160),
    ("so4_d256_b32_t8k", dict(batch=1, hq=4, hkv=1, quant="asym", block=64, scale_dtype="e4m3"), 99, [60, 39], 39),
    # code widths 2 and 4
    ("gqa_h32kv8_t32k", dict(hq=8, hkv=2, bits=4), 200, [150, 50], 50),
    ("gqa_h32kv8_t32k", dict(hq=8, hkv=2, bits=2), 130, [130], 130),
    ("gqa_b16h64kv8_t128k_asym", dict(batch=1, hq=16, hkv=2, bits=4), 150, [150], 70),
    ("gqa_b16h64kv8_t128k_asym", dict(batch=1, hq=16, hkv=2, bits=2), 100, [64, 36], 36),
    ("so4_d256_b32_t8k", dict(batch=1, hq=4, hkv=1, bits=4), 96, [96], 96),
    ("tiny_d128_t256", dict(bits=2), 256, [256], 256),
    # no rotation (U = I)
    ("gqa_h32kv8_t32k", dict(hq=8, hkv=2, rotation="none"), 140, [100, 40], 40),
    ("so4_d256_b32_t8k", dict(batch=1, hq=4, hkv=1, rotation="none", block=256), 90, [90], 90),
]


@pytest.mark.parametrize("name,over,t,chunks,n_q", CASES)
def test_prefill_parity(name, over, t, chunks, n_q):
    wl = okv_synth.workload(name).with_(**over)
    run_prefill(wl, t, chunks, n_q)


def test_prefill_errors():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_okv_amd as okv
    wl = okv_synth.workload("tiny_d128_t256")
    p32, _ = params_of(wl)
    cache = make_cache(wl, 64, p32)
    q = okv_synth.query_rows(wl, 0, 4, device="cuda")
    out = torch.empty((1, 4, 1, 128), dtype=torch.float32, device="cuda")
    say("prefill error paths")
    assert okv.okv_prefill_attn(cache.handle, q.data_ptr(), 4, out.data_ptr()) == okv.OKV_E_INVALID  # empty
    k, v = okv_synth.kv_tokens(wl, 0, 3, device="cuda")
    cache.write(k, v)
    assert okv.okv_prefill_attn(cache.handle, q.data_ptr(), 4, out.data_ptr()) == okv.OKV_E_INVALID  # n > len
    assert okv.okv_prefill_attn(cache.handle, q.data_ptr(), 0, out.data_ptr()) == okv.OKV_E_INVALID
    assert okv.okv_prefill_attn(cache.handle, q.data_ptr() + 4, 3, out.data_ptr()) == okv.OKV_E_ALIGN
    cache.close()
