"""okv_decode_attn_noalloc (split partials in the library's static device scratch)
against okv_decode_attn (the handle's workspace): the same kernels and split count, so
the outputs must agree bit for bit (within the read path's 2e-3 RMS bound a fortiori).
Two calls in a row, the second on a smaller cache (fewer sequences, heads and tokens),
then a size beyond the 16 MiB scratch, which is refused before any launch.  Every call
goes through the C ABI."""
import numpy as np
import pytest
import torch

import okv_synth
from okv_parity import decode_ref_unit, free_gpu, make_cache, out_error, params_of, say, unit_inputs

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(cache, q):
    import decode_attention_okv_amd as okv
    ref = cache.decode_attn(q)
    got = torch.full_like(ref, float("nan"))
    st = okv.okv_decode_attn_noalloc(cache.handle, q.data_ptr(), got.data_ptr())
    assert st == okv.OKV_OK, okv.okv_strerror(st)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_decode_attn_two_calls():
    _need_gpu()
    import oracle
    cases = [
        # first call: grouped kernel, 2 x 16 query heads over 2 KV heads, 3,000 tokens
        ("gqa_b16h64kv8_t128k_asym", dict(batch=2, hq=16, hkv=2), 3000, 0),
        # second call: smaller (1 sequence, 4 heads, 500 tokens, per-head kernel)
        ("mha_b4h32_t128k", dict(batch=1, hq=4, hkv=4), 500, 0),
    ]
    for name, over, t, splits in cases:
        wl = okv_synth.workload(name).with_(**over)
        p32, u = params_of(wl)
        cache = make_cache(wl, -(-(t + 1) // 32) * 32, p32)
        k, v = okv_synth.kv_tokens(wl, 0, t, device="cuda")
        cache.write(k, v)
        q = okv_synth.queries(wl, 0, device="cuda")
        say("okv_decode_attn / okv_decode_attn_noalloc", name, over, "T", t, "splits", cache.splits(),
            cache.decode_kernel())
        ref, got = _both(cache, q)
        assert torch.equal(ref, got), (name, float((ref - got).abs().max()))
        # and the shared output against the oracle (one unit)
        kh, vh = unit_inputs(k, v, 0, 0)
        r = oracle.write_unit(kh, vh, wl, p32)
        y_ref = decode_ref_unit(wl, okv_synth.host_f32(q), 0, 0, r, t, u)
        err, _ = out_error(got.cpu().numpy()[0, :wl.group], y_ref)
        say(name, f"noalloc unit (0, 0) max_err/rms={err:.3e}")
        assert err <= 2e-3
        cache.close()
        free_gpu()


def test_noalloc_refuses_beyond_scratch():
    _need_gpu()
    import decode_attention_okv_amd as okv
    # batch 64 x 512 query heads x 1 split x 130 floats = 4,259,840 > 4,194,304
    wl = okv_synth.workload("mha_b4h32_t128k").with_(batch=64, hq=512, hkv=512)
    p32, _ = params_of(wl)
    cache = make_cache(wl, 32, p32)
    k, v = okv_synth.kv_tokens(wl, 0, 1, device="cuda")
    cache.write(k, v)
    assert cache.splits() == 1
    q = okv_synth.queries(wl, 0, device="cuda")
    out = torch.zeros((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    say("okv_decode_attn_noalloc beyond the scratch")
    assert okv.okv_decode_attn_noalloc(cache.handle, q.data_ptr(), out.data_ptr()) == okv.OKV_E_CAPACITY
    torch.cuda.synchronize()
    assert not out.any()
    # the allocating entry point serves it
    assert okv.okv_decode_attn(cache.handle, q.data_ptr(), out.data_ptr()) == okv.OKV_OK
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    cache.close()
    free_gpu()
