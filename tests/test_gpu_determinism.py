"""Run-to-run determinism of the library on the GPU (no oracle involved).

- `okv_write`: the same inputs, written in the same chunks into two caches whose buffers
  start with different contents, give identical bytes (codes, scales, zero-points) over
  the written rows and value tiles, the ragged last tile included.
- `okv_decode_attn` and `okv_prefill_attn`: for a fixed split count and kernel, repeated
  calls give bit-identical outputs (no atomics decide an order of summation).
Every call goes through the C ABI."""
import pytest
import torch

import okv_synth
from okv_parity import free_gpu, make_cache, params_of, round_up, say

pytestmark = pytest.mark.gpu

CASES = {
    "mha_b4h32_t128k": dict(batch=2, hq=8, hkv=8),
    "gqa_b16h64kv8_t128k_asym": dict(batch=2),
    "so4_d256_b32_t8k": dict(batch=2),
}


def written(cache, t):
    ntile = -(-t // 32)
    return (cache.k_codes[:, :, :t], cache.v_codes[:, :, :ntile], cache.k_meta[:, :, :t],
            cache.v_meta[:, :, :t])


@pytest.mark.parametrize("name", list(CASES))
def test_repeatable(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = okv_synth.workload(name).with_(**CASES[name])
    p32, _ = params_of(wl)
    t, chunks = 1500, [700, 1, 799]
    k, v = okv_synth.kv_tokens(wl, 0, t, device="cuda")
    caches = []
    for fill in (0x00, 0xFF):
        cache = make_cache(wl, round_up(t + 1, 32), p32)
        for buf in (cache.k_codes, cache.v_codes, cache.k_meta, cache.v_meta):
            buf.view(torch.uint8).fill_(fill)
        pos = 0
        for n in chunks:
            say(name, "okv_write", "fill", hex(fill), pos, n)
            cache.write(k[:, pos:pos + n].contiguous(), v[:, pos:pos + n].contiguous())
            pos += n
        caches.append(cache)
    torch.cuda.synchronize()
    for a, b, what in zip(written(caches[0], t), written(caches[1], t), ("k_codes", "v_codes", "k_meta", "v_meta")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (name, what)

    cache = caches[0]
    q = okv_synth.queries(wl, 0, device="cuda")
    kernels = ["per_head"] + (["grouped"] if wl.group in (2, 4, 8) else [])
    for kernel in kernels:
        cache.set_decode_kernel(kernel)
        for splits in (0, 7):           # 0: the automatic count
            cache.set_splits(splits)
            say(name, "okv_decode_attn", kernel, "splits", cache.splits(), "x3")
            outs = [cache.decode_attn(q) for _ in range(3)]
            torch.cuda.synchronize()
            for o in outs[1:]:
                assert torch.equal(outs[0], o), (name, kernel, splits)
    qp = okv_synth.query_rows(wl, t - 45, 45, device="cuda")
    say(name, "okv_prefill_attn", "n_q", 45, "x2")
    p1 = cache.prefill_attn(qp)
    p2 = cache.prefill_attn(qp)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2), name
    for c in caches:
        c.close()
    free_gpu()
