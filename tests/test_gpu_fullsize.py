"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (automatic split count).  Whole (sequence, KV head) units are checked
byte-exact against the oracle and their decode outputs within 2e-3 RMS; in
addition random tokens from every part of the cache are checked byte-exact."""
import multiprocessing as mp
import time

import numpy as np
import pytest
import torch

import okv_synth
import oracle
from okv_parity import free_gpu, make_cache, out_error, params_of, round_up, say
from oracle_pool import token_job, unit_job

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _spec(wl):
    return dict(d=wl.d, block=wl.block, quant=wl.quant, scale_dtype=wl.scale_dtype, eps=wl.eps,
                rotation=wl.rotation)


def _pool(n):
    return mp.get_context("spawn").Pool(n)


def check_random_tokens(cache, wl, k, v, p32, n=96, seed=0):
    rng = np.random.default_rng(seed)
    t = cache.length
    bs = rng.integers(0, wl.batch, n)
    hs = rng.integers(0, wl.hkv, n)
    ts = rng.integers(0, t, n)
    ts[:4] = [0, t - 1, min(31, t - 1), min(32, t - 1)]
    kh = np.stack([okv_synth.host_f32(k[b, tt, h]) for b, h, tt in zip(bs, hs, ts)])
    vh = np.stack([okv_synth.host_f32(v[b, tt, h]) for b, h, tt in zip(bs, hs, ts)])
    ref = token_job((kh, vh, _spec(wl), p32))
    bad = 0
    for i, (b, h, tt) in enumerate(zip(bs, hs, ts)):
        krow = cache.k_codes[b, h, tt].cpu().numpy()
        vgrp = cache.v_codes[b, h, tt // 32].cpu().numpy()            # (d, 12)
        vcodes = oracle.unpack_g32(vgrp)[:, tt % 32]
        km = cache.k_meta[b, h, tt].cpu().numpy().view(np.uint8)
        vm = cache.v_meta[b, h, tt].cpu().numpy().view(np.uint8)
        bad += int(np.count_nonzero(krow != ref["k_row"][i]))
        bad += int(np.count_nonzero(vcodes != ref["v_u"][i]))
        bad += int(np.count_nonzero(km != ref["k_meta"][i].view(np.uint8)))
        bad += int(np.count_nonzero(vm != ref["v_meta"][i].view(np.uint8)))
    say(wl.name, f"random tokens checked: {n}, byte mismatches: {bad}")
    assert bad == 0


def check_units(cache, wl, units, k_all, v_all, p32, u, qsteps):
    """units: list of (b, h); qsteps: list of (t, q tensor) decode calls whose
    outputs are in `outs` (list of host arrays [B][Hq][d])."""
    jobs = []
    g = wl.group
    for (b, h) in units:
        kh = okv_synth.host_f32(k_all[b, :, h])
        vh = okv_synth.host_f32(v_all[b, :, h])
        qs = [(t, okv_synth.host_f32(q)[b, h * g:(h + 1) * g]) for t, q, _ in qsteps]
        jobs.append(((b, h), kh, vh, _spec(wl), p32, u, qs))
    t0 = time.time()
    with _pool(min(len(jobs), 4)) as pool:
        results = pool.map(unit_job, jobs)
    say(wl.name, f"oracle for {len(jobs)} unit(s): {time.time() - t0:.1f} s")
    t_final = cache.length
    for (b, h), ref, outs in results:
        ntile = -(-t_final // 32)
        mism = {
            "k_codes": int(np.count_nonzero(cache.k_codes[b, h, :t_final].cpu().numpy() != ref["k_codes"])),
            "v_codes": int(np.count_nonzero(cache.v_codes[b, h, :ntile].cpu().numpy() != ref["v_codes"])),
            "k_meta": int(np.count_nonzero(cache.k_meta[b, h, :t_final].cpu().numpy().view(np.uint8)
                                           != np.asarray(ref["k_meta"]).view(np.uint8))),
            "v_meta": int(np.count_nonzero(cache.v_meta[b, h, :t_final].cpu().numpy().view(np.uint8)
                                           != np.asarray(ref["v_meta"]).view(np.uint8))),
        }
        say(wl.name, f"unit b={b} h={h} T={t_final} mismatches {mism}")
        assert all(x == 0 for x in mism.values())
        for (t, _, out_h), y_ref in zip(qsteps, outs):
            err, worst = out_error(out_h[b, h * g:(h + 1) * g], y_ref)
            say(wl.name, f"unit b={b} h={h} decode T={t} max_err/rms={err:.3e} worst_head={worst:.3e}")
            assert err <= TOL


def prefill_and_step(wl, steps=1, also_per_head=False):
    """Prefill wl.tokens tokens in one okv_write, then `steps` x (append one token,
    decode), as the benchmark does (automatic kernel and split count).  With
    also_per_head, the last query is decoded once more with the per-head kernel.
    Returns the cache, all keys/values and the decode calls [(t, q, out_host)]."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p32, u = params_of(wl)
    cap = round_up(wl.tokens + steps + 32, 32)
    say(wl.name, "full size: batch", wl.batch, "kv", wl.hkv, "q", wl.hq, "T", wl.tokens, "cap", cap)
    cache = make_cache(wl, cap, p32)
    k, v = okv_synth.kv_tokens(wl, 0, wl.tokens, device="cuda")
    say(wl.name, "okv_write prefill")
    cache.write(k, v)
    calls = []
    ks, vs = [k], [v]
    for i in range(steps):
        kn, vn = okv_synth.kv_tokens(wl, wl.tokens + i, 1, device="cuda", step=i)
        cache.write(kn, vn)
        ks.append(kn)
        vs.append(vn)
        q = okv_synth.queries(wl, i, device="cuda")
        say(wl.name, "okv_decode_attn", cache.decode_kernel(), "T", cache.length, "splits", cache.splits())
        out = cache.decode_attn(q)
        calls.append((cache.length, q, out))
    if also_per_head and calls:
        cache.set_decode_kernel("per_head")
        t, q, _ = calls[-1]
        say(wl.name, "okv_decode_attn per_head T", t, "splits", cache.splits())
        calls.append((t, q, cache.decode_attn(q)))
        cache.set_decode_kernel("auto")
    torch.cuda.synchronize()
    calls = [(t, q, o.cpu().numpy()) for t, q, o in calls]
    k_all = torch.cat(ks, 1) if steps else k
    v_all = torch.cat(vs, 1) if steps else v
    return cache, k_all, v_all, p32, u, calls


@pytest.mark.parametrize("name,units", [
    ("mha_b4h32_t128k", [(0, 0), (3, 31)]),
    ("gqa_b16h64kv8_t128k_asym", [(0, 0), (15, 7)]),
    ("so4_d256_b32_t8k", [(0, 0), (31, 7), (17, 3)]),
])
def test_fullsize_prefill_decode(name, units):
    wl = okv_synth.workload(name)
    cache, k, v, p32, u, calls = prefill_and_step(wl, steps=1, also_per_head=wl.group > 1)
    check_random_tokens(cache, wl, k, v, p32)
    check_units(cache, wl, units, k, v, p32, u, calls)
    cache.close()
    del k, v
    free_gpu()


def test_fullsize_gqa_32k_decode_steps():
    # 32K context, then 256 decode steps (append one token, decode); outputs of
    # steps 1, 2, 128 and 256 are checked on two KV-head units
    wl = okv_synth.workload("gqa_h32kv8_t32k")
    cache, k, v, p32, u, calls = prefill_and_step(wl, steps=wl.decode_steps)
    check_random_tokens(cache, wl, k, v, p32)
    pick = [calls[i] for i in (0, 1, 127, 255)]
    check_units(cache, wl, [(0, 0), (0, 5)], k, v, p32, u, pick)
    cache.close()
    free_gpu()
