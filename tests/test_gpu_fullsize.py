"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (automatic kernel and split count).  Every (sequence, KV head) unit of every
workload is checked: its codes, scales and zero-points byte for byte against the
oracle's write of the same raw inputs, and every checked decode call's output within
2e-3 of the output RMS against the oracle's float64 read path (max |y - y_ref| over
all sequences, query heads and dims of the call).  Exact ties among the codes are
counted and reported.  The oracle runs in worker processes on the host cores."""
import multiprocessing as mp
import os
import time

import numpy as np
import pytest
import torch

import okv_synth
from okv_parity import free_gpu, make_cache, out_error, params_of, round_up, say
from oracle_pool import full_unit_job

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _spec(wl):
    return dict(d=wl.d, block=wl.block, quant=wl.quant, scale_dtype=wl.scale_dtype, eps=wl.eps,
                rotation=wl.rotation, bits=wl.bits)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pool(n):
    # one BLAS thread per worker: the workers already fill the cores
    old = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in old:
        os.environ[k] = "1"
    try:
        return mp.get_context("spawn").Pool(n)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _host_raw(x):
    """Host copy of an input tensor: float32 as it is, bfloat16 as uint16 bits."""
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def check_every_unit(cache, wl, k_all, v_all, p32, u, calls):
    """Byte-exact cache and decode outputs of every (sequence, KV head) unit.
    calls: [(t, q tensor, out host [B][Hq][d])] decode calls made at length t."""
    t_final = cache.length
    g = wl.group
    kh, vh = _host_raw(k_all), _host_raw(v_all)
    ntile = -(-t_final // 32)
    gk = cache.k_codes[:, :, :t_final].cpu().numpy()
    gv = cache.v_codes[:, :, :ntile].cpu().numpy()
    gkm = cache.k_meta[:, :, :t_final].cpu().numpy().view(np.uint8).reshape(wl.batch, wl.hkv, t_final, -1)
    gvm = cache.v_meta[:, :, :t_final].cpu().numpy().view(np.uint8).reshape(wl.batch, wl.hkv, t_final, -1)
    qh = [okv_synth.host_f32(q) for _, q, _ in calls]
    units = [(b, h) for b in range(wl.batch) for h in range(wl.hkv)]

    def jobs():
        for (b, h) in units:
            qs = [(t, q[b, h * g:(h + 1) * g]) for (t, _, _), q in zip(calls, qh)]
            gpu = {"k_codes": gk[b, h], "v_codes": gv[b, h], "k_meta": gkm[b, h], "v_meta": gvm[b, h]}
            yield ((b, h), np.ascontiguousarray(kh[b, :, h]), np.ascontiguousarray(vh[b, :, h]), _spec(wl), p32,
                   u, qs, gpu)

    y_ref = [np.zeros((wl.batch, wl.hq, wl.d)) for _ in calls]
    tot = {"k_codes": 0, "v_codes": 0, "k_meta": 0, "v_meta": 0}
    ties = codes = 0
    nw = min(_workers(), len(units))
    t0 = time.time()
    say(wl.name, f"oracle over all {len(units)} units, {len(calls)} decode call(s), {nw} workers")
    with _pool(nw) as pool:
        for i, ((b, h), mism, nt, nc, outs) in enumerate(pool.imap_unordered(full_unit_job, jobs())):
            for kk in tot:
                tot[kk] += mism[kk]
            if any(mism.values()):
                say(wl.name, f"unit b={b} h={h} mismatches {mism}")
            ties += nt
            codes += nc
            for c, y in enumerate(outs):
                y_ref[c][b, h * g:(h + 1) * g] = y
            if (i + 1) % 32 == 0:
                say(wl.name, f"{i + 1}/{len(units)} units checked, {time.time() - t0:.1f} s")
    say(wl.name, f"all units T={t_final}: byte mismatches {tot}, codes {codes}, exact ties {ties} "
                 f"({ties / max(codes, 1):.2e} of codes), oracle {time.time() - t0:.1f} s")
    assert all(x == 0 for x in tot.values()), tot
    worst = 0.0
    for c, ((t, _, out_h), yr) in enumerate(zip(calls, y_ref)):
        err, head = out_error(out_h, yr)
        worst = max(worst, err)
        if c < 4 or c == len(calls) - 1 or err > TOL:
            say(wl.name, f"decode call {c} T={t}: max_err/rms={err:.3e} worst_head={head:.3e}")
        assert err <= TOL, (c, t, err)
    say(wl.name, f"{len(calls)} decode call(s): worst max_err/rms {worst:.3e}")


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
        if i < 2 or i == steps - 1:
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
    del ks, vs
    return cache, k_all, v_all, p32, u, calls


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mha_b4h32_t128k", "gqa_b16h64kv8_t128k_asym", "so4_d256_b32_t8k"])
def test_fullsize_prefill_decode_every_unit(name):
    wl = okv_synth.workload(name)
    cache, k, v, p32, u, calls = prefill_and_step(wl, steps=1, also_per_head=wl.group > 1)
    check_every_unit(cache, wl, k, v, p32, u, calls)
    cache.close()
    del k, v
    free_gpu()


@pytest.mark.timeout(900)
def test_fullsize_gqa_32k_decode_steps_every_unit():
    # 32K context, then 256 decode steps (append one token, decode); every step's
    # output and the final cache of every KV-head unit are checked
    wl = okv_synth.workload("gqa_h32kv8_t32k")
    cache, k, v, p32, u, calls = prefill_and_step(wl, steps=wl.decode_steps)
    check_every_unit(cache, wl, k, v, p32, u, calls)
    cache.close()
    free_gpu()
