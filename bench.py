"""Benchmark of the rotated 3-bit KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: okv_write appends one new
token per sequence (rotate, quantise, pack), then okv_decode_attn attends with one
query per (sequence, query head) over the whole cache (rotate q, fused unpack /
scale / dot, online softmax, P.V, split-K reduce, rotate back).  The append may run
on a second stream, concurrently with the previous step's decode (the warm-up picks
that schedule or a single stream, whichever is faster; "append_schedule" says which).

Default workload: 7B MHA shape at 128K context (batch 4, 32 heads, d 128,
131,072 cached tokens per sequence, 8.3 % outlier channels, block 32, fp16 scales).
Prints one JSON line.  `value` is decode-attention GB/s over the algorithmic bytes
of the packed cache (codes + scales read, q read, output written), timed over
whole steps.  A second leg times chunked-prefill attention over the packed cache
(okv_prefill_attn: the last 2,048 positions of a 32,768-token GQA context attend
causally) and reports it under "prefill_attn"; "code_widths" times the decode kernel
at 2- and 4-bit codes on the same workload (the pages' method is 3-bit), and
"rotations" the unrotated per-token variant and U = B H (SO(4) after the transform);
"so4_calibration" times the SO(4) calibration search on 16,384 key vectors.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_PEAK_TFLOPS = 2500.0   # dense f16 MFMA
METRIC = "decode attn GB/s over packed 3-bit KV (% HBM peak); okv_write tokens/s"


def algorithmic_decode_bytes(wl, t):
    in_b = 4 if wl.in_dtype == "f32" else 2
    cache = 2 * wl.batch * wl.hkv * t * wl.row_bytes()
    q = wl.batch * wl.hq * wl.d * in_b
    out = wl.batch * wl.hq * wl.d * 4
    return cache, q, out


def write_bytes_per_position(wl):
    in_b = 4 if wl.in_dtype == "f32" else 2
    return wl.batch * wl.hkv * 2 * (wl.d * in_b + wl.row_bytes())


# source files of each decode kernel (the recorded HBM counters hold for these bytes)
KERNEL_SOURCES = {
    "per_head": ["okv_decode_head.hip", "okv_decode_common.hpp", "okv_device.hpp"],
    "grouped": ["okv_decode_mfma.hip", "okv_decode_common.hpp", "okv_device.hpp"],
}


def recorded_traffic(wl, kernel):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3 counter
    record (profiles/traffic_<workload>.txt: FETCH_SIZE and WRITE_SIZE scaled by a
    calibration copy), or None when there is none or the kernel source has changed
    since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.txt")
    if not os.path.exists(path):
        return None
    rec = json.loads(open(path).read())
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "decode_attention_okv_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return int(rec["read_bytes"]) + int(rec["write_bytes"])


def prefill_attn_leg(name, rows, reps=5):
    """Chunked-prefill attention over the packed cache: the last `rows` positions of a
    full context attend causally (okv_prefill_attn).  Algorithmic work: 4 d flops per
    (query head, causal query-key pair), QK^T and P.V; the kernel issues each product
    twice (float16 hi + lo), which the f16 MFMA peak fraction does not count."""
    import numpy as np
    import torch

    import decode_attention_okv_amd as okv
    import okv_synth
    wl = okv_synth.workload(name)
    t = wl.tokens
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    cache = okv.OkvCache(batch=wl.batch, num_q_heads=wl.hq, num_kv_heads=wl.hkv, head_dim=wl.d,
                         max_tokens=t, block=wl.block, quant=wl.quant, scale_dtype=wl.scale_dtype,
                         in_dtype=wl.in_dtype, rotation=wl.rotation, eps=wl.eps, rot_params=p32,
                         device="cuda")
    step = 4096
    for pos in range(0, t, step):
        k, v = okv_synth.kv_tokens(wl, pos, min(step, t - pos), device="cuda")
        cache.write(k, v)
    q = okv_synth.query_rows(wl, t - rows, rows, device="cuda")
    out = torch.empty((wl.batch, rows, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    cache.prefill_attn(q, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        cache.prefill_attn(q, out=out)
    e1.record()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ms = e0.elapsed_time(e1) / reps
    pairs = rows * (t - rows) + rows * (rows + 1) // 2
    flops = 4.0 * wl.d * wl.hq * wl.batch * pairs
    cache.close()
    return {
        "workload": wl.name, "context": t, "rows": rows, "calls": reps, "ms": round(ms, 3),
        "tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 1),
        "frac_f16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS, 4),
    }


def variant_leg(wl, calls=10, **over):
    """One variant of the workload (another code width, rotation or block): write the
    context (timed with events around all write calls), then time `calls` decode calls
    at full length with HIP events on the attention kernel's own dispatch."""
    import numpy as np
    import torch

    import decode_attention_okv_amd as okv
    import okv_synth
    wb = wl.with_(**over)
    t = wb.tokens
    p32 = okv_synth.rotation_params(wb, dtype=np.float32)
    cache = okv.OkvCache(batch=wb.batch, num_q_heads=wb.hq, num_kv_heads=wb.hkv, head_dim=wb.d,
                         max_tokens=t, block=wb.block, quant=wb.quant, scale_dtype=wb.scale_dtype,
                         in_dtype=wb.in_dtype, rotation=wb.rotation, eps=wb.eps, rot_params=p32,
                         device="cuda", bits=wb.bits)
    step = 16384
    chunks = [okv_synth.kv_tokens(wb, pos, min(step, t - pos), device="cuda") for pos in range(0, t, step)]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k, v in chunks:
        cache.write(k, v)
    e1.record()
    torch.cuda.synchronize()
    write_ms = e0.elapsed_time(e1)
    del chunks
    q = okv_synth.queries(wb, 0, device="cuda")
    out = torch.empty((wb.batch, wb.hq, wb.d), dtype=torch.float32, device="cuda")
    for _ in range(3):
        cache.decode_attn(q, out)
    torch.cuda.synchronize()
    cache.timing(True)
    for _ in range(calls):
        cache.decode_attn(q, out)
    torch.cuda.synchronize()
    n, attn_ms, red_ms = cache.timing_read()
    cache.timing(False)
    assert n == calls and torch.isfinite(out).all()
    kern = cache.decode_kernel()
    cache.close()
    torch.cuda.empty_cache()
    byt = sum(algorithmic_decode_bytes(wb, t)[:2])
    us = 1e3 * attn_ms / calls
    return {**over, "decode_kernel": kern, "decode_kernel_us": round(us, 2),
            "reduce_kernel_us": round(1e3 * red_ms / calls, 2), "bytes_per_call": byt,
            "achieved_GBs": round(byt / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "write_ms": round(write_ms, 3),
            "write_GBs": round(write_bytes_per_position(wb) * t / (write_ms * 1e-3) / 1e9, 1)}


def calibration_leg(name="so4_d256_b32_t8k", n=16384, sweeps=4, n_cand=16):
    """SO(4) calibration (okv_so4_calibrate) on n key vectors of the workload (KV head 0
    of sequences 0, 1, ...): wall time of the call, which runs sweeps x d/4 search steps
    of n_cand candidate evaluations over all n vectors, and the error it removes."""
    import numpy as np
    import torch

    import decode_attention_okv_amd as okv
    import okv_synth
    wl = okv_synth.workload(name)
    t = min(n, wl.tokens)
    k, _ = okv_synth.kv_tokens(wl.with_(batch=-(-n // t)), 0, t, device="cuda")
    x = k[:, :, 0].float().reshape(-1, wl.d)[:n].contiguous()
    del k
    rot0 = okv_synth.rotation_params(wl.with_(rotation="so4"))
    cand = okv_synth.so4_candidates(wl.d, sweeps, n_cand)
    okv.so4_calibrate(x, rot0, cand[:1, :, :2], block=wl.block, bits=wl.bits, eps=wl.eps)   # load
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, trace = okv.so4_calibrate(x, rot0, cand, block=wl.block, bits=wl.bits, eps=wl.eps)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0)
    steps = sweeps * wl.d // 4
    return {"workload": wl.name, "vectors": n, "head_dim": wl.d, "block": wl.block, "sweeps": sweeps,
            "candidates": n_cand, "ms": round(ms, 2), "us_per_step": round(1e3 * ms / steps, 1),
            "error_before": round(float(trace[0]), 1), "error_after": round(float(trace[-1]), 1)}


def cpu_baseline(wl, target_s=12.0):
    """Time the CPU oracle's decode on (sequence, KV head) units of the workload at
    its full context length (same distributions; values drawn on the host)."""
    import numpy as np

    import okv_synth
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    unit = wl.with_(batch=1, hkv=1, hq=wl.group)
    p32 = okv_synth.rotation_params(unit, dtype=np.float32)
    u = oracle.rotation_matrix(unit.rotation, p32.astype(np.float64), unit.d)
    k, v = okv_synth.kv_tokens(unit, 0, unit.tokens)
    ref = oracle.write_unit(okv_synth.host_f32(k)[0, :, 0], okv_synth.host_f32(v)[0, :, 0], unit, p32)
    q = okv_synth.host_f32(okv_synth.queries(unit, 0))[0]
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.attend_unit(q, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"],
                           unit.tokens, unit, u)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s or n >= 64:
            break
    unit_bytes = 2 * unit.tokens * unit.row_bytes()
    # write path: the oracle's bit-exact float32 rotation, quantisation and packing of
    # every key and value vector of the unit (about a second of CPU work at 128K)
    nw = unit.tokens
    kh, vh = okv_synth.host_f32(k)[0, :nw, 0], okv_synth.host_f32(v)[0, :nw, 0]
    tw = time.perf_counter()
    oracle.write_unit(kh, vh, unit, p32)
    elw = time.perf_counter() - tw
    hv_s = 2 * nw / elw                      # head vectors (keys and values) per second
    return {
        "value": round(n * unit_bytes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} decode call(s) of one (sequence, KV head) unit: {unit.group} query head(s) "
                  f"over {unit.tokens} tokens (NumPy, float64 attention from packed codes), "
                  f"{el:.1f} s; BLAS threads {threads}, unpack/dequantise single-threaded",
        "write_head_vectors_per_s": round(hv_s, 1),
        "write_tokens_per_s": round(hv_s / (2 * wl.hkv), 2),
        "write_sample": f"okv_write of {nw} key and {nw} value vectors of one unit (NumPy float32 "
                        f"bit-exact path, {elw:.2f} s); a token is one position of one sequence: "
                        f"tokens/s = head vectors/s / (2 x {wl.hkv} KV heads)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mha_b4h32_t128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--prefill-workload", default="gqa_h32kv8_t32k",
                    help="workload of the chunked-prefill attention leg ('' to skip)")
    ap.add_argument("--prefill-rows", type=int, default=2048)
    ap.add_argument("--widths", default="2,4",
                    help="other code widths to time decode at on the same workload ('' to skip)")
    ap.add_argument("--calibration", type=int, default=1,
                    help="also time the SO(4) calibration on 16,384 key vectors (0 to skip)")
    ap.add_argument("--rotations", type=int, default=1,
                    help="also time the unrotated per-token variant and U = B H (0 to skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "copies": 5}))
        return

    import decode_attention_okv_amd as okv
    import okv_synth

    wl = okv_synth.workload(args.workload)
    W, K = args.warmup, args.steps
    T0 = wl.tokens
    cap = -(-(T0 + W + K + 1) // 32) * 32
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cache = okv.OkvCache(batch=wl.batch, num_q_heads=wl.hq, num_kv_heads=wl.hkv, head_dim=wl.d,
                         max_tokens=cap, block=wl.block, quant=wl.quant, scale_dtype=wl.scale_dtype,
                         in_dtype=wl.in_dtype, rotation=wl.rotation, eps=wl.eps, rot_params=p32,
                         device=dev)
    if args.splits:
        cache.set_splits(args.splits)

    # ---- prefill (timed separately: okv_write tokens/s).  One untimed prefill loads
    # the kernels; the cache is then rewound and written again under the timer.
    k, v = okv_synth.kv_tokens(wl, 0, T0, device=dev)
    cache.write(k, v)
    cache.set_length(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    cache.write(k, v)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    del k, v
    torch.cuda.empty_cache()
    print(f"# prefill {T0} tokens x {wl.batch} seq: {prefill_ms:.3f} ms", file=sys.stderr, flush=True)

    # ---- decode steps: inputs resident before timing
    steps = W + K
    news = [okv_synth.kv_tokens(wl, T0 + i, 1, device=dev, step=i) for i in range(steps)]
    qs = [okv_synth.queries(wl, i, device=dev) for i in range(steps)]
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    # Two schedules of a step.  "overlapped": the one-token append runs on its own stream,
    # concurrently with the previous step's decode (the append writes position len only
    # and rewrites the earlier codes of the current value tile unchanged; the decode
    # reads positions < len), and the step's decode waits for it.  "serial": both on one
    # stream.  The overlap hides the append when the GPU is the bottleneck; its extra
    # event calls cost host time, which bounds short steps.  The warm-up measures the GPU
    # time of a serial step and the host time to issue an overlapped one, and overlaps
    # only while the host keeps well ahead of the GPU.  Both streams keep the default
    # priority.
    s_main = torch.cuda.current_stream()
    s_app = torch.cuda.Stream()
    app_done = [torch.cuda.Event() for _ in range(steps)]

    def step(i, overlapped):
        if overlapped:
            cache.write(*news[i], stream=s_app)
            app_done[i].record(s_app)
            s_main.wait_event(app_done[i])
        else:
            cache.write(*news[i], stream=s_main)
        cache.decode_attn(qs[i], out, stream=s_main)

    overlap = False
    if W >= 4:
        step(0, False)                  # first uses of both schedules: kernel loading,
        step(1, True)                   # stream and event set-up
        half = 2 + (W - 2) // 2
        torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for i in range(2, half):
            step(i, False)
        w1.record()
        torch.cuda.synchronize()
        gpu_step_ms = w0.elapsed_time(w1) / (half - 2)
        h0 = time.perf_counter()
        for i in range(half, W):
            step(i, True)
        host_step_ms = 1e3 * (time.perf_counter() - h0) / (W - half)
        overlap = host_step_ms < 0.5 * gpu_step_ms
    else:
        for i in range(W):
            step(i, False)
    torch.cuda.synchronize()
    splits = cache.splits()
    kernel = cache.decode_kernel()
    ts, te = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts.record()
    s_app.wait_event(ts)
    for i in range(W, steps):
        step(i, overlap)
    te.record()
    torch.cuda.synchronize()
    step_ms_total = ts.elapsed_time(te)
    assert torch.isfinite(out).all()
    # attention-kernel duration: K more decode calls back to back at the final
    # length, with HIP events attached to the kernel's own dispatch
    t_fin = T0 + steps
    cache.timing(True)
    for i in range(K):
        cache.decode_attn(qs[W + i], out)
    torch.cuda.synchronize()
    ncalls, attn_ms, red_ms = cache.timing_read()
    cache.timing(False)
    assert ncalls == K, (ncalls, K)

    lens = [T0 + i + 1 for i in range(W, steps)]
    tot_bytes = sum(sum(algorithmic_decode_bytes(wl, t)) for t in lens)
    value = tot_bytes / (step_ms_total * 1e-3) / 1e9
    kern_bytes = K * (algorithmic_decode_bytes(wl, t_fin)[0] + algorithmic_decode_bytes(wl, t_fin)[1])
    achieved = kern_bytes / (attn_ms * 1e-3) / 1e9
    write_tok_s = wl.batch * T0 / (prefill_ms * 1e-3)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_ms_total / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.hq, "kv_heads": wl.hkv,
                   "head_dim": wl.d, "context": T0, "quant": wl.quant, "block": wl.block,
                   "scale_dtype": wl.scale_dtype, "rotation": wl.rotation, "splits": splits},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_kernel_us": round(1e3 * attn_ms / K, 2),
        "reduce_kernel_us": round(1e3 * red_ms / K, 2),
        "write_tokens_per_s": round(write_tok_s, 1),
        "write_head_vectors_per_s": round(write_tok_s * 2 * wl.hkv, 1),
        "write_prefill_ms": round(prefill_ms, 3),
        "write_prefill_GBs": round(write_bytes_per_position(wl) * T0 / (prefill_ms * 1e-3) / 1e9, 2),
        "decode_kernel": kernel,
        "append_schedule": "overlapped" if overlap else "serial",
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(wl, kernel),
        },
    }
    cache.close()
    del cache, news, qs, out
    torch.cuda.empty_cache()
    if args.widths:
        res["code_widths"] = [variant_leg(wl, bits=int(b)) for b in args.widths.split(",")]
    if args.rotations:
        # the unrotated per-token baseline and U = B H (the Hadamard-only variant is the
        # sign rotation with D = I: same kernels and bytes as the headline)
        res["rotations"] = [variant_leg(wl, rotation="none", block=wl.d), variant_leg(wl, rotation="so4")]
    if args.prefill_workload:
        res["prefill_attn"] = prefill_attn_leg(args.prefill_workload, args.prefill_rows)
    if args.calibration:
        res["so4_calibration"] = calibration_leg()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
