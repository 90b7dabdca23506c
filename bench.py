"""Benchmark of the rotated 3-bit KV cache on one MI355X.

A step is one pass of the whole hot path over one batch, in the order an
autoregressive decoder runs it: okv_write appends one new token per sequence
(rotate, quantise, pack), then okv_decode_attn attends with one query per
(sequence, query head) over the whole cache (rotate q, fused unpack / scale / dot,
online softmax, P.V, split-K reduce, rotate back).  Both run on one stream, one after
the other (the next token would depend on this step's output).

Default workload: 7B MHA shape at 128K context (batch 4, 32 heads, d 128, 131,072
cached tokens per sequence, 8.3 % outlier channels, block 32, fp16 scales).  Prints
one JSON line.  `value` is decode-attention GB/s over the algorithmic bytes of the
packed cache (codes + scales read, q read, output written), timed over whole serial
steps (append + decode + merge + launch gaps).  Extra objects on the same line:
"decode_call" (the decode call alone, back to back), "workloads" (the 70B-shaped
asymmetric 128K decode, the 32K GQA append-and-decode steps, the SO(4) d = 256
prefill write and decode, the tiny one-head case), "hbm_read_probe" (a plain
streaming-read kernel on the same GPU), "prefill_attn" (chunked-prefill attention
over the packed cache), "code_widths" and "rotations" (2-/4-bit codes, the
unrotated and SO(4) variants on the headline workload), "so4_calibration",
"cpu_baseline" (the CPU oracle on a bounded sample), "oracle_spot_check" (the oracle's
write and decode of one (sequence, KV head) of the timed cache, compared with the
library's bytes and output) and "gpu_under_load" (the
firmware's clock, power and temperature tables during 2.5 s of untimed decode calls on
the headline and the asymmetric 128K workloads, after every timed leg).
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


def prefill_attn_leg(name, rows, reps=5, settle_s=1.5):
    """Chunked-prefill attention over the packed cache: the last `rows` positions of a
    full context attend causally (okv_prefill_attn).  Algorithmic work: 4 d flops per
    (query head, causal query-key pair), QK^T and P.V; the kernel issues the products
    two or three times (float16 hi + lo parts), which the f16 MFMA peak fraction does
    not count.  `ms` is the median of 2 reps calls after `settle_s` seconds of untimed
    calls; `ms_first_calls` the mean of the first `reps` calls after one untimed call."""
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

    def timed(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            cache.prefill_attn(q, out=out)
            ev[i + 1].record()
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))

    first = timed(reps)
    # then untimed calls for `settle_s` seconds, so that the timed calls run at the
    # clocks the GPU holds under this load, as for the decode legs
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        timed(10)
    ms = timed(2 * reps)[reps]
    assert torch.isfinite(out).all()
    pairs = rows * (t - rows) + rows * (rows + 1) // 2
    flops = 4.0 * wl.d * wl.hq * wl.batch * pairs
    cache.close()
    return {
        "workload": wl.name, "context": t, "rows": rows, "calls": 2 * reps, "ms": round(ms, 3),
        "ms_first_calls": round(sum(first) / reps, 3), "settle_s": settle_s,
        "tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 1),
        "frac_f16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS, 4),
    }


def variant_leg(wl, calls=10, settle_ms=0.0, **over):
    """One variant of the workload (another code width, rotation or block): write the
    context (timed with events around all write calls), then, after `settle_ms` of
    untimed decode calls, time `calls` decode calls at full length with HIP events on
    the attention kernel's own dispatch."""
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
    if settle_ms > 0:
        settle(cache, q, out, settle_ms)
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


def capture_unit(cache, wl, unit_kv, news, q, out):
    """Host copies, for the oracle spot check, of (sequence 0, KV head 0) of the timed
    cache at its final length: the raw keys and values written (prefill and every
    append, in order), the cache bytes, and the last decode call's query and output for
    the KV head's query heads."""
    import numpy as np

    import okv_synth
    t, g = cache.length, wl.group
    ntile = -(-t // 32)
    app_k = np.stack([okv_synth.host_f32(n[0][0, 0, 0]) for n in news])
    app_v = np.stack([okv_synth.host_f32(n[1][0, 0, 0]) for n in news])
    assert unit_kv["k"].shape[0] + app_k.shape[0] == t, (unit_kv["k"].shape, app_k.shape, t)
    return {"t": t, "k": np.concatenate([unit_kv["k"], app_k]), "v": np.concatenate([unit_kv["v"], app_v]),
            "k_codes": cache.k_codes[0, 0, :t].cpu().numpy(), "v_codes": cache.v_codes[0, 0, :ntile].cpu().numpy(),
            "k_meta": cache.k_meta[0, 0, :t].cpu().numpy(), "v_meta": cache.v_meta[0, 0, :t].cpu().numpy(),
            "q": okv_synth.host_f32(q)[0, :g], "y": out[0, :g].cpu().numpy()}


def oracle_spot_check(wl, spot):
    """The CPU oracle's write of the captured unit's raw keys and values, compared byte
    for byte with the library's cache of that unit; the exact rounding ties among its
    values (a rotated value on a threshold of its stored scale); and the oracle's decode
    of the last query against the library's output (max |y - y_ref| / RMS(y_ref))."""
    import numpy as np

    import okv_synth
    import oracle
    unit = wl.with_(batch=1, hkv=1, hq=wl.group)
    p32 = okv_synth.rotation_params(unit, dtype=np.float32)
    u = oracle.rotation_matrix(unit.rotation, p32.astype(np.float64), unit.d)
    t0 = time.perf_counter()
    ref = oracle.write_unit(spot["k"], spot["v"], unit, p32)
    mism = {}
    for key in ("k_codes", "v_codes", "k_meta", "v_meta"):
        a = np.ascontiguousarray(spot[key]).view(np.uint8)
        b = np.ascontiguousarray(np.asarray(ref[key])).view(np.uint8)
        mism[key] = int(np.count_nonzero(a != b)) if a.shape == b.shape else -1
    ties = 0
    for key, mkey in (("k_rot", "k_meta"), ("v_rot", "v_meta")):
        y = ref[key].astype(np.float64)
        sc, off = oracle.meta_values(ref[mkey], unit)
        yb = y.reshape(y.shape[0], unit.d // unit.block, unit.block)
        if unit.quant == "sym":
            x = yb / sc[..., None]
        else:
            x = (yb.astype(np.float32) - off[..., None].astype(np.float32)).astype(np.float64) / sc[..., None]
        with np.errstate(invalid="ignore", divide="ignore"):
            ties += int(np.count_nonzero(x - np.floor(x) == 0.5))
    y_ref = oracle.attend_unit(spot["q"], ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"],
                               spot["t"], unit, u)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.abs(spot["y"].astype(np.float64) - y_ref).max() / rms)
    return {"unit": "sequence 0, KV head 0 of the timed cache", "tokens": spot["t"],
            "byte_mismatches": mism, "exact_ties": ties, "decode_max_err_over_rms": float("%.3g" % err),
            "bound": 2e-3, "ok": all(v == 0 for v in mism.values()) and err <= 2e-3,
            "oracle_s": round(time.perf_counter() - t0, 1)}


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


def new_cache(wl, cap, dev, bits=None):
    import numpy as np

    import decode_attention_okv_amd as okv
    import okv_synth
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    return okv.OkvCache(batch=wl.batch, num_q_heads=wl.hq, num_kv_heads=wl.hkv, head_dim=wl.d,
                        max_tokens=cap, block=wl.block, quant=wl.quant, scale_dtype=wl.scale_dtype,
                        in_dtype=wl.in_dtype, rotation=wl.rotation, eps=wl.eps, rot_params=p32,
                        device=dev, bits=wl.bits if bits is None else bits)


def timed_prefill(cache, wl, dev, warm=20, reps=10, keep_unit=None):
    """okv_write of the workload's whole context in one call.  A first untimed call on
    the first 32 positions loads the kernel; the first whole write is timed on its own
    (the GPU comes from idle), then `warm` untimed and `reps` timed whole writes, each
    rewinding the cache to 0 first (the same work every time: the clocks pass through
    the same transient as for decode calls, and settle within about 20 writes).
    Returns (median ms of the timed writes, ms of the first one).  `keep_unit`, a dict,
    receives float32 host copies of the keys and values of (sequence 0, KV head 0)."""
    import torch

    import okv_synth
    k, v = okv_synth.kv_tokens(wl, 0, wl.tokens, device=dev)
    if keep_unit is not None:
        keep_unit["k"], keep_unit["v"] = okv_synth.host_f32(k[0, :, 0]), okv_synth.host_f32(v[0, :, 0])
    cache.write(k[:, :32].contiguous(), v[:, :32].contiguous())
    torch.cuda.synchronize()

    def once():
        cache.set_length(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.write(k, v)
        e1.record()
        return e0, e1

    first = once()
    torch.cuda.synchronize()
    for _ in range(warm):
        cache.set_length(0)
        cache.write(k, v)
    evs = [once() for _ in range(reps)]
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    del k, v
    torch.cuda.empty_cache()
    return ms[len(ms) // 2], first[0].elapsed_time(first[1])


def write_record(wl, ms_pair):
    """Write-path rates of a prefill of wl.tokens positions per sequence (the median of
    the timed writes), and the first write's time."""
    ms, first = ms_pair
    pos_s = wl.batch * wl.tokens / (ms * 1e-3)
    return {"write_prefill_ms": round(ms, 3), "write_prefill_first_ms": round(first, 3),
            "write_tokens_per_s": round(pos_s, 1),
            "write_head_vectors_per_s": round(pos_s * 2 * wl.hkv, 1),
            "write_GBs": round(write_bytes_per_position(wl) * wl.tokens / (ms * 1e-3) / 1e9, 1)}


class GpuMonitor:
    """Clock, power and temperature of the benchmarked GPU from the power-management
    firmware's metrics table (amdsmi, read-only; no HIP call).  The firmware refreshes
    that table about once a second, so a daemon thread polls it while sustained untimed
    work runs (never inside a timed region) and keeps each fresh table (a new firmware
    timestamp).  If amdsmi is missing, cannot see the GPU, or does not answer within two
    seconds, the record says so and the benchmark goes on."""

    def __init__(self, pci):
        import threading
        self.pci, self.err, self.h = tuple(pci), None, None
        self.samples, self.last_ts, self.on = [], None, threading.Event()
        self.ready, self.stop = threading.Event(), threading.Event()
        threading.Thread(target=self._run, daemon=True).start()
        if not self.ready.wait(2.0):
            self.err = "amdsmi did not answer within 2 s"

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            for h in amdsmi.amdsmi_get_processor_handles():
                # "domain:bus:device.function", hexadecimal
                dom, bus, dev_fn = str(amdsmi.amdsmi_get_gpu_device_bdf(h)).split(":")
                if (int(dom, 16), int(bus, 16), int(dev_fn.split(".")[0], 16)) == self.pci:
                    self.h = h
                    break
            if self.h is None:
                raise RuntimeError("no amdsmi device at PCI %04x:%02x:%02x" % self.pci)
            self.get = amdsmi.amdsmi_get_gpu_metrics_info
            self.idle = self._read()[1]
        except Exception as e:   # noqa: BLE001 - any failure only disables the record
            self.err = " ".join(f"{type(e).__name__}: {e}".split())[:200]
        self.ready.set()
        while self.h is not None and not self.stop.is_set():
            if self.on.wait(0.5) and not self.stop.is_set():
                try:
                    ts, rec = self._read()
                    if ts != self.last_ts:
                        self.last_ts = ts
                        self.samples.append(rec)
                except Exception:   # noqa: BLE001
                    pass
                time.sleep(0.005)

    def _read(self):
        m = self.get(self.h)
        clk = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 65535]

        def num(k):
            v = m.get(k)
            return v if isinstance(v, int) and 0 <= v < 65535 else None
        return m.get("firmware_timestamp"), {
            "gfxclk_mhz_per_xcd": clk, "socket_power_w": num("current_socket_power"),
            "hotspot_c": num("temperature_hotspot"), "mem_c": num("temperature_mem")}

    def start(self):
        self.samples = []
        if self.h is not None:
            try:
                self.last_ts = self._read()[0]     # the table current now predates the load
            except Exception:   # noqa: BLE001 - a failed read only loses this table
                self.last_ts = None
        self.on.set()

    def record(self):
        """Stop polling; the fresh tables seen since start()."""
        self.on.clear()
        time.sleep(0.01)
        if self.err or self.h is None:
            return {"unavailable": self.err or "no device"}
        return {"idle_before": self.idle, "tables_under_load": list(self.samples)}

    def close(self):
        self.stop.set()
        self.on.set()


def gpu_clock_leg(name, dev, seconds=2.5):
    """The workload's cache (prefill untimed), then untimed decode calls back to back for
    `seconds` of wall time while the monitor collects the firmware's tables: the clock
    and power the GPU holds under this load.  Runs after every timed leg."""
    import torch

    import okv_synth
    wl = okv_synth.workload(name)
    print(f"# leg {name}: {seconds} s of decode calls, clock and power", file=sys.stderr, flush=True)
    cache = new_cache(wl, -(-(wl.tokens + 32) // 32) * 32, dev)
    k, v = okv_synth.kv_tokens(wl, 0, wl.tokens, device=dev)
    cache.write(k, v)
    del k, v
    q = okv_synth.queries(wl, 0, device=dev)
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    MONITOR.start()
    t_end, n = time.perf_counter() + seconds, 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            cache.decode_attn(q, out)
        torch.cuda.synchronize()
        n += 10
    rec = {"workload": name, "decode_kernel": cache.decode_kernel(), "decode_calls": n, **MONITOR.record()}
    cache.close()
    del cache, q, out
    torch.cuda.empty_cache()
    return rec


MONITOR = None


def settle(cache, q, out, ms):
    """Untimed decode calls back to back for about `ms` milliseconds of GPU time, so that
    timed regions start at the steady state a decoder serving continuously runs in.
    Under sustained load the GPU's power management changes its clocks twice: a dip a
    few milliseconds in that recovers after about 10 ms, then a slower rise; on the 128K
    MHA decode the call time settles after about half a second of continuous load (in
    runs of thousands of calls, 297-299 us per call over the first 0.5 s against 287-289
    us after it).  Returns the call count."""
    import torch
    n, el = 0, 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while el < ms:
        e0.record()
        for _ in range(10):
            cache.decode_attn(q, out)
        e1.record()
        torch.cuda.synchronize()
        el += e0.elapsed_time(e1)
        n += 10
    return n


def series_leg(name, dev, n=150):
    """Sustained load: the streaming-read probe, then `n` decode calls of the workload
    back to back, each timed with its own events; GB/s over windows of call indices
    (the clock transient of the first tens of calls shows here)."""
    import numpy as np
    import torch

    import decode_attention_okv_amd as okv
    import okv_synth
    wl = okv_synth.workload(name)
    cache = new_cache(wl, -(-(wl.tokens + 32) // 32) * 32, dev)
    timed_prefill(cache, wl, dev)
    q = okv_synth.queries(wl, 0, device=dev)
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    nb = 2 << 30
    buf = torch.ones(nb // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def run(fn, k):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
        ev[0].record()
        for i in range(k):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(k)])

    okv.read_probe(buf, sink)
    cache.decode_attn(q, out)
    torch.cuda.synchronize()
    time.sleep(2.0)
    tp = run(lambda: okv.read_probe(buf, sink), 100)
    time.sleep(2.0)
    td = run(lambda: cache.decode_attn(q, out), n)
    byt = sum(algorithmic_decode_bytes(wl, wl.tokens))
    wins = [(1, 6), (10, 20), (20, 40), (40, 60), (n - 20, n)]
    rec = {"workload": name, "calls": n,
           "probe_GBs": round(nb / (float(np.mean(tp)) * 1e-3) / 1e9, 1),
           "decode_GBs_by_call": {f"{a}-{b}": round(byt / (float(np.mean(td[a:b])) * 1e-3) / 1e9, 1) for a, b in wins},
           "decode_us_by_call": {f"{a}-{b}": round(1e3 * float(np.mean(td[a:b])), 1) for a, b in wins}}
    cache.close()
    del buf, cache
    torch.cuda.empty_cache()
    return rec


def decode_calls(cache, wl, q, out, calls):
    """`calls` okv_decode_attn calls back to back at the current length, twice: bare,
    with torch events around the loop (whole call: attention + merge + gaps), then with
    the library's HIP events on each kernel's own dispatch (kernel durations; those
    events add launch gaps, so they stay out of the first loop).  Returns (call_us,
    attn_kernel_us, reduce_kernel_us)."""
    import torch
    for _ in range(2):
        cache.decode_attn(q, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        cache.decode_attn(q, out)
    e1.record()
    torch.cuda.synchronize()
    cache.timing(True)
    for _ in range(calls):
        cache.decode_attn(q, out)
    torch.cuda.synchronize()
    n, attn_ms, red_ms = cache.timing_read()
    cache.timing(False)
    assert n == calls and torch.isfinite(out).all(), (n, calls)
    return 1e3 * e0.elapsed_time(e1) / calls, 1e3 * attn_ms / calls, 1e3 * red_ms / calls


def decode_record(wl, t, call_us, attn_us, red_us, kernel, splits):
    cache_b, qb, ob = algorithmic_decode_bytes(wl, t)
    kern_b = cache_b + qb
    return {"decode_kernel": kernel, "splits": splits, "context": t,
            "decode_call_us": round(call_us, 2), "decode_kernel_us": round(attn_us, 2),
            "reduce_kernel_us": round(red_us, 2),
            "call_GBs": round((kern_b + ob) / (call_us * 1e-6) / 1e9, 1),
            "kernel_GBs": round(kern_b / (attn_us * 1e-6) / 1e9, 1),
            "kernel_frac_hbm_peak": round(kern_b / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "call_frac_hbm_peak": round((kern_b + ob) / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def decode_workload_leg(name, dev, calls=100, settle_ms=0.0):
    """A decode workload at its full size: prefill write (timed), then `calls` decode
    calls back to back.  Reports write rates, decode call / kernel times, GB/s and the
    fraction of the HBM peak, and the recorded HBM traffic of the decode kernel."""
    import torch

    import okv_synth
    wl = okv_synth.workload(name)
    print(f"# leg {name}: prefill write", file=sys.stderr, flush=True)
    cache = new_cache(wl, -(-(wl.tokens + 32) // 32) * 32, dev)
    ms = timed_prefill(cache, wl, dev)
    q = okv_synth.queries(wl, 0, device=dev)
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    print(f"# leg {name}: decode x {calls}", file=sys.stderr, flush=True)
    if settle_ms > 0:
        settle(cache, q, out, settle_ms)
    call_us, attn_us, red_us = decode_calls(cache, wl, q, out, calls)
    kern = cache.decode_kernel()
    rec = {"workload": name, "batch": wl.batch, "q_heads": wl.hq, "kv_heads": wl.hkv, "head_dim": wl.d,
           "quant": wl.quant, "block": wl.block, "scale_dtype": wl.scale_dtype, "rotation": wl.rotation,
           **decode_record(wl, wl.tokens, call_us, attn_us, red_us, kern, cache.splits()),
           "traffic": recorded_traffic(wl, kern), **write_record(wl, ms)}
    cache.close()
    del cache, q, out
    torch.cuda.empty_cache()
    return rec


def steps_leg(name, dev, settle_ms=0.0):
    """The 32K GQA workload as its configuration runs it: prefill write (timed), then,
    after `settle_ms` of untimed decode calls, wl.decode_steps serial steps of (append
    one token, decode), timed as a whole."""
    import torch

    import okv_synth
    wl = okv_synth.workload(name)
    n = wl.decode_steps
    print(f"# leg {name}: prefill write, {n} steps", file=sys.stderr, flush=True)
    cache = new_cache(wl, -(-(wl.tokens + n + 34) // 32) * 32, dev)
    ms = timed_prefill(cache, wl, dev)
    news = [okv_synth.kv_tokens(wl, wl.tokens + i, 1, device=dev, step=i) for i in range(n + 2)]
    qs = [okv_synth.queries(wl, i, device=dev) for i in range(n + 2)]
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    if settle_ms > 0:
        settle(cache, qs[0], out, settle_ms)
    for i in range(2):                      # warm-up steps (appended tokens stay)
        cache.write(*news[i])
        cache.decode_attn(qs[i], out)
    torch.cuda.synchronize()
    t_start = cache.length
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(2, n + 2):
        cache.write(*news[i])
        cache.decode_attn(qs[i], out)
    e1.record()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    step_ms = e0.elapsed_time(e1) / n
    byt = sum(sum(algorithmic_decode_bytes(wl, t_start + i + 1)) for i in range(n))
    call_us, attn_us, red_us = decode_calls(cache, wl, qs[-1], out, 20)
    rec = {"workload": name, "batch": wl.batch, "q_heads": wl.hq, "kv_heads": wl.hkv, "head_dim": wl.d,
           "steps": n, "step_us": round(1e3 * step_ms, 2),
           "step_GBs": round(byt / (step_ms * 1e-3 * n) / 1e9, 1),
           **decode_record(wl, cache.length, call_us, attn_us, red_us, cache.decode_kernel(), cache.splits()),
           "traffic": recorded_traffic(wl, cache.decode_kernel()), **write_record(wl, ms),
           "note": "the 29 MB cache fits the GPU's last-level cache: not an HBM figure"}
    cache.close()
    del cache, news, qs, out
    torch.cuda.empty_cache()
    return rec


def tiny_leg(dev, reps=20):
    """The one-head d = 128 case: write its 256 tokens, then one decode; latency of
    each (median of `reps` repetitions, the cache rewound in between)."""
    import torch

    import okv_synth
    wl = okv_synth.workload("tiny_d128_t256")
    cache = new_cache(wl, 288, dev)
    k, v = okv_synth.kv_tokens(wl, 0, wl.tokens, device=dev)
    q = okv_synth.queries(wl, 0, device=dev)
    out = torch.empty((1, 1, wl.d), dtype=torch.float32, device=dev)
    wr, dc = [], []
    for _ in range(reps + 2):
        cache.set_length(0)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        cache.write(k, v)
        e[1].record()
        cache.decode_attn(q, out)
        e[2].record()
        torch.cuda.synchronize()
        wr.append(e[0].elapsed_time(e[1]))
        dc.append(e[1].elapsed_time(e[2]))
    cache.close()
    wr, dc = sorted(wr[2:]), sorted(dc[2:])
    return {"workload": wl.name, "write_256_us": round(1e3 * wr[len(wr) // 2], 2),
            "decode_us": round(1e3 * dc[len(dc) // 2], 2), "reps": reps,
            "note": "latency only (32 KiB cache)"}


def read_probe_leg(dev, gib=2, reps=10):
    """okv_read_probe: a plain streaming-read kernel over `gib` GiB, the HBM read rate
    a simple kernel reaches on this GPU (best and median of `reps` launches)."""
    import torch

    import decode_attention_okv_amd as okv
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    okv.read_probe(buf, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        okv.read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    del buf
    torch.cuda.empty_cache()
    return {"bytes": n, "launches": reps, "best_GBs": round(n / (ts[0] * 1e-3) / 1e9, 1),
            "median_GBs": round(n / (ts[len(ts) // 2] * 1e-3) / 1e9, 1),
            "frac_hbm_peak_best": round(n / (ts[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mha_b4h32_t128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--legs", default="gqa_b16h64kv8_t128k_asym,gqa_h32kv8_t32k,so4_d256_b32_t8k,tiny_d128_t256",
                    help="other workloads to run at full size ('' to skip)")
    ap.add_argument("--read-probe", type=int, default=1, help="run the streaming-read probe (0 to skip)")
    ap.add_argument("--series", type=int, default=0,
                    help="also time this many back-to-back decode calls one by one after the probe "
                         "(the clock transient under sustained load; 0 to skip)")
    ap.add_argument("--gpu-monitor", type=int, default=1,
                    help="after the timed regions, 2.5 s of untimed decode calls while the "
                         "firmware's clock / power / temperature tables are read (amdsmi, "
                         "read-only; 0 to skip)")
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="untimed decode calls (GPU milliseconds) before the warm-up steps, until the "
                         "GPU's clocks have settled under the load; the prefill-attention leg runs "
                         "untimed calls for as many wall-clock milliseconds (0 to skip)")
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

    import okv_synth

    wl = okv_synth.workload(args.workload)
    W, K = args.warmup, args.steps
    T0 = wl.tokens
    cap = -(-(T0 + W + 2 * K + 1) // 32) * 32
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    global MONITOR
    if args.gpu_monitor:
        pr = torch.cuda.get_device_properties(0)
        MONITOR = GpuMonitor((pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id))
    cache = new_cache(wl, cap, dev)
    if args.splits:
        cache.set_splits(args.splits)

    # ---- prefill (timed separately: okv_write tokens/s)
    unit_kv = None if args.no_cpu_baseline else {}
    prefill_ms = timed_prefill(cache, wl, dev, keep_unit=unit_kv)
    print(f"# prefill {T0} tokens x {wl.batch} seq: {prefill_ms[0]:.3f} ms (first {prefill_ms[1]:.3f} ms)",
          file=sys.stderr, flush=True)

    # ---- decode steps: inputs resident before timing.  A step appends one token to
    # every sequence, then decodes; one stream, in that order.  The first timed region
    # of K steps, bare, gives `value`.  Then K decode calls back to back at the final
    # length, bare and then with the library's HIP events attached to each kernel's own
    # dispatch: their attention-kernel duration is behind `roofline`.  Last, K more steps
    # with those events (reported apart): there the events' bookkeeping between the
    # append and the decode leaves gaps of tens of microseconds per step, and the decode
    # kernel they bracket reads several per cent slower than the whole bare step allows.
    steps = W + 2 * K
    news = [okv_synth.kv_tokens(wl, T0 + i, 1, device=dev, step=i) for i in range(steps)]
    qs = [okv_synth.queries(wl, i, device=dev) for i in range(steps)]
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)

    def step(i):
        cache.write(*news[i])
        cache.decode_attn(qs[i], out)

    settle_calls = settle(cache, qs[0], out, args.settle_ms) if args.settle_ms > 0 else 0
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    splits = cache.splits()
    kernel = cache.decode_kernel()
    ts, te = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts.record()
    for i in range(W, W + K):
        step(i)
    te.record()
    torch.cuda.synchronize()
    step_ms_total = ts.elapsed_time(te)
    assert torch.isfinite(out).all()
    lens = [T0 + i + 1 for i in range(W, W + K)]
    tot_bytes = sum(sum(algorithmic_decode_bytes(wl, t)) for t in lens)
    value = tot_bytes / (step_ms_total * 1e-3) / 1e9
    # the decode call alone, K calls back to back at the final length
    t_fin = cache.length
    call_us, c_attn_us, c_red_us = decode_calls(cache, wl, qs[W + K - 1], out, K)
    achieved = sum(algorithmic_decode_bytes(wl, t_fin)[:2]) / (c_attn_us * 1e-6) / 1e9
    cache.timing(True)
    t2s, t2e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t2s.record()
    for i in range(W + K, steps):
        step(i)
    t2e.record()
    torch.cuda.synchronize()
    ncalls, attn_ms, red_ms = cache.timing_read()
    cache.timing(False)
    assert ncalls == K, (ncalls, K)
    assert torch.isfinite(out).all()
    spot = None if unit_kv is None else capture_unit(cache, wl, unit_kv, news, qs[steps - 1], out)

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
        "seeds": "okv_synth: NumPy SeedSequence([workload id, stream, ...]) per draw (rotation, "
                 "channel scales, outliers); torch generators seeded from SeedSequence([workload id, "
                 "stream, step + 1, first position]) for keys and values, ([workload id, stream, "
                 "step]) for decode queries",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.hq, "kv_heads": wl.hkv,
                   "head_dim": wl.d, "context": T0, "quant": wl.quant, "block": wl.block,
                   "scale_dtype": wl.scale_dtype, "rotation": wl.rotation, "splits": splits},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_schedule": "serial: append 1 token, then decode, one stream",
        "settle": {"ms": args.settle_ms, "decode_calls": settle_calls},
        "decode_kernel": kernel,
        "decode_kernel_us": round(c_attn_us, 2),
        "reduce_kernel_us": round(c_red_us, 2),
        **write_record(wl, prefill_ms),
        "decode_call": decode_record(wl, t_fin, call_us, c_attn_us, c_red_us, kernel, cache.splits()),
        "steps_with_kernel_events": {"ms_per_step": round(t2s.elapsed_time(t2e) / K, 4),
                                     "decode_kernel_us": round(1e3 * attn_ms / K, 2),
                                     "reduce_kernel_us": round(1e3 * red_ms / K, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(wl, kernel),
            "launches": K,
            "kernel_us": round(c_attn_us, 2),
        },
    }
    cache.close()
    del cache, news, qs, out
    torch.cuda.empty_cache()
    legs = [x for x in args.legs.split(",") if x and x != wl.name]
    if legs:
        res["workloads"] = []
        for name in legs:
            if name == "gqa_h32kv8_t32k":
                res["workloads"].append(steps_leg(name, dev, settle_ms=args.settle_ms))
            elif name == "tiny_d128_t256":
                res["workloads"].append(tiny_leg(dev))
            else:
                res["workloads"].append(decode_workload_leg(name, dev, settle_ms=args.settle_ms))
    if args.read_probe:
        res["hbm_read_probe"] = read_probe_leg(dev)
    if args.series:
        res["sustained_series"] = series_leg(wl.name, dev, args.series)
    if args.widths:
        res["code_widths"] = [variant_leg(wl, settle_ms=args.settle_ms, bits=int(b)) for b in args.widths.split(",")]
    if args.rotations:
        # the unrotated per-token baseline and U = B H (the Hadamard-only variant is the
        # sign rotation with D = I: same kernels and bytes as the headline)
        res["rotations"] = [variant_leg(wl, settle_ms=args.settle_ms, rotation="none", block=wl.d),
                            variant_leg(wl, settle_ms=args.settle_ms, rotation="so4")]
    if args.prefill_workload:
        res["prefill_attn"] = prefill_attn_leg(args.prefill_workload, args.prefill_rows,
                                               settle_s=args.settle_ms / 1000.0)
    if args.calibration:
        res["so4_calibration"] = calibration_leg()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
        res["oracle_spot_check"] = oracle_spot_check(wl, spot)
    if MONITOR is not None:
        if MONITOR.err or MONITOR.h is None:
            res["gpu_under_load"] = {"unavailable": MONITOR.err or "no device"}
        else:
            res["gpu_under_load"] = [gpu_clock_leg(n, dev) for n in
                                     [wl.name] + [x for x in legs if x == "gqa_b16h64kv8_t128k_asym"]]
        MONITOR.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
