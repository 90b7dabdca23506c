"""Quality diagnostics of the rotation variants on the synthetic workloads (CPU,
oracle only; writes a Markdown table to stdout).

    python3 oracle/ablation_report.py [tokens]

Variants (the idea card, Implementation notes: standard per-token 3-bit KV,
Hadamard-only 3-bit KV and Hadamard-plus-SO(4) 3-bit KV; the OIQ report, Section
6.4: the transform without its random sign flip):
  none / per-token    U = I, one scale per token and head (m = d)
  none / m 32         U = I, blocks of 32
  H (D = I)           U = H_d, blocks of 32
  H D                 U = H_d D with random signs, blocks of 32
  B H                 U = B H_d with random SO(4) blocks, blocks of 32
  B H calibrated      the same blocks after the coordinate search (3 sweeps, 12
                      candidates) on held-out keys of the same head
For each: the Gini coefficient of the keys' per-channel magnitudes after U (the
OIQ report, Section 6.1), the worst block maximum of U k relative to its RMS (the
idea card's Verification), the relative reconstruction error of the keys, and the
relative RMSE of decode attention over the packed cache against unquantised
attention (Frobenius over 64 query rows).  Symmetric codes with fp16 scales; b = 3 unless stated.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import okv_synth  # noqa: E402
import oracle  # noqa: E402

VARIANTS = [
    ("none / per-token", dict(rotation="none", block=None), "none"),
    ("none / m 32", dict(rotation="none", block=32), "none"),
    ("H (D = I)", dict(rotation="sign", block=32), "ones"),
    ("H D", dict(rotation="sign", block=32), "seeded"),
    ("B H", dict(rotation="so4", block=32), "seeded"),
    ("B H calibrated", dict(rotation="so4", block=32), "calibrated"),
]


NQ = 64   # query rows per measurement (query head 0 of rows 0 .. 63)


def unit_data(wl, tokens):
    k, v = okv_synth.kv_tokens(wl, 0, tokens)
    q = okv_synth.query_rows(wl, 0, NQ)
    return (okv_synth.host_f32(k)[0, :, 0], okv_synth.host_f32(v)[0, :, 0],
            okv_synth.host_f32(q)[0, :, 0])


def calibrated(wl, tokens, sweeps=3, n_cand=12):
    """SO(4) blocks calibrated by the coordinate search on held-out keys (positions
    tokens .. 2 tokens - 1 of the same KV head), starting from the seeded rotations."""
    w = wl.with_(rotation="so4")
    k, _ = okv_synth.kv_tokens(w, tokens, tokens)
    x = okv_synth.host_f32(k)[0, :, 0]
    rot, _, _ = oracle.calibrate_so4(x, okv_synth.rotation_params(w), okv_synth.so4_candidates(w.d, sweeps, n_cand),
                                     32, w.eps, 3)
    return rot.astype(np.float32)


def row(name, wl, tokens, over, params, bits=3):
    w = wl.with_(rotation=over["rotation"], block=over["block"] or wl.d, bits=bits,
                 scale_dtype="f16", quant="sym")
    k, v, q = unit_data(wl, tokens)
    if params == "ones":
        p32 = np.ones(w.d, np.float32)
    elif params == "calibrated":
        p32 = calibrated(wl, tokens)
    else:
        p32 = okv_synth.rotation_params(w, dtype=np.float32)
    y = oracle.rotate_f32(k, w.rotation, p32)
    ref = oracle.write_unit(k, v, w, p32)
    u = oracle.rotation_matrix(w.rotation, p32.astype(np.float64), w.d)
    k_hat = oracle.dequantize(ref["k_u"], ref["k_meta"], w) @ u    # rows of U^T k1_hat
    rec = float(np.linalg.norm(k_hat - k) / np.linalg.norm(k))
    att = oracle.attention_rel_rmse(q, k, v, w, p32)
    bm = oracle.block_max_stats(y, 32)["worst_over_rms"]
    return (f"| {name} | {bits} | {oracle.channel_gini(y):.3f} | {bm:.2f} | {rec:.4f} | {att:.4f} |")


def main():
    tokens = int(sys.argv[1]) if len(sys.argv) > 1 else 2048
    for wname in ("mha_b4h32_t128k", "gqa_h32kv8_t32k"):
        wl = okv_synth.workload(wname).with_(batch=1, hkv=1, hq=okv_synth.workload(wname).group)
        k, _, _ = unit_data(wl, tokens)
        print(f"\n{wname}: one KV head, {tokens} tokens, {NQ} queries; raw keys: "
              f"channel Gini {oracle.channel_gini(k):.3f}, worst block max / RMS "
              f"{oracle.block_max_stats(k, 32)['worst_over_rms']:.2f}\n")
        print("| variant | b | channel Gini of U k | worst block max / RMS | key rel. error | attention rel. RMSE |")
        print("|---|---|---|---|---|---|")
        for name, over, params in VARIANTS:
            print(row(name, wl, tokens, over, params), flush=True)
        for bits in (2, 4):
            print(row("H D", wl, tokens, dict(rotation="sign", block=32), "seeded", bits), flush=True)


if __name__ == "__main__":
    main()
