"""Benchmark bookkeeping on the CPU: the algorithmic bytes bench.py divides by, and
its single-GPU contract.

The per-token and per-position byte counts follow from the packed layout (3-bit codes:
3 d / 8 bytes per head vector, plus d/m block scales of 4, 2 or 2 x 1 bytes) and the
input types of the five workloads; they are typed here from that arithmetic, not taken
from bench.py.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import okv_synth  # noqa: E402

# name: (decode bytes per cached token per KV head (K + V), write bytes per position)
EXPECTED = {
    # d 128: 48 B codes + 4 fp32 scales (16 B); fp32 inputs; 1 KV head
    "tiny_d128_t256": (2 * (48 + 16), 1 * 2 * (128 * 4 + 48 + 16)),
    # d 128: 48 B codes + 4 fp16 scales (8 B); bf16 inputs; 8 KV heads
    "gqa_h32kv8_t32k": (2 * (48 + 8), 8 * 2 * (128 * 2 + 48 + 8)),
    # 32 KV heads, same rows
    "mha_b4h32_t128k": (2 * (48 + 8), 32 * 2 * (128 * 2 + 48 + 8)),
    # 2 blocks of 64, each an E4M3 (scale, zero-point) pair: 4 B
    "gqa_b16h64kv8_t128k_asym": (2 * (48 + 4), 8 * 2 * (128 * 2 + 48 + 4)),
    # d 256: 96 B codes + 8 fp16 scales (16 B)
    "so4_d256_b32_t8k": (2 * (96 + 16), 8 * 2 * (256 * 2 + 96 + 16)),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    wl = okv_synth.workload(name)
    per_token, per_position = EXPECTED[name]
    cache, q, out = bench.algorithmic_decode_bytes(wl, 1000)
    assert cache == wl.batch * wl.hkv * 1000 * per_token
    in_b = 4 if wl.in_dtype == "f32" else 2
    assert q == wl.batch * wl.hq * wl.d * in_b
    assert out == wl.batch * wl.hq * wl.d * 4
    assert bench.write_bytes_per_position(wl) == wl.batch * per_position


def test_headline_per_token_figures():
    # per cached token and KV head: 128 / 112 / 112 / 104 / 224 B for the five workloads
    got = [EXPECTED[n][0] for n in ("tiny_d128_t256", "gqa_h32kv8_t32k", "mha_b4h32_t128k",
                                    "gqa_b16h64kv8_t128k_asym", "so4_d256_b32_t8k")]
    assert got == [128, 112, 112, 104, 224]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _spot(name, t):
    """A spot-check record built from the oracle's own write and decode of a small unit
    (what the library would report if it matched the oracle exactly)."""
    import numpy as np

    import oracle
    wl = okv_synth.workload(name)
    unit = wl.with_(batch=1, hkv=1, hq=wl.group)
    p32 = okv_synth.rotation_params(unit, dtype=np.float32)
    u = oracle.rotation_matrix(unit.rotation, p32.astype(np.float64), unit.d)
    k, v = okv_synth.kv_tokens(unit, 0, t)
    kh, vh = okv_synth.host_f32(k)[0, :, 0], okv_synth.host_f32(v)[0, :, 0]
    ref = oracle.write_unit(kh, vh, unit, p32)
    q = okv_synth.host_f32(okv_synth.queries(unit, 0))[0]
    y = oracle.attend_unit(q, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], t, unit, u)
    return wl, {"t": t, "k": kh, "v": vh, "k_codes": ref["k_codes"].copy(), "v_codes": ref["v_codes"].copy(),
                "k_meta": np.array(ref["k_meta"]), "v_meta": np.array(ref["v_meta"]), "q": q,
                "y": y.astype(np.float32)}


@pytest.mark.parametrize("name", ["tiny_d128_t256", "gqa_b16h64kv8_t128k_asym"])
def test_oracle_spot_check_flags_mismatches(name):
    """bench.py's spot check passes a faithful unit and flags a flipped code bit, a
    changed scale byte and an output off by 1 % of its RMS."""
    import numpy as np
    wl, spot = _spot(name, 97)
    rec = bench.oracle_spot_check(wl, spot)
    assert rec["ok"] and rec["byte_mismatches"] == {"k_codes": 0, "v_codes": 0, "k_meta": 0, "v_meta": 0}
    assert rec["decode_max_err_over_rms"] < 1e-6
    bad = dict(spot, v_codes=spot["v_codes"].copy())
    bad["v_codes"].reshape(-1)[7] ^= 4
    rec = bench.oracle_spot_check(wl, bad)
    assert not rec["ok"] and rec["byte_mismatches"]["v_codes"] == 1
    bad = dict(spot, k_meta=spot["k_meta"].copy())
    bad["k_meta"].view(np.uint8).reshape(-1)[3] ^= 1
    rec = bench.oracle_spot_check(wl, bad)
    assert not rec["ok"] and rec["byte_mismatches"]["k_meta"] == 1
    y = spot["y"].astype(np.float64)
    bad = dict(spot, y=(y + 0.01 * np.sqrt(np.mean(y ** 2))).astype(np.float32))
    rec = bench.oracle_spot_check(wl, bad)
    assert not rec["ok"] and 0.009 < rec["decode_max_err_over_rms"] < 0.011
