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
