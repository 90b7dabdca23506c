"""The seeded input generator is deterministic and has the stated shapes (CPU only)."""
import numpy as np
import torch

import okv_synth


def test_workload_table():
    names = list(okv_synth.WORKLOADS)
    assert len(names) == 5
    w = okv_synth.workload("mha_b4h32_t128k")
    assert (w.batch, w.hq, w.hkv, w.d, w.tokens) == (4, 32, 32, 128, 131072)
    assert w.row_bytes() == 56 and w.cache_bytes() == 1879048192
    w4 = okv_synth.workload("gqa_b16h64kv8_t128k_asym")
    assert w4.row_bytes() == 52 and w4.group == 8


def test_deterministic_and_shapes():
    w = okv_synth.workload("gqa_h32kv8_t32k")
    k1, v1 = okv_synth.kv_tokens(w, 100, 16)
    k2, v2 = okv_synth.kv_tokens(w, 100, 16)
    assert k1.shape == (1, 16, 8, 128) and k1.dtype == torch.bfloat16
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    k3, _ = okv_synth.kv_tokens(w, 100, 16, step=3)
    assert not torch.equal(k1, k3)
    q = okv_synth.queries(w, 5)
    assert q.shape == (1, 32, 128)
    s = okv_synth.channel_model(w, "k", 3)
    assert (s > 5).sum() >= 4             # the persistent outlier channels (x20)
    p = okv_synth.rotation_params(w)
    assert set(np.unique(p)) <= {-1.0, 1.0}
