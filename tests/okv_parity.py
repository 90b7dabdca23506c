"""Helpers of the GPU parity tests: run the library on seeded inputs and compare
with the CPU oracle.  Inputs come from okv_synth; expected values come from the
oracle only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import okv_synth
import oracle


def say(*a):
    print("[okv-test]", *a, flush=True)
    sys.stdout.flush()


def round_up(n, m):
    return -(-n // m) * m


def make_cache(wl, max_tokens, params32):
    import decode_attention_okv_amd as okv
    return okv.OkvCache(batch=wl.batch, num_q_heads=wl.hq, num_kv_heads=wl.hkv, head_dim=wl.d,
                        max_tokens=max_tokens, block=wl.block, quant=wl.quant,
                        scale_dtype=wl.scale_dtype, in_dtype=wl.in_dtype, rotation=wl.rotation,
                        eps=wl.eps, rot_params=params32, device="cuda", bits=wl.bits)


def params_of(wl):
    p32 = okv_synth.rotation_params(wl, dtype=np.float32)
    u = oracle.rotation_matrix(wl.rotation, p32.astype(np.float64), wl.d)
    return p32, u


def unit_inputs(k, v, b, h):
    """Host float32 copies of the keys / values of one (sequence, KV head)."""
    return (okv_synth.host_f32(k[b, :, h]), okv_synth.host_f32(v[b, :, h]))


def compare_unit(cache, wl, b, h, t, ref):
    """Byte-exact comparison of one unit's cache against the oracle's write.
    Returns a dict of mismatch counts (all must be 0)."""
    ntile = -(-t // 32)
    kc = cache.k_codes[b, h, :t].cpu().numpy()
    bits = oracle.bits_of(wl)
    vc = cache.v_codes[b, h, :ntile].cpu().numpy()
    km = cache.k_meta[b, h, :t].cpu().numpy()
    vm = cache.v_meta[b, h, :t].cpu().numpy()
    res = {
        "k_codes": int(np.count_nonzero(kc != ref["k_codes"])),
        "v_codes": int(np.count_nonzero(vc != ref["v_codes"])),
        "k_meta": int(np.count_nonzero(km.view(np.uint8) != np.asarray(ref["k_meta"]).view(np.uint8))),
        "v_meta": int(np.count_nonzero(vm.view(np.uint8) != np.asarray(ref["v_meta"]).view(np.uint8))),
    }
    if res["k_codes"] or res["v_codes"]:
        # code-level detail for the report
        gk = oracle.unpack_rows(kc, wl.d, bits)
        gv = oracle.unpack_vtiles(vc, t, bits)
        res["k_code_mismatch"] = int(np.count_nonzero(gk != ref["k_u"]))
        res["v_code_mismatch"] = int(np.count_nonzero(gv != ref["v_u"]))
    return res


def exact_ties(ref, wl):
    """Number of rotated values on an exact rounding threshold (oracle_pool.exact_ties)."""
    from oracle_pool import exact_ties as _ties
    return _ties(ref, wl)


def decode_ref_unit(wl, q_host, b, hk, ref, t, u):
    """Oracle outputs (G, d) of the query heads of KV head hk of sequence b."""
    g = wl.group
    qh = q_host[b, hk * g:(hk + 1) * g]
    return oracle.attend_unit(qh, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], t, wl, u)


def out_error(y, y_ref):
    """(max |y - y_ref| / RMS(y_ref), worst per-head ratio)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.abs(y - y_ref).max() / rms
    per_head = np.abs(y - y_ref).max(axis=-1) / np.sqrt(np.mean(y_ref ** 2, axis=-1))
    return float(err), float(per_head.max())


def free_gpu():
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def zero_token_attention(q1, k_hat, v_hat, n_zero, v_zero=None):
    """Softmax attention of the rows q1 (G, d) over the given keys / values plus n_zero
    tokens whose key is the zero vector and whose value is v_zero (zero by default),
    in float64: such a token has logit 0, weight exp(-m) (m = max(0, largest logit)),
    and adds exp(-m) v_zero to the numerator."""
    logits = q1 @ k_hat.T / np.sqrt(q1.shape[-1])
    m = np.maximum(logits.max(axis=1, keepdims=True), 0.0)
    p = np.exp(logits - m)
    num = p @ v_hat
    if v_zero is not None:
        num = num + n_zero * np.exp(-m) * np.asarray(v_zero, dtype=np.float64)[None, :]
    return num / (p.sum(axis=1, keepdims=True) + n_zero * np.exp(-m))
