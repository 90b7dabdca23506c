"""Oracle work for the full-size GPU tests, run in spawned worker processes.

Imports only NumPy and the oracle (no torch, no GPU)."""
from types import SimpleNamespace

import numpy as np

import oracle


def unit_job(args):
    """Oracle write of one (sequence, KV head) and its decode outputs at the given
    lengths.  args: (key, k (T, d) f32, v (T, d) f32, spec dict, params f32,
    u (d, d) f64, [(t, q (G, d) f32), ...])."""
    key, k, v, spec, p32, u, queries = args
    wl = SimpleNamespace(**spec)
    ref = oracle.write_unit(k, v, wl, p32)
    outs = [oracle.attend_unit(q, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], t, wl, u)
            for t, q in queries]
    keep = {n: ref[n] for n in ("k_codes", "v_codes", "k_meta", "v_meta", "k_u", "v_u")}
    return key, keep, outs


def token_job(args):
    """Oracle codes and metadata of single key/value vectors: (n, d) f32 each."""
    k, v, spec, p32 = args
    wl = SimpleNamespace(**spec)
    res = {}
    for name, x in (("k", k), ("v", v)):
        y = oracle.rotate_f32(x, wl.rotation, p32)
        u, meta = oracle.quantize_f32(y, wl)
        res[name + "_u"] = u
        res[name + "_meta"] = np.asarray(meta)
        res[name + "_row"] = oracle.pack_rows(u)
    return res
