"""Oracle work for the full-size GPU tests, run in spawned worker processes.

Imports only NumPy and the oracle (no torch, no GPU)."""
from types import SimpleNamespace

import numpy as np

import oracle


def widen(x):
    """Exact float32 values of an input array: float32 as it is, bfloat16 given as its
    uint16 bit patterns (the high half of the float32 bits)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def exact_ties(ref, spec):
    """Number of rotated values that lie exactly on a rounding threshold of their
    stored scale (the oracle's own count; reported, expected ~0)."""
    n = 0
    for key, mkey in (("k_rot", "k_meta"), ("v_rot", "v_meta")):
        y = ref[key].astype(np.float64)
        s, off = oracle.meta_values(ref[mkey], spec)
        t, d = y.shape
        yb = y.reshape(t, d // spec.block, spec.block)
        if spec.quant == "sym":
            q = yb / s[..., None]
        else:
            q = (yb.astype(np.float32) - off[..., None].astype(np.float32)).astype(np.float64) / s[..., None]
        with np.errstate(invalid="ignore", divide="ignore"):
            frac = q - np.floor(q)
        n += int(np.count_nonzero(frac == 0.5))
    return n


def full_unit_job(args):
    """One (sequence, KV head) at full size: the oracle's write of its raw keys and
    values, compared byte for byte with the library's cache of that unit; the number
    of exact ties among its codes; the oracle's decode outputs of the unit's query heads
    at every checked call.

    args: (key, k, v, spec dict, params f32, u (d, d) f64, [(t, q (G, d) f32), ...],
    gpu) with k, v (T, d) raw inputs (float32, or bfloat16 as uint16 bits) and gpu a
    dict of the unit's cache bytes: k_codes (T, row bytes), v_codes (tiles, d, group
    bytes), k_meta, v_meta (T, ...) viewed as uint8.
    Returns (key, mismatch counts, ties, codes checked, [y_ref (G, d), ...])."""
    key, k, v, spec, p32, u, queries, gpu = args
    wl = SimpleNamespace(**spec)
    ref = oracle.write_unit(widen(k), widen(v), wl, p32)
    t = ref["k_u"].shape[0]
    ntile = ref["v_codes"].shape[0]
    mism = {
        "k_codes": int(np.count_nonzero(gpu["k_codes"][:t] != ref["k_codes"])),
        "v_codes": int(np.count_nonzero(gpu["v_codes"][:ntile] != ref["v_codes"])),
        "k_meta": int(np.count_nonzero(gpu["k_meta"][:t] != np.asarray(ref["k_meta"]).view(np.uint8).reshape(t, -1))),
        "v_meta": int(np.count_nonzero(gpu["v_meta"][:t] != np.asarray(ref["v_meta"]).view(np.uint8).reshape(t, -1))),
    }
    if mism["k_codes"] or mism["v_codes"]:
        bits = oracle.bits_of(wl)
        mism["k_code_mismatch"] = int(np.count_nonzero(
            oracle.unpack_rows(gpu["k_codes"][:t], wl.d, bits) != ref["k_u"]))
        mism["v_code_mismatch"] = int(np.count_nonzero(
            oracle.unpack_vtiles(gpu["v_codes"][:ntile], t, bits) != ref["v_u"]))
    ties = exact_ties(ref, wl)
    outs = oracle.attend_unit_lengths(queries, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"],
                                      wl, u)
    return key, mism, ties, 2 * ref["k_u"].size, outs


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
