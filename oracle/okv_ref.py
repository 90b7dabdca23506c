"""Reference implementation (CPU, NumPy) of the rotated 3-bit KV cache.

TEST INFRASTRUCTURE -- see the package docstring.  Nothing here is used by the
HIP library.

A "spec" argument is any object with the attributes ``d``, ``block``, ``quant``
('sym' | 'asym'), ``scale_dtype`` ('f32' | 'f16' | 'e4m3'), ``eps`` and
``rotation`` ('sign' | 'so4' | 'none'), and optionally ``bits`` (the code width b: 2, 3 or
4; 3 when absent).

Readings of points the pages leave open are marked READING; the list of all of
them, with reasons, is kept with the design notes of the repository.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "hadamard", "rotation_matrix", "fwht_f32", "rotate_f32", "c_norm_f32",
    "f16_store", "e4m3_encode", "e4m3_decode",
    "rne_codes", "quantize_f32", "dequantize", "bits_of", "group_bytes",
    "G32_BIT_POSITIONS", "group_bit_positions", "pack_g32", "unpack_g32", "pack_rows", "unpack_rows",
    "pack_vtiles", "unpack_vtiles",
    "write_unit", "meta_values", "attend_unit", "attend_unit_lengths", "attend_exact",
    "attend_prefill_unit",
    "gini", "channel_gini", "block_max_stats", "attention_rel_rmse",
]

F32 = np.float32
TILE = 32          # tokens per V tile
GROUP = 32         # codes per packed group (4 b bytes: 12 for b = 3)
BITS = (2, 3, 4)   # code widths


def bits_of(spec) -> int:
    """Code width b of a spec (3 unless the spec says otherwise)."""
    b = int(getattr(spec, "bits", 3))
    if b not in BITS:
        raise ValueError(f"code width {b} not in {BITS}")
    return b


def group_bytes(bits: int) -> int:
    """Bytes of one packed group of 32 b-bit codes."""
    return 4 * bits


# ---------------------------------------------------------------------------
# Rotation: float64 mathematics
# ---------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix H_d, float64, Sylvester construction.

    The OIQ report, Section 3.1: FWHT(x) = H_d x with H_d the d x d normalised
    Hadamard matrix, d a power of two, self-inverse.  The idea card, Mathematical
    statement: H_d^T H_d = I_d.
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def rotation_matrix(rotation: str, params, d: int) -> np.ndarray:
    """U as a dense float64 matrix.

    'sign': U = H_d D with D = diag(params) -- the OIQ report, Section 3.2, stores
    FWHT(D k), i.e. the sign flip first, then the transform.
    'so4':  U = B H_d with B = diag(R_1, ..., R_{d/4}) -- the idea card,
    Mathematical statement and Key formulas.
    'none': U = I, the unrotated baseline the idea card's Implementation notes
    compare against (per-token 3-bit KV); params are ignored.
    """
    if rotation == "none":
        return np.eye(d)
    h = hadamard(d)
    p = np.asarray(params, dtype=np.float64)
    if rotation == "sign":
        return h @ np.diag(p.reshape(d))
    if rotation == "so4":
        r = p.reshape(d // 4, 4, 4)
        b = np.zeros((d, d))
        for i in range(d // 4):
            b[4 * i:4 * i + 4, 4 * i:4 * i + 4] = r[i]
        return b @ h
    raise ValueError(rotation)


# ---------------------------------------------------------------------------
# Rotation: float32 bit specification of the write path
# ---------------------------------------------------------------------------

def c_norm_f32(d: int) -> np.float32:
    """The normalisation constant of H_d rounded to float32: RN32(1/sqrt(d))."""
    return F32(1.0 / np.sqrt(np.float64(d)))


def fwht_f32(x) -> np.ndarray:
    """Normalised fast Walsh-Hadamard transform of the last axis, in float32.

    The idea card, Implementation notes, computes the transform by the recursive
    butterfly scheme; the recursion H_{2n} = [[H_n, H_n], [H_n, -H_n]] transforms
    both halves first and combines them last.  READING (fp32 evaluation order): butterfly stages of stride
    h = 1, 2, 4, ..., d/2 in that order; in a stage every pair (i, i + h) with
    i & h == 0 becomes (a + b, a - b), each a single float32 rounding; after the
    last stage one multiply by c_d = RN32(1/sqrt(d)) (normalisation, OIQ report
    Section 3.1).
    """
    y = np.array(x, dtype=F32, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return y * c_norm_f32(d)


def rotate_f32(x, rotation: str, params32) -> np.ndarray:
    """y = U x in float32, the write path's rotation (bit specification).

    'sign' (OIQ report Section 3.2): multiply by the signs (exact), then fwht_f32.
    'so4'  (idea card, Implementation notes: the normalised transform first, the
    block-diagonal SO(4) rotations after it): fwht_f32, then for each 4-block r
    of the output
    y_r = ((R_r0 x_0 + R_r1 x_1) + R_r2 x_2) + R_r3 x_3, every product and sum
    rounded separately (READING: this order, no fused multiply-add).
    'none': y = x.
    """
    x = np.asarray(x, dtype=F32)
    if rotation == "none":
        return x.copy()
    d = x.shape[-1]
    p = np.asarray(params32, dtype=F32)
    if rotation == "sign":
        return fwht_f32(x * p.reshape(d))
    if rotation != "so4":
        raise ValueError(rotation)
    h = fwht_f32(x)
    r = p.reshape(d // 4, 4, 4)
    h4 = h.reshape(h.shape[:-1] + (d // 4, 4))
    out = np.empty_like(h4)
    for row in range(4):
        acc = r[:, row, 0] * h4[..., 0]
        acc = acc + r[:, row, 1] * h4[..., 1]
        acc = acc + r[:, row, 2] * h4[..., 2]
        acc = acc + r[:, row, 3] * h4[..., 3]
        out[..., row] = acc
    return out.reshape(h.shape)


# ---------------------------------------------------------------------------
# Storage number formats
# ---------------------------------------------------------------------------

def f16_store(s32) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of float32 values (subnormals kept,
    overflow to infinity), returned as float16."""
    with np.errstate(over="ignore"):
        return np.asarray(s32, dtype=F32).astype(np.float16)


def e4m3_encode(x) -> np.ndarray:
    """float32 -> OCP FP8 E4M3FN bit patterns (uint8), round-to-nearest-even,
    saturating: magnitudes at or above 448 (the largest finite value) become
    +-448; NaN becomes 0x7F.

    Format (OCP 8-bit floating point specification): 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9;
    S.1111.111 is NaN and there is no infinity.  The news item, third paragraph,
    stores each 64-element sub-block's scale and zero-point in FP8; READING: this
    is the E4M3FN flavour with round-to-nearest-even.
    """
    x = np.asarray(x, dtype=F32).astype(np.float64)
    nan = np.isnan(x)
    sign = np.signbit(x)
    a = np.where(nan, 0.0, np.abs(x))
    sat = a >= 448.0
    a = np.where(sat, 0.0, a)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -6)                 # exponent of the binade, floor at the subnormal one
    quantum = np.ldexp(1.0, e - 3)             # spacing of representable values in that binade
    v = np.rint(a / quantum) * quantum         # exact quotient, round half to even
    v = np.where(sat, 448.0, v)
    sub = v < 2.0 ** -6
    mant_sub = np.rint(v / 2.0 ** -9).astype(np.int64)
    _, ev = np.frexp(np.where(v > 0, v, 1.0))
    ev = ev - 1
    mant_norm = np.rint((v / np.ldexp(1.0, ev) - 1.0) * 8.0).astype(np.int64)
    bits = np.where(sub, mant_sub, ((ev + 7) << 3) | mant_norm)
    bits = np.where(v == 0, 0, bits)
    bits = bits | np.where(sign, 0x80, 0)
    bits = np.where(nan, 0x7F, bits)
    return bits.astype(np.uint8)


def e4m3_decode(bits) -> np.ndarray:
    """OCP FP8 E4M3FN bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (s * val).astype(F32)


def _store_scale(s32, scale_dtype: str):
    """Round a float32 scale into its storage type; returns (stored array, value as float32)."""
    if scale_dtype == "f32":
        st = np.asarray(s32, dtype=F32)
        return st, st
    if scale_dtype == "f16":
        st = f16_store(s32)
        return st, st.astype(F32)
    if scale_dtype == "e4m3":
        st = e4m3_encode(s32)
        return st, e4m3_decode(st)
    raise ValueError(scale_dtype)


# ---------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------

def rne_codes(y, s, lo: int, hi: int) -> np.ndarray:
    """clip(round(y / s), lo, hi) with round-half-to-even of the EXACT quotient.

    Counts the thresholds (k + 1/2) s, k = lo .. hi-1, that y lies above; at an
    exact tie y == (k + 1/2) s it rounds to the even one of k, k + 1.  The
    thresholds are exact in float64 (s has at most 24 significant bits).  s == 0
    gives code 0 (READING: a block whose scale is zero carries no information).
    y: (..., m) float32, s: (...) float32 > = 0.  Returns int64 codes.
    """
    y64 = np.asarray(y, dtype=F32).astype(np.float64)
    s64 = np.asarray(s, dtype=F32).astype(np.float64)[..., None]
    c = np.full(y64.shape, lo, dtype=np.int64)
    for k in range(lo, hi):
        thr = (k + 0.5) * s64
        up = (y64 > thr) | ((y64 == thr) & (k % 2 != 0))
        c += up.astype(np.int64)
    zero_scale = np.broadcast_to(s64 == 0, y64.shape)
    return np.where(zero_scale, 0, c)


def quantize_f32(y, spec):
    """Blockwise b-bit quantisation of rotated vectors (last axis d).

    Symmetric ('sym'; the idea card, Mathematical statement / Key formulas, with
    L = 2^(b-1) - 1 levels on each side; the card fixes b = 3, L = 3):
      s   = RN32(RN32(max_j |y_j| + eps) / L), stored as scale_dtype (RNE);
      c_j = clip(round(y_j / s_st), -L, L), stored as u_j = c_j + 2^(b-1).
    Asymmetric ('asym'; the news item, third paragraph: unsigned 3-bit codes with
    an FP8 scale and zero-point per 64-element sub-block; for b bits the 2^b codes
    0 .. 2^b - 1 span max - min):
      s   = RN32(RN32(max - min) / (2^b - 1)), z = min, both stored as E4M3 (RNE, sat);
      u_j = clip(round(RN32(y_j - z_st) / s_st), 0, 2^b - 1).
    READING: the codes are taken against the *stored* scale (and zero-point), so
    the reconstruction x_hat = s_st * c (or s_st * u + z_st) uses exactly what is
    kept; eps is added for 'sym' only.
    READING: widths other than 3 keep every other choice of the 3-bit path (the
    same excess code u = c + 2^(b-1), the same rounding and scale storage).
    Returns (u uint8 (..., d), meta): meta is the stored scale array (..., d/m)
    for 'sym' and a uint8 (..., d/m, 2) array of (scale, zero-point) E4M3 bits
    for 'asym'.
    """
    b = bits_of(spec)
    y = np.asarray(y, dtype=F32)
    d = y.shape[-1]
    m = spec.block
    yb = y.reshape(y.shape[:-1] + (d // m, m))
    if spec.quant == "sym":
        lev = 2 ** (b - 1) - 1
        mx = np.max(np.abs(yb), axis=-1)
        s32 = (mx + F32(spec.eps)) / F32(lev)
        stored, s_val = _store_scale(s32, spec.scale_dtype)
        c = rne_codes(yb, s_val, -lev, lev)
        u = (c + 2 ** (b - 1)).astype(np.uint8)
        return u.reshape(y.shape), stored
    if spec.quant == "asym":
        if spec.scale_dtype != "e4m3":
            raise ValueError("asymmetric quantiser stores E4M3 meta")
        top = 2 ** b - 1
        mn = np.min(yb, axis=-1)
        mx = np.max(yb, axis=-1)
        s32 = (mx - mn) / F32(top)
        s_bits = e4m3_encode(s32)
        z_bits = e4m3_encode(mn)
        s_val = e4m3_decode(s_bits)
        z_val = e4m3_decode(z_bits)
        t = yb - z_val[..., None]                       # float32, one rounding
        u = rne_codes(t, s_val, 0, top).astype(np.uint8)
        return u.reshape(y.shape), np.stack([s_bits, z_bits], axis=-1)
    raise ValueError(spec.quant)


def meta_values(meta, spec):
    """(scale, offset) float64 arrays (..., d/m) such that x_hat = scale * u + offset.

    'sym':  x_hat = s (u - 2^(b-1))     -> (s, -2^(b-1) s)
    'asym': x_hat = s u + z             -> (s, z)
    """
    if spec.quant == "sym":
        s = np.asarray(meta).astype(np.float64)
        return s, -float(2 ** (bits_of(spec) - 1)) * s
    s = e4m3_decode(meta[..., 0]).astype(np.float64)
    z = e4m3_decode(meta[..., 1]).astype(np.float64)
    return s, z


def dequantize(u, meta, spec) -> np.ndarray:
    """x_hat (float64) from stored codes and metadata (idea card, Key formulas:
    the reconstruction is the scale times the clipped rounded code; news item,
    third paragraph: scale and zero-point)."""
    u = np.asarray(u).astype(np.float64)
    d = u.shape[-1]
    m = spec.block
    sc, off = meta_values(meta, spec)
    ub = u.reshape(u.shape[:-1] + (d // m, m))
    return (ub * sc[..., None] + off[..., None]).reshape(u.shape)


# ---------------------------------------------------------------------------
# Packing: 32 b-bit codes -> 4 b bytes
# ---------------------------------------------------------------------------

def group_bit_positions(bits: int = 3) -> np.ndarray:
    """Bit index (little-endian over the 4 b bytes) of bit q of code i: (32, b).

    READING: the idea card (Implementation notes) only says that the codes are
    packed into bytes; the layouts chosen here keep the codes in byte lanes of
    32-bit words, so that byte j of unpacked word k holds code 4 k + j:
      b = 4: word k = i // 8, r = i % 8, byte r % 4, field f = r // 4:
             bits 8 (r % 4) + 4 f .. + 3 of word k (two codes per byte);
      b = 2: word k = i // 16, r = i % 16, byte r % 4, field f = r // 4:
             bits 8 (r % 4) + 2 f .. + 1 of word k (four codes per byte);
      b = 3: codes 0..23: word k = i // 8, r = i % 8, byte r % 4, field f = r // 4,
             bits 8 (r % 4) + 3 f .. + 2 of word k;
             codes 24..27 (j = i - 24): bits 0-1 -> bits 8j+6, 8j+7 of word 0,
             bit 2 -> bit 8j+6 of word 2;
             codes 28..31 (j = i - 28): bits 0-1 -> bits 8j+6, 8j+7 of word 1,
             bit 2 -> bit 8j+7 of word 2.
    """
    pos = np.zeros((GROUP, bits), dtype=np.int64)
    for i in range(GROUP):
        if bits in (2, 4):
            per_word = 32 // bits
            k, r = divmod(i, per_word)
            byte, f = r % 4, r // 4
            for q in range(bits):
                pos[i, q] = 32 * k + 8 * byte + bits * f + q
        elif i < 24:
            k, r = divmod(i, 8)
            byte, f = r % 4, r // 4
            for q in range(3):
                pos[i, q] = 32 * k + 8 * byte + 3 * f + q
        elif i < 28:
            j = i - 24
            pos[i] = [8 * j + 6, 8 * j + 7, 64 + 8 * j + 6]
        else:
            j = i - 28
            pos[i] = [32 + 8 * j + 6, 32 + 8 * j + 7, 64 + 8 * j + 7]
    return pos


G32_BIT_POSITIONS = group_bit_positions(3)
_POSITIONS = {b: group_bit_positions(b) for b in BITS}


def pack_g32(e, bits: int = 3) -> np.ndarray:
    """(..., 32) codes in 0 .. 2^b - 1 -> (..., 4 b) bytes (layout of
    group_bit_positions)."""
    e = np.asarray(e).astype(np.int64)
    if e.shape[-1] != GROUP or np.any((e < 0) | (e >= 2 ** bits)):
        raise ValueError(f"need (..., 32) codes in 0..{2 ** bits - 1}")
    pos = _POSITIONS[bits]
    out = np.zeros(e.shape[:-1] + (32 * bits,), dtype=np.uint8)
    for q in range(bits):
        out[..., pos[:, q]] = ((e >> q) & 1).astype(np.uint8)
    return np.packbits(out, axis=-1, bitorder="little")


def unpack_g32(g, bits: int = 3) -> np.ndarray:
    """(..., 4 b) bytes -> (..., 32) codes (uint8)."""
    g = np.asarray(g, dtype=np.uint8)
    raw = np.unpackbits(g, axis=-1, bitorder="little").astype(np.int64)
    pos = _POSITIONS[bits]
    e = np.zeros(g.shape[:-1] + (GROUP,), dtype=np.int64)
    for q in range(bits):
        e |= raw[..., pos[:, q]] << q
    return e.astype(np.uint8)


def pack_rows(u, bits: int = 3) -> np.ndarray:
    """Key cache rows: (..., d) codes -> (..., b d/8) bytes; dims 32g..32g+31 form
    group g at bytes 4 b g .. 4 b g + 4 b - 1."""
    u = np.asarray(u)
    d = u.shape[-1]
    g = pack_g32(u.reshape(u.shape[:-1] + (d // GROUP, GROUP)), bits)
    return g.reshape(u.shape[:-1] + (bits * d // 8,))


def unpack_rows(r, d: int, bits: int = 3) -> np.ndarray:
    r = np.asarray(r, dtype=np.uint8)
    e = unpack_g32(r.reshape(r.shape[:-1] + (d // GROUP, group_bytes(bits))), bits)
    return e.reshape(r.shape[:-1] + (d,))


def pack_vtiles(u, bits: int = 3) -> np.ndarray:
    """Value cache tiles: (T, d) codes of one (sequence, head) -> (ceil(T/32), d, 4 b).

    READING (layout): tokens are grouped 32 to a tile; inside a tile, dim j holds
    the codes of the tile's 32 tokens as one group (token 32 tau + i is code i).
    Token slots past T in the last tile hold code 0.
    """
    u = np.asarray(u)
    t, d = u.shape
    nt = -(-t // TILE)
    full = np.zeros((nt * TILE, d), dtype=np.uint8)
    full[:t] = u
    tiles = full.reshape(nt, TILE, d).transpose(0, 2, 1)      # (tile, dim, token-in-tile)
    return pack_g32(tiles, bits)


def unpack_vtiles(v, t: int, bits: int = 3) -> np.ndarray:
    """(ntiles, d, 4 b) -> (t, d) codes."""
    e = unpack_g32(np.asarray(v, dtype=np.uint8), bits)      # (tile, dim, 32)
    nt, d, _ = e.shape
    return e.transpose(0, 2, 1).reshape(nt * TILE, d)[:t]


# ---------------------------------------------------------------------------
# Write path of one (sequence, KV head)
# ---------------------------------------------------------------------------

def write_unit(k, v, spec, params32):
    """Rotate, quantise and pack the keys and values of one (sequence, KV head).

    The idea card, Implementation notes (write path): each new key and value
    vector is rotated by U, given one scale per block, rounded to signed b-bit
    codes (b = 3 on the card) and packed; only codes and scales are kept.  k, v:
    (T, d) float32 (exact widening of the inputs).
    Returns a dict: k_codes (T, b d/8) uint8, v_codes (ceil(T/32), d, 4 b) uint8,
    k_meta / v_meta (T, d/m) scales or (T, d/m, 2) E4M3 bytes, plus the code
    arrays k_u / v_u (T, d) and the rotated float32 vectors k_rot / v_rot.
    """
    k_rot = rotate_f32(k, spec.rotation, params32)
    v_rot = rotate_f32(v, spec.rotation, params32)
    k_u, k_meta = quantize_f32(k_rot, spec)
    v_u, v_meta = quantize_f32(v_rot, spec)
    b = bits_of(spec)
    return {
        "k_codes": pack_rows(k_u, b), "v_codes": pack_vtiles(v_u, b),
        "k_meta": k_meta, "v_meta": v_meta,
        "k_u": k_u, "v_u": v_u, "k_rot": k_rot, "v_rot": v_rot,
    }


# ---------------------------------------------------------------------------
# Read path (float64 mathematics)
# ---------------------------------------------------------------------------

def attend_exact(q, k, v) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v in float64 for query rows q (G, d) over (T, d)
    keys and values; max-subtracted softmax over every row (idea card, Key
    formulas: Attn(Q, K, V) = softmax(Q K^T / sqrt d) V; decode attends to all
    cached tokens, no mask)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = q @ k.T / np.sqrt(q.shape[-1])
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def attend_unit(q, k_codes, k_meta, v_codes, v_meta, t: int, spec, u_mat) -> np.ndarray:
    """Decode attention of the query heads q (G, d) of one KV head over its t
    cached tokens, from the packed cache.

    The idea card, Implementation notes (read path): the query is rotated by U,
    logits come from it and the decoded rotated keys, the softmax weights
    multiply the decoded rotated values, and U^T maps the result back.  The OIQ
    report, Section 2.3, explains why this equals attention on the unrotated
    vectors.
    Returns (G, d) float64.
    """
    d, b = spec.d, bits_of(spec)
    k_hat = dequantize(unpack_rows(np.asarray(k_codes)[:t], d, b), np.asarray(k_meta)[:t], spec)
    v_hat = dequantize(unpack_vtiles(v_codes, t, b), np.asarray(v_meta)[:t], spec)
    q1 = np.asarray(q, dtype=np.float64) @ u_mat.T          # rows of U q
    y1 = attend_exact(q1, k_hat, v_hat)
    return y1 @ u_mat                                       # rows of U^T y1


def attend_unit_lengths(queries, k_codes, k_meta, v_codes, v_meta, spec, u_mat) -> list:
    """Decode attention of one KV head at several cache lengths: queries is a list of
    (t, q) with q (G, d) the query heads of a decode step that saw t cached tokens.
    Each entry is attend_unit(q, ..., t, ...): the read path of the idea card's
    Implementation notes over tokens 0 .. t-1 (the cache is append-only, so a step at
    length t reads the first t tokens of the final cache).  The cache is decoded once.
    Returns a list of (G, d) float64 arrays."""
    if not queries:
        return []
    d, b = spec.d, bits_of(spec)
    t_max = max(int(t) for t, _ in queries)
    k_hat = dequantize(unpack_rows(np.asarray(k_codes)[:t_max], d, b), np.asarray(k_meta)[:t_max], spec)
    v_hat = dequantize(unpack_vtiles(v_codes, t_max, b), np.asarray(v_meta)[:t_max], spec)
    outs = []
    for t, q in queries:
        q1 = np.asarray(q, dtype=np.float64) @ u_mat.T
        outs.append(attend_exact(q1, k_hat[:int(t)], v_hat[:int(t)]) @ u_mat)
    return outs


def attend_prefill_unit(q, positions, k_codes, k_meta, v_codes, v_meta, spec, u_mat) -> np.ndarray:
    """Causal attention of new query rows over the packed cache of one KV head (the
    prefill half of serving, over the same stored codes and metadata).

    q: (n, G, d) query heads of n new positions; query row i sits at cache position
    positions[i] (its own key and value are already stored) and attends to the
    cached tokens 0 .. positions[i].  Each row is the read path of the idea card's
    Implementation notes over that prefix: rotate q by U, softmax of the logits with
    the decoded rotated keys, weights on the decoded rotated values, U^T back.
    Returns (n, G, d) float64.
    """
    positions = [int(x) for x in positions]
    t = max(positions) + 1
    d, b = spec.d, bits_of(spec)
    k_hat = dequantize(unpack_rows(np.asarray(k_codes)[:t], d, b), np.asarray(k_meta)[:t], spec)
    v_hat = dequantize(unpack_vtiles(v_codes, t, b), np.asarray(v_meta)[:t], spec)
    q = np.asarray(q, dtype=np.float64)
    out = np.empty(q.shape, dtype=np.float64)
    for i, pos in enumerate(positions):
        q1 = q[i] @ u_mat.T
        out[i] = attend_exact(q1, k_hat[:pos + 1], v_hat[:pos + 1]) @ u_mat
    return out


# ---------------------------------------------------------------------------
# Quality diagnostics of the ablation variants (float64)
# ---------------------------------------------------------------------------

def gini(x) -> float:
    """Gini coefficient of the magnitudes |x| (all elements): the mean absolute
    difference of two draws over twice the mean, sum_ij |a_i - a_j| / (2 n^2 mean a).
    0 for equal magnitudes, (n - 1) / n for one nonzero among n.  The OIQ report,
    Section 6.1, measures it on key tensors before and after the transform."""
    a = np.sort(np.abs(np.asarray(x, dtype=np.float64)).ravel())
    n = a.size
    tot = a.sum()
    if n == 0 or tot == 0.0:
        return 0.0
    # sum_ij |a_i - a_j| = 2 sum_i (2 i - n + 1) a_(i) over the ascending order (i from 0)
    i = np.arange(n, dtype=np.float64)
    return float(2.0 * np.sum((2.0 * i - n + 1.0) * a) / (2.0 * n * tot))


def channel_gini(x) -> float:
    """Gini coefficient of the per-channel magnitudes of a (T, d) tensor: the RMS of
    each channel over the T rows.  READING: the OIQ report, Section 6.1, measures "the
    Gini coefficient of key tensor magnitude distribution" before and after the
    transform; outlier channels concentrate that distribution and the transform
    spreads their energy over all channels, so the per-channel magnitudes are taken."""
    x = np.asarray(x, dtype=np.float64)
    return gini(np.sqrt(np.mean(x.reshape(-1, x.shape[-1]) ** 2, axis=0)))


def block_max_stats(y, block: int) -> dict:
    """Block maxima of |y| over blocks of `block` values along the last axis: the
    worst one and the mean one, also relative to the RMS of y (the quantity the
    scale follows; the idea card's Verification reports the worst block maximum)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    bm = np.abs(y.reshape(y.shape[:-1] + (d // block, block))).max(axis=-1)
    rms = float(np.sqrt(np.mean(y ** 2)))
    return {"worst": float(bm.max()), "mean": float(bm.mean()),
            "worst_over_rms": float(bm.max()) / rms if rms > 0 else 0.0,
            "mean_over_rms": float(bm.mean()) / rms if rms > 0 else 0.0}


def attention_rel_rmse(q, k, v, spec, params32) -> float:
    """||y_cache - y_exact|| / ||y_exact|| (Frobenius over the query heads) of one
    (sequence, KV head): y_cache is the read path over the packed cache written from
    k, v (write_unit, attend_unit), y_exact the unquantised attention of the raw
    vectors (idea card, Key formulas).  q: (G, d), k, v: (T, d) float32."""
    u = rotation_matrix(spec.rotation, np.asarray(params32, dtype=np.float64), spec.d)
    ref = write_unit(k, v, spec, params32)
    t = np.asarray(k).shape[0]
    y_c = attend_unit(q, ref["k_codes"], ref["k_meta"], ref["v_codes"], ref["v_meta"], t, spec, u)
    y_e = attend_exact(q, k, v)
    return float(np.linalg.norm(y_c - y_e) / np.linalg.norm(y_e))
