// Device helpers shared by the write and decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "okv_kernels.hpp"

namespace okv {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Load 8 consecutive input elements (bf16 or f32) starting at element index `idx`
// (a multiple of 8, so the load is 16- or 32-byte aligned) and widen them exactly.
__device__ __forceinline__ void load8(const void* base, size_t idx, int in_bf16, float x[8]) {
  if (in_bf16) {
    const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    const float4 a = f[0], b = f[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 holds
// subnormals m * 2^-9; S.1111.111 is NaN; no infinity.  Round half to even,
// magnitudes >= 448 saturate to 448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  if (abits > 0x7F800000u) return 0x7Fu;
  const float a = __uint_as_float(abits);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {
    // below 2^-6 the spacing is 2^-9; a * 512 is exact, rint rounds half to even.
    // The count 0..8 is the encoding itself (8 = exponent field 1, mantissa 0).
    return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  }
  // keep 3 of the 23 fraction bits, round half to even; a carry moves into the exponent
  const uint32_t lsb = (abits >> 20) & 1u;
  const uint32_t r = (abits + 0x7FFFFu + lsb) >> 20;   // (float32 exponent << 3) | mantissa
  return sign | (r - (120u << 3));                    // rebias 127 -> 7
}

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0) v = static_cast<float>(m) * 0.001953125f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return (b & 0x80u) ? -v : v;
}

// Round-half-to-even of the exact quotient y / s, clipped to [lo, hi].
// A candidate from the approximate reciprocal is within one of the answer; the
// signs of y - (k0 +- 1/2) s, each computed by one fused multiply-add and hence
// exact in sign, decide the final code.  s == 0 (or NaN) gives 0.
__device__ __forceinline__ int rne_code(float y, float s, float rs, int lo, int hi) {
  if (!(s > 0.0f)) return 0;
  float k0 = __builtin_rintf(y * rs);
  k0 = fminf(fmaxf(k0, static_cast<float>(lo - 1)), static_cast<float>(hi + 1));
  const float up = __builtin_fmaf(-(k0 + 0.5f), s, y);
  const float dn = __builtin_fmaf(-(k0 - 0.5f), s, y);
  int k = static_cast<int>(k0);
  const bool odd = (k & 1) != 0;
  if (up > 0.0f || (up == 0.0f && odd)) k += 1;
  else if (dn < 0.0f || (dn == 0.0f && odd)) k -= 1;
  return k < lo ? lo : (k > hi ? hi : k);
}

// 12-byte group -> the 32 codes as 8 words of byte lanes: byte b of D[k] is code 4k+b.
__device__ __forceinline__ void g32_to_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t d[8]) {
  d[0] = w0 & 0x07070707u;
  d[1] = (w0 >> 3) & 0x07070707u;
  d[2] = w1 & 0x07070707u;
  d[3] = (w1 >> 3) & 0x07070707u;
  d[4] = w2 & 0x07070707u;
  d[5] = (w2 >> 3) & 0x07070707u;
  d[6] = ((w0 >> 6) & 0x03030303u) | ((w2 >> 4) & 0x04040404u);
  d[7] = ((w1 >> 6) & 0x03030303u) | ((w2 >> 5) & 0x04040404u);
}

// b-bit groups (b = 2, 3, 4): 32 codes in 4 b bytes.  Byte j of unpacked word k is
// code 4k + j in every width.  b = 4: byte j of word k holds code 8k + j in bits 0-3
// and code 8k + 4 + j in bits 4-7; b = 2: byte j of word k holds codes 16k + 4f + j
// in bits 2f, 2f + 1 (f = 0..3); b = 3: the 12-byte layout above.
template <int BITS>
__device__ __forceinline__ void group_to_bytes(const uint32_t* w, uint32_t d[8]) {
  static_assert(BITS >= 2 && BITS <= 4, "code width");
  if constexpr (BITS == 3) {
    g32_to_bytes(w[0], w[1], w[2], d);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      d[2 * k] = w[k] & 0x0F0F0F0Fu;
      d[2 * k + 1] = (w[k] >> 4) & 0x0F0F0F0Fu;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int f = 0; f < 4; ++f) d[4 * k + f] = (w[k] >> (2 * f)) & 0x03030303u;
  }
}

// Same, but the byte-lane words are made opaque to the optimiser so that byte
// extraction stays a single v_cvt_f32_ubyteN instead of a 3-bit field extract.
__device__ __forceinline__ void g32_to_bytes_opaque(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t d[8]) {
  g32_to_bytes(w0, w1, w2, d);
#pragma unroll
  for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(d[k]));
}

// Code i (0..31) of a 12-byte group.
__device__ __forceinline__ uint32_t g32_code(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
  if (i < 24) {
    const uint32_t w = i < 8 ? w0 : (i < 16 ? w1 : w2);
    const int r = i & 7;
    return (w >> (8 * (r & 3) + 3 * (r >> 2))) & 7u;
  }
  const int b = i & 3;
  if (i < 28) return ((w0 >> (8 * b + 6)) & 3u) | (((w2 >> (8 * b + 6)) & 1u) << 2);
  return ((w1 >> (8 * b + 6)) & 3u) | (((w2 >> (8 * b + 7)) & 1u) << 2);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// Scale (and zero-point) of block `blk` of cache row `row`.
__device__ __forceinline__ void load_meta(const void* meta, size_t row, int nblk, int blk,
                                          int sdt, float& s, float& z) {
  const size_t i = row * nblk + blk;
  if (sdt == kScaleF32) {
    s = reinterpret_cast<const float*>(meta)[i];
    z = 0.0f;
  } else if (sdt == kScaleF16) {
    s = static_cast<float>(reinterpret_cast<const _Float16*>(meta)[i]);
    z = 0.0f;
  } else {
    const uint32_t sz = reinterpret_cast<const uint16_t*>(meta)[i];
    s = e4m3_decode(sz & 0xFFu);
    z = e4m3_decode(sz >> 8);
  }
}

}  // namespace okv
