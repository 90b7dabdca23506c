// Helpers shared by the decode and reduce kernels (included by okv_decode_head.hip,
// okv_decode_mfma.hip and okv_reduce.hip).
#pragma once

#include "okv_device.hpp"

namespace okv {
namespace dec {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWMax = 4194303.0f;   // value weights: 22-bit fixed point per step (2^22 - 1)
constexpr int kQMax = 8000000;        // |q| fixed-point limit: three balanced int8 digits

// Fixed-point limit of q for sums of q times a code term over `span` dims: the int32
// digit combinations wrap, so only the final sum must fit, and |sum| <= span * limit *
// cmax where cmax bounds |code term| (code_max).  Capped at kQMax.
constexpr int q_limit(int span, int cmax) {
  return 2147483647LL / (static_cast<long long>(span) * cmax) < kQMax
             ? static_cast<int>(2147483647LL / (static_cast<long long>(span) * cmax))
             : kQMax;
}
// Same for the value weights (64 tokens per product), capped at `cap`.
constexpr int w_limit(int cmax, int cap) {
  return 2147483647LL / (64LL * cmax) < cap ? static_cast<int>(2147483647LL / (64LL * cmax)) : cap;
}
constexpr int kMaxSplitsDev = 256;    // must match the host's split-K capacity

enum : int { kFmtSymF32 = 0, kFmtSymF16 = 1, kFmtAsym = 2 };

// (scale, offset) of a block from its raw metadata bits.
template <int FMT>
__device__ __forceinline__ void meta_decode(uint32_t raw, float& s, float& o) {
  if constexpr (FMT == kFmtSymF32) {
    s = __uint_as_float(raw);
    o = 0.0f;
  } else if constexpr (FMT == kFmtSymF16) {
    s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(raw)));
    o = 0.0f;
  } else {
    // v_cvt_f32_fp8 decodes OCP E4M3FN on gfx950 (byte 0: scale, byte 1: zero-point)
    s = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(raw), 0);
    o = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(raw), 1) + 4.0f * s;
  }
}

__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float swz_xor4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}

__device__ __forceinline__ float dpp_ror4(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
}

// Maximum / sum over the 16 lanes of each row (all lanes active): quad xor 1 and 2,
// then rotations by 4 and 8 inside the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, dpp_ror4(v));
  return fmaxf(v, dpp_ror8(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_xor1(v);
  v += dpp_xor2(v);
  v += dpp_ror4(v);
  return v + dpp_ror8(v);
}
__device__ __forceinline__ int row16_sum(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true);
  return v + __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
}
__device__ __forceinline__ float swz_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Maximum over the 64 lanes, returned wave-uniform (DPP / swizzle within each half,
// then the two halves through readlane).
__device__ __forceinline__ float wave_max_fast(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, swz_xor4(v));
  v = fmaxf(v, dpp_ror8(v));
  v = fmaxf(v, swz_xor16(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return fmaxf(a, b);
}

// Unnormalised in-place FWHT of D floats in shared memory.
template <int D>
__device__ __forceinline__ void lds_fwht(float* x) {
#pragma unroll
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int pidx = threadIdx.x; pidx < D / 2; pidx += blockDim.x) {
      const int i = (pidx / hs) * 2 * hs + (pidx % hs);
      const float a = x[i], c = x[i + hs];
      x[i] = a + c;
      x[i + hs] = a - c;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, `bytes` valid bytes (loads past them return 0)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i mfma64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// a * 2^sa + b * 2^sb + c in wrapping int32 arithmetic (the true value fits).  The
// empty asm keeps the two shift-adds apart, so each maps to one v_lshl_add_u32
// instead of two shifts and an add3.
template <int SA, int SB>
__device__ __forceinline__ int combine3(int a, int b, int c) {
  uint32_t t = (static_cast<uint32_t>(b) << SB) + static_cast<uint32_t>(c);
  asm("" : "+v"(t));
  return static_cast<int>((static_cast<uint32_t>(a) << SA) + t);
}

// 16-byte slot of chunk c (16 tokens) in a 64-byte LDS row r: rotating the chunk
// order by bits 2-3 of the row spreads 16 consecutive rows over all 64 banks.
__device__ __forceinline__ int slot16(int c, int r) { return (c ^ (r >> 2)) & 3; }

// Cache policy (the loads' aux bits) for data read once per call: non-temporal.  The
// per-head decode reads every code and scale exactly once and gains from it; kernels
// that re-read the cache (prefill) or that measured no gain (grouped decode) keep 0.
constexpr int kStreamAux = 2;

// One b-bit code group (4 b bytes) at byte offset voff of a buffer resource; zero past
// the resource's range.  AUX: cache policy of the load.
template <int BITS, int AUX = 0>
__device__ __forceinline__ void buf_group(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* w) {
  if constexpr (BITS == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, AUX);
    w[0] = x[0];
    w[1] = x[1];
  } else if constexpr (BITS == 3) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b96(r, voff, 0, AUX);
    w[0] = x[0];
    w[1] = x[1];
    w[2] = x[2];
  } else {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX);
    w[0] = x[0];
    w[1] = x[1];
    w[2] = x[2];
    w[3] = x[3];
  }
}

// Largest |code term| of b-bit codes: |u - 2^(b-1)| <= 2^(b-1) - 1 (symmetric, centred)
// or u <= 2^b - 1 (asymmetric).
constexpr int code_max(bool asym, int bits) { return asym ? (1 << bits) - 1 : (1 << (bits - 1)) - 1; }

template <int FMT, int AUX = 0>
__device__ __forceinline__ uint32_t buf_meta(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (FMT == kFmtSymF32) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
  else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX);
}

}  // namespace dec
}  // namespace okv
