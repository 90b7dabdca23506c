// Write path: rotate each new key and value head vector with U, quantise it
// blockwise to b-bit codes (b = 2, 3, 4; the pages' method uses 3) and pack the codes.
//
// Pages: "Orthogonally mixed 3-bit KV cache", Implementation notes (k1 = U(k),
// v1 = U(v), one scale per block, signed 3-bit codes, pack, store codes and scales)
// and Key formulas (the quantiser); "Orthogonal Invariance in Activation Space",
// Sections 3.1-3.2 (normalised FWHT after a random sign flip); the news item on
// hardware-fused transforms, third paragraph (asymmetric unsigned 3-bit codes per
// 64-element sub-block with an FP8 scale and zero-point).
//
// Every float32 operation of the transform and the statistics is rounded on its
// own, in a fixed order, so the result matches the bit specification exactly:
// contraction into fused multiply-adds is disabled for this file (the explicit
// fmaf calls below only serve the code rounding, where their exactness is used).
#pragma clang fp contract(off)

#include "okv_device.hpp"

namespace okv {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;   // quad_perm [2,3,0,1]

// x[e] = RN(x[e] + sg * (x[e] of the partner lane)) for 16 elements, one v_fmac_f32 with
// a DPP source each (quad_perm [1,0,3,2]: partner lane ^ 1; [2,3,0,1]: lane ^ 2).  The
// compiler does not fold a DPP move into v_fmac_f32 (a move and an fma per element).
// The hazard check does not see inside inline asm: the leading s_nop gives the wait
// states a DPP read needs after a VALU or EXEC write of its sources, the trailing one
// covers a DPP read of the results right after the block.
#define OKV_FMAC_DPP(i, perm) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " perm " row_mask:0xf bank_mask:0xf\n"
#define OKV_FMAC_DPP16(perm)                                                                 \
  "s_nop 4\n" OKV_FMAC_DPP(0, perm) OKV_FMAC_DPP(1, perm) OKV_FMAC_DPP(2, perm)               \
      OKV_FMAC_DPP(3, perm) OKV_FMAC_DPP(4, perm) OKV_FMAC_DPP(5, perm) OKV_FMAC_DPP(6, perm)  \
      OKV_FMAC_DPP(7, perm) OKV_FMAC_DPP(8, perm) OKV_FMAC_DPP(9, perm) OKV_FMAC_DPP(10, perm) \
      OKV_FMAC_DPP(11, perm) OKV_FMAC_DPP(12, perm) OKV_FMAC_DPP(13, perm)                    \
      OKV_FMAC_DPP(14, perm) OKV_FMAC_DPP(15, perm) "s_nop 1"
template <int CTRL>
__device__ __forceinline__ void fmac_dpp16(float* x, float sg) {
  static_assert(CTRL == kXor1 || CTRL == kXor2, "lane partner");
  if constexpr (CTRL == kXor1) {
    asm(OKV_FMAC_DPP16("quad_perm:[1,0,3,2]")
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
          "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15])
        : "v"(sg));
  } else {
    asm(OKV_FMAC_DPP16("quad_perm:[2,3,0,1]")
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
          "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15])
        : "v"(sg));
  }
}
#undef OKV_FMAC_DPP16
#undef OKV_FMAC_DPP

// Distance from a half-integer below which the fast code rounding defers to the exact
// one: the approximate quotient is within ~2e-6 of the exact one for |q| <= 8.
constexpr float kNear = 0.5f - 0x1.0p-17f;

// Four codes (integer-valued floats 0..15) as the bytes of one word.
__device__ __forceinline__ uint32_t bytes_of(const float* u) {
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(u[0], 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(u[1], 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(u[2], 2, w);
  return __builtin_amdgcn_cvt_pk_u8_f32(u[3], 3, w);
}

// 32 codes as byte lanes (byte j of d[k] = code 4k+j) -> the 4b-byte group (the
// layouts of group_to_bytes).
template <int BITS>
__device__ __forceinline__ void pack_group(const uint32_t d[8], uint32_t* w) {
  if constexpr (BITS == 3) {
    w[0] = d[0] | (d[1] << 3) | ((d[6] & 0x03030303u) << 6);
    w[1] = d[2] | (d[3] << 3) | ((d[7] & 0x03030303u) << 6);
    w[2] = d[4] | (d[5] << 3) | ((d[6] & 0x04040404u) << 4) | ((d[7] & 0x04040404u) << 5);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = d[2 * k] | (d[2 * k + 1] << 4);
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) w[k] = d[4 * k] | (d[4 * k + 1] << 2) | (d[4 * k + 2] << 4) | (d[4 * k + 3] << 6);
  }
}

// Bits of a group that hold the codes of tokens 0 .. n-1.
template <int BITS>
__device__ __forceinline__ void keep_mask(int n, uint32_t* m) {
#pragma unroll
  for (int k = 0; k < BITS; ++k) m[k] = 0u;
  if constexpr (BITS == 3) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int sh = 8 * b;
      if (b < n) m[0] |= 0x07u << sh;
      if (4 + b < n) m[0] |= 0x38u << sh;
      if (24 + b < n) { m[0] |= 0xC0u << sh; m[2] |= 0x40u << sh; }
      if (8 + b < n) m[1] |= 0x07u << sh;
      if (12 + b < n) m[1] |= 0x38u << sh;
      if (28 + b < n) { m[1] |= 0xC0u << sh; m[2] |= 0x80u << sh; }
      if (16 + b < n) m[2] |= 0x07u << sh;
      if (20 + b < n) m[2] |= 0x38u << sh;
    }
  } else {
    // code i: word i / (32 / b), byte i % 4, field (i % (32 / b)) / 4
    constexpr int PW = 32 / BITS;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (i < n) m[i / PW] |= ((1u << BITS) - 1u) << (8 * (i % 4) + BITS * ((i % PW) / 4));
  }
}

// Elements of a vector per lane: 32 at d = 128 (four lanes per vector, two cross-lane
// butterfly stages, about 76 registers: six waves per SIMD) and 64 at d = 256.  Holding
// 64 elements at d = 128 saves one butterfly stage but takes about 143 registers (three
// waves per SIMD), which left the loads less overlap with the arithmetic.
constexpr int write_epl(int d) { return d == 128 ? 32 : 64; }
constexpr int write_threads(int d) { return 64 * (d / write_epl(d)); }

// One workgroup owns one 32-token tile of one (sequence, KV head).  Each of the tile's
// 32 key and 32 value vectors is held by LPV = D / EPL lanes; lane r of a vector holds
// elements EPL r .. EPL r + EPL - 1.  New slots are quantised; key rows are stored
// straight from the lanes; value codes go through LDS to be regrouped per dimension
// (old codes of earlier tokens are kept, slots after the new tokens stay zero).
//
// SIGN_BF16: the sign-flip rotation with bfloat16 inputs, fixed at compile time, so that
// the other rotations' and float32 inputs' code leaves this variant.
template <int D, int BLOCK, bool ASYM, int BITS, bool SIGN_BF16>
__global__ __launch_bounds__(write_threads(D)) void write_kernel(const WriteParams p) {
  const int rotation = SIGN_BF16 ? static_cast<int>(kRotSign) : p.rotation;
  const bool in_bf16 = SIGN_BF16 || p.in_bf16 != 0;
  constexpr int EPL = write_epl(D);                   // elements per lane
  constexpr int LPV = D / EPL;                        // lanes per vector (4)
  constexpr int NT = 64 * LPV;                        // threads: 64 vectors of the tile
  constexpr int GPL = EPL / 32;                       // 32-code groups per lane
  constexpr int BPL = EPL >= BLOCK ? EPL / BLOCK : 1; // quantisation blocks per lane
  constexpr int LPB = BLOCK > EPL ? BLOCK / EPL : 1;  // lanes per block
  constexpr int NBLK = D / BLOCK;
  constexpr int BE = BLOCK < EPL ? BLOCK : EPL;       // a block's elements in one lane
  constexpr int GB = 4 * BITS;                        // bytes per 32-code group
  constexpr int EXC = 1 << (BITS - 1);                // excess of symmetric codes
  constexpr int LEV = EXC - 1;                        // symmetric levels: codes -LEV .. LEV
  constexpr int TOP = (1 << BITS) - 1;                // largest code
  static_assert(NT >= D && (LPV == 2 || LPV == 4), "one thread per dim of the tile stage");
  __shared__ __align__(16) uint8_t vt[kTile][D];      // value codes u of the tile, [slot][dim]

  const int tile = p.tile0 + static_cast<int>(blockIdx.x);
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int tile_base = tile * kTile;
  const int s_lo = max(p.len - tile_base, 0);
  const int s_hi = min(p.len + p.n_new - tile_base, kTile);
  const size_t unit = static_cast<size_t>(b) * p.hkv + h;

  const int vi = tid / LPV, r = tid % LPV;
  const int tensor = vi >> 5, slot = vi & 31;
  const bool active = slot >= s_lo && slot < s_hi;    // uniform over the vector's lanes
  uint32_t* vdst = reinterpret_cast<uint32_t*>(&vt[slot][EPL * r]);

  // SO(4) matrices of B (every lane reads those of its dims for each vector), or the
  // sign flips of D as bit masks over pairs of bfloat16 inputs: staged in LDS once per
  // workgroup
  __shared__ __align__(16) float rot_s[SIGN_BF16 ? 1 : 4 * D];
  __shared__ __align__(16) uint32_t sgn_s[SIGN_BF16 ? D / 2 : 1];
  if constexpr (SIGN_BF16) {
    if (tid < D / 2) {
      sgn_s[tid] = (p.rot[2 * tid] < 0.0f ? 0x8000u : 0u) | (p.rot[2 * tid + 1] < 0.0f ? 0x80000000u : 0u);
    }
    __syncthreads();
  } else if (rotation == kRotSo4) {                   // uniform over the workgroup
    for (int e = tid; e < 4 * D; e += NT) rot_s[e] = p.rot[e];
    __syncthreads();
  }

  if (active) {
    const int pos = tile_base + slot;
    const size_t src = ((static_cast<size_t>(b) * p.n_new + (pos - p.len)) * p.hkv + h) * D + EPL * r;
    float x[EPL];
    if (in_bf16) {
      const uint4* s4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(tensor ? p.v : p.k) + src);
#pragma unroll
      for (int i = 0; i < EPL / 8; ++i) {
        const uint4 w = s4[i];
        uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        if constexpr (SIGN_BF16) {
          // the sign flip of two elements at once: x D is exact, a sign bit each
          const uint4 g = reinterpret_cast<const uint4*>(sgn_s + EPL / 2 * r)[i];
          ws[0] ^= g.x; ws[1] ^= g.y; ws[2] ^= g.z; ws[3] ^= g.w;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * i + 2 * k] = bf16_bits_to_f32(ws[k] & 0xFFFFu);
          x[8 * i + 2 * k + 1] = bf16_bits_to_f32(ws[k] >> 16);
        }
      }
    } else {
      const float4* s4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(tensor ? p.v : p.k) + src);
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        const float4 w = s4[i];
        x[4 * i] = w.x; x[4 * i + 1] = w.y; x[4 * i + 2] = w.z; x[4 * i + 3] = w.w;
      }
    }
    if (!SIGN_BF16 && rotation == kRotSign) {
      const float4* sg = reinterpret_cast<const float4*>(p.rot + EPL * r);
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        const float4 g = sg[i];
        x[4 * i] *= g.x; x[4 * i + 1] *= g.y; x[4 * i + 2] *= g.z; x[4 * i + 3] *= g.w;
      }
    }
    const bool rotated = rotation != kRotNone;     // U = I: y = x (uniform)
    if (rotated) {
      // butterfly stages of stride 1 .. EPL/2 inside the lane
#pragma unroll
      for (int hs = 1; hs < EPL; hs <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          if (!(e & hs)) {
            const float a = x[e], c = x[e + hs];
            x[e] = a + c;
            x[e + hs] = a - c;
          }
        }
      }
      // strides EPL (partner lane r ^ 1) and, with four lanes, 2 EPL (r ^ 2).  Each
      // stage is one fma(sg, partner, own) = RN(own +- partner): the lower lane gets
      // a + b, the upper one b - a = -(a - b).  Lanes whose index has odd parity end
      // up holding their values negated (RN is odd, so the magnitudes are exactly the
      // specified ones); sigma undoes it.
      {
        const float sg1 = (r & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < EPL; e += 16) fmac_dpp16<kXor1>(x + e, sg1);
      }
      if constexpr (LPV == 4) {
        const float sg2 = (r & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < EPL; e += 16) fmac_dpp16<kXor2>(x + e, sg2);
      }
    }
    const float cnorm = (D == 128) ? __uint_as_float(0x3DB504F3u) : 0.0625f;  // RN32(1/sqrt(D))
    const bool neg = LPV == 4 ? ((r ^ (r >> 1)) & 1) != 0 : (r & 1) != 0;
    const float sc = neg ? -cnorm : cnorm;           // sigma * c
    // With the sign-flip rotation the values stay unnormalised: the block statistics of
    // RN(x c) follow from those of x (rounding is monotone), and the code quotient folds
    // c in.  SO(4) needs y = RN(x c) as the input of its 4 x 4 products.
    const bool normalized = rotation == kRotSo4;
    if (normalized && rotated) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = x[e] * sc;
    }
    if (rotation == kRotSo4) {
      // y_row = ((R_row0 x0 + R_row1 x1) + R_row2 x2) + R_row3 x3 per 4-block
#pragma unroll
      for (int q4 = 0; q4 < EPL / 4; ++q4) {
        const float4* R = reinterpret_cast<const float4*>(rot_s + 16 * (EPL / 4 * r + q4));
        const float x0 = x[4 * q4], x1 = x[4 * q4 + 1], x2 = x[4 * q4 + 2], x3 = x[4 * q4 + 3];
#pragma unroll
        for (int row = 0; row < 4; ++row) {
          const float4 rr = R[row];
          float acc = rr.x * x0;
          acc = acc + rr.y * x1;
          acc = acc + rr.z * x2;
          acc = acc + rr.w * x3;
          x[4 * q4 + row] = acc;
        }
      }
    }
    const float xs = (normalized || !rotated) ? 1.0f : sc;    // y = RN(x xs) for every element

    // ---- block statistics, scales and metadata
    const size_t row = unit * p.tcap + pos;
    void* meta = tensor ? p.v_meta : p.k_meta;
    const bool meta_lane = (r % LPB) == 0;
    float sblk[BPL], rsblk[BPL], zblk[BPL], mblk[BPL], nzblk[BPL], ymax[BPL];
    bool exact = false;   // this lane's blocks need the exact rounding (see below)
#pragma unroll
    for (int bb = 0; bb < BPL; ++bb) {
      const int blk = (EPL * r) / BLOCK + bb;
      if constexpr (!ASYM) {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < BE; ++e) amax = fmaxf(amax, fabsf(x[bb * BE + e]));
        if constexpr (LPB >= 2) amax = fmaxf(amax, dpp<kXor1>(amax));
        if constexpr (LPB >= 4) amax = fmaxf(amax, dpp<kXor2>(amax));
        if (!normalized && rotated) amax = amax * cnorm;
        const float s32 = (amax + p.eps) / static_cast<float>(LEV);
        float s;
        if (p.scale_dtype == kScaleF16) {
          const _Float16 s16 = static_cast<_Float16>(s32);
          s = static_cast<float>(s16);
          if (meta_lane) reinterpret_cast<_Float16*>(meta)[row * NBLK + blk] = s16;
        } else {
          s = s32;
          if (meta_lane) reinterpret_cast<float*>(meta)[row * NBLK + blk] = s32;
        }
        sblk[bb] = s;
        zblk[bb] = 0.0f;
      } else {
        float mn = x[bb * BE], mx = x[bb * BE];
#pragma unroll
        for (int e = 1; e < BE; ++e) {
          mn = fminf(mn, x[bb * BE + e]);
          mx = fmaxf(mx, x[bb * BE + e]);
        }
        {
          // the extremes of y = RN(x xs): RN is monotone, decreasing in x when xs < 0
          const float a = mn * xs, c = mx * xs;
          mn = fminf(a, c);
          mx = fmaxf(a, c);
        }
        if constexpr (LPB >= 2) {
          mn = fminf(mn, dpp<kXor1>(mn));
          mx = fmaxf(mx, dpp<kXor1>(mx));
        }
        if constexpr (LPB >= 4) {
          mn = fminf(mn, dpp<kXor2>(mn));
          mx = fmaxf(mx, dpp<kXor2>(mx));
        }
        ymax[bb] = fmaxf(fabsf(mn), fabsf(mx));
        const float s32 = (mx - mn) / static_cast<float>(TOP);
        const uint32_t sb = e4m3_encode(s32), zb = e4m3_encode(mn);
        if (meta_lane) reinterpret_cast<uint16_t*>(meta)[row * NBLK + blk] = static_cast<uint16_t>(sb | (zb << 8));
        sblk[bb] = e4m3_decode(sb);
        zblk[bb] = e4m3_decode(zb);
      }
      rsblk[bb] = __builtin_amdgcn_rcpf(sblk[bb]);
      mblk[bb] = xs * rsblk[bb];      // quotient multiplier: y / s ~ x mblk
      if constexpr (ASYM) {
        // (y - z) / s ~ x mblk - z / s in one fma.  Its error is at most
        // (|y| + |z|) / s 1.5 2^-23 + 2^-21 (reciprocal, two products, the fma), and the
        // exact quotient of RN(y - z) differs from (y - z) / s by at most
        // (|y| / s + 8) 2^-24; with (max|y| + |z|) / s <= 16 (blocks that hold values of
        // both signs stay below 15) both stay under 4.8e-6, inside the near-tie margin.
        // Other blocks, and zero scales, take the exact rounding.
        nzblk[bb] = -zblk[bb] * rsblk[bb];
        const float big = (ymax[bb] + fabsf(zblk[bb])) * rsblk[bb];
        exact = exact || !(big <= 16.0f);
      }
    }

    // ---- codes u (0 .. 2^b - 1) of each 32-code group as bytes of eight words (byte j
    // of word k = code 4 k + j).  Fast rounding: rint of the approximate quotient
    // (within ~3e-6 of the exact one, |q| <= 16); the excess 2^(b-1) added before rint
    // is even, so ties keep their parity.  If any value of the wave lies within kNear
    // of a rounding boundary, the wave takes the exact rounding of the exact quotient
    // instead.
    auto quotient = [&](int e) {
      const int bb = e / BE;
      if constexpr (!ASYM) return __builtin_fmaf(x[e], mblk[bb], static_cast<float>(EXC));   // 2^(b-1) + y / s
      else return __builtin_fmaf(x[e], mblk[bb], nzblk[bb]);                  // (y - z) / s
    };
    // Symmetric codes skip the clipping in the fast rounding: |y| <= max|y| + eps, so
    // |y / s| exceeds 2^(b-1) - 1 by at most the scale's rounding (2^-11 relative for a
    // normal float16, 2^-24 for a normal float32), and rint stays within the code range.
    // A block whose scale is zero or subnormal in its storage type (less relative
    // precision) sends the wave to the exact rounding, which clips.
    if constexpr (!ASYM) {
      const float smin = p.scale_dtype == kScaleF16 ? 0x1.0p-14f : 0x1.0p-125f;
#pragma unroll
      for (int bb = 0; bb < BPL; ++bb) exact = exact || !(sblk[bb] >= smin);
    }
    uint32_t pk[GPL][8];
    float dist = 0.0f;
#pragma unroll
    for (int g = 0; g < GPL; ++g)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float t = quotient(32 * g + 4 * k + i);
          const float kk = __builtin_rintf(t);
          dist = fmaxf(dist, fabsf(t - kk));
          u[i] = ASYM ? __builtin_amdgcn_fmed3f(kk, 0.0f, static_cast<float>(TOP)) : kk;
        }
        pk[g][k] = bytes_of(u);
      }
    if (__any(exact || dist > kNear)) {
#pragma unroll
      for (int g = 0; g < GPL; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 32 * g + 4 * k + i, bb = e / BE;
            const float y = x[e] * xs;
            if constexpr (ASYM) {
              u[i] = static_cast<float>(rne_code(y - zblk[bb], sblk[bb], rsblk[bb], 0, TOP));
            } else {
              // a float32 scale below 2^-64 (it can be subnormal; its reciprocal can
              // overflow) is taken together with y times 2^64, which is exact
              const bool tiny = sblk[bb] < 0x1.0p-64f;
              const float f = tiny ? 0x1.0p64f : 1.0f;
              const float s2 = sblk[bb] * f;
              u[i] = static_cast<float>(rne_code(y * f, s2, tiny ? __builtin_amdgcn_rcpf(s2) : rsblk[bb], -LEV, LEV) + EXC);
            }
          }
          pk[g][k] = bytes_of(u);
        }
    }

    // ---- pack
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      if (tensor == 0) {
        uint32_t w[BITS];
        pack_group<BITS>(pk[g], w);
        uint32_t* dst = reinterpret_cast<uint32_t*>(p.k_codes + row * (BITS * D / 8) + GB * (GPL * r + g));
#pragma unroll
        for (int k = 0; k < BITS; ++k) dst[k] = w[k];
      } else {
        reinterpret_cast<uint4*>(vdst)[2 * g] = make_uint4(pk[g][0], pk[g][1], pk[g][2], pk[g][3]);
        reinterpret_cast<uint4*>(vdst)[2 * g + 1] = make_uint4(pk[g][4], pk[g][5], pk[g][6], pk[g][7]);
      }
    }
  } else if (tensor == 1) {
    // value slot without a new token: code 0
#pragma unroll
    for (int i = 0; i < EPL / 16; ++i) reinterpret_cast<uint4*>(vdst)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  // ---- value tile: dim j is one group over the tile's 32 tokens (threads j < D)
  uint8_t* vtile = p.v_codes + (unit * p.ntile_cap + tile) * static_cast<size_t>(D) * GB;
  if (tid < D) {
    const int j = tid;
    uint32_t d[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      d[k] = static_cast<uint32_t>(vt[4 * k][j]) | (static_cast<uint32_t>(vt[4 * k + 1][j]) << 8) |
             (static_cast<uint32_t>(vt[4 * k + 2][j]) << 16) | (static_cast<uint32_t>(vt[4 * k + 3][j]) << 24);
    }
    uint32_t w[BITS];
    pack_group<BITS>(d, w);
    uint32_t* g = reinterpret_cast<uint32_t*>(vtile + GB * j);
    if (s_lo > 0) {
      // keep the codes of the tile's earlier tokens
      uint32_t m[BITS];
      keep_mask<BITS>(s_lo, m);
#pragma unroll
      for (int k = 0; k < BITS; ++k) w[k] |= g[k] & m[k];
    }
#pragma unroll
    for (int k = 0; k < BITS; ++k) g[k] = w[k];
  }
}

template <int D, int BLOCK, int BITS>
void launch_b(const WriteParams& p, dim3 grid, hipStream_t s) {
  const bool sb = p.rotation == kRotSign && p.in_bf16;
  if (p.quant == kQuantAsym) {
    if (sb) hipLaunchKernelGGL((write_kernel<D, BLOCK, true, BITS, true>), grid, dim3(write_threads(D)), 0, s, p);
    else hipLaunchKernelGGL((write_kernel<D, BLOCK, true, BITS, false>), grid, dim3(write_threads(D)), 0, s, p);
  } else {
    if (sb) hipLaunchKernelGGL((write_kernel<D, BLOCK, false, BITS, true>), grid, dim3(write_threads(D)), 0, s, p);
    else hipLaunchKernelGGL((write_kernel<D, BLOCK, false, BITS, false>), grid, dim3(write_threads(D)), 0, s, p);
  }
}

template <int D, int BLOCK>
void launch_q(const WriteParams& p, dim3 grid, hipStream_t s) {
  if (p.bits == 2) launch_b<D, BLOCK, 2>(p, grid, s);
  else if (p.bits == 4) launch_b<D, BLOCK, 4>(p, grid, s);
  else launch_b<D, BLOCK, 3>(p, grid, s);
}

template <int D>
bool launch_d(const WriteParams& p, dim3 grid, hipStream_t s) {
  switch (p.block) {
    case 32: launch_q<D, 32>(p, grid, s); return true;
    case 64: launch_q<D, 64>(p, grid, s); return true;
    case 128: launch_q<D, 128>(p, grid, s); return true;
    case 256:
      if constexpr (D >= 256) {
        launch_q<D, 256>(p, grid, s);
        return true;
      }
      return false;
    default: return false;
  }
}

}  // namespace

hipError_t launch_write(const WriteParams& p, int ntiles, int batch, int d, hipStream_t s) {
  const dim3 grid(ntiles, p.hkv, batch);
  bool ok = false;
  if (d == 128) ok = launch_d<128>(p, grid, s);
  else if (d == 256) ok = launch_d<256>(p, grid, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
