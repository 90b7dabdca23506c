// Prefill attention over the packed cache: the rows of a chunk of new tokens (already
// written by okv_write) attend causally to the cached tokens up to their own position.
// With many queries per sequence, Q.K and P.V are dense contractions: a workgroup
// unpacks each 64-token tile of key and value codes once into LDS and runs f16 MFMA
// (v_mfma_f32_16x16x32_f16) for its 64 query rows (16 per wave).
//
// Precision.  A float16 copy of the dequantised keys, values or probabilities is not
// accurate enough (each alone gives errors of 0.3% to 3% of the output RMS on caches
// with outliers), so nothing that carries a scale is rounded to 11 bits:
//  * the 3-bit codes are held exactly as float16 integers;
//  * each query row is normalised by its largest element and split into float16
//    hi + lo parts (22 significant bits): two products per 32-dim chunk;
//  * per key block the code.query dot product (exact integers times hi + lo) is scaled
//    by the token's block scale in float32 (asymmetric blocks add z times the block sum
//    of the query);
//  * P.V folds the value scale of (token, block) into the weight w = p s_v, normalised
//    per (query, tile, block) by its maximum and split into hi + lo; the float32 result
//    of the tile is scaled back by that maximum (asymmetric blocks add p z_v, summed
//    per block in float32).
//
//  * S^T = K Q^T per wave and tile: A = 16 tokens x 32 dims of codes, B = the wave's 16
//    queries.  Lane (query j, lq) holds 16 logits of query j, so the row maximum and
//    sum need two cross-lane steps only, and the lane's weights are already the A
//    operand of P.V (token order inside the K chunk is the lane's own: tokens 4 lq ..
//    4 lq + 3 of each 16-token half, matched by the value reads).
//  * Base-2 online softmax with a lazy maximum (threshold 8), as in the decode kernels.
//  * The outputs are normalised and rotated back with U^T in LDS, like the reduce kernel.
//
// Method: the idea card ("Orthogonally mixed 3-bit KV cache"), Implementation notes
// (read path) and Key formulas, applied to every row of the chunk with a causal mask;
// the OIQ report, Section 2.3 (the rotation leaves attention unchanged).
#include <hip/hip_ext.h>

#include "okv_decode_common.hpp"
#include "okv_kernels.hpp"

namespace okv {

namespace {

using namespace dec;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kQT = 64;   // query rows per workgroup (16 per wave)
constexpr int kKT = 64;   // tokens per key/value tile

__device__ __forceinline__ f4 mfma_f16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int FMT>
__device__ __forceinline__ void meta_pair(uint32_t raw, float& s, float& z) {
  if constexpr (FMT == kFmtSymF32) {
    s = __uint_as_float(raw);
    z = 0.0f;
  } else if constexpr (FMT == kFmtSymF16) {
    s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(raw)));
    z = 0.0f;
  } else {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(raw), false);   // OCP E4M3FN
    s = f[0];
    z = f[1];
  }
}

// The 32 codes of a 12-byte group as exact float16 integers: u - 4 for symmetric codes,
// u for asymmetric ones.  Half 0x6400 | u is 1024 + u, so one packed subtraction of
// 1024 + bias gives the integer.
template <bool ASYM>
__device__ __forceinline__ void codes_h16(const uint32_t w0, const uint32_t w1, const uint32_t w2, h8 out[4]) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  uint32_t d[8];
  g32_to_bytes(w0, w1, w2, d);
  const h2 bias = {static_cast<_Float16>(ASYM ? 1024.0f : 1028.0f), static_cast<_Float16>(ASYM ? 1024.0f : 1028.0f)};
  uint32_t hw[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t lo = (d[k] & 0xFFu) | ((d[k] & 0xFF00u) << 8) | 0x64006400u;
    const uint32_t hi = ((d[k] >> 16) & 0xFFu) | ((d[k] >> 8) & 0xFF0000u) | 0x64006400u;
    hw[2 * k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, lo) - bias);
    hw[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, hi) - bias);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w4[4] = {hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]};
    out[k] = __builtin_bit_cast(h8, w4);
  }
}

// x (|x| <= 1) as float16 hi + lo.  x is pinned in a register first: otherwise the
// compiler may fuse the product that made x into one conversion (one rounding) and
// compute the lo part from the separately rounded float32 x, and at an exact float16
// tie of x the two hi values differ by an ulp.
struct H2 {
  _Float16 hi, lo;
};
__device__ __forceinline__ H2 split_h16(float x) {
  asm volatile("" : "+v"(x));
  H2 r;
  r.hi = static_cast<_Float16>(x);
  r.lo = static_cast<_Float16>(x - static_cast<float>(r.hi));
  return r;
}

// One workgroup = 64 consecutive query rows of one (sequence, query head).
template <int D, int FMT, int BLOCK>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
  constexpr int NG = D / 32;               // 32-dim groups per key row
  constexpr int NBLK = D / BLOCK;
  constexpr int CPB = BLOCK / 32;          // 32-dim chunks per block
  constexpr int TPB = BLOCK / 16;          // 16-dim output tiles per block
  constexpr int ROWB = 3 * D / 8;
  constexpr int MB = FMT == kFmtSymF32 ? 4 : 2;
  constexpr bool ASYM = FMT == kFmtAsym;
  constexpr int KROW = D + 8;              // halves per LDS key row (16 bytes of padding; rows 16-byte aligned)
  constexpr int VROW = kKT + 4;            // halves per LDS value row (8 bytes of padding; rows 8-byte aligned)
  constexpr int NT = D / 16;               // 16-dim output tiles
  constexpr int KTB = kKT * KROW * 2;      // bytes of the key tile
  constexpr int VTB = D * VROW * 2;        // bytes of the value tile
  constexpr int QB = kQT * D * 4;          // bytes of the float32 query / output rows
  constexpr int UB = (KTB + VTB > QB) ? KTB + VTB : QB;
  constexpr int NZ = ASYM ? NBLK : 1;

  // u_s: float32 query rows (prologue), then the key and value code tiles, then
  // float32 output rows (end)
  __shared__ __align__(16) uint8_t u_s[UB];
  __shared__ __align__(16) float kms_s[NBLK][kKT];   // key scales of the tile, [block][token]
  __shared__ __align__(16) float kmz_s[NZ][kKT];
  __shared__ __align__(16) float vms_s[NBLK][kKT];   // value scales
  __shared__ __align__(16) float vmz_s[NZ][kKT];

  const int qt = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15, lq = lane >> 4;
  const int hk = hq / (p.hq / p.hkv);
  const size_t unit = static_cast<size_t>(b) * p.hkv + hk;
  const int row0 = qt * kQT;                          // first query row of the workgroup
  const int nrows = min(kQT, p.n_q - row0);
  const int pos_first = p.pos0 + row0;
  const int pos_last = pos_first + nrows - 1;

  // ---- query rows: q1 = U q, prescaled by log2(e) / sqrt(D) (base-2 logits); the
  // transform below is unnormalised, so the prescale is log2(e) / D
  float* qs = reinterpret_cast<float*>(u_s);          // [kQT][D]
  const float qscale = kLog2e / static_cast<float>(D);
  for (int e = tid; e < kQT * D; e += 256) {
    const int r = e / D, dim = e % D;
    float x = 0.0f;
    if (r < nrows) {
      const size_t src = ((static_cast<size_t>(b) * p.n_q + row0 + r) * p.hq + hq) * D + dim;
      x = p.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[src])
                    : reinterpret_cast<const float*>(p.q)[src];
      if (p.rotation == kRotSign) x *= p.rot[dim];
    }
    qs[e] = x * qscale;
  }
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int e = tid; e < kQT * D / 2; e += 256) {
      const int r = e / (D / 2), pi = e % (D / 2);
      const int i = (pi / hs) * 2 * hs + (pi % hs);
      const float a = qs[r * D + i], c = qs[r * D + i + hs];
      qs[r * D + i] = a + c;
      qs[r * D + i + hs] = a - c;
    }
    __syncthreads();
  }
  if (p.rotation == kRotSo4) {   // q1 = B (H q): 4 x 4 blocks along the row
    float t[kQT * D / 256];
#pragma unroll
    for (int u = 0; u < kQT * D / 256; ++u) {
      const int e = tid + 256 * u, r = e / D, dim = e % D;
      const float* R = p.rot + 16 * (dim >> 2) + 4 * (dim & 3);
      const float* xs = qs + r * D + (dim & ~3);
      t[u] = R[0] * xs[0] + R[1] * xs[1] + R[2] * xs[2] + R[3] * xs[3];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kQT * D / 256; ++u) qs[tid + 256 * u] = t[u];
    __syncthreads();
  }
  // B operand of S^T = K Q^T: lane (query j, lq) holds dims 32 c + 8 lq .. + 7 of the
  // row divided by its largest magnitude qmax, as float16 hi + lo
  h8 qh[NG], ql[NG];
  float qmax = 0.0f;
  float qsum[NZ];                           // asymmetric keys: block sums of q1
  {
    const float* qr = qs + (16 * wave + j) * D;
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(qr[32 * c + 8 * lq + e]));
    qmax = fmaxf(qmax, swz_xor16(qmax));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
    const float qinv = qmax > 0.0f ? 1.0f / qmax : 0.0f;
#pragma unroll
    for (int z = 0; z < NZ; ++z) qsum[z] = 0.0f;
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qr[32 * c + 8 * lq + e];
        const H2 xs = split_h16(x * qinv);
        qh[c][e] = xs.hi;
        ql[c][e] = xs.lo;
        if constexpr (ASYM) qsum[(32 * c) / BLOCK] += x;
      }
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
      qsum[z] += swz_xor16(qsum[z]);
      qsum[z] += __shfl_xor(qsum[z], 32, 64);
    }
  }

  // per lane: softmax state of query j (replicated over lq, partial sums per lane);
  // accumulators of queries 4 lq + r, dims 16 nt + j
  const int my_pos = pos_first + 16 * wave + j;      // position of this lane's query
  float m_run = -INFINITY, l_run = 0.0f;
  float zacc[NZ];                                     // asymmetric values: sum of p z_v per block
#pragma unroll
  for (int z = 0; z < NZ; ++z) zacc[z] = 0.0f;
  f4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int T = p.len;
  const int ntiles = (T + kTile - 1) / kTile;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_codes + unit * p.tcap * ROWB, static_cast<uint32_t>(T) * ROWB);
  const __amdgpu_buffer_rsrc_t rkm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.k_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rvm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.v_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_codes + unit * p.ntile_cap * static_cast<size_t>(D) * 12,
                                              static_cast<uint32_t>(ntiles) * D * 12);
  _Float16* kt = reinterpret_cast<_Float16*>(u_s);              // [kKT][KROW] key codes
  _Float16* vt = reinterpret_cast<_Float16*>(u_s + KTB);        // [D][VROW] value codes

  const int n_kt = pos_last / kKT + 1;                // key tiles any row of the group sees
  for (int it = 0; it < n_kt; ++it) {
    const int t0 = it * kKT;
    __syncthreads();   // the previous tile (or the query rows) is no longer read
    // ---- scales of the tile (zero past T); codes of the tile as float16 integers
    for (int e = tid; e < kKT * NBLK; e += 256) {
      const int tok = e / NBLK, blk = e % NBLK;
      const uint32_t off = static_cast<uint32_t>(((t0 + tok) * NBLK + blk) * MB);
      float s, z;
      meta_pair<FMT>(buf_meta<FMT>(rkm, off, 0), s, z);
      kms_s[blk][tok] = s;
      if constexpr (ASYM) kmz_s[blk][tok] = z;
      meta_pair<FMT>(buf_meta<FMT>(rvm, off, 0), s, z);
      vms_s[blk][tok] = s;
      if constexpr (ASYM) vmz_s[blk][tok] = z;
    }
    for (int e = tid; e < kKT * NG; e += 256) {
      const int tok = e / NG, g = e % NG;
      const auto w = __builtin_amdgcn_raw_buffer_load_b96(rk, static_cast<uint32_t>((t0 + tok) * ROWB + 12 * g), 0, 0);
      h8 hv[4];
      codes_h16<ASYM>(w[0], w[1], w[2], hv);
      h8* dst = reinterpret_cast<h8*>(kt + tok * KROW + 32 * g);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = hv[k];
    }
    for (int e = tid; e < 2 * D; e += 256) {          // (dim, 32-token half) groups
      const int dim = e % D, half = e / D;
      const auto w = __builtin_amdgcn_raw_buffer_load_b96(
          rv, static_cast<uint32_t>((t0 / kTile + half) * D * 12 + 12 * dim), 0, 0);
      h8 hv[4];
      codes_h16<ASYM>(w[0], w[1], w[2], hv);
      // value rows are 8-byte aligned only (VROW * 2 = 136 bytes): 8-byte stores
      uint2* dst = reinterpret_cast<uint2*>(vt + dim * VROW + 32 * half);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 x = __builtin_bit_cast(uint4, hv[k]);
        dst[2 * k] = make_uint2(x.x, x.y);
        dst[2 * k + 1] = make_uint2(x.z, x.w);
      }
    }
    __syncthreads();

    // ---- S^T for the wave's 16 queries: 4 token tiles of 16; per key block the exact
    // code products are scaled by the tokens' block scales
    float sv[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      float z4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        f4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int cc = blk * CPB; cc < (blk + 1) * CPB; ++cc) {
          const h8 a = *reinterpret_cast<const h8*>(kt + (16 * tt + j) * KROW + 32 * cc + 8 * lq);
          c = mfma_f16(a, qh[cc], c);
          c = mfma_f16(a, ql[cc], c);
        }
        const float4 ks = *reinterpret_cast<const float4*>(&kms_s[blk][16 * tt + 4 * lq]);
        s4[0] = __builtin_fmaf(c[0], ks.x, s4[0]);
        s4[1] = __builtin_fmaf(c[1], ks.y, s4[1]);
        s4[2] = __builtin_fmaf(c[2], ks.z, s4[2]);
        s4[3] = __builtin_fmaf(c[3], ks.w, s4[3]);
        if constexpr (ASYM) {
          const float4 kz = *reinterpret_cast<const float4*>(&kmz_s[blk][16 * tt + 4 * lq]);
          z4[0] = __builtin_fmaf(kz.x, qsum[blk], z4[0]);
          z4[1] = __builtin_fmaf(kz.y, qsum[blk], z4[1]);
          z4[2] = __builtin_fmaf(kz.z, qsum[blk], z4[2]);
          z4[3] = __builtin_fmaf(kz.w, qsum[blk], z4[3]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = t0 + 16 * tt + 4 * lq + r;
        const float lg = __builtin_fmaf(s4[r], qmax, z4[r]);
        sv[tt][r] = tok <= my_pos ? lg : -INFINITY;    // causal mask (and tokens past T)
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sv[tt][r]);
    tmax = fmaxf(tmax, swz_xor16(tmax));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__any(tmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int z = 0; z < NZ; ++z) zacc[z] *= alpha;
      m_run = m_new;
      // accumulator rows of this lane are queries 4 lq + r: their factors
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * lq + r, 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] *= al[r];
    }
    // ---- probabilities of query j; tokens 16 tt + 4 lq + r
    float pr[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[tt][r] = __builtin_amdgcn_exp2f(sv[tt][r] - m_run);
        l_run += pr[tt][r];
      }
    // ---- P.V per value block: weights w = p s_v relative to their maximum over the
    // tile, as float16 hi + lo packed as the A operand (K chunk cc covers tokens
    // 32 cc + 4 lq + r and 32 cc + 16 + 4 lq + r of this lane's query j)
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      float w[4][4];
      float wm = 0.0f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 vs = *reinterpret_cast<const float4*>(&vms_s[blk][16 * tt + 4 * lq]);
        const float vsr[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          w[tt][r] = pr[tt][r] * vsr[r];
          wm = fmaxf(wm, w[tt][r]);
        }
        if constexpr (ASYM) {
          const float4 vz = *reinterpret_cast<const float4*>(&vmz_s[blk][16 * tt + 4 * lq]);
          zacc[blk] = __builtin_fmaf(pr[tt][0], vz.x, zacc[blk]);
          zacc[blk] = __builtin_fmaf(pr[tt][1], vz.y, zacc[blk]);
          zacc[blk] = __builtin_fmaf(pr[tt][2], vz.z, zacc[blk]);
          zacc[blk] = __builtin_fmaf(pr[tt][3], vz.w, zacc[blk]);
        }
      }
      wm = fmaxf(wm, swz_xor16(wm));
      wm = fmaxf(wm, __shfl_xor(wm, 32, 64));
      // weights below 1e-30 of a whole tile and block are dropped (no reciprocal overflow)
      const float winv = wm > 1.0e-30f ? 1.0f / wm : 0.0f;
      h8 ph[2], pl[2];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const H2 xs = split_h16(w[tt][r] * winv);
          ph[tt >> 1][4 * (tt & 1) + r] = xs.hi;
          pl[tt >> 1][4 * (tt & 1) + r] = xs.lo;
        }
      float wq[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wq[r] = __shfl(wm > 1.0e-30f ? wm : 0.0f, 4 * lq + r, 64);
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        const int nt = blk * TPB + t;
        const _Float16* vr = vt + (16 * nt + j) * VROW + 4 * lq;
        f4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vr + 32 * cc);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 32 * cc + 16);
          const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
          const h8 bv = __builtin_bit_cast(h8, w4);
          c = mfma_f16(ph[cc], bv, c);
          c = mfma_f16(pl[cc], bv, c);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] = __builtin_fmaf(c[r], wq[r], acc[nt][r]);
      }
    }
  }

  // ---- normalise: l (and the zero-point sums) of query j sum the four lanes of the query
  l_run += swz_xor16(l_run);
  l_run += __shfl_xor(l_run, 32, 64);
  float inv_l[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = __shfl(l_run, 4 * lq + r, 64);
    inv_l[r] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  if constexpr (ASYM) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      float z = zacc[blk];
      z += swz_xor16(z);
      z += __shfl_xor(z, 32, 64);
      float zr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) zr[r] = __shfl(z, 4 * lq + r, 64);
#pragma unroll
      for (int t = 0; t < TPB; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[blk * TPB + t][r] += zr[r];
    }
  }
  __syncthreads();   // every wave is done with the tiles
  float* ys = reinterpret_cast<float*>(u_s);          // [kQT][D]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) ys[(16 * wave + 4 * lq + r) * D + 16 * nt + j] = acc[nt][r] * inv_l[r];
  __syncthreads();
  // ---- y = U^T y1: B^T then the transform (SO(4)), or the transform then the signs
  if (p.rotation == kRotSo4) {
    float t[kQT * D / 256];
#pragma unroll
    for (int u = 0; u < kQT * D / 256; ++u) {
      const int e = tid + 256 * u, r = e / D, dim = e % D;
      const float* R = p.rot + 16 * (dim >> 2) + (dim & 3);
      const float* yr = ys + r * D + (dim & ~3);
      t[u] = R[0] * yr[0] + R[4] * yr[1] + R[8] * yr[2] + R[12] * yr[3];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kQT * D / 256; ++u) ys[tid + 256 * u] = t[u];
    __syncthreads();
  }
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int e = tid; e < kQT * D / 2; e += 256) {
      const int r = e / (D / 2), pi = e % (D / 2);
      const int i = (pi / hs) * 2 * hs + (pi % hs);
      const float a = ys[r * D + i], c = ys[r * D + i + hs];
      ys[r * D + i] = a + c;
      ys[r * D + i + hs] = a - c;
    }
    __syncthreads();
  }
  const float cn = rsqrtf(static_cast<float>(D));
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, dim = e % D;
    float y = ys[e] * cn;
    if (p.rotation == kRotSign) y *= p.rot[dim];
    p.out[((static_cast<size_t>(b) * p.n_q + row0 + r) * p.hq + hq) * D + dim] = y;
  }
}

template <int D, int FMT, int BLOCK>
void launch_t(const PrefillParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, FMT, BLOCK>), grid, dim3(256), 0, s, p);
}

template <int D, int BLOCK>
void launch_fmt(const PrefillParams& p, dim3 grid, hipStream_t s) {
  if (p.quant == kQuantAsym) launch_t<D, kFmtAsym, BLOCK>(p, grid, s);
  else if (p.scale_dtype == kScaleF32) launch_t<D, kFmtSymF32, BLOCK>(p, grid, s);
  else launch_t<D, kFmtSymF16, BLOCK>(p, grid, s);
}

template <int D>
bool launch_d(const PrefillParams& p, dim3 grid, hipStream_t s) {
  switch (p.block) {
    case 32: launch_fmt<D, 32>(p, grid, s); return true;
    case 64: launch_fmt<D, 64>(p, grid, s); return true;
    case 128: launch_fmt<D, 128>(p, grid, s); return true;
    case 256:
      if constexpr (D >= 256) {
        launch_fmt<D, 256>(p, grid, s);
        return true;
      }
      return false;
    default: return false;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int batch, int d, hipStream_t s) {
  if (p.n_q < 1 || p.n_q > p.len || p.pos0 != p.len - p.n_q) return hipErrorInvalidValue;
  if (p.hkv < 1 || p.hq % p.hkv != 0) return hipErrorInvalidValue;
  const dim3 grid((p.n_q + kQT - 1) / kQT, p.hq, batch);
  bool ok = false;
  if (d == 128) ok = launch_d<128>(p, grid, s);
  else if (d == 256) ok = launch_d<256>(p, grid, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
