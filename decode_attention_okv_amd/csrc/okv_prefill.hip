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
constexpr int kFold = 1024;   // tiles per run of the first-level P.V sums (a power of 2)

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

// The 32 codes of a group as exact float16 integers: u - 2^(b-1) for symmetric codes,
// u for asymmetric ones.  Half 0x64uu is 1024 + u: one v_perm_b32 places two code bytes
// under 0x64 bytes, then one packed subtraction of 1024 + bias gives the integers.
template <bool ASYM, int BITS>
__device__ __forceinline__ void codes_h16(const uint32_t* w, h8 out[4]) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  uint32_t d[8];
  group_to_bytes<BITS>(w, d);
  constexpr float kBias = ASYM ? 1024.0f : 1024.0f + (1 << (BITS - 1));
  const h2 bias = {static_cast<_Float16>(kBias), static_cast<_Float16>(kBias)};
  uint32_t hw[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // selector bytes 0..3 pick bytes of d[k], 4 picks a byte of 0x64646464
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, d[k], 0x04010400u);   // u0, u1
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, d[k], 0x04030402u);   // u2, u3
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
template <int D, int FMT, int BLOCK, int BITS>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
  constexpr int NG = D / 32;               // 32-dim groups per key row
  constexpr int NBLK = D / BLOCK;
  constexpr int CPB = BLOCK / 32;          // 32-dim chunks per block
  constexpr int TPB = BLOCK / 16;          // 16-dim output tiles per block
  constexpr int ROWB = BITS * D / 8;       // bytes per key row
  constexpr int GB = 4 * BITS;             // bytes per 32-code group
  constexpr int MB = FMT == kFmtSymF32 ? 4 : 2;
  constexpr bool ASYM = FMT == kFmtAsym;
  constexpr int KROW = D + 8;              // halves per LDS key row (16 bytes of padding; rows 16-byte aligned)
  constexpr int VROW = kKT + 4;            // halves per LDS value row (8 bytes of padding; rows 8-byte aligned)
  constexpr int NT = D / 16;               // 16-dim output tiles
  constexpr int KTB = kKT * KROW * 2;      // bytes of the key tile
  constexpr int VTB = D * VROW * 2;        // bytes of one value plane
  constexpr int QB = kQT * D * 4;          // bytes of the float32 query / output rows
  constexpr int UB = (KTB + 2 * VTB > QB) ? KTB + 2 * VTB : QB;
  constexpr int NZ = ASYM ? NBLK : 1;
  // value unpacking: wave w owns dims [w D / 4, (w + 1) D / 4) and the blocks they lie in
  constexpr int WD = D / 4;                // dims per wave
  constexpr int NBW = WD >= BLOCK ? WD / BLOCK : 1;   // value blocks per wave
  constexpr int VGW = WD * 2 / 64;         // (dim, 32-token half) groups per lane
  constexpr int NTW = NT / 4;              // output tiles per wave's dims
  // significant bits of the scale's hi part: code x hi must be exact in float16 (11 bits)
  constexpr int CMAX = ASYM ? (1 << BITS) - 1 : (1 << (BITS - 1)) - 1;
  constexpr int HIB = 11 - (CMAX >= 8 ? 4 : CMAX >= 4 ? 3 : CMAX >= 2 ? 2 : 1);
  constexpr uint32_t HIMASK = 0xFFFFFFFFu << (24 - HIB);

  // u_s: float32 query rows (prologue), then the key codes and the two value planes,
  // then float32 output rows (end)
  __shared__ __align__(16) uint8_t u_s[UB];
  __shared__ __align__(16) float kms_s[NBLK][kKT];      // key scales of the tile, [block][token]
  __shared__ __align__(16) float kmz_s[NZ][kKT];
  __shared__ __align__(16) float vmz_s[NZ][kKT];        // value zero-points (asymmetric)
  __shared__ __align__(16) _Float16 sfh_s[NBLK][kKT];   // normalised value scales, hi part
  __shared__ __align__(16) _Float16 sfl_s[NBLK][kKT];   // and lo part
  __shared__ float g_s[4];                              // per wave: 1 / normaliser
  __shared__ float mf_s[kQT];                           // per row: running maximum at the last fold

  // workgroups start longest first: the flat index runs over the query heads fastest,
  // then over the row tiles from the last (the longest causal prefix) to the first
  const size_t lin = static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const int hq = static_cast<int>(lin % static_cast<size_t>(p.hq));
  const int qt = static_cast<int>(gridDim.x - 1 - lin / static_cast<size_t>(p.hq));
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
  // transform below is unnormalised, so the prescale is log2(e) / D (U = I: no transform)
  float* qs = reinterpret_cast<float*>(u_s);          // [kQT][D]
  const bool rot = p.rotation != kRotNone;            // uniform
  const float qscale = rot ? kLog2e / static_cast<float>(D) : kLog2e * rsqrtf(static_cast<float>(D));
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
  for (int hs = 1; hs < D && rot; hs <<= 1) {
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
  // l_run: the row's running softmax sum, added to once per tile with a compensated
  // (Kahan) sum, l_cmp holding the part rounded away: one float32 sum over a prefix of
  // millions of near-equal terms would otherwise drift by up to n 2^-24 of itself
  float m_run = -INFINITY, l_run = 0.0f, l_cmp = 0.0f;
  // asymmetric values: sum of p z_v per block, compensated like l_run (the zero-points
  // of a block mostly share a sign)
  float zacc[NZ], zcmp[NZ];
#pragma unroll
  for (int z = 0; z < NZ; ++z) zacc[z] = zcmp[z] = 0.0f;
  // P.V sums in two levels: acc holds the current run of kFold tiles; at the end of a
  // run it is added into the lane's elements of its (not yet written) output rows in
  // global memory, the second level, so that no float32 sum takes more than about 1,400
  // terms even on a 90-million-token prefix (a value dim whose terms share a sign would
  // otherwise drift by up to n 2^-24 of itself over n tiles).  The folded sums are in
  // the frame of the row's running maximum at the last fold, kept in mf_s.
  f4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // out += the folded sums, rescaled to the current maximum (first: out = acc), element
  // by element; the offset is opaque so that none of the addressing is kept live across
  // the tile loop, and each dim's loads wait for the previous dim's stores (a handful of
  // registers at any time: this runs once per kFold tiles)
  auto fold = [&](bool first, bool store) {
    const float mf = mf_s[16 * wave + j];
    const float f_own = first || mf == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mf - m_run);
    float fm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) fm[r] = __shfl(f_own, 4 * lq + r, 64);
    size_t o = ((static_cast<size_t>(b) * p.n_q + row0 + 16 * wave + 4 * lq) * p.hq + hq) * D + j;
    asm volatile("" : "+v"(o));
    const size_t rs = static_cast<size_t>(p.hq) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (16 * wave + 4 * lq + r < nrows) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float* e = p.out + o + r * rs + 16 * nt;
          const float x = first ? acc[nt][r] : __builtin_fmaf(*e, fm[r], acc[nt][r]);
          if (store) *e = x;
          else acc[nt][r] = x;
          asm volatile("" ::: "memory");
        }
      }
    }
  };

  const int T = p.len;
  const int ntiles = (T + kTile - 1) / kTile;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_codes + unit * p.tcap * ROWB, static_cast<uint32_t>(T) * ROWB);
  const __amdgpu_buffer_rsrc_t rkm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.k_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rvm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.v_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_codes + unit * p.ntile_cap * static_cast<size_t>(D) * GB,
                                              static_cast<uint32_t>(ntiles) * D * GB);
  _Float16* kt = reinterpret_cast<_Float16*>(u_s);                   // [kKT][KROW] key codes
  _Float16* vh = reinterpret_cast<_Float16*>(u_s + KTB);             // [D][VROW] u sf_hi
  _Float16* vl = reinterpret_cast<_Float16*>(u_s + KTB + VTB);       // [D][VROW] u sf_lo
  const int blk0 = (wave * WD) / BLOCK;                              // first value block of the wave

  const int n_kt = pos_last / kKT + 1;                // key tiles any row of the group sees
  // ---- raw tile data in registers, loaded one tile ahead: key code groups, the wave's
  // value code groups, and the metadata of the wave's blocks (token = lane).  Byte
  // offsets are unsigned 32-bit: a slice of packed codes reaches up to 4 GiB.
  constexpr int KGT = (kKT * NG + 255) / 256;         // key groups per thread
  uint32_t kw[KGT][BITS], vw[VGW][BITS], kmr[NBW], vmr[NBW];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < KGT; ++i) {
      const int e = tid + 256 * i;
      buf_group<BITS>(rk, static_cast<uint32_t>(t0 + e / NG) * ROWB + GB * (e % NG), kw[i]);
    }
#pragma unroll
    for (int i = 0; i < VGW; ++i) {
      const int grp = lane + 64 * i, dim = wave * WD + grp % WD, half = grp / WD;
      buf_group<BITS>(rv, (static_cast<uint32_t>(t0 / kTile) + half) * (D * GB) + GB * dim, vw[i]);
    }
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const uint32_t off = (static_cast<uint32_t>(t0 + lane) * NBLK + blk0 + i) * MB;
      kmr[i] = buf_meta<FMT>(rkm, off, 0);
      vmr[i] = buf_meta<FMT>(rvm, off, 0);
    }
  };
  load_tile(0);
  for (int it = 0; it < n_kt; ++it) {
    const int t0 = it * kKT;
    __syncthreads();   // the previous tile (or the query rows) is no longer read
    // ---- scales of the wave's blocks, token = lane.  Value scales are normalised by a
    // power of two f (largest scale of the wave's blocks in [1/2, 1)) and split into
    // a hi part of HIB significant bits and a float16 lo part, so that code x hi is
    // exact in float16.
    float vsr[NBW];
    float vmax = 0.0f;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int blk = blk0 + i;
      float s, z;
      meta_pair<FMT>(kmr[i], s, z);
      kms_s[blk][lane] = s;
      if constexpr (ASYM) kmz_s[blk][lane] = z;
      meta_pair<FMT>(vmr[i], s, z);
      vsr[i] = s;
      vmax = fmaxf(vmax, s);
      if constexpr (ASYM) vmz_s[blk][lane] = z;
    }
    vmax = wave_max_fast(vmax);
    const int ex = vmax > 0.0f ? static_cast<int>((__float_as_uint(vmax) >> 23) & 0xFFu) - 126 : 0;
    const float fnorm = __builtin_amdgcn_ldexpf(1.0f, -ex);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const float sf = vsr[i] * fnorm;                              // exact (power of two)
      const float hi = __uint_as_float(__float_as_uint(sf) & HIMASK);
      sfh_s[blk0 + i][lane] = static_cast<_Float16>(hi);
      sfl_s[blk0 + i][lane] = static_cast<_Float16>(sf - hi);
    }
    if (lane == 0) g_s[wave] = __builtin_amdgcn_ldexpf(1.0f, ex);
    // ---- key codes as float16 integers
#pragma unroll
    for (int i = 0; i < KGT; ++i) {
      const int e = tid + 256 * i;
      h8 hv[4];
      codes_h16<ASYM, BITS>(kw[i], hv);
      h8* dst = reinterpret_cast<h8*>(kt + (e / NG) * KROW + 32 * (e % NG));
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = hv[k];
    }
    // the wave reads back only the scales it wrote itself
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- value planes: u sf_hi (exact) and u sf_lo, [dim][token]
#pragma unroll
    for (int i = 0; i < VGW; ++i) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const int grp = lane + 64 * i, dim = wave * WD + grp % WD, half = grp / WD;
      const int blk = dim / BLOCK;
      h8 hv[4];
      codes_h16<ASYM, BITS>(vw[i], hv);
      const uint4* sh = reinterpret_cast<const uint4*>(&sfh_s[blk][32 * half]);
      const uint4* sl = reinterpret_cast<const uint4*>(&sfl_s[blk][32 * half]);
      uint2* dh = reinterpret_cast<uint2*>(vh + dim * VROW + 32 * half);   // 8-byte aligned rows
      uint2* dl = reinterpret_cast<uint2*>(vl + dim * VROW + 32 * half);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 c = __builtin_bit_cast(uint4, hv[k]);
        const uint4 a = sh[k], b = sl[k];
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w}, aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t oh[4], ol[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const h2 cc = __builtin_bit_cast(h2, cw[m]);
          oh[m] = __builtin_bit_cast(uint32_t, cc * __builtin_bit_cast(h2, aw[m]));
          ol[m] = __builtin_bit_cast(uint32_t, cc * __builtin_bit_cast(h2, bw[m]));
        }
        dh[2 * k] = make_uint2(oh[0], oh[1]);
        dh[2 * k + 1] = make_uint2(oh[2], oh[3]);
        dl[2 * k] = make_uint2(ol[0], ol[1]);
        dl[2 * k + 1] = make_uint2(ol[2], ol[3]);
      }
    }
    if (it > 0 && (it & (kFold - 1)) == 0) {    // uniform; acc holds tiles it - kFold .. it - 1
      fold(it == kFold, true);
      if (lq == 0) mf_s[16 * wave + j] = m_run;   // rows of this wave only: no barrier
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (it + 1 < n_kt) load_tile(t0 + kKT);
    __syncthreads();

    // ---- S^T for the wave's 16 queries: 4 token tiles of 16; per key block the exact
    // code products are scaled by the tokens' block scales
    const bool masked = t0 + kKT - 1 > pos_first + 16 * wave;   // some token after a query
    float sv[4][4];
    // The two matrix-product stretches (Q.K here, P.V below) run at a raised wave
    // priority: the two workgroups sharing a CU then drift out of step, one in its
    // products while the other converts codes or takes its softmax, instead of both
    // waiting on the same unit (3 % faster on the 32K GQA prefill).
    __builtin_amdgcn_s_setprio(1);
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
      for (int r = 0; r < 4; ++r) sv[tt][r] = __builtin_fmaf(s4[r], qmax, z4[r]);
    }
    __builtin_amdgcn_s_setprio(0);
    if (masked) {   // causal mask (and tokens past T)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 16 * tt + 4 * lq + r > my_pos) sv[tt][r] = -INFINITY;
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
      l_cmp *= alpha;
#pragma unroll
      for (int z = 0; z < NZ; ++z) {
        zacc[z] *= alpha;
        zcmp[z] *= alpha;
      }
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
    // ---- probabilities of query j (tokens 16 tt + 4 lq + r) as float16 hi + lo, packed
    // as the A operand of P.V: K chunk cc covers tokens 32 cc + 4 lq + r and
    // 32 cc + 16 + 4 lq + r.  They are taken 2^7 times p: p <= 2^8 (lazy maximum), so
    // 2^7 p <= 2^15 still fits float16, while the weights of tokens down to 2^-21 of the
    // running maximum stay normal numbers (below 2^-14 a float16 keeps an absolute error
    // of up to 2^-25, which many equal small weights would add up).  Every sum formed
    // from them (P.V, the softmax sum, the zero-point sums) carries the same factor, and
    // the normalisation removes it.
    const float m_p = m_run - 7.0f;
    h8 ph[2], pl[2];
    float l_tile = 0.0f, z_tile[NZ];
#pragma unroll
    for (int z = 0; z < NZ; ++z) z_tile[z] = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(sv[tt][r] - m_p);
        l_tile += pr;
        const H2 xs = split_h16(pr);
        ph[tt >> 1][4 * (tt & 1) + r] = xs.hi;
        pl[tt >> 1][4 * (tt & 1) + r] = xs.lo;
        if constexpr (ASYM) {
          // zero-points: sum of p z_v per block, in float32
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            z_tile[blk] = __builtin_fmaf(pr, vmz_s[blk][16 * tt + 4 * lq + r], z_tile[blk]);
        }
      }
    {
      const float y = l_tile - l_cmp;
      const float t = l_run + y;
      l_cmp = (t - l_run) - y;
      l_run = t;
    }
    if constexpr (ASYM) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const float y = z_tile[blk] - zcmp[blk];
        const float t = zacc[blk] + y;
        zcmp[blk] = (t - zacc[blk]) - y;
        zacc[blk] = t;
      }
    }
    // ---- P.V: ph vh + ph vl + pl vh per 32-token chunk, scaled back by the normaliser
    // of the wave that unpacked the dims
    float gw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) gw[w] = g_s[w];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const _Float16* rh = vh + (16 * nt + j) * VROW + 4 * lq;
      const _Float16* rl = vl + (16 * nt + j) * VROW + 4 * lq;
      f4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const uint2 h0 = *reinterpret_cast<const uint2*>(rh + 32 * cc);
        const uint2 h1 = *reinterpret_cast<const uint2*>(rh + 32 * cc + 16);
        const uint2 l0 = *reinterpret_cast<const uint2*>(rl + 32 * cc);
        const uint2 l1 = *reinterpret_cast<const uint2*>(rl + 32 * cc + 16);
        const uint32_t wh[4] = {h0.x, h0.y, h1.x, h1.y};
        const uint32_t wl[4] = {l0.x, l0.y, l1.x, l1.y};
        const h8 bh = __builtin_bit_cast(h8, wh);
        const h8 bl = __builtin_bit_cast(h8, wl);
        c = mfma_f16(ph[cc], bh, c);
        c = mfma_f16(ph[cc], bl, c);
        c = mfma_f16(pl[cc], bh, c);
      }
      const float g = gw[nt / NTW];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nt][r] = __builtin_fmaf(c[r], g, acc[nt][r]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if (n_kt > kFold) fold(false, false);           // acc += the folded sums

  // ---- normalise: l (and the zero-point sums) of query j sum the four lanes of the query
  l_run -= l_cmp;
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
      float z = zacc[blk] - zcmp[blk];
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
  // (U = I: y = y1)
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
  for (int hs = 1; hs < D && rot; hs <<= 1) {
    for (int e = tid; e < kQT * D / 2; e += 256) {
      const int r = e / (D / 2), pi = e % (D / 2);
      const int i = (pi / hs) * 2 * hs + (pi % hs);
      const float a = ys[r * D + i], c = ys[r * D + i + hs];
      ys[r * D + i] = a + c;
      ys[r * D + i + hs] = a - c;
    }
    __syncthreads();
  }
  const float cn = rot ? rsqrtf(static_cast<float>(D)) : 1.0f;
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, dim = e % D;
    float y = ys[e] * cn;
    if (p.rotation == kRotSign) y *= p.rot[dim];
    p.out[((static_cast<size_t>(b) * p.n_q + row0 + r) * p.hq + hq) * D + dim] = y;
  }
}

template <int D, int FMT, int BLOCK>
void launch_t(const PrefillParams& p, dim3 grid, hipStream_t s) {
  if (p.bits == 2) hipLaunchKernelGGL((prefill_kernel<D, FMT, BLOCK, 2>), grid, dim3(256), 0, s, p);
  else if (p.bits == 4) hipLaunchKernelGGL((prefill_kernel<D, FMT, BLOCK, 4>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((prefill_kernel<D, FMT, BLOCK, 3>), grid, dim3(256), 0, s, p);
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
