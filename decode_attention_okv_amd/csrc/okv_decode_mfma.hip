// Decode attention for query groups: G query heads share one key/value head, so
// the packed keys and values of a (sequence, KV head) are streamed once for all G
// heads and both contractions run on int8 MFMA (v_mfma_i32_16x16x64_i8).  A wave
// works on steps of 64 tokens (two 32-token value tiles):
//
//  * Q.K as C = Q K^T: A = 16 rows (head h, block b) holding one int8 digit of q_h
//    restricted to block b (zero elsewhere), B = key codes of 16 tokens (columns) x 64
//    dims.  A lane decodes one whole 32-code key group and feeds two instructions; the
//    (head, block) rows keep the per-block scales separable.  A query group with more
//    than 16 (head, block) pairs per 128-dim quad takes several 16-row sets (G = 8 with
//    blocks of 32: two sets); a smaller one leaves rows zero.  Three instruction
//    chains take the three balanced digits of the 24-bit fixed-point query and
//    combine exactly in int32.  Each lane ends with whole logits (every block of its
//    heads) of four consecutive tokens, so the softmax runs once per (token, head).
//  * P.V: the step's weights p s of each (head, block) row become 21-bit integers
//    (relative to one scale per head, or per row, and step) in three balanced int8
//    digit planes in LDS.  A = rows (head, digit) of one block:
//    instruction i takes heads 4 i .. 4 i + 3, row 4 hh + d holding digit d of head
//    4 i + hh; B = value codes of 64 tokens x 16 dims of that block, decoded once per
//    step into LDS; C = int32, so lane (dim j, lq) holds the three digit sums of head
//    4 i + lq and combines them exactly, then scales back to float once per step.
//
// Block metadata is decoded once per (token, block) into LDS as floats.  With the
// asymmetric quantiser the zero-point enters directly (s u + z); with the symmetric
// one the codes are centred (s (u - 2^(b-1))) through the integer accumulators.
//
// Method: "Orthogonally mixed 3-bit KV cache" (idea card), Implementation notes,
// read path, and Key formulas; "Orthogonal Invariance in Activation Space",
// Sections 2.3 and 4.3.  Split partials go to the same workspace, merged by the
// same reduce kernel as the per-head path.
#include <hip/hip_ext.h>

#include <type_traits>

#include "okv_decode_common.hpp"
#include "okv_kernels.hpp"

namespace okv {

namespace {

using namespace dec;

constexpr int kStep = 64;                 // tokens per wave step (two value tiles)
constexpr int kW7 = (1 << 21) - 1;        // P.V weights: 21-bit integers per step and row
// 2^23 + 0x8080: for 0 <= x < 2^21, x + kDigitBias lies in [2^23, 2^24), where floats are
// spaced by 1, so the sum rounds x to the nearest integer wi and its low 23 bits are
// wi + 0x8080.  Bytes 0 and 1 of those bits with bit 7 flipped, and byte 2 as it is, are
// the balanced base-256 digits of wi as int8: wi = 65536 d2 + 256 d1 + d0 with d0, d1 in
// [-128, 127] and 0 <= d2 < 128.
constexpr float kDigitBias = 8421504.0f;


__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
// Maximum over the 16 lanes of each row (quad xor 1 and 2, then row rotations by 4 and 8).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true)));
  v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true)));
  v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x124, 0xF, 0xF, true)));
  return umax(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, true)));
}

// Storage row of weight row r (16 rows of 64 bytes): rows keep their group of four and
// rotate inside it by r / 4.
__device__ __forceinline__ int wrow(int r) { return (r & ~3) | ((r + (r >> 2)) & 3); }

// Four consecutive metadata values of LDS as floats (float32 or float16 rows).
__device__ __forceinline__ void meta4(const float* m, float v[4]) {
  const float4 x = *reinterpret_cast<const float4*>(m);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void meta4(const _Float16* m, float v[4]) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 x = *reinterpret_cast<const h4*>(m);
  v[0] = static_cast<float>(x[0]); v[1] = static_cast<float>(x[1]);
  v[2] = static_cast<float>(x[2]); v[3] = static_cast<float>(x[3]);
}

// Balanced base-256 digits: q = 65536 hi + 256 mi + lo, each in [-128, 127].
__device__ __forceinline__ void digits_q(int q, int& hi, int& mi, int& lo) {
  lo = ((q + 128) & 255) - 128;
  const int q2 = (q - lo) >> 8;
  mi = ((q2 + 128) & 255) - 128;
  hi = (q2 - mi) >> 8;
}

// A token's metadata row of MDB bytes (2, 4, 8 or a multiple of 16) into dwords (a
// 2-byte row goes to the low half of w[0]).
template <int MDB>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  constexpr int MDW = MDB / 4;
  if constexpr (MDB == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (MDW == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (MDW == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = x[0]; w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < MDW / 4; ++i) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
      w[4 * i] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
    }
  }
}

// Scale s (and zero-point z) of block `bb` from a token's raw metadata row `w`.
template <int FMT>
__device__ __forceinline__ void meta_entry(const uint32_t* w, int bb, float& s, float& z) {
  if constexpr (FMT == kFmtSymF32) {
    s = __uint_as_float(w[bb]);
    z = 0.0f;
  } else if constexpr (FMT == kFmtSymF16) {
    const uint32_t x = w[bb >> 1];
    s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>((bb & 1) ? (x >> 16) : x)));
    z = 0.0f;
  } else {
    // v_cvt_pk_f32_fp8 decodes two OCP E4M3FN bytes on gfx950: entry = (scale, zero-point)
    const int x = static_cast<int>(w[bb >> 1]);
    const auto f = (bb & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(x, true) : __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
    s = f[0];
    z = f[1];
  }
}

template <int NQ, int DPL, int MDW, int BITS>
struct StepRaw {
  uint32_t kw[4][NQ][BITS];  // token 4 (lane % 16) + hf of the step, key group 4 qd + lane / 16
  uint32_t vw[2][DPL][BITS]; // value tile tt of the step, dims lane + 64 k
  uint32_t km[MDW];       // key metadata row of token `lane` of the step
  uint32_t vm[MDW];       // value metadata row of token `lane`
};

// Static shape of the grouped kernel for head dim D, quantisation block BLOCK and query
// group G.  Q.K runs per 128-dim quad on 16-row sets of (head, block) pairs; P.V runs on
// (head, digit) rows, four heads per instruction.
template <int D, int FMT, int BLOCK, int G, int BITS>
struct GroupShape {
  static constexpr int NQ = D / 128;              // 128-dim quads
  static constexpr int BPQ = 128 / BLOCK;         // quantisation blocks per quad (4, 2, 1)
  static constexpr int NBLK = D / BLOCK;
  static constexpr int ROWS = G * BPQ;            // (head, block) rows per quad
  static constexpr int S = (ROWS + 15) / 16;      // 16-row sets
  static constexpr int HPL = 4 / BPQ;             // heads per lane and set (C rows 4 lq .. 4 lq + 3)
  static constexpr int NI = (G + 3) / 4;          // P.V instructions per 16 dims (4 heads x 3 digits)
  static constexpr int NBPB = 8 / BPQ;            // 16-dim output blocks per quantisation block
  static constexpr bool ASYM = FMT == kFmtAsym;
  static constexpr int NS = ASYM ? 2 : 1;         // decoded metadata floats per entry: s (, z)
  static constexpr int MST = ASYM ? 72 : 80;      // padded LDS row of one block's metadata
  // bytes per decoded metadata value in LDS
  static constexpr int MSZ = FMT == kFmtSymF32 || (ASYM && NBLK <= 2) ? 4 : 2;
  static constexpr int UB0 = 4 * 64 * 64;         // per-wave value rows of half a quad
  static constexpr int UB1 = 4 * G * D * 4;       // wave partials in the final combine
  static constexpr int UB2 = G * D * 7;           // prologue: q1 floats and digits
  static constexpr int UB = UB0 > UB1 ? (UB0 > UB2 ? UB0 : UB2) : (UB1 > UB2 ? UB1 : UB2);
  // LDS of one workgroup (bytes): value rows / prologue / partials, weight digits, block
  // metadata, Q operands, small per-head arrays
  static constexpr int LDS = UB + 4 * NQ * S * 3 * 16 * 64 + 4 * 2 * NBLK * NS * MST * MSZ +
                             NQ * S * 2 * 3 * 64 * 16 + 4 * NQ * S * 16 * 4 + 52 * G + 20 * G * NBLK;
};

// Resident waves per SIMD the register allocation aims for at d = 128 and b <= 3: as
// many workgroups as the LDS footprint lets share a CU, up to four with blocks of 32
// dims and three with wider blocks (whose lanes keep two or four heads' rows live: at
// four waves, 128 registers, they spill loop-invariant values and run slower).  At
// d = 256 and b = 4, no constraint.  The kernel streams one step ahead per wave, so
// resident waves set the bytes in flight.
template <int D, int FMT, int BLOCK, int G, int BITS>
constexpr int waves_per_eu() {
  using SH = GroupShape<D, FMT, BLOCK, G, BITS>;
  if (D != 128 || BITS > 3) return 1;
  const int wg = (160 * 1024) / SH::LDS;
  const int cap = BLOCK == 32 ? 4 : 3;
  return wg >= cap ? cap : (wg >= 1 ? wg : 1);
}

// P.V weight scales: one per (head, step), shared by the head's blocks of a quad, so a
// head's row maximum is taken once instead of once per block.  A block whose weights
// reach only 2^-k of the head's largest keeps 21 - k bits, and its share of the output
// is smaller in the same proportion, so the error relative to the output stays that of
// 21-bit weights (on the workloads' caches the blocks' scales are of one magnitude).
// Not where the kernel runs at four waves per SIMD or with 4-bit codes: there the extra
// live values spill or cost a resident wave, and one scale per (head, block) row is
// faster.
template <int D, int FMT, int BLOCK, int G, int BITS>
constexpr bool shared_weight_scale() {
  return BITS <= 3 && waves_per_eu<D, FMT, BLOCK, G, BITS>() < 4;
}

// One workgroup = one (split, KV head, sequence) and all G query heads of that KV
// head; its four waves take the split's 64-token steps in turn.
template <int D, int FMT, int BLOCK, int G, int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D, FMT, BLOCK, G, BITS>())))
void decode_grouped_kernel(const DecodeParams p) {
  using SH = GroupShape<D, FMT, BLOCK, G, BITS>;
  constexpr int NQ = SH::NQ, BPQ = SH::BPQ, NBLK = SH::NBLK, ROWS = SH::ROWS, S = SH::S, HPL = SH::HPL;
  constexpr int NI = SH::NI, NBPB = SH::NBPB, NS = SH::NS, MST = SH::MST, UB = SH::UB;
  constexpr bool ASYM = SH::ASYM;
  constexpr bool SHW = shared_weight_scale<D, FMT, BLOCK, G, BITS>();
  // P.V results combined one 16-dim block late (a few more live registers: the same
  // shapes as the shared weight scale)
  constexpr bool DEFER = SHW;
  constexpr int NSC = SHW ? 1 : BPQ;   // weight scales per (lane head, quad)
  static_assert(BPQ >= 1 && BPQ <= 4 && G >= 2, "blocks of 32 .. 128 dims, query groups of two or more");
  constexpr int ROWB = BITS * D / 8;   // bytes per key row
  constexpr int GB = 4 * BITS;         // bytes per 32-code group
  constexpr int EXC = 1 << (BITS - 1); // excess of symmetric codes
  constexpr int MB = FMT == kFmtSymF32 ? 4 : 2;      // bytes per metadata entry
  constexpr int MDB = NBLK * MB;                     // metadata bytes per token (2 .. 64)
  constexpr int MDW = (MDB + 3) / 4;                 // metadata dwords per token
  constexpr int NBQ = 8;               // 16-dim output blocks per quad
  constexpr int DPL = D / 64;          // value groups per lane and tile
  constexpr int NU = G * D / 256;      // query elements per thread in the prologue
  constexpr int SPAN = BLOCK < 64 ? BLOCK : 64;      // lanes of one block inside a wave
  // fixed-point limit that keeps every int32 block sum exact (see q_limit)
  constexpr int QMAX = q_limit(BLOCK, code_max(ASYM, BITS));
  constexpr int WMAX = w_limit(code_max(ASYM, BITS), kW7);
  static_assert(NU >= 1 && G * D % 256 == 0, "prologue: whole waves per head");
  // fp16 scales stay float16 in LDS (half-size rows, no conversion); E4M3 pairs decode
  // to float32 (v_cvt_pk_f32_fp8) and are kept as float32 when there are at most two
  // blocks (no conversion back), else as float16 (exact) to keep the LDS footprint
  using MT = typename std::conditional<SH::MSZ == 4, float, _Float16>::type;
  using Raw = StepRaw<NQ, DPL, MDW, BITS>;

  // u_s: q1 and its digits (prologue), decoded value rows (steps), wave partials (end)
  __shared__ __align__(16) uint8_t u_s[UB];
  // weight digit planes per (quad, row set, digit): 16 (head, block) rows of 64 tokens;
  // row r is stored at wrow(r), which moves the four rows r with the same r % 4 (written
  // by one instruction from the four lane rows) to different banks
  __shared__ __align__(16) uint8_t wq_s[4][NQ][S][3][16][kStep];
  __shared__ __align__(16) MT mf_s[4][2][NBLK][NS][MST];        // [key/value][block][s, z][token]
  // Q operands (the same for every wave, indexed by lane; in registers they would cost
  // resident waves)
  __shared__ __align__(16) v4i qbs_s[NQ][S][2][3][64];
  // P.V weight scales per quad: per head (first G entries) or per (head, block) row
  __shared__ __align__(16) float wsg_s[4][NQ][16 * S];
  __shared__ float alpha_s[4][G];                                // softmax rescaling per head
  __shared__ float cm_s[4][G], cl_s[4][G];
  __shared__ float cob_s[4][G][NBLK];
  __shared__ int32_t qds_s[G][NBLK];                 // per (head, block): sum of q
  __shared__ uint32_t qam_s[G];                      // per head: max |q1| (float bits)

  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const size_t unit = static_cast<size_t>(b) * p.hkv + hk;

  // ---- q1 = U q for the G heads of the group; 24-bit fixed point per head
  float(*q_s)[D] = reinterpret_cast<float(*)[D]>(u_s);
  uint8_t(*qd_s)[G][D] = reinterpret_cast<uint8_t(*)[G][D]>(u_s + G * D * 4);
  const size_t qoff = (static_cast<size_t>(b) * p.hq + static_cast<size_t>(hk) * G) * D;
  for (int e = tid; e < G * D; e += 256) {
    const int jd = e % D;
    float x = p.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff + e])
                        : reinterpret_cast<const float*>(p.q)[qoff + e];
    if (p.rotation == kRotSign) x *= p.rot[jd];
    q_s[e / D][jd] = x;
  }
  if (tid < G) qam_s[tid] = 0u;
  for (int e = tid; e < G * NBLK; e += 256) (&qds_s[0][0])[e] = 0;
  __syncthreads();
  for (int hs = 1; hs < D && p.rotation != kRotNone; hs <<= 1) {   // U = I: no transform
    for (int e = tid; e < G * D / 2; e += 256) {
      const int h = e / (D / 2), pi = e % (D / 2);
      const int i = (pi / hs) * 2 * hs + (pi % hs);
      const float a = q_s[h][i], c = q_s[h][i + hs];
      q_s[h][i] = a + c;
      q_s[h][i + hs] = a - c;
    }
    __syncthreads();
  }
  const float cn = rsqrtf(static_cast<float>(D));
  float yq[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    // a wave's 64 consecutive elements belong to one head (64 | D)
    const int e = tid + 256 * u, h = e / D, jd = e % D;
    float y;
    if (p.rotation == kRotSo4) {
      const float* R = p.rot + 16 * (jd >> 2) + 4 * (jd & 3);
      const float* xs = &q_s[h][jd & ~3];
      y = R[0] * xs[0] + R[1] * xs[1] + R[2] * xs[2] + R[3] * xs[3];
    } else {
      y = q_s[h][jd];
    }
    yq[u] = p.rotation == kRotNone ? y : y * cn;
    const float am = wave_max_fast(fabsf(yq[u]));
    if (lane == 0) atomicMax(&qam_s[h], __float_as_uint(am));
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = tid + 256 * u, h = e / D, jd = e % D;
    const float am = __uint_as_float(qam_s[h]);
    const float inv = am > 0.0f ? static_cast<float>(QMAX) / am : 0.0f;
    int qi = static_cast<int>(__builtin_rintf(yq[u] * inv));
    qi = qi > QMAX ? QMAX : (qi < -QMAX ? -QMAX : qi);
    int hi, mi, lo;
    digits_q(qi, hi, mi, lo);
    qd_s[0][h][jd] = static_cast<uint8_t>(hi);
    qd_s[1][h][jd] = static_cast<uint8_t>(mi);
    qd_s[2][h][jd] = static_cast<uint8_t>(lo);
    // block sums: over the SPAN consecutive lanes of the block in this wave, then
    // across waves (blocks of 128 dims span two waves) in LDS
    int s0 = qi;
#pragma unroll
    for (int m = 1; m < SPAN; m <<= 1) s0 += __shfl_xor(s0, m, 64);
    if (jd % SPAN == 0) atomicAdd(&qds_s[h][jd / BLOCK], s0);
  }
  __syncthreads();

  // ---- lane roles.  Q.K runs as C = Q K^T per row set s: C rows are the (head, block)
  // pairs r = 16 s + row (head r / BPQ, block r % BPQ of the quad), C columns 16 tokens.
  // Column j of 16-token group hf is token 4 j + hf of the step, so lane (j, lq) ends with
  // the logits of four consecutive tokens for C rows 4 lq .. 4 lq + 3 of each set: heads
  // (16 s + 4 lq) / BPQ .. + HPL - 1, every block of the quad.  A head's logit is summed
  // over its blocks inside the lane; the weights the lane forms are those rows.  P.V
  // runs on (head, digit) rows: instruction i takes heads 4 i .. 4 i + 3, row 4 hh + d
  // = digit d of head 4 i + hh (d = 3: zero), so lane (dim j, lq) ends with the three
  // digit sums of head 4 i + lq.
  const int j = lane & 15;             // Q row / token column / dim within 16
  const int lq = lane >> 4;            // k-chunk of the operands; lane row group of the results
  // head of set s, head slot hl of this lane (valid when < G)
  auto head_of = [&](int s, int hl) { return (16 * s + 4 * lq) / BPQ + hl; };
  // base-2 logit per integer unit of each head this lane holds (kept positive: a zero
  // query has all-zero logits)
  float c_logit[S][HPL];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hl = 0; hl < HPL; ++hl) {
      const int h = head_of(s, hl) < G ? head_of(s, hl) : G - 1;
      const float am = __uint_as_float(qam_s[h]);
      c_logit[s][hl] = fmaxf((am / static_cast<float>(QMAX)) * kLog2e * cn, 1.0e-30f);
    }
  int cinit[NQ][S][4];   // initial value of the low-digit chain per C row
  float qsum_f[NQ][S][4];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      // Q operand row j of set s: digit d of q_h at dims 32 (4 qd + lq) + 16 c + e (e < 16),
      // zero outside the row's block and for rows past the group
      const int rA = 16 * s + j;
      const int hA = rA / BPQ < G ? rA / BPQ : G - 1;
      const int blkA = qd * BPQ + rA % BPQ;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int dim0 = 32 * (4 * qd + lq) + 16 * c;
        const bool in_blk = rA < ROWS && dim0 / BLOCK == blkA;   // 16 dims never straddle a block
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          const uint4 w = *reinterpret_cast<const uint4*>(&qd_s[d][hA][dim0]);
          const v4i x = in_blk ? v4i{static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                                     static_cast<int>(w.w)}
                               : v4i{0, 0, 0, 0};
          if (wave == 0) qbs_s[qd][s][c][d][lane] = x;
        }
      }
      // C row 4 lq + rr of set s; symmetric codes are centred (u - 2^(b-1)) by the
      // low-digit chain's initial value -2^(b-1) sum(q) (the digit combination wraps in
      // int32; only the centred total must fit)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * s + 4 * lq + rr;
        const bool ok = r < ROWS;
        const int hr = ok ? r / BPQ : 0, br = qd * BPQ + r % BPQ;
        cinit[qd][s][rr] = (ASYM || !ok) ? 0 : static_cast<int>(static_cast<uint32_t>(-EXC) * static_cast<uint32_t>(qds_s[hr][br]));
        qsum_f[qd][s][rr] = ok ? static_cast<float>(qds_s[hr][br]) : 0.0f;
      }
    }
  }
  __syncthreads();   // u_s is reused for value rows below

  float m_run[S][HPL], l_run[S][HPL];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hl = 0; hl < HPL; ++hl) {
      m_run[s][hl] = -INFINITY;
      l_run[s][hl] = 0.0f;
    }
  float ob[NQ][S][4];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ob[qd][s][rr] = 0.0f;
  float acc[NQ][NI][NBQ];   // head 4 i + lq, dim 128 qd + 16 nb + j
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) acc[qd][i][nb] = 0.0f;
  // P.V centring of symmetric codes: the byte -2^(b-1) in every lane of a B operand
  // (a product with it gives -2^(b-1) times each weight row's sum)
  const int exc_b = static_cast<int>(0x01010101u * static_cast<uint32_t>((256 - EXC) & 255));
  const v4i excv = {exc_b, exc_b, exc_b, exc_b};
  // P.V A operand of this lane: row j = 4 hh + d; the (head, block) row it reads is
  // fixed per (instruction i, block) and the digit plane is d
  const int pv_hh = j >> 2, pv_d = j & 3;

  const int T = p.T;
  const int ntiles = (T + kTile - 1) / kTile;
  // buffer resources of this (sequence, KV head); offsets carry the step base in the
  // vector offset, so rows past T (and tiles past the last) read as zero
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_codes + unit * p.tcap * ROWB, static_cast<uint32_t>(T) * ROWB);
  const __amdgpu_buffer_rsrc_t rkm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.k_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rvm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.v_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_codes + unit * p.ntile_cap * static_cast<size_t>(D) * GB,
                                              static_cast<uint32_t>(ntiles) * D * GB);
  const uint32_t koff = static_cast<uint32_t>(4 * j * ROWB + GB * lq);
  uint8_t* vrow = u_s + wave * (64 * 64);        // this wave's value rows [64 dims][64 tokens]
  MT(*mf)[NBLK][NS][MST] = mf_s[wave];

  // key groups of token 4 j + hf of the step (one per 16-token group hf)
  auto load_k = [&](Raw& r, int st, int hf) {
    const uint32_t tok0 = static_cast<uint32_t>(st) * kStep;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      buf_group<BITS>(rk, tok0 * ROWB + koff + (hf * ROWB + 4 * GB * qd), r.kw[hf][qd]);
    }
  };
  // value groups of dim 128 qd + 64 kk + lane of both tiles
  auto load_v = [&](Raw& r, int st, int qd, int kk) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tv = (2 * static_cast<uint32_t>(st) + tt) * D * GB;
      buf_group<BITS>(rv, tv + GB * lane + 64 * GB * (2 * qd + kk), r.vw[tt][2 * qd + kk]);
    }
  };
  // value rows of dims 128 qd + 64 kk .. + 63 to LDS: [dim][64 tokens] bytes, 16-byte
  // chunks rotated
  auto decode_v = [&](const Raw& r, int qd, int kk) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      uint32_t dv[8];
      group_to_bytes<BITS>(r.vw[tt][2 * qd + kk], dv);
      *reinterpret_cast<uint4*>(vrow + lane * 64 + 16 * slot16(2 * tt, lane)) = make_uint4(dv[0], dv[1], dv[2], dv[3]);
      *reinterpret_cast<uint4*>(vrow + lane * 64 + 16 * slot16(2 * tt + 1, lane)) =
          make_uint4(dv[4], dv[5], dv[6], dv[7]);
    }
  };
  auto load_m = [&](Raw& r, int st) {
    const uint32_t tok0 = static_cast<uint32_t>(st) * kStep;
    load_row<MDB>(rkm, (tok0 + lane) * MDB, r.km);
    load_row<MDB>(rvm, (tok0 + lane) * MDB, r.vm);
  };

  // one step from the raw data in `r`; each part of `r` is refilled with step `nx`
  // as soon as it has been consumed
  auto compute_step = [&](Raw& r, int st, int nx) {
    const int base = st * kStep;
    const bool tail = base + kStep > T;            // wave-uniform
    // ---- metadata of token `lane`: decode once, to LDS as floats [block][s, z][token]
#pragma unroll
    for (int bb = 0; bb < NBLK; ++bb) {
      float s, z;
      meta_entry<FMT>(r.km, bb, s, z);
      mf[0][bb][0][lane] = static_cast<MT>(s);
      if constexpr (ASYM) mf[0][bb][1][lane] = static_cast<MT>(z);
      meta_entry<FMT>(r.vm, bb, s, z);
      mf[1][bb][0][lane] = static_cast<MT>(s);
      if constexpr (ASYM) mf[1][bb][1][lane] = static_cast<MT>(z);
    }
    load_m(r, nx);
    // the first value rows go to LDS at once, so their registers refill early
    decode_v(r, 0, 0);
    load_v(r, nx, 0, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    // ---- logits (integer units of c_logit): head slot hl of set s, token 4 j + hf
    float L[S][HPL][4];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hl = 0; hl < HPL; ++hl)
#pragma unroll
        for (int hf = 0; hf < 4; ++hf) L[s][hl][hf] = 0.0f;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      // Q operands of a single row set stay in registers over the quad's four token
      // groups; with two or more sets they are read from LDS where they are used
      v4i qq1[2][3];
      if constexpr (S == 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int d = 0; d < 3; ++d) qq1[c][d] = qbs_s[qd][0][c][d][lane];
      }
      // key scales (and zero-points) of the lane's four tokens, every block of the quad
      float sk[BPQ][4], zk[BPQ][4];
#pragma unroll
      for (int bq = 0; bq < BPQ; ++bq) {
        meta4(&mf[0][qd * BPQ + bq][0][4 * j], sk[bq]);
        if constexpr (ASYM) meta4(&mf[0][qd * BPQ + bq][NS - 1][4 * j], zk[bq]);
      }
#pragma unroll
      for (int hf = 0; hf < 4; ++hf) {
        uint32_t dk[8];
        group_to_bytes<BITS>(r.kw[hf][qd], dk);
        if (qd == NQ - 1) load_k(r, nx, hf);
        const v4i a0 = {static_cast<int>(dk[0]), static_cast<int>(dk[1]), static_cast<int>(dk[2]),
                        static_cast<int>(dk[3])};
        const v4i a1 = {static_cast<int>(dk[4]), static_cast<int>(dk[5]), static_cast<int>(dk[6]),
                        static_cast<int>(dk[7])};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          v4i c[3];
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            const v4i ci = d == 2 ? v4i{cinit[qd][s][0], cinit[qd][s][1], cinit[qd][s][2], cinit[qd][s][3]}
                                  : v4i{0, 0, 0, 0};
            c[d] = mfma64(S == 1 ? qq1[0][d] : qbs_s[qd][s][0][d][lane], a0, ci);
            c[d] = mfma64(S == 1 ? qq1[1][d] : qbs_s[qd][s][1][d][lane], a1, c[d]);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int hl = rr / BPQ, bq = rr % BPQ;
            // sum over the block of q (u - 2^(b-1)) (symmetric) or q u (asymmetric), exact
            const int comb = combine3<16, 8>(c[0][rr], c[1][rr], c[2][rr]);
            float v = __builtin_fmaf(sk[bq][hf], static_cast<float>(comb), L[s][hl][hf]);
            if constexpr (ASYM) v = __builtin_fmaf(zk[bq][hf], qsum_f[qd][s][rr], v);
            L[s][hl][hf] = v;
          }
        }
      }
    }
    if (tail) {
      // a real branch: the empty volatile asm keeps the compiler from turning the
      // masking into selects executed on every step
      asm volatile("");
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int hl = 0; hl < HPL; ++hl)
#pragma unroll
          for (int hf = 0; hf < 4; ++hf)
            if (base + 4 * j + hf >= T) L[s][hl][hf] = -INFINITY;
    }
    // ---- online softmax per head (base 2), lazy maximum: the running maximum moves
    // only when a logit exceeds it by more than 8, which each lane can test on its own
    // tokens; the step maximum over the 16 token columns is needed only then
    float tl[S][HPL];
    bool up = false;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hl = 0; hl < HPL; ++hl) {
        const float t = fmaxf(fmaxf(L[s][hl][0], L[s][hl][1]), fmaxf(L[s][hl][2], L[s][hl][3])) * c_logit[s][hl];
        tl[s][hl] = t;
        up = up || t > m_run[s][hl] + 8.0f;
      }
    if (__any(up)) {
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int hl = 0; hl < HPL; ++hl) {
          // finite: every step holds a valid token
          const float m_new = fmaxf(m_run[s][hl], row16_max(tl[s][hl]));
          const float alpha = __builtin_amdgcn_exp2f(m_run[s][hl] - m_new);
          l_run[s][hl] *= alpha;
#pragma unroll
          for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
            for (int bq = 0; bq < BPQ; ++bq) ob[qd][s][hl * BPQ + bq] *= alpha;
          m_run[s][hl] = m_new;
          const int h = head_of(s, hl);
          if (j == 0 && h < G) alpha_s[wave][h] = alpha;
        }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
      // the P.V accumulators of head 4 i + lq follow their head's rescaling
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int h = 4 * i + lq < G ? 4 * i + lq : G - 1;
        const float a = alpha_s[wave][h];
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
          for (int nb = 0; nb < NBQ; ++nb) acc[qd][i][nb] *= a;
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
    }
    float pr[S][HPL][4];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hl = 0; hl < HPL; ++hl) {
#pragma unroll
        for (int hf = 0; hf < 4; ++hf)
          pr[s][hl][hf] = __builtin_amdgcn_exp2f(__builtin_fmaf(L[s][hl][hf], c_logit[s][hl], -m_run[s][hl]));
        // one term per step in the running float32 sum (its rounding drift grows with
        // the number of terms it takes)
        l_run[s][hl] += (pr[s][hl][0] + pr[s][hl][1]) + (pr[s][hl][2] + pr[s][hl][3]);
      }
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      // ---- weights w = p s_v of row (head, block) as 21-bit integers, byte digits
      float sv[BPQ][4], zv[BPQ][4];
#pragma unroll
      for (int bq = 0; bq < BPQ; ++bq) {
        meta4(&mf[1][qd * BPQ + bq][0][4 * j], sv[bq]);
        if constexpr (ASYM) meta4(&mf[1][qd * BPQ + bq][NS - 1][4 * j], zv[bq]);
      }
      // shared scales: per token, the largest value scale over the quad's blocks
      // (scales are >= 0)
      float svm[4];
#pragma unroll
      for (int hf = 0; hf < 4; ++hf) {
        uint32_t m = __float_as_uint(sv[0][hf]);
        if constexpr (SHW) {
#pragma unroll
          for (int bq = 1; bq < BPQ; ++bq) m = umax(m, __float_as_uint(sv[bq][hf]));
        }
        svm[hf] = __uint_as_float(m);
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int hl = 0; hl < HPL; ++hl) {
          // the largest weight of the scale's rows over the step's 64 tokens: p >= 0 and
          // rounding is monotonic, so with a shared scale it is p svm of the largest
          // product per token; w >= 0, so float bits order as unsigned integers (no NaN
          // quieting).  w winv <= WMAX - 1 up to an ulp of rcp
          const int hw = head_of(s, hl);
          float winv[NSC];
#pragma unroll
          for (int k = 0; k < NSC; ++k) {
            uint32_t mx = 0u;
#pragma unroll
            for (int hf = 0; hf < 4; ++hf)
              mx = umax(mx, __float_as_uint(__builtin_fmaf(pr[s][hl][hf], SHW ? svm[hf] : sv[k][hf], 0.0f)));
            const float wm = __uint_as_float(row16_max_u32(mx));
            winv[k] = wm > 1.0e-30f ? static_cast<float>(WMAX - 1) * __builtin_amdgcn_rcpf(wm) : 0.0f;
            if (j == 0 && hw < G)
              wsg_s[wave][qd][SHW ? hw : 16 * s + 4 * lq + hl * BPQ + k] = wm * (1.0f / static_cast<float>(WMAX - 1));
          }
#pragma unroll
          for (int bq = 0; bq < BPQ; ++bq) {
            const int rr = hl * BPQ + bq;
            // weights w = p s_v, zero past T (the scale reads as zero); fmas, so that a
            // float16 scale enters v_fma_mix_f32 without a separate conversion.  Integer
            // wi and its three digits from one float addition (kDigitBias)
            uint32_t f[4];
#pragma unroll
            for (int hf = 0; hf < 4; ++hf) {
              const float w = __builtin_fmaf(pr[s][hl][hf], sv[bq][hf], 0.0f);
              if constexpr (ASYM) ob[qd][s][rr] = __builtin_fmaf(pr[s][hl][hf], zv[bq][hf], ob[qd][s][rr]);
              f[hf] = __float_as_uint(__builtin_fmaf(w, winv[SHW ? 0 : bq], kDigitBias));
            }
            // byte transpose: digit plane k gets byte k of the four tokens' words; planes 0
            // and 1 then flip bit 7 of every byte (the xor 0x80 of the digit rule)
            const uint32_t x01 = __builtin_amdgcn_perm(f[1], f[0], 0x05010400u);   // f0.b0 f1.b0 f0.b1 f1.b1
            const uint32_t x23 = __builtin_amdgcn_perm(f[3], f[2], 0x05010400u);
            const uint32_t y01 = __builtin_amdgcn_perm(f[1], f[0], 0x07030602u);   // f0.b2 f1.b2 f0.b3 f1.b3
            const uint32_t y23 = __builtin_amdgcn_perm(f[3], f[2], 0x07030602u);
            const int prow = 4 * lq + rr;
            const int off = 16 * slot16(j >> 2, prow) + 4 * (j & 3);
            *reinterpret_cast<uint32_t*>(&wq_s[wave][qd][s][0][wrow(prow)][off]) =
                __builtin_amdgcn_perm(y23, y01, 0x05040100u);                                      // d2
            *reinterpret_cast<uint32_t*>(&wq_s[wave][qd][s][1][wrow(prow)][off]) =
                __builtin_amdgcn_perm(x23, x01, 0x07060302u) ^ 0x80808080u;                        // d1
            *reinterpret_cast<uint32_t*>(&wq_s[wave][qd][s][2][wrow(prow)][off]) =
                __builtin_amdgcn_perm(x23, x01, 0x05040100u) ^ 0x80808080u;                        // d0
          }
        }
      }
      if (qd > 0) {
        // the previous quad's P.V is done with the value rows
        decode_v(r, qd, 0);
        load_v(r, nx, qd, 0);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
      // ---- P.V: rows (head, digit) of one quantisation block, K = the step's 64
      // tokens, 16 dims per instruction
      v4i pa[NI], pc[NI];
      float pw[NI];   // weight scale of head 4 i + lq and the block
      // rows 4 lq + d of ev: the three digit sums of head 4 i + lq for dims 16 nbx + j
      auto combine = [&](const v4i* ev, const float* pws, int nbx) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int ai = combine3<16, 8>(ev[i][0], ev[i][1], ev[i][2]);
          acc[qd][i][nbx] = __builtin_fmaf(pws[i], static_cast<float>(ai), acc[qd][i][nbx]);
        }
      };
      // with DEFER, the products of the previous 16 dims are combined after this
      // block's products are issued, so their results are read an instruction later
      v4i ep[NI];
      float pwp[NI];
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        if (nb == NBQ / 2) {
          // second half of the quad's dims: rows of the first half are done
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_wave_barrier();
          decode_v(r, qd, 1);
          load_v(r, nx, qd, 1);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_wave_barrier();
        }
        if (nb % NBPB == 0) {
          // first 16 dims of block bq: A operands, centring and scales of its rows
          const int bq = nb / NBPB;
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            // rows 4 hh + 3 and rows of heads past the group only feed result rows that
            // are never read, so they take any valid row's digits (no masking)
            const int h = 4 * i + pv_hh < G ? 4 * i + pv_hh : G - 1;
            const int r = h * BPQ + bq;                // (head, block) row of the weights
            const uint4 x = *reinterpret_cast<const uint4*>(
                &wq_s[wave][qd][r >> 4][pv_d < 3 ? pv_d : 2][wrow(r & 15)][16 * slot16(lq, r & 15)]);
            pa[i] = v4i{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z), static_cast<int>(x.w)};
            // symmetric: start each product at -2^(b-1) times the rows' digit sums
            pc[i] = ASYM ? v4i{0, 0, 0, 0} : mfma64(pa[i], excv, v4i{0, 0, 0, 0});
            const int hw = 4 * i + lq < G ? 4 * i + lq : 0;
            pw[i] = wsg_s[wave][qd][SHW ? hw : hw * BPQ + bq];
          }
        }
        const int rrow = 16 * (nb % (NBQ / 2)) + j;
        const uint4 x = *reinterpret_cast<const uint4*>(vrow + rrow * 64 + 16 * slot16(lq, rrow));
        const v4i bv = {static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z), static_cast<int>(x.w)};
        v4i e[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) e[i] = mfma64(pa[i], bv, pc[i]);
        if constexpr (DEFER) {
          if (nb > 0) combine(ep, pwp, nb - 1);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            ep[i] = e[i];
            pwp[i] = pw[i];
          }
        } else {
          combine(e, pw, nb);
        }
      }
      if constexpr (DEFER) combine(ep, pwp, NBQ - 1);
      // the next quad or step overwrites this wave's LDS rows
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
    }
  };

  // Steps are interleaved over the workgroups of a (sequence, KV head): wave w of
  // split s takes steps 4 s + w, then every 4 nsplit-th, so the running workgroups
  // sweep the cache together.  After a wave's last step its prefetch names step
  // s_end, wholly past the buffer ranges: those loads return zeros without touching
  // memory.
  const int s_end = (ntiles + 1) / 2;
  const int sstr = 4 * p.nsplit;
  Raw r;
  int st = split * 4 + wave;
  if (st < s_end) {
    load_m(r, st);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      load_v(r, st, qd, 0);
      load_v(r, st, qd, 1);
    }
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) load_k(r, st, hf);
  }
  for (; st < s_end; st += sstr) compute_step(r, st, st + sstr < s_end ? st + sstr : s_end);

  // ---- combine the four waves; partials per query head (sums over the 16 token
  // columns of each lane row)
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hl = 0; hl < HPL; ++hl) l_run[s][hl] = row16_sum(l_run[s][hl]);
  if constexpr (ASYM) {
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ob[qd][s][rr] = row16_sum(ob[qd][s][rr]);
  }
  __syncthreads();   // every wave is done with its value rows
  float* cacc = reinterpret_cast<float*>(u_s);      // [4][G][D]
  if (j == 0) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hl = 0; hl < HPL; ++hl) {
        const int h = head_of(s, hl);
        if (h < G) {
          cm_s[wave][h] = m_run[s][hl];
          cl_s[wave][h] = l_run[s][hl];
        }
      }
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * s + 4 * lq + rr;
          if (r < ROWS) cob_s[wave][r / BPQ][qd * BPQ + r % BPQ] = ob[qd][s][rr];
        }
  }
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int h = 4 * i + lq;
      if (h < G) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) cacc[(wave * G + h) * D + 128 * qd + 16 * nb + j] = acc[qd][i][nb];
      }
    }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int hh = e / D, dim = e % D;
    const float mx = fmaxf(fmaxf(cm_s[0][hh], cm_s[1][hh]), fmaxf(cm_s[2][hh], cm_s[3][hh]));
    float a = 0.0f, l = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float al = __builtin_amdgcn_exp2f(cm_s[wv][hh] - mx);
        a += al * (cacc[(wv * G + hh) * D + dim] + cob_s[wv][hh][dim / BLOCK]);
        l += al * cl_s[wv][hh];
      }
    }
    const size_t hq = static_cast<size_t>(hk) * G + hh;
    float* out = p.ws + ((static_cast<size_t>(b) * p.hq + hq) * p.nsplit + split) * (D + 2);
    out[dim] = a;
    if (dim == 0) {
      out[D] = mx;
      out[D + 1] = l;
    }
  }
}

template <int D, int FMT, int BLOCK, int G>
void launch_t(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.bits == 2) hipExtLaunchKernelGGL((decode_grouped_kernel<D, FMT, BLOCK, G, 2>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else if (p.bits == 4) hipExtLaunchKernelGGL((decode_grouped_kernel<D, FMT, BLOCK, G, 4>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else hipExtLaunchKernelGGL((decode_grouped_kernel<D, FMT, BLOCK, G, 3>), grid, dim3(256), 0, s, e0, e1, 0, p);
}

template <int D, int BLOCK, int G>
void launch_fmt(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.quant == kQuantAsym) launch_t<D, kFmtAsym, BLOCK, G>(p, grid, s, e0, e1);
  else if (p.scale_dtype == kScaleF32) launch_t<D, kFmtSymF32, BLOCK, G>(p, grid, s, e0, e1);
  else launch_t<D, kFmtSymF16, BLOCK, G>(p, grid, s, e0, e1);
}

template <int D, int G>
bool launch_g(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.block) {
    case 32: launch_fmt<D, 32, G>(p, grid, s, e0, e1); return true;
    case 64: launch_fmt<D, 64, G>(p, grid, s, e0, e1); return true;
    case 128: launch_fmt<D, 128, G>(p, grid, s, e0, e1); return true;
    default: return false;
  }
}

template <int D>
bool launch_d(const DecodeParams& p, int group, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (group) {
    case 2: return launch_g<D, 2>(p, grid, s, e0, e1);
    case 4: return launch_g<D, 4>(p, grid, s, e0, e1);
    case 8: return launch_g<D, 8>(p, grid, s, e0, e1);
    default: return false;
  }
}

}  // namespace

bool grouped_decode_supported(int d, int block, int group) {
  return (d == 128 || d == 256) && (block == 32 || block == 64 || block == 128) &&
         (group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_grouped(const DecodeParams& p, int batch, int d, hipStream_t s, hipEvent_t e0,
                                 hipEvent_t e1) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  if (p.hkv < 1 || p.hq % p.hkv != 0) return hipErrorInvalidValue;
  const int group = p.hq / p.hkv;
  if (!grouped_decode_supported(d, p.block, group)) return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.hkv, batch);
  bool ok = false;
  if (d == 128) ok = launch_d<128>(p, group, grid, s, e0, e1);
  else ok = launch_d<256>(p, group, grid, s, e0, e1);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
