// Decode attention for one query head per workgroup on int8 MFMA
// (v_mfma_i32_16x16x64_i8).  A wave works on steps of 64 tokens (two value tiles).
//
//  * Q.K: the three balanced int8 digits of the 24-bit fixed-point query and the
//    segments of one 128-dim quad (its quantisation blocks, or the quad itself when a
//    block spans quads) give 3 x (128/seg) <= 12 rows: row 4 b + d holds digit d of
//    q restricted to segment b (row 4 b + 3 is zero).
//    B = key codes, 64 dims x 16 tokens (a lane decodes one whole 32-code group and
//    feeds two instructions).  In the result, lane (token j, lq) holds the three
//    digit sums of block lq: they combine exactly in int32 in the lane, the block
//    scale multiplies the sum and two cross-lane adds sum the blocks.
//  * Softmax: base 2, lazy maximum; the maximum is uniform over the wave.
//  * P.V: lane (token j, lq) forms the weight p s of block lq, 22 bits as three
//    balanced int8 digits, into LDS rows (block, digit) x 64 tokens.  A = those
//    rows, B = value codes 64 tokens x 16 dims (decoded once per step into LDS), so
//    lane (dim j, lq) again holds the three digit sums of block lq; it keeps the
//    result when block lq holds its dims.  The block scale and centring of each
//    block live in the same lanes that formed the weights.
//
// Method: "Orthogonally mixed 3-bit KV cache" (idea card), Implementation notes,
// read path, and Key formulas; "Orthogonal Invariance in Activation Space",
// Sections 2.3 and 4.3.  Split partials go to the workspace merged by the reduce
// kernel.
#include <hip/hip_ext.h>

#include "okv_decode_common.hpp"
#include "okv_kernels.hpp"

namespace okv {

namespace {

using namespace dec;

constexpr int kStep = 64;           // tokens per wave step (two value tiles)
constexpr int kWRow = 80;           // bytes per LDS weight row (64 tokens + padding)

template <int NQ, int DPL, int BITS>
struct HeadRaw {
  uint32_t kw[4][NQ][BITS];  // token 16 hf + (lane % 16), key group 4 qd + lane / 16
  uint32_t vw[2][DPL][BITS]; // value tile tt of the step, dims lane + 64 k
};

template <int NQ>
struct HeadMeta {
  uint32_t k[4][NQ];      // raw metadata of (token 16 hf + lane % 16, block of segment qd BPQ + lane / 16)
  uint32_t v[4][NQ];
};

// (scale, zero-point) from a raw metadata entry.
template <int FMT>
__device__ __forceinline__ void meta_sz(uint32_t raw, float& s, float& z) {
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

// One workgroup = one (split, query head, sequence); its four waves take the split's
// 64-token steps in turn.
// STREAM: every code and scale is read by exactly one workgroup (one query head per KV
// head), so the loads are marked non-temporal; with query groups the heads of a group
// re-read the same cache lines and keep the default policy.
template <int D, int FMT, int BLOCK, int BITS, bool STREAM>
__global__ __launch_bounds__(256) void decode_head_kernel(const DecodeParams p) {
  constexpr int kAux = STREAM ? kStreamAux : 0;
  constexpr int NQ = D / 128;          // 128-dim quads
  constexpr int SEG = BLOCK < 128 ? BLOCK : 128;   // block part inside one quad
  constexpr int BPQ = 128 / SEG;       // segments per quad (1, 2 or 4)
  constexpr int NSEG = D / SEG;
  constexpr int NBLK = D / BLOCK;
  constexpr int ROWB = BITS * D / 8;    // bytes per key row
  constexpr int GB = 4 * BITS;         // bytes per 32-code group
  constexpr int EXC = 1 << (BITS - 1); // excess of symmetric codes
  constexpr int MB = FMT == kFmtSymF32 ? 4 : 2;
  constexpr bool ASYM = FMT == kFmtAsym;
  constexpr int NBQ = 8;               // 16-dim output blocks per quad
  constexpr int DPL = D / 64;          // value groups per lane and tile
  constexpr int WPLANE = 16 * kWRow;   // bytes of one quad's 16 weight rows
  // fixed-point limits that keep every int32 sum exact (see q_limit)
  constexpr int QMAX = q_limit(SEG, code_max(ASYM, BITS));
  constexpr int WMAX = w_limit(code_max(ASYM, BITS), static_cast<int>(kWMax));
  using Raw = HeadRaw<NQ, DPL, BITS>;
  using Meta = HeadMeta<NQ>;
  static_assert(D * 7 + 64 <= 4 * 128 * 64, "prologue fits the value-row region");

  // u_s: q1 and its digits (prologue), value rows of one quad per wave (steps),
  // wave partials (end)
  __shared__ __align__(16) uint8_t u_s[4 * 128 * 64];
  // per wave and quad: weight rows 4 b + d (d = 3: zero) of 64 tokens
  __shared__ __align__(16) uint8_t wq_s[4][NQ][WPLANE];
  __shared__ int32_t qds_s[NSEG][4];   // per segment: sum q, hi, mid, lo
  __shared__ float red_s[4];
  __shared__ float cm_s[4], cl_s[4];
  __shared__ float cob_s[4][NSEG];

  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hk = hq / (p.hq / p.hkv);
  const size_t unit = static_cast<size_t>(b) * p.hkv + hk;

  // ---- q1 = U q in float32, then 24-bit fixed point as three balanced int8 digits
  float* q_s = reinterpret_cast<float*>(u_s);
  uint8_t(*qd_s)[D] = reinterpret_cast<uint8_t(*)[D]>(u_s + 4 * D);
  const size_t qoff = (static_cast<size_t>(b) * p.hq + hq) * D;
  if (tid < D) {
    float x = p.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff + tid])
                        : reinterpret_cast<const float*>(p.q)[qoff + tid];
    if (p.rotation == kRotSign) x *= p.rot[tid];
    q_s[tid] = x;
  }
  for (int e = tid; e < NSEG * 4; e += 256) (&qds_s[0][0])[e] = 0;
  // the digit-3 rows of the weight planes stay zero
  for (int e = tid; e < 4 * NQ * WPLANE / 4; e += 256) reinterpret_cast<uint32_t*>(&wq_s[0][0][0])[e] = 0u;
  __syncthreads();
  if (p.rotation != kRotNone) lds_fwht<D>(q_s);   // uniform over the workgroup
  const float cn = rsqrtf(static_cast<float>(D));
  float yq = 0.0f;
  if (tid < D) {
    if (p.rotation == kRotNone) {
      yq = q_s[tid];
    } else if (p.rotation == kRotSo4) {
      const float* R = p.rot + 16 * (tid >> 2) + 4 * (tid & 3);
      const float* xs = q_s + (tid & ~3);
      yq = R[0] * xs[0] + R[1] * xs[1] + R[2] * xs[2] + R[3] * xs[3];
    } else {
      yq = q_s[tid];
    }
    if (p.rotation != kRotNone) yq *= cn;
  }
  float amax_q = wave_max(fabsf(yq));
  if (lane == 0) red_s[wave] = amax_q;
  __syncthreads();
  amax_q = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  if (tid < D) {
    const float inv = amax_q > 0.0f ? static_cast<float>(QMAX) / amax_q : 0.0f;
    int qi = static_cast<int>(__builtin_rintf(yq * inv));
    qi = qi > QMAX ? QMAX : (qi < -QMAX ? -QMAX : qi);
    const int lo = ((qi + 128) & 255) - 128;
    const int q2 = (qi - lo) >> 8;
    const int mi = ((q2 + 128) & 255) - 128;
    const int hi = (q2 - mi) >> 8;
    qd_s[0][tid] = static_cast<uint8_t>(hi);
    qd_s[1][tid] = static_cast<uint8_t>(mi);
    qd_s[2][tid] = static_cast<uint8_t>(lo);
    // segment sums: over min(SEG, 64) lanes, then across waves in LDS
    int s0 = qi, s1 = hi, s2 = mi, s3 = lo;
    constexpr int SPAN = SEG < 64 ? SEG : 64;
#pragma unroll
    for (int m = 1; m < SPAN; m <<= 1) {
      s0 += __shfl_xor(s0, m, 64);
      s1 += __shfl_xor(s1, m, 64);
      s2 += __shfl_xor(s2, m, 64);
      s3 += __shfl_xor(s3, m, 64);
    }
    if (tid % SPAN == 0) {
      const int sg = tid / SEG;
      atomicAdd(&qds_s[sg][0], s0);
      atomicAdd(&qds_s[sg][1], s1);
      atomicAdd(&qds_s[sg][2], s2);
      atomicAdd(&qds_s[sg][3], s3);
    }
  }
  __syncthreads();

  // ---- lane roles
  const int j = lane & 15;             // token (Q.K) / dim in the 16-dim block (P.V); A row
  const int lq = lane >> 4;            // k-chunk of the operands; block of the result rows
  const bool bvalid = lq < BPQ;        // lane's result rows belong to segment lq of the quad
  const float c_logit = fmaxf((amax_q / static_cast<float>(QMAX)) * kLog2e * cn, 1.0e-30f);
  // A operands of Q.K: row j = 4 bA + d, dims 32 (4 qd + lq) + 16 c + e (e < 16)
  v4i qa[NQ][2];
  int cinit[NQ][4];
  float qsum_f[NQ];
  {
    const int d = j & 3, bA = j >> 2;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int dim0 = 32 * (4 * qd + lq) + 16 * c;
        const bool use = d < 3 && bA < BPQ && dim0 / SEG == qd * BPQ + bA;
        const uint4 w = *reinterpret_cast<const uint4*>(&qd_s[d < 3 ? d : 0][dim0]);
        qa[qd][c] = use ? v4i{static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                              static_cast<int>(w.w)}
                        : v4i{0, 0, 0, 0};
      }
      // result rows 4 lq + r = (segment lq, digit r); symmetric codes centred by
      // -2^(b-1) sum(digits) over the segment
      const int sg = qd * BPQ + (bvalid ? lq : 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) cinit[qd][r] = (!ASYM && bvalid && r < 3) ? -EXC * qds_s[sg][1 + r] : 0;
      qsum_f[qd] = bvalid ? static_cast<float>(qds_s[sg][0]) : 0.0f;
    }
  }
  __syncthreads();   // u_s is reused for value rows below

  float m_run = -INFINITY, l_run = 0.0f;
  float ob[NQ];
  float acc[NQ][NBQ];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    ob[qd] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) acc[qd][nb] = 0.0f;
  }

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
  const uint32_t koff = static_cast<uint32_t>(j * ROWB + GB * lq);
  const uint32_t moff = static_cast<uint32_t>(j * NBLK * MB);
  uint8_t* vrow = u_s + wave * (128 * 64);       // this wave's value rows [128 dims][64 tokens]

  auto load_k = [&](Raw& r, int st, int hf) {
    const uint32_t tok0 = static_cast<uint32_t>(st) * kStep;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      buf_group<BITS, kAux>(rk, tok0 * ROWB + koff + (16 * hf * ROWB + 4 * GB * qd), r.kw[hf][qd]);
    }
  };
  auto load_v = [&](Raw& r, int st, int qd) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tv = (2 * static_cast<uint32_t>(st) + tt) * D * GB;
#pragma unroll
      for (int k = 2 * qd; k < 2 * qd + 2; ++k) buf_group<BITS, kAux>(rv, tv + GB * lane + 64 * GB * k, r.vw[tt][k]);
    }
  };
  auto load_m = [&](Meta& m, int st) {
    const uint32_t tok0 = static_cast<uint32_t>(st) * kStep;
#pragma unroll
    for (int hf = 0; hf < 4; ++hf)
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        // block of segment qd BPQ + lq (lanes with lq >= BPQ read a neighbouring
        // entry, or zero past T; unused)
        const uint32_t o = (tok0 + 16 * hf) * (NBLK * MB) + moff + ((qd * BPQ + lq) * SEG / BLOCK) * MB;
        m.k[hf][qd] = buf_meta<FMT, kAux>(rkm, o, 0);
        m.v[hf][qd] = buf_meta<FMT, kAux>(rvm, o, 0);
      }
  };
  // value rows of quad qd to LDS: [dim][64 tokens] bytes, 16-byte chunks rotated
  auto decode_v = [&](const Raw& r, int qd) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int rrow = lane + 64 * kk;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t dv[8];
        group_to_bytes<BITS>(r.vw[tt][2 * qd + kk], dv);
        *reinterpret_cast<uint4*>(vrow + rrow * 64 + 16 * slot16(2 * tt, rrow)) =
            make_uint4(dv[0], dv[1], dv[2], dv[3]);
        *reinterpret_cast<uint4*>(vrow + rrow * 64 + 16 * slot16(2 * tt + 1, rrow)) =
            make_uint4(dv[4], dv[5], dv[6], dv[7]);
      }
    }
  };

  // one step from `r` and `mc`; the parts of `r` are refilled with step `nx` as soon as
  // they are consumed, and `mn` receives the metadata of step `nx`
  auto compute_step = [&](Raw& r, const Meta& mc, Meta& mn, int st, int nx) {
    const int base = st * kStep;
    const bool tail = base + kStep > T;          // wave-uniform
    load_m(mn, nx);
    decode_v(r, 0);
    load_v(r, nx, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    // ---- logits of tokens 16 hf + j: block partials in lane lq, summed across lanes
    float L[4];
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) {
      float val = 0.0f;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        uint32_t dk[8];
        group_to_bytes<BITS>(r.kw[hf][qd], dk);
        if (qd == NQ - 1) load_k(r, nx, hf);
        const v4i b0 = {static_cast<int>(dk[0]), static_cast<int>(dk[1]), static_cast<int>(dk[2]),
                        static_cast<int>(dk[3])};
        const v4i b1 = {static_cast<int>(dk[4]), static_cast<int>(dk[5]), static_cast<int>(dk[6]),
                        static_cast<int>(dk[7])};
        v4i c = {cinit[qd][0], cinit[qd][1], cinit[qd][2], cinit[qd][3]};
        c = mfma64(qa[qd][0], b0, c);
        c = mfma64(qa[qd][1], b1, c);
        // sum over block lq of q (u - 2^(b-1)) (symmetric) or q u (asymmetric), exact
        const int comb = combine3<16, 8>(c[0], c[1], c[2]);
        float s, z;
        meta_sz<FMT>(mc.k[hf][qd], s, z);
        float v = s * static_cast<float>(comb);
        if constexpr (ASYM) v = __builtin_fmaf(z, qsum_f[qd], v);
        val += bvalid ? v : 0.0f;
      }
      L[hf] = val;
    }
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) L[hf] += swz_xor16(L[hf]);
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) L[hf] += __shfl_xor(L[hf], 32, 64);
    if (tail) {
#pragma unroll
      for (int hf = 0; hf < 4; ++hf)
        if (base + 16 * hf + j >= T) L[hf] = -INFINITY;
    }
    // ---- online softmax (base 2), lazy maximum; the step maximum is wave-uniform
    float tmax = fmaxf(fmaxf(L[0], L[1]), fmaxf(L[2], L[3]));
    tmax = row16_max(tmax) * c_logit;     // finite: every step holds a valid token
    if (__any(tmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        ob[qd] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) acc[qd][nb] *= alpha;
      }
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) pr[hf] = __builtin_amdgcn_exp2f(__builtin_fmaf(L[hf], c_logit, -m_run));
    // the step's four weights are summed first, so that the running float32 sum takes
    // one term per step (its rounding drift grows with the number of terms it takes)
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      if (qd > 0) {
        // the previous quad's P.V is done with the value rows
        decode_v(r, qd);
        load_v(r, nx, qd);
      }
      // ---- weights w = p s_v of (token 16 hf + j, segment lq): 22-bit integers relative
      // to the segment's step maximum, three balanced int8 digits
      float w[4];
      float wm = 0.0f;
#pragma unroll
      for (int hf = 0; hf < 4; ++hf) {
        float s, z;
        meta_sz<FMT>(mc.v[hf][qd], s, z);
        w[hf] = bvalid ? pr[hf] * s : 0.0f;        // zero past T (scale reads as zero)
        if constexpr (ASYM) ob[qd] = __builtin_fmaf(bvalid ? pr[hf] : 0.0f, z, ob[qd]);
        wm = fmaxf(wm, w[hf]);
      }
      wm = row16_max(wm);
      // w winv + 1/2 stays below WMAX + 1 (rcp is within an ulp), so truncation rounds
      const float winv = wm > 1.0e-30f ? (WMAX - 1.0f) * __builtin_amdgcn_rcpf(wm) : 0.0f;
      int ws = 0;
      uint8_t* wrow = &wq_s[wave][qd][0];
#pragma unroll
      for (int hf = 0; hf < 4; ++hf) {
        const uint32_t wi = static_cast<uint32_t>(__builtin_fmaf(w[hf], winv, 0.5f));
        if constexpr (!ASYM) ws += static_cast<int>(wi);
        // balanced digits: lo = byte 0 of w, mid = byte 1 of w + 128, hi = byte 2 of w + 32896
        const int tok = 16 * hf + j;
        wrow[(4 * lq + 0) * kWRow + tok] = static_cast<uint8_t>((wi + 32896u) >> 16);
        wrow[(4 * lq + 1) * kWRow + tok] = static_cast<uint8_t>((wi + 128u) >> 8);
        wrow[(4 * lq + 2) * kWRow + tok] = static_cast<uint8_t>(wi);
      }
      int wcen = 0;
      // centring of (u - 2^(b-1)); unsigned: only the centred sum below must fit in int32
      if constexpr (!ASYM) wcen = static_cast<int>(static_cast<uint32_t>(EXC) * static_cast<uint32_t>(row16_sum(ws)));
      const float wsig = wm * (1.0f / (WMAX - 1.0f));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
      // ---- P.V: A = weight rows 4 b + d (lane row j), K = the step's 64 tokens
      const uint4 xa = *reinterpret_cast<const uint4*>(wrow + j * kWRow + 16 * lq);
      const v4i a = {static_cast<int>(xa.x), static_cast<int>(xa.y), static_cast<int>(xa.z),
                     static_cast<int>(xa.w)};
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        const int rrow = 16 * nb + j;
        const uint4 xb = *reinterpret_cast<const uint4*>(vrow + rrow * 64 + 16 * slot16(lq, rrow));
        const v4i bv = {static_cast<int>(xb.x), static_cast<int>(xb.y), static_cast<int>(xb.z),
                        static_cast<int>(xb.w)};
        const v4i e = mfma64(a, bv, v4i{0, 0, 0, 0});
        // valid in the lanes whose segment lq holds dims 16 nb .. 16 nb + 15
        const int ai = static_cast<int>(static_cast<uint32_t>(combine3<16, 8>(e[0], e[1], e[2])) -
                                        static_cast<uint32_t>(wcen));
        acc[qd][nb] = __builtin_fmaf(wsig, static_cast<float>(ai), acc[qd][nb]);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
    }
  };

  // Steps are interleaved over the workgroups of a (sequence, head): wave w of split s
  // takes steps 4 s + w, then every 4 nsplit-th, so the running workgroups sweep the
  // cache together.  After a wave's last step its prefetch names step s_end, wholly
  // past the buffer ranges: those loads return zeros without touching memory.
  const int s_end = (ntiles + 1) / 2;
  const int sstr = 4 * p.nsplit;
  Raw r;
  Meta ma, mb;
  int st = split * 4 + wave;
  if (st < s_end) {
    load_m(ma, st);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) load_v(r, st, qd);
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) load_k(r, st, hf);
  }
  while (st < s_end) {
    compute_step(r, ma, mb, st, st + sstr < s_end ? st + sstr : s_end);
    st += sstr;
    if (st >= s_end) break;
    compute_step(r, mb, ma, st, st + sstr < s_end ? st + sstr : s_end);
    st += sstr;
  }

  // ---- combine the four waves
  const float lsum = row16_sum(l_run);          // the four lane rows hold the same tokens
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) ob[qd] = row16_sum(ob[qd]);
  __syncthreads();   // every wave is done with its value rows
  float* cacc = reinterpret_cast<float*>(u_s);  // [4][D]
  if (lane == 0) {
    cm_s[wave] = m_run;
    cl_s[wave] = lsum;
  }
  if (j == 0 && bvalid) {
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) cob_s[wave][qd * BPQ + lq] = ob[qd];   // per segment
  }
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb)
      if (lq == (16 * nb) / SEG) cacc[wave * D + 128 * qd + 16 * nb + j] = acc[qd][nb];
  __syncthreads();
  if (tid < D) {
    const int dim = tid;
    const float mx = fmaxf(fmaxf(cm_s[0], cm_s[1]), fmaxf(cm_s[2], cm_s[3]));
    float a = 0.0f, l = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float al = __builtin_amdgcn_exp2f(cm_s[wv] - mx);
        a += al * (cacc[wv * D + dim] + cob_s[wv][dim / SEG]);
        l += al * cl_s[wv];
      }
    }
    float* out = p.ws + ((static_cast<size_t>(b) * p.hq + hq) * p.nsplit + split) * (D + 2);
    out[dim] = a;
    if (dim == 0) {
      out[D] = mx;
      out[D + 1] = l;
    }
  }
}

template <int D, int FMT, int BLOCK, bool STREAM>
void launch_s(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.bits == 2) {
    hipExtLaunchKernelGGL((decode_head_kernel<D, FMT, BLOCK, 2, STREAM>), grid, dim3(256), 0, s, e0, e1, 0, p);
  } else if (p.bits == 4) {
    hipExtLaunchKernelGGL((decode_head_kernel<D, FMT, BLOCK, 4, STREAM>), grid, dim3(256), 0, s, e0, e1, 0, p);
  } else {
    hipExtLaunchKernelGGL((decode_head_kernel<D, FMT, BLOCK, 3, STREAM>), grid, dim3(256), 0, s, e0, e1, 0, p);
  }
}

template <int D, int FMT, int BLOCK>
void launch_t(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.hq == p.hkv) launch_s<D, FMT, BLOCK, true>(p, grid, s, e0, e1);
  else launch_s<D, FMT, BLOCK, false>(p, grid, s, e0, e1);
}

template <int D, int BLOCK>
void launch_fmt(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.quant == kQuantAsym) launch_t<D, kFmtAsym, BLOCK>(p, grid, s, e0, e1);
  else if (p.scale_dtype == kScaleF32) launch_t<D, kFmtSymF32, BLOCK>(p, grid, s, e0, e1);
  else launch_t<D, kFmtSymF16, BLOCK>(p, grid, s, e0, e1);
}

template <int D>
bool launch_d(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.block) {
    case 32: launch_fmt<D, 32>(p, grid, s, e0, e1); return true;
    case 64: launch_fmt<D, 64>(p, grid, s, e0, e1); return true;
    case 128: launch_fmt<D, 128>(p, grid, s, e0, e1); return true;
    case 256:
      if constexpr (D >= 256) {
        launch_fmt<D, 256>(p, grid, s, e0, e1);
        return true;
      }
      return false;
    default: return false;
  }
}

}  // namespace

bool head_decode_supported(int d, int block) {
  return (d == 128 || d == 256) && block >= 32 && block <= d && d % block == 0 && (block & (block - 1)) == 0;
}

hipError_t launch_decode_head(const DecodeParams& p, int batch, int d, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  if (p.hkv < 1 || p.hq % p.hkv != 0) return hipErrorInvalidValue;
  if (!head_decode_supported(d, p.block)) return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.hq, batch);
  bool ok = false;
  if (d == 128) ok = launch_d<128>(p, grid, s, e0, e1);
  else ok = launch_d<256>(p, grid, s, e0, e1);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
