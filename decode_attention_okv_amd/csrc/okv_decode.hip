// Read path: decode attention directly over the packed 3-bit cache.
//
// Pages: "Orthogonally mixed 3-bit KV cache", Implementation notes (the read
// path: the query is rotated by U, the packed keys are decoded and scaled inside
// the dot product, the softmax weights multiply the decoded rotated values and U^T
// maps the result back; full-precision K/V never exist in memory) and Key
// formulas (attention as softmax of the scaled logits times V); "Orthogonal
// Invariance in Activation Space", Section 2.3 (rotating q together with k, and
// rotating the output back, leaves attention unchanged) and Section 4.3
// (dequantisation fused into the attention kernel).
//
// Split-K: the token range of each (sequence, query head) is cut into splits; one
// workgroup per split produces (m, l, acc[D]) with m the running maximum of the
// base-2 logits, l = sum 2^(logit - m) and acc the matching weighted sum of the
// dequantised rotated values; the reduce kernel merges the splits, normalises
// and applies U^T.
//
// Both quantisers are handled in one centred form: x_hat = s (u - 4) + o with
// o = 0 (symmetric codes) or o = z + 4 s (asymmetric codes; exact in float32).
#include <hip/hip_ext.h>

#include "okv_decode_common.hpp"

namespace okv {

namespace {

using namespace dec;

// Raw loads of one compute step: NT consecutive 32-token tiles.
template <int D, int NT>
struct StepRaw {
  static constexpr int NG = D / 32;
  static constexpr int IPL = NT * kTile / (64 / NG);   // key items per lane
  static constexpr int DPL = D / 64;                   // value dims per lane (per tile)
  uint32_t kw[IPL][3];
  uint32_t km[IPL];
  uint32_t vw[NT][DPL][3];
  uint32_t vm[IPL];
};

// One workgroup = one (split, query head, sequence); its four waves take the split's
// steps of NT 32-token tiles in turn, each wave double-buffering the raw loads of
// its next step.
//  * keys: lane (token slot, 32-dim group g) unpacks its group to byte lanes and
//    takes int8 dot products against q in 24-bit fixed point (three balanced int8
//    digits, each centred by its digit sum: exact in int32); the block scale is
//    applied to the integer result; the D/32 partials of a token are summed across
//    lanes;
//  * softmax in base 2; the running maximum is raised only when a logit exceeds it
//    by more than 8, so weights stay <= 256 and rescaling is rare;
//  * values: each lane owns D/64 dims of the dim-major value tiles; the step's
//    weights w = p s become 22-bit integers relative to the step maximum, stored as
//    three byte planes in LDS, and meet the codes in unsigned int8 dot products
//    (exact in int32); one float multiply-add per dim and step.
template <int D, int FMT, int BLOCK, int NT>
__global__ __launch_bounds__(256) void decode_valu_kernel(const DecodeParams p) {
  using Raw = StepRaw<D, NT>;
  constexpr int STEP = NT * kTile;      // tokens per compute step
  constexpr int NG = Raw::NG;           // 32-dim groups per key row
  constexpr int TPR = 64 / NG;          // token slots covered by the 64 lanes per round
  constexpr int IPL = Raw::IPL;         // key items per lane per step
  constexpr int LPG = 64 / NG;          // lanes per 32-dim value group
  constexpr int DPL = Raw::DPL;         // value dims per lane
  constexpr int GPB = BLOCK / 32;       // 32-dim groups per quantisation block
  constexpr int NBLK = D / BLOCK;
  constexpr int ROWB = 3 * D / 8;       // bytes of a key code row
  constexpr int MB = FMT == kFmtSymF32 ? 4 : 2;   // metadata bytes per block
  static_assert(D <= 256, "one thread per q element");

  __shared__ float q_s[D];
  __shared__ __align__(16) uint8_t qd_s[3][D];    // q digit planes (hi, mid, lo)
  __shared__ int32_t qsum_s[NG][4];               // per group: sum of q, of hi, mid, lo
  __shared__ float red_s[4];
  __shared__ __align__(16) uint8_t wq[4][NBLK][3][STEP];  // per-wave weight planes (lo, mid, hi)
  __shared__ int32_t wsum_s[4][NBLK];
  __shared__ float cm_s[4], cl_s[4];
  __shared__ float cacc_s[4][D];
  __shared__ float cob_s[4][NBLK];

  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hk = hq / (p.hq / p.hkv);
  const size_t unit = static_cast<size_t>(b) * p.hkv + hk;

  // ---- q1 = U q in float32, then 24-bit fixed point as three balanced int8 digits
  const size_t qoff = (static_cast<size_t>(b) * p.hq + hq) * D;
  if (tid < D) {
    float x = p.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff + tid])
                        : reinterpret_cast<const float*>(p.q)[qoff + tid];
    if (p.rotation == kRotSign) x *= p.rot[tid];
    q_s[tid] = x;
  }
  __syncthreads();
  lds_fwht<D>(q_s);
  const float cn = rsqrtf(static_cast<float>(D));
  float yq = 0.0f;
  if (tid < D) {
    if (p.rotation == kRotSo4) {
      const float* R = p.rot + 16 * (tid >> 2) + 4 * (tid & 3);
      const float* xs = q_s + (tid & ~3);
      yq = R[0] * xs[0] + R[1] * xs[1] + R[2] * xs[2] + R[3] * xs[3];
    } else {
      yq = q_s[tid];
    }
    yq *= cn;
  }
  float amax_q = wave_max(fabsf(yq));
  if (lane == 0) red_s[wave] = amax_q;
  __syncthreads();
  amax_q = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  if (tid < D) {
    const float inv = amax_q > 0.0f ? static_cast<float>(kQMax) / amax_q : 0.0f;
    int qi = static_cast<int>(__builtin_rintf(yq * inv));
    qi = qi > kQMax ? kQMax : (qi < -kQMax ? -kQMax : qi);
    const int lo = ((qi + 128) & 255) - 128;
    const int q2 = (qi - lo) >> 8;
    const int mi = ((q2 + 128) & 255) - 128;
    const int hi = (q2 - mi) >> 8;
    qd_s[0][tid] = static_cast<uint8_t>(hi);
    qd_s[1][tid] = static_cast<uint8_t>(mi);
    qd_s[2][tid] = static_cast<uint8_t>(lo);
    // group sums over the 32 consecutive threads of the group
    int s0 = qi, s1 = hi, s2 = mi, s3 = lo;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      s0 += __shfl_xor(s0, m, 64);
      s1 += __shfl_xor(s1, m, 64);
      s2 += __shfl_xor(s2, m, 64);
      s3 += __shfl_xor(s3, m, 64);
    }
    if ((tid & 31) == 0) {
      qsum_s[tid >> 5][0] = s0; qsum_s[tid >> 5][1] = s1; qsum_s[tid >> 5][2] = s2; qsum_s[tid >> 5][3] = s3;
    }
  }
  __syncthreads();
  const float c_logit = (amax_q > 0.0f ? amax_q / static_cast<float>(kQMax) : 0.0f) * kLog2e * cn;

  // per-lane q digits of key group g (dim 32g + 4k + byte)
  const int g = lane % NG;
  uint32_t qh[8], qm[8], ql[8];
  {
    const uint4* ph = reinterpret_cast<const uint4*>(&qd_s[0][32 * g]);
    const uint4* pm = reinterpret_cast<const uint4*>(&qd_s[1][32 * g]);
    const uint4* pl = reinterpret_cast<const uint4*>(&qd_s[2][32 * g]);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 a = ph[c], bm = pm[c], l4 = pl[c];
      qh[4 * c] = a.x; qh[4 * c + 1] = a.y; qh[4 * c + 2] = a.z; qh[4 * c + 3] = a.w;
      qm[4 * c] = bm.x; qm[4 * c + 1] = bm.y; qm[4 * c + 2] = bm.z; qm[4 * c + 3] = bm.w;
      ql[4 * c] = l4.x; ql[4 * c + 1] = l4.y; ql[4 * c + 2] = l4.z; ql[4 * c + 3] = l4.w;
    }
  }
  const float qsum_f = static_cast<float>(qsum_s[g][0]);
  const int h_init = -4 * qsum_s[g][1], m_init = -4 * qsum_s[g][2], l_init = -4 * qsum_s[g][3];
  const int blk_k = g / GPB;
  const bool wlane = (g % GPB) == 0;    // lane computes value weights of block blk_k

  int vdim[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) vdim[dd] = 32 * (lane / LPG) + (lane % LPG) + LPG * dd;
  const int blk_v = vdim[0] / BLOCK;

  float m_run = -INFINITY, l_run = 0.0f, ob = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.0f;

  const int T = p.T;
  const int ntiles = (T + kTile - 1) / kTile;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(t_begin + p.tiles_per_split, ntiles);
  // buffer resources of this (sequence, KV head); offsets carry the step base in the
  // vector offset (the range check covers it), so rows past T read as zero
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_codes + unit * p.tcap * ROWB, static_cast<uint32_t>(T) * ROWB);
  const __amdgpu_buffer_rsrc_t rkm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.k_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rvm = make_rsrc(
      reinterpret_cast<const uint8_t*>(p.v_meta) + unit * p.tcap * NBLK * MB, static_cast<uint32_t>(T) * NBLK * MB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_codes + unit * p.ntile_cap * static_cast<size_t>(D) * 12,
                                              static_cast<uint32_t>(ntiles) * D * 12);
  const uint32_t koff = static_cast<uint32_t>((lane / NG) * ROWB + 12 * g);
  const uint32_t moff = static_cast<uint32_t>(((lane / NG) * NBLK + blk_k) * MB);

  // step `st` covers tiles NT st .. NT st + NT - 1
  auto load_step = [&](Raw& r, int st) {
    const uint32_t sk = static_cast<uint32_t>(st) * STEP * ROWB;
    const uint32_t sm = static_cast<uint32_t>(st) * STEP * NBLK * MB;
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b96(rk, sk + koff + it * TPR * ROWB, 0, 0);
      r.kw[it][0] = w[0]; r.kw[it][1] = w[1]; r.kw[it][2] = w[2];
      r.km[it] = buf_meta<FMT>(rkm, sm + moff + it * TPR * NBLK * MB, 0);
      r.vm[it] = buf_meta<FMT>(rvm, sm + moff + it * TPR * NBLK * MB, 0);
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint32_t sv = static_cast<uint32_t>(NT * st + tt) * D * 12;
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b96(rv, sv + 12 * vdim[dd], 0, 0);
        r.vw[tt][dd][0] = w[0]; r.vw[tt][dd][1] = w[1]; r.vw[tt][dd][2] = w[2];
      }
    }
  };

  auto compute_step = [&](const Raw& r, int st) {
    const int base = st * STEP;
    // ---- keys
    float L[IPL];
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      uint32_t dw[8];
      g32_to_bytes(r.kw[it][0], r.kw[it][1], r.kw[it][2], dw);
      int ah = h_init, am = m_init, al = l_init;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ah = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(qh[k]), ah, false);
        am = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(qm[k]), am, false);
        al = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(ql[k]), al, false);
      }
      const int comb = (ah << 16) + (am << 8) + al;   // sum_j q_j (u_j - 4), exact
      float s, o;
      meta_decode<FMT>(r.km[it], s, o);
      float val = s * static_cast<float>(comb);
      if constexpr (FMT == kFmtAsym) val = __builtin_fmaf(o, qsum_f, val);
      val += dpp_xor1(val);
      val += dpp_xor2(val);
      if constexpr (NG == 8) val += swz_xor4(val);
      L[it] = base + lane / NG + it * TPR < T ? val * c_logit : -INFINITY;
    }
    // ---- online softmax (base 2)
    float tmax = L[0];
#pragma unroll
    for (int it = 1; it < IPL; ++it) tmax = fmaxf(tmax, L[it]);
    if (__any(tmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, wave_max_fast(tmax));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) acc[dd] *= alpha;
      l_run *= alpha;
      ob *= alpha;
      m_run = m_new;
    }
    float pr[IPL];
#pragma unroll
    for (int it = 0; it < IPL; ++it) pr[it] = __builtin_amdgcn_exp2f(L[it] - m_run);
    if (g == 0) {
#pragma unroll
      for (int it = 0; it < IPL; ++it) l_run += pr[it];
    }
    // ---- value weights w = p s_v (one lane per token and block), as 22-bit
    // integers relative to the step's largest weight
    float wv[IPL];
    float wmax = 0.0f;
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      float sv, ov;
      meta_decode<FMT>(r.vm[it], sv, ov);   // zero past T
      wv[it] = wlane ? pr[it] * sv : 0.0f;
      if constexpr (FMT == kFmtAsym) ob += wlane ? pr[it] * ov : 0.0f;
      wmax = fmaxf(wmax, wv[it]);
    }
    wmax = wave_max_fast(wmax);
    const float winv = wmax > 0.0f ? kWMax * __builtin_amdgcn_rcpf(wmax) : 0.0f;
    const float wsig = wmax * (1.0f / kWMax);
    int wsum = 0;
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      const uint32_t wi = static_cast<uint32_t>(__builtin_rintf(wv[it] * winv));
      wsum += static_cast<int>(wi);
      if (wlane) {
        const int slot = lane / NG + it * TPR;
        wq[wave][blk_k][0][slot] = static_cast<uint8_t>(wi);
        wq[wave][blk_k][1][slot] = static_cast<uint8_t>(wi >> 8);
        wq[wave][blk_k][2][slot] = static_cast<uint8_t>(wi >> 16);
      }
    }
    // sum of the block's integer weights: lanes of equal g
#pragma unroll
    for (int mk = NG; mk < 64; mk <<= 1) wsum += __shfl_xor(wsum, mk, 64);
    if (lane < NG && wlane) wsum_s[wave][blk_k] = wsum;
    // the weights are read back by other lanes of this wave: LDS operations of a
    // wave execute in order, so only compiler reordering has to be prevented
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    // ---- values: acc[j] += wsig * sum_t w_t (u_tj - 4), w_t = sum_d 256^d digit_d,t;
    // byte b of pl[d][k] is digit d of token 4k + b of the tile
    const int wcen = 4 * wsum_s[wave][blk_v];
    int ai[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) ai[dd] = -wcen;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      uint32_t pl[3][8];
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) {
        const uint4* wr = reinterpret_cast<const uint4*>(&wq[wave][blk_v][dg][kTile * tt]);
        const uint4 x0 = wr[0], x1 = wr[1];
        pl[dg][0] = x0.x; pl[dg][1] = x0.y; pl[dg][2] = x0.z; pl[dg][3] = x0.w;
        pl[dg][4] = x1.x; pl[dg][5] = x1.y; pl[dg][6] = x1.z; pl[dg][7] = x1.w;
      }
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        uint32_t dw[8];
        g32_to_bytes(r.vw[tt][dd][0], r.vw[tt][dd][1], r.vw[tt][dd][2], dw);
        uint32_t a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          a0 = __builtin_amdgcn_udot4(dw[k], pl[0][k], a0, false);
          a1 = __builtin_amdgcn_udot4(dw[k], pl[1][k], a1, false);
          a2 = __builtin_amdgcn_udot4(dw[k], pl[2][k], a2, false);
        }
        // one tile's sum w u <= 7 * 32 * 2^22 < 2^30, and every partial sum lies in
        // [-4 sum(w), 3 sum(w)] with 4 sum(w) <= 4 * 64 * 2^22 = 2^30: exact in int32
        ai[dd] += 65536 * static_cast<int>(a2) + 256 * static_cast<int>(a1) + static_cast<int>(a0);
      }
    }
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = __builtin_fmaf(wsig, static_cast<float>(ai[dd]), acc[dd]);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
  };

  // steps of NT tiles; the four waves take steps in turn; two register buffers
  // alternate so that the loads of step s+4 are in flight while step s is computed
  // (past the split's end the prefetch reloads its last step)
  const int s_begin = t_begin / NT;
  const int s_end = (t_end + NT - 1) / NT;
  Raw ra, rb;
  int st = s_begin + wave;
  if (st < s_end) load_step(ra, st);
  while (st < s_end) {
    load_step(rb, min(st + 4, s_end - 1));
    compute_step(ra, st);
    st += 4;
    if (st >= s_end) break;
    load_step(ra, min(st + 4, s_end - 1));
    compute_step(rb, st);
    st += 4;
  }

  // ---- combine the four waves
  const float lsum = wave_sum(l_run);
  // offsets: lanes with g % GPB == 0 hold block blk_k's sum; add lanes of equal g
#pragma unroll
  for (int mk = NG; mk < 64; mk <<= 1) ob += shfl_xor(ob, mk);
  if (lane == 0) {
    cm_s[wave] = m_run;
    cl_s[wave] = lsum;
  }
  if (lane < NG && wlane) cob_s[wave][blk_k] = ob;  // lane g < NG holds group g
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) cacc_s[wave][vdim[dd]] = acc[dd];
  __syncthreads();
  if (tid < D) {
    const int j = tid;
    const float mx = fmaxf(fmaxf(cm_s[0], cm_s[1]), fmaxf(cm_s[2], cm_s[3]));
    float a = 0.0f, l = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float al = __builtin_amdgcn_exp2f(cm_s[wv] - mx);
        a += al * (cacc_s[wv][j] + cob_s[wv][j / BLOCK]);
        l += al * cl_s[wv];
      }
    }
    float* out = p.ws + ((static_cast<size_t>(b) * p.hq + hq) * p.nsplit + split) * (D + 2);
    out[j] = a;
    if (j == 0) {
      out[D] = mx;
      out[D + 1] = l;
    }
  }
}

// Merge the splits of one (sequence, query head), normalise, apply U^T.
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceParams p) {
  constexpr int P = 256 / D;           // partial sums per output element
  __shared__ float al_s[kMaxSplitsDev];
  __shared__ float part_s[P][D];
  __shared__ float y_s[D];
  __shared__ float t_s[D];
  __shared__ float red_s[2];
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int ns = p.nsplit;
  const float* base = p.ws + (static_cast<size_t>(b) * p.hq + hq) * ns * (D + 2);
  // split maxima and weights, loaded in parallel
  for (int s = tid; s < ns; s += 256) al_s[s] = base[s * (D + 2) + D];
  __syncthreads();
  if (tid < 64) {
    float mx = -INFINITY;
    for (int s = tid; s < ns; s += 64) mx = fmaxf(mx, al_s[s]);
    mx = wave_max(mx);
    if (tid == 0) red_s[0] = mx;
  }
  __syncthreads();
  const float mx = red_s[0];
  __syncthreads();
  for (int s = tid; s < ns; s += 256) al_s[s] = __builtin_amdgcn_exp2f(al_s[s] - mx);
  __syncthreads();
  if (tid < 64) {
    float den = 0.0f;
    for (int s = tid; s < ns; s += 64) den += al_s[s] * base[s * (D + 2) + D + 1];
    den = wave_sum(den);
    if (tid == 0) red_s[1] = den;
  }
  {
    const int j = tid % D, part = tid / D;
    float num = 0.0f;
#pragma unroll 8
    for (int s = part; s < ns; s += P) num += al_s[s] * base[s * (D + 2) + j];
    part_s[part][j] = num;
  }
  __syncthreads();
  if (tid < D) {
    float num = 0.0f;
#pragma unroll
    for (int q = 0; q < P; ++q) num += part_s[q][tid];
    y_s[tid] = num / red_s[1];
  }
  __syncthreads();
  if (tid < D) {
    const int j = tid;
    if (p.rotation == kRotSo4) {
      // B^T y: (B^T y)_{4r+c} = sum_row R_r[row][c] y_{4r+row}
      const float* R = p.rot + 16 * (j >> 2) + (j & 3);
      const float* ys = y_s + (j & ~3);
      t_s[j] = R[0] * ys[0] + R[4] * ys[1] + R[8] * ys[2] + R[12] * ys[3];
    } else {
      t_s[j] = y_s[j];
    }
  }
  __syncthreads();
  lds_fwht<D>(t_s);
  if (tid < D) {
    const int j = tid;
    float y = t_s[j] * rsqrtf(static_cast<float>(D));
    if (p.rotation == kRotSign) y *= p.rot[j];
    p.out[(static_cast<size_t>(b) * p.hq + hq) * D + j] = y;
  }
}

template <int D, int FMT, int BLOCK>
void launch_decode_t(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL((decode_valu_kernel<D, FMT, BLOCK, kStepTiles>), grid, dim3(256), 0, s, e0, e1, 0, p);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  int fmt;
  if (p.quant == kQuantAsym) fmt = kFmtAsym;
  else fmt = p.scale_dtype == kScaleF32 ? kFmtSymF32 : kFmtSymF16;
  if (p.block == 32) {
    if (fmt == kFmtSymF32) launch_decode_t<D, kFmtSymF32, 32>(p, grid, s, e0, e1);
    else if (fmt == kFmtSymF16) launch_decode_t<D, kFmtSymF16, 32>(p, grid, s, e0, e1);
    else launch_decode_t<D, kFmtAsym, 32>(p, grid, s, e0, e1);
  } else if (p.block == 64) {
    if (fmt == kFmtSymF32) launch_decode_t<D, kFmtSymF32, 64>(p, grid, s, e0, e1);
    else if (fmt == kFmtSymF16) launch_decode_t<D, kFmtSymF16, 64>(p, grid, s, e0, e1);
    else launch_decode_t<D, kFmtAsym, 64>(p, grid, s, e0, e1);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int batch, int d, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.hq, batch);
  if (d == 128) return launch_decode_d<128>(p, grid, s, e0, e1);
  if (d == 256) return launch_decode_d<256>(p, grid, s, e0, e1);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceParams& p, int batch, int d, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  const dim3 grid(p.hq, batch);
  if (d == 128) hipExtLaunchKernelGGL(reduce_kernel<128>, grid, dim3(256), 0, s, e0, e1, 0, p);
  else if (d == 256) hipExtLaunchKernelGGL(reduce_kernel<256>, grid, dim3(256), 0, s, e0, e1, 0, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
