// Read path: decode attention directly over the packed 3-bit cache.
//
// Pages: "Orthogonally mixed 3-bit KV cache", Implementation notes (q1 = U(q);
// unpack and scale keys inside the attention dot product; logits from q1 and the
// reconstructed transformed keys; softmax; multiply by the reconstructed
// transformed values; rotate the output back with U.T; never materialise full
// K/V) and Key formulas (softmax(QK^T / sqrt d) V); "Orthogonal Invariance in
// Activation Space", Section 2.3 (rotating q and rotating the output back leaves
// attention unchanged) and Section 4.3 (dequantisation fused into the attention
// kernel).
//
// Split-K: the token range of each (sequence, query head) is cut into splits; one
// workgroup per split produces (m, l, acc[D]) with m the running maximum of the
// base-2 logits, l = sum 2^(logit - m) and acc the matching weighted sum of the
// dequantised rotated values; the reduce kernel merges the splits, normalises
// and applies U^T.
//
// Both quantisers are handled in one centred form: x_hat = s (u - 4) + o with
// o = 0 (symmetric codes) or o = z + 4 s (asymmetric codes; exact in float32).
#include "okv_device.hpp"

namespace okv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWStride = 36;          // floats per row of the per-wave weight buffer
constexpr int kQMax = 8000000;        // |q| fixed-point limit: three balanced int8 digits
constexpr int kMaxSplitsDev = 256;    // must match the host's split-K capacity

enum : int { kFmtSymF32 = 0, kFmtSymF16 = 1, kFmtAsym = 2 };

template <int FMT>
__device__ __forceinline__ uint32_t load_meta_raw(const void* meta, size_t i) {
  if constexpr (FMT == kFmtSymF32) return reinterpret_cast<const uint32_t*>(meta)[i];
  else return reinterpret_cast<const uint16_t*>(meta)[i];
}

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
    s = e4m3_decode(raw & 0xFFu);
    o = e4m3_decode(raw >> 8) + 4.0f * s;
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

template <int D>
struct TileRaw {
  static constexpr int NG = D / 32;
  static constexpr int IPL = kTile / (64 / NG);
  static constexpr int DPL = D / 64;
  uint32_t kw[IPL][3];
  uint32_t km[IPL];
  uint32_t vw[DPL][3];
  uint32_t vm[IPL];
};

// One workgroup = one (split, query head, sequence); its four waves take the split's
// 32-token tiles in turn, each wave double-buffering the raw loads of its next tile.
//  * keys: lane (token slot, 32-dim group g) unpacks its group to byte lanes and
//    takes int8 dot products against q in 24-bit fixed point (three balanced int8
//    digits, each centred by its digit sum: exact in int32); the block scale is
//    applied to the integer result; the D/32 partials of a token are summed across
//    lanes;
//  * softmax in base 2; the running maximum is raised only when a logit exceeds it
//    by more than 8, so weights stay <= 256 and rescaling is rare;
//  * values: each lane owns D/64 dims of the dim-major value tile, weights
//    w = p s come from a per-wave shared buffer; codes are centred per tile.
template <int D, int FMT, int BLOCK>
__global__ __launch_bounds__(256) void decode_valu_kernel(const DecodeParams p) {
  using Raw = TileRaw<D>;
  constexpr int NG = Raw::NG;           // 32-dim groups per key row
  constexpr int TPR = 64 / NG;          // token slots covered by the 64 lanes per round
  constexpr int IPL = Raw::IPL;         // key items per lane per tile
  constexpr int LPG = 64 / NG;          // lanes per 32-dim value group
  constexpr int DPL = Raw::DPL;         // value dims per lane
  constexpr int GPB = BLOCK / 32;       // 32-dim groups per quantisation block
  constexpr int NBLK = D / BLOCK;

  __shared__ float q_s[D];
  __shared__ float q_t[D];
  __shared__ int32_t qi_s[D];
  __shared__ int32_t qg_s[NG][4];
  __shared__ float red_s[4];
  __shared__ __align__(16) float wbuf[4][NBLK][kWStride];
  __shared__ float cm_s[4], cl_s[4];
  __shared__ float cacc_s[4][D];
  __shared__ float cob_s[4][NBLK];

  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hk = hq / (p.hq / p.hkv);
  const size_t unit = static_cast<size_t>(b) * p.hkv + hk;

  // ---- q1 = U q in float32, then 24-bit fixed point
  const size_t qoff = (static_cast<size_t>(b) * p.hq + hq) * D;
  for (int j = tid; j < D; j += 256) {
    float x = p.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff + j])
                        : reinterpret_cast<const float*>(p.q)[qoff + j];
    if (p.rotation == kRotSign) x *= p.rot[j];
    q_s[j] = x;
  }
  __syncthreads();
  lds_fwht<D>(q_s);
  const float cn = rsqrtf(static_cast<float>(D));
  for (int j = tid; j < D; j += 256) {
    float y;
    if (p.rotation == kRotSo4) {
      const float* R = p.rot + 16 * (j >> 2) + 4 * (j & 3);
      const float* xs = q_s + (j & ~3);
      y = R[0] * xs[0] + R[1] * xs[1] + R[2] * xs[2] + R[3] * xs[3];
    } else {
      y = q_s[j];
    }
    q_t[j] = y * cn;
  }
  __syncthreads();
  float amax_q = 0.0f;
  for (int j = tid; j < D; j += 256) amax_q = fmaxf(amax_q, fabsf(q_t[j]));
  amax_q = wave_max(amax_q);
  if (lane == 0) red_s[wave] = amax_q;
  __syncthreads();
  amax_q = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  {
    const float inv = amax_q > 0.0f ? static_cast<float>(kQMax) / amax_q : 0.0f;
    for (int j = tid; j < D; j += 256) {
      int qi = static_cast<int>(__builtin_rintf(q_t[j] * inv));
      qi = qi > kQMax ? kQMax : (qi < -kQMax ? -kQMax : qi);
      qi_s[j] = qi;
    }
    __syncthreads();
    if (tid < NG) {
      // per group: sum of q and of each of its three digits
      int sq = 0, sh = 0, sm = 0, sl = 0;
      for (int j = 0; j < 32; ++j) {
        const int qi = qi_s[32 * tid + j];
        const int l = ((qi + 128) & 255) - 128;
        const int q2 = (qi - l) >> 8;
        const int m = ((q2 + 128) & 255) - 128;
        const int h = (q2 - m) >> 8;
        sq += qi; sh += h; sm += m; sl += l;
      }
      qg_s[tid][0] = sq; qg_s[tid][1] = sh; qg_s[tid][2] = sm; qg_s[tid][3] = sl;
    }
    __syncthreads();
  }
  const float c_logit = (amax_q > 0.0f ? amax_q / static_cast<float>(kQMax) : 0.0f) * kLog2e * cn;

  // per-lane q digits of key group g (dim 32g + 4k + byte)
  const int g = lane % NG;
  uint32_t qh[8], qm[8], ql[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t hv = 0, mv = 0, lv = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int qi = qi_s[32 * g + 4 * k + bb];
      const int l = ((qi + 128) & 255) - 128;
      const int q2 = (qi - l) >> 8;
      const int m = ((q2 + 128) & 255) - 128;
      const int h = (q2 - m) >> 8;
      hv |= (static_cast<uint32_t>(h) & 0xFFu) << (8 * bb);
      mv |= (static_cast<uint32_t>(m) & 0xFFu) << (8 * bb);
      lv |= (static_cast<uint32_t>(l) & 0xFFu) << (8 * bb);
    }
    qh[k] = hv; qm[k] = mv; ql[k] = lv;
  }
  const float qsum_f = static_cast<float>(qg_s[g][0]);
  const int h_init = -4 * qg_s[g][1], m_init = -4 * qg_s[g][2], l_init = -4 * qg_s[g][3];
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
  const uint8_t* kc = p.k_codes + unit * p.tcap * (3 * D / 8);
  const uint8_t* vc = p.v_codes + unit * p.ntile_cap * static_cast<size_t>(D) * 12;
  const size_t mrow0 = unit * p.tcap;

  auto load_tile = [&](Raw& r, int tile) {
    const int base = tile * kTile;
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      const int pos = base + lane / NG + it * TPR;
      r.kw[it][0] = r.kw[it][1] = r.kw[it][2] = 0u;
      r.km[it] = 0u;
      r.vm[it] = 0u;
      if (pos < T) {
        const uint3 w = *reinterpret_cast<const uint3*>(kc + static_cast<size_t>(pos) * (3 * D / 8) + 12 * g);
        r.kw[it][0] = w.x; r.kw[it][1] = w.y; r.kw[it][2] = w.z;
        const size_t mi = (mrow0 + pos) * NBLK + blk_k;
        r.km[it] = load_meta_raw<FMT>(p.k_meta, mi);
        if (wlane) r.vm[it] = load_meta_raw<FMT>(p.v_meta, mi);
      }
    }
    const uint8_t* vt = vc + static_cast<size_t>(tile) * D * 12;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const uint3 w = *reinterpret_cast<const uint3*>(vt + 12 * vdim[dd]);
      r.vw[dd][0] = w.x; r.vw[dd][1] = w.y; r.vw[dd][2] = w.z;
    }
  };

  Raw cur, nxt;
  int tile = t_begin + wave;
  if (tile < t_end) load_tile(cur, tile);
  for (; tile < t_end; tile += 4) {
    if (tile + 4 < t_end) load_tile(nxt, tile + 4);
    const int base = tile * kTile;
    // ---- keys
    float L[IPL];
#pragma unroll
    for (int it = 0; it < IPL; ++it) {
      uint32_t dw[8];
      g32_to_bytes(cur.kw[it][0], cur.kw[it][1], cur.kw[it][2], dw);
      int ah = h_init, am = m_init, al = l_init;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ah = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(qh[k]), ah, false);
        am = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(qm[k]), am, false);
        al = __builtin_amdgcn_sdot4(static_cast<int>(dw[k]), static_cast<int>(ql[k]), al, false);
      }
      const int comb = (ah << 16) + (am << 8) + al;   // sum_j q_j (u_j - 4), exact
      float s, o;
      meta_decode<FMT>(cur.km[it], s, o);
      float val = s * static_cast<float>(comb);
      if constexpr (FMT == kFmtAsym) val = __builtin_fmaf(o, qsum_f, val);
      val += dpp_xor1(val);
      val += dpp_xor2(val);
      if constexpr (NG == 8) val += swz_xor4(val);
      const int pos = base + lane / NG + it * TPR;
      L[it] = pos < T ? val * c_logit : -INFINITY;
    }
    // ---- online softmax (base 2)
    float tmax = L[0];
#pragma unroll
    for (int it = 1; it < IPL; ++it) tmax = fmaxf(tmax, L[it]);
    if (__any(tmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, wave_max(tmax));
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
    // ---- value weights w = p s_v (one lane per token and block)
    if (wlane) {
#pragma unroll
      for (int it = 0; it < IPL; ++it) {
        float s, o;
        meta_decode<FMT>(cur.vm[it], s, o);
        const bool valid = base + lane / NG + it * TPR < T;
        const float w = valid ? pr[it] * s : 0.0f;
        if constexpr (FMT == kFmtAsym) ob += valid ? pr[it] * o : 0.0f;
        wbuf[wave][blk_k][lane / NG + it * TPR] = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- values: acc[j] += sum_t w_t (u_tj - 4)
    float w[kTile];
    {
      const float4* wr = reinterpret_cast<const float4*>(&wbuf[wave][blk_v][0]);
#pragma unroll
      for (int i = 0; i < kTile / 4; ++i) {
        const float4 v4 = wr[i];
        w[4 * i] = v4.x; w[4 * i + 1] = v4.y; w[4 * i + 2] = v4.z; w[4 * i + 3] = v4.w;
      }
    }
    float wsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kTile; ++i) wsum += w[i];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      uint32_t dw[8];
      g32_to_bytes_opaque(cur.vw[dd][0], cur.vw[dd][1], cur.vw[dd][2], dw);
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < kTile; ++i) {
        const uint32_t x = dw[i >> 2];
        float u;
        if ((i & 3) == 0) u = static_cast<float>(x & 0xFFu);
        else if ((i & 3) == 1) u = static_cast<float>((x >> 8) & 0xFFu);
        else if ((i & 3) == 2) u = static_cast<float>((x >> 16) & 0xFFu);
        else u = static_cast<float>(x >> 24);
        t = __builtin_fmaf(w[i], u, t);
      }
      acc[dd] += __builtin_fmaf(-4.0f, wsum, t);
    }
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
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
void launch_decode_t(const DecodeParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_valu_kernel<D, FMT, BLOCK>), grid, dim3(256), 0, s, p);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, dim3 grid, hipStream_t s) {
  int fmt;
  if (p.quant == kQuantAsym) fmt = kFmtAsym;
  else fmt = p.scale_dtype == kScaleF32 ? kFmtSymF32 : kFmtSymF16;
  if (p.block == 32) {
    if (fmt == kFmtSymF32) launch_decode_t<D, kFmtSymF32, 32>(p, grid, s);
    else if (fmt == kFmtSymF16) launch_decode_t<D, kFmtSymF16, 32>(p, grid, s);
    else launch_decode_t<D, kFmtAsym, 32>(p, grid, s);
  } else if (p.block == 64) {
    if (fmt == kFmtSymF32) launch_decode_t<D, kFmtSymF32, 64>(p, grid, s);
    else if (fmt == kFmtSymF16) launch_decode_t<D, kFmtSymF16, 64>(p, grid, s);
    else launch_decode_t<D, kFmtAsym, 64>(p, grid, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int batch, int d, hipStream_t s) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.hq, batch);
  if (d == 128) return launch_decode_d<128>(p, grid, s);
  if (d == 256) return launch_decode_d<256>(p, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceParams& p, int batch, int d, hipStream_t s) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  const dim3 grid(p.hq, batch);
  if (d == 128) hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(256), 0, s, p);
  else if (d == 256) hipLaunchKernelGGL(reduce_kernel<256>, grid, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
