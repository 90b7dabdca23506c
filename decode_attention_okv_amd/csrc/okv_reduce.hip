// Split-K merge of the decode partials and the rotation back.
//
// Pages: "Orthogonally mixed 3-bit KV cache", Implementation notes (read path: the
// attention output is rotated back with U^T); "Orthogonal Invariance in Activation
// Space", Section 2.3 (rotating q together with k and the output back leaves
// attention unchanged).
//
// Each decode split leaves (m, l, acc[D]): m the running maximum of its base-2
// logits, l = sum 2^(logit - m) and acc the matching weighted sum of the dequantised
// rotated values.  The merge rescales every split to the common maximum, divides by
// the total weight and applies U^T.
#include <hip/hip_ext.h>

#include "okv_decode_common.hpp"

namespace okv {

namespace {

using namespace dec;

// Merge the splits of one (sequence, query head), normalise, apply U^T.
//
// Thread (j, part) owns output element j and the splits part, part + P, ...; it merges
// them online (running maximum, rescaled numerator and denominator), up to NB splits per
// batch with all their loads in flight together (indices clamped into range, so the
// loads need no branches).  The P parts meet in LDS; wave 0 then applies U^T with the
// transform's cross-lane stages as lane shuffles (no workgroup barriers).
template <int D, int NB>
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceParams p) {
  constexpr int P = 256 / D;           // threads per output element
  constexpr int EPW = D / 64;          // elements per lane of wave 0 in the transform
  __shared__ float pm_s[P][D], pn_s[P][D], pd_s[P][D];
  __shared__ float y_s[D];
  const int tid = threadIdx.x;
  const int ns = p.nsplit;
  const int j = tid % D, part = tid / D;
  const size_t uq = static_cast<size_t>(blockIdx.y) * p.hq + blockIdx.x;
  const float* base = p.ws + uq * ns * (D + 2);
  float mrun = -INFINITY, num = 0.0f, den = 0.0f;
  for (int s0 = part; s0 < ns; s0 += NB * P) {
    float mv[NB], lv[NB], av[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float* row = base + static_cast<size_t>(min(s0 + k * P, ns - 1)) * (D + 2);
      mv[k] = row[D];
      lv[k] = row[D + 1];
      av[k] = row[j];
    }
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (s0 + k * P >= ns) mv[k] = -INFINITY;   // past the last split: no weight
      mb = fmaxf(mb, mv[k]);
    }
    const float mnew = fmaxf(mrun, mb);
    if (mnew != -INFINITY) {           // splits without tokens carry m = -inf, l = 0
      const float sc = __builtin_amdgcn_exp2f(mrun - mnew);
      num *= sc;
      den *= sc;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float w = mv[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv[k] - mnew);
        num = __builtin_fmaf(w, av[k], num);
        den = __builtin_fmaf(w, lv[k], den);
      }
      mrun = mnew;
    }
  }
  pm_s[part][j] = mrun;
  pn_s[part][j] = num;
  pd_s[part][j] = den;
  __syncthreads();
  if (tid < D) {
    float mx = pm_s[0][j];
#pragma unroll
    for (int q = 1; q < P; ++q) mx = fmaxf(mx, pm_s[q][j]);
    float n = 0.0f, d = 0.0f;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const float w = pm_s[q][j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pm_s[q][j] - mx);
      n = __builtin_fmaf(w, pn_s[q][j], n);
      d = __builtin_fmaf(w, pd_s[q][j], d);
    }
    y_s[j] = n / d;
  }
  __syncthreads();
  if (tid >= 64) return;
  // wave 0: lane l holds elements l + 64 e of t = B^T y (SO(4)) or y
  const int l = tid;
  float t[EPW];
#pragma unroll
  for (int e = 0; e < EPW; ++e) {
    const int jj = l + 64 * e;
    if (p.rotation == kRotSo4) {
      // (B^T y)_{4r+c} = sum_row R_r[row][c] y_{4r+row}
      const float* R = p.rot + 16 * (jj >> 2) + (jj & 3);
      const float* ys = y_s + (jj & ~3);
      t[e] = R[0] * ys[0] + R[4] * ys[1] + R[8] * ys[2] + R[12] * ys[3];
    } else {
      t[e] = y_s[jj];
    }
  }
  float* out = p.out + uq * D;
  if (p.rotation == kRotNone) {        // U = I: y = y1 (uniform over the workgroup)
#pragma unroll
    for (int e = 0; e < EPW; ++e) out[l + 64 * e] = t[e];
    return;
  }
  // unnormalised Walsh-Hadamard transform: strides of 64 and up inside the lane,
  // strides 1 .. 32 across lanes (each stage pairs lane l with l ^ h)
#pragma unroll
  for (int h = 1; h < EPW; h <<= 1) {
#pragma unroll
    for (int e = 0; e < EPW; ++e) {
      if (!(e & h)) {
        const float a = t[e], c = t[e + h];
        t[e] = a + c;
        t[e + h] = a - c;
      }
    }
  }
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const bool upper = (l & h) != 0;
#pragma unroll
    for (int e = 0; e < EPW; ++e) {
      const float o = __shfl_xor(t[e], h, 64);
      t[e] = upper ? o - t[e] : t[e] + o;
    }
  }
  const float cn = rsqrtf(static_cast<float>(D));
#pragma unroll
  for (int e = 0; e < EPW; ++e) {
    const int jj = l + 64 * e;
    float y = t[e] * cn;
    if (p.rotation == kRotSign) y *= p.rot[jj];
    out[jj] = y;
  }
}

template <int D>
void launch_nb(const ReduceParams& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // splits per thread: one load batch of the smallest size that holds them (up to 32)
  const int k = (p.nsplit + 256 / D - 1) / (256 / D);
  if (k <= 2) hipExtLaunchKernelGGL((reduce_kernel<D, 2>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else if (k <= 4) hipExtLaunchKernelGGL((reduce_kernel<D, 4>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else if (k <= 8) hipExtLaunchKernelGGL((reduce_kernel<D, 8>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else if (k <= 16) hipExtLaunchKernelGGL((reduce_kernel<D, 16>), grid, dim3(256), 0, s, e0, e1, 0, p);
  else hipExtLaunchKernelGGL((reduce_kernel<D, 32>), grid, dim3(256), 0, s, e0, e1, 0, p);
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, int batch, int d, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  if (p.nsplit < 1 || p.nsplit > kMaxSplitsDev) return hipErrorInvalidValue;
  const dim3 grid(p.hq, batch);
  if (d == 128) launch_nb<128>(p, grid, s, e0, e1);
  else if (d == 256) launch_nb<256>(p, grid, s, e0, e1);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
