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
  if (p.rotation == kRotNone) {   // U = I: y = y1 (uniform over the workgroup)
    if (tid < D) p.out[(static_cast<size_t>(b) * p.hq + hq) * D + tid] = y_s[tid];
    return;
  }
  lds_fwht<D>(t_s);
  if (tid < D) {
    const int j = tid;
    float y = t_s[j] * rsqrtf(static_cast<float>(D));
    if (p.rotation == kRotSign) y *= p.rot[j];
    p.out[(static_cast<size_t>(b) * p.hq + hq) * D + j] = y;
  }
}

}  // namespace

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
