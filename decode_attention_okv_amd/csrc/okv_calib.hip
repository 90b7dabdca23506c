// SO(4) calibration: choose the rotations R_i of U = B H_d (B = diag(R_1 .. R_{d/4}))
// that minimise the reconstruction error of y = B (H x) after b-bit quantisation over
// a set of calibration vectors x.
//
// Method: "Orthogonally mixed 3-bit KV cache" (idea card), Implementation notes: start
// from fixed random rotations, calibrate them on representative vectors by minimising
// the reconstruction MSE after 3-bit quantisation, each SO(4) block a quaternion pair.
// The search is a coordinate search over given candidate perturbations: the error
// splits over quantisation blocks, so a change of R_g only changes the block that
// holds group g, and every candidate of a step is one evaluation of that block.
//
//  * hx_kernel: H x once per calibration vector (normalised FWHT in LDS, float32).
//  * eval_kernel: grid (vector chunk, candidate); a thread takes one vector and sums
//    the squared error of the block, y computed group by group from hx twice (block
//    maximum, then error), with group g's matrix replaced by cand_c R_g.  Partial sums
//    per (candidate, chunk) are added on the host in a fixed order.
//  * The host takes each step's decision (first minimum) and updates R_g.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "okv.h"
#include "okv_decode_common.hpp"

namespace okv {

namespace {

constexpr int kVec = 8;          // calibration vectors per hx workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
constexpr int kEvalThreads = 256;

template <int D>
__global__ __launch_bounds__(256) void hx_kernel(const float* __restrict__ x, float* __restrict__ hx, int n) {
  __shared__ float xs[kVec][D];
  const int v0 = blockIdx.x * kVec;
  for (int e = threadIdx.x; e < kVec * D; e += 256) {
    const int v = v0 + e / D;
    xs[e / D][e % D] = v < n ? x[static_cast<size_t>(v) * D + e % D] : 0.0f;
  }
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int e = threadIdx.x; e < kVec * D / 2; e += 256) {
      const int r = e / (D / 2), pi = e % (D / 2);
      const int i = (pi / hs) * 2 * hs + (pi % hs);
      const float a = xs[r][i], c = xs[r][i + hs];
      xs[r][i] = a + c;
      xs[r][i + hs] = a - c;
    }
    __syncthreads();
  }
  const float cn = rsqrtf(static_cast<float>(D));
  for (int e = threadIdx.x; e < kVec * D; e += 256) {
    const int v = v0 + e / D;
    if (v < n) hx[static_cast<size_t>(v) * D + e % D] = xs[e / D][e % D] * cn;
  }
}

struct EvalParams {
  const float* hx;      // [n][d] H x
  const float* rot;     // [d/4][16] current rows of B's blocks
  const float* cand;    // [n_cand][16] perturbations of group `group`
  float* part;          // [n_cand][nchunk] partial error sums
  int n, d, block, group, nchunk, lev;
  float eps;
};

__global__ __launch_bounds__(kEvalThreads) void eval_kernel(const EvalParams p) {
  __shared__ float mg[16];                 // cand_c R_g
  __shared__ float red[kEvalThreads / 64];
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < 16) {
    const int r = tid / 4, col = tid % 4;
    const float* P = p.cand + 16 * c;
    const float* R = p.rot + 16 * p.group;
    mg[tid] = P[4 * r] * R[col] + P[4 * r + 1] * R[4 + col] + P[4 * r + 2] * R[8 + col] + P[4 * r + 3] * R[12 + col];
  }
  __syncthreads();
  const int v = blockIdx.x * kEvalThreads + tid;
  float err = 0.0f;
  if (v < p.n) {
    const int g0 = (4 * p.group) / p.block * (p.block / 4);
    const int ng = p.block / 4;
    const float* row = p.hx + static_cast<size_t>(v) * p.d;
    auto group_y = [&](int g, float y[4]) {
      const float4 h = *reinterpret_cast<const float4*>(row + 4 * g);
      const float* M = (g == p.group) ? mg : p.rot + 16 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = M[4 * r] * h.x + M[4 * r + 1] * h.y + M[4 * r + 2] * h.z + M[4 * r + 3] * h.w;
    };
    float amax = 0.0f;
    for (int g = g0; g < g0 + ng; ++g) {
      float y[4];
      group_y(g, y);
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(y[r]));
    }
    const float s = (amax + p.eps) / static_cast<float>(p.lev);
    const float rs = s > 0.0f ? 1.0f / s : 0.0f;
    const float lev = static_cast<float>(p.lev);
    for (int g = g0; g < g0 + ng; ++g) {
      float y[4];
      group_y(g, y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the error is continuous across rounding thresholds, so the float32 quotient
        // only moves it by rounding noise
        const float q = fminf(fmaxf(__builtin_rintf(y[r] * rs), -lev), lev);
        const float e = y[r] - s * q;
        err = __builtin_fmaf(e, e, err);
      }
    }
  }
  err = wave_sum(err);
  if ((tid & 63) == 0) red[tid >> 6] = err;
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f;
    for (int w = 0; w < kEvalThreads / 64; ++w) t += red[w];
    p.part[static_cast<size_t>(c) * p.nchunk + blockIdx.x] = t;
  }
}

bool hip_ok(hipError_t e) { return e == hipSuccess; }

// Device workspace of one calibration call.
struct Work {
  float* hx = nullptr;
  float* rot = nullptr;
  float* cand = nullptr;
  float* part = nullptr;
  ~Work() {
    if (hx) (void)hipFree(hx);
    if (rot) (void)hipFree(rot);
    if (cand) (void)hipFree(cand);
    if (part) (void)hipFree(part);
  }
};

int check_args(const float* x, int32_t n, int32_t d, int32_t block, int32_t bits, float eps, int32_t n_cand) {
  if (x == nullptr || n < 1 || n_cand < 1 || n_cand > 1024) return OKV_E_INVALID;
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return OKV_E_ALIGN;
  if (bits < 2 || bits > 4 || !std::isfinite(eps) || eps < 0.0f) return OKV_E_INVALID;
  if (d != 128 && d != 256) return OKV_E_UNSUPPORTED;
  if (block < 4 || block % 4 != 0 || d % block != 0) return OKV_E_INVALID;
  if (static_cast<int64_t>(n) * d >= (int64_t{1} << 31)) return OKV_E_UNSUPPORTED;
  return OKV_OK;
}

int setup(Work& w, const float* x, int32_t n, int32_t d, int32_t n_cand, size_t cand_floats, hipStream_t s) {
  const int nchunk = (n + kEvalThreads - 1) / kEvalThreads;
  if (!hip_ok(hipMalloc(&w.hx, static_cast<size_t>(n) * d * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.rot, static_cast<size_t>(d) * 4 * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.cand, cand_floats * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.part, static_cast<size_t>(n_cand) * nchunk * sizeof(float)))) {
    return OKV_E_HIP;
  }
  const dim3 grid((n + kVec - 1) / kVec);
  if (d == 128) hipLaunchKernelGGL(hx_kernel<128>, grid, dim3(256), 0, s, x, w.hx, n);
  else hipLaunchKernelGGL(hx_kernel<256>, grid, dim3(256), 0, s, x, w.hx, n);
  return hip_ok(hipGetLastError()) ? OKV_OK : OKV_E_HIP;
}

// Errors of the block holding `group` for n_cand candidates at dev_cand (device).
int evaluate(const Work& w, int32_t n, int32_t d, int32_t block, int32_t bits, float eps, const float* dev_cand,
             int32_t n_cand, int32_t group, std::vector<float>& part, double* err, hipStream_t s) {
  EvalParams p{};
  p.hx = w.hx;
  p.rot = w.rot;
  p.cand = dev_cand;
  p.part = w.part;
  p.n = n;
  p.d = d;
  p.block = block;
  p.group = group;
  p.nchunk = (n + kEvalThreads - 1) / kEvalThreads;
  p.lev = (1 << (bits - 1)) - 1;
  p.eps = eps;
  hipLaunchKernelGGL(eval_kernel, dim3(p.nchunk, n_cand), dim3(kEvalThreads), 0, s, p);
  if (!hip_ok(hipGetLastError())) return OKV_E_HIP;
  part.resize(static_cast<size_t>(n_cand) * p.nchunk);
  if (!hip_ok(hipMemcpyAsync(part.data(), w.part, part.size() * sizeof(float), hipMemcpyDeviceToHost, s)) ||
      !hip_ok(hipStreamSynchronize(s))) {
    return OKV_E_HIP;
  }
  for (int c = 0; c < n_cand; ++c) {
    double t = 0.0;
    for (int k = 0; k < p.nchunk; ++k) t += part[static_cast<size_t>(c) * p.nchunk + k];
    err[c] = t;
  }
  return OKV_OK;
}

}  // namespace
}  // namespace okv

extern "C" {

int okv_so4_eval(const float* x, int32_t n, int32_t head_dim, int32_t block, int32_t bits, float eps,
                 const float* rot, const float* cand, int32_t n_cand, int32_t group, double* err,
                 void* hip_stream) {
  int st = okv::check_args(x, n, head_dim, block, bits, eps, n_cand);
  if (st != OKV_OK) return st;
  if (rot == nullptr || cand == nullptr || err == nullptr || group < 0 || group >= head_dim / 4) {
    return OKV_E_INVALID;
  }
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  okv::Work w;
  st = okv::setup(w, x, n, head_dim, n_cand, static_cast<size_t>(n_cand) * 16, s);
  if (st != OKV_OK) return st;
  if (!okv::hip_ok(hipMemcpyAsync(w.rot, rot, static_cast<size_t>(head_dim) * 4 * sizeof(float),
                                  hipMemcpyHostToDevice, s)) ||
      !okv::hip_ok(hipMemcpyAsync(w.cand, cand, static_cast<size_t>(n_cand) * 16 * sizeof(float),
                                  hipMemcpyHostToDevice, s))) {
    return OKV_E_HIP;
  }
  std::vector<float> part;
  return okv::evaluate(w, n, head_dim, block, bits, eps, w.cand, n_cand, group, part, err, s);
}

int okv_so4_calibrate(const float* x, int32_t n, int32_t head_dim, int32_t block, int32_t bits, float eps,
                      float* rot, const float* cand, int32_t sweeps, int32_t n_cand, double* trace,
                      void* hip_stream) {
  int st = okv::check_args(x, n, head_dim, block, bits, eps, n_cand);
  if (st != OKV_OK) return st;
  if (rot == nullptr || cand == nullptr || sweeps < 1 || sweeps > 1024) return OKV_E_INVALID;
  const int ng = head_dim / 4;
  const size_t per_group = static_cast<size_t>(n_cand) * 16;
  const size_t cand_floats = static_cast<size_t>(sweeps) * ng * per_group + 16;   // + identity
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  okv::Work w;
  st = okv::setup(w, x, n, head_dim, n_cand, cand_floats, s);
  if (st != OKV_OK) return st;
  static const float kIdentity[16] = {1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1};
  float* dev_identity = w.cand + cand_floats - 16;
  if (!okv::hip_ok(hipMemcpyAsync(w.rot, rot, static_cast<size_t>(ng) * 16 * sizeof(float),
                                  hipMemcpyHostToDevice, s)) ||
      !okv::hip_ok(hipMemcpyAsync(w.cand, cand, (cand_floats - 16) * sizeof(float), hipMemcpyHostToDevice, s)) ||
      !okv::hip_ok(hipMemcpyAsync(dev_identity, kIdentity, sizeof(kIdentity), hipMemcpyHostToDevice, s))) {
    return OKV_E_HIP;
  }
  std::vector<float> part;
  std::vector<double> err(static_cast<size_t>(n_cand));
  std::vector<double> R(static_cast<size_t>(ng) * 16);
  for (size_t i = 0; i < R.size(); ++i) R[i] = rot[i];
  auto total = [&](double* out) {
    double t = 0.0;
    for (int b = 0; b < head_dim / block; ++b) {
      double e = 0.0;
      const int r = okv::evaluate(w, n, head_dim, block, bits, eps, dev_identity, 1, b * block / 4, part, &e, s);
      if (r != OKV_OK) return r;
      t += e;
    }
    *out = t;
    return static_cast<int>(OKV_OK);
  };
  if (trace != nullptr && (st = total(&trace[0])) != OKV_OK) return st;
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int g = 0; g < ng; ++g) {
      const float* dc = w.cand + (static_cast<size_t>(sw) * ng + g) * per_group;
      st = okv::evaluate(w, n, head_dim, block, bits, eps, dc, n_cand, g, part, err.data(), s);
      if (st != OKV_OK) return st;
      int best = 0;
      for (int c = 1; c < n_cand; ++c) {
        if (err[c] < err[best]) best = c;   // first minimum
      }
      if (best != 0) {
        // R_g <- P_best R_g (double on the host), then the float32 copy to the device
        const float* P = cand + (static_cast<size_t>(sw) * ng + g) * per_group + 16 * best;
        double Rn[16];
        for (int r = 0; r < 4; ++r)
          for (int c = 0; c < 4; ++c) {
            double a = 0.0;
            for (int k = 0; k < 4; ++k) a += static_cast<double>(P[4 * r + k]) * R[16 * g + 4 * k + c];
            Rn[4 * r + c] = a;
          }
        float Rf[16];
        for (int i = 0; i < 16; ++i) {
          R[16 * g + i] = Rn[i];
          Rf[i] = static_cast<float>(Rn[i]);
        }
        if (!okv::hip_ok(hipMemcpyAsync(w.rot + 16 * g, Rf, sizeof(Rf), hipMemcpyHostToDevice, s)) ||
            !okv::hip_ok(hipStreamSynchronize(s))) {
          return OKV_E_HIP;
        }
      }
    }
    if (trace != nullptr && (st = total(&trace[sw + 1])) != OKV_OK) return st;
  }
  for (size_t i = 0; i < R.size(); ++i) rot[i] = static_cast<float>(R[i]);
  return OKV_OK;
}

}  // extern "C"
