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
//    per (candidate, chunk) are added in a fixed order (chunk ascending, in double).
//  * Steps in different quantisation blocks are independent (a group's error and update
//    touch its own block only), so step k of every block runs in one launch, the block
//    on grid z; each block still takes its groups in ascending order.
//  * select_kernel (a workgroup per block, after each search evaluation) takes the step's
//    decision (first minimum over the candidates) and sets R_g <- P_best R_g in double,
//    with its float32 copy for the next evaluation; trace_kernel adds a block's error to
//    a trace entry (the blocks' errors in ascending order).  The search is queued on the
//    stream with no host round trip; the double arithmetic is unfused and in the same
//    order as a host loop would take it.  (Replaying the search as a captured HIP graph
//    removes the per-launch host cost, but capturing and instantiating ~600 nodes per
//    call costs more than it saves.)
//    (Taking the decision in the last eval workgroup to finish instead costs a
//    device-wide fence in every workgroup, which is slower than the extra launch.)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
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

// dst <- src, n16 16-byte words; src may be pinned host memory (read over the bus).
__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; i < n16; i += static_cast<size_t>(gridDim.x) * 256)
    dst[i] = src[i];
}

struct EvalParams {
  const float* hx;      // [n][d] H x
  const float* rot;     // [d/4][16] current rows of B's blocks
  const float* cand;    // [n_cand][16] perturbations of group `group`
  float* part;          // [n_cand][nchunk] partial error sums
  int n, d, block, group, nchunk, lev, n_cand;
  int cand_zstride;     // floats from the candidates of grid-z block z to z + 1 (0: shared)
  float eps;
};

// Sum of the chunk partials of candidate c, chunk ascending, in double; the loads of a
// batch of 32 chunks are in flight together (the additions stay in order).
__device__ __forceinline__ double cand_error(const float* part, int nchunk, int c) {
  constexpr int NB = 32;
  const float* pc = part + static_cast<size_t>(c) * nchunk;
  double t = 0.0;
  for (int k0 = 0; k0 < nchunk; k0 += NB) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = pc[min(k0 + i, nchunk - 1)];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (k0 + i < nchunk) t = __dadd_rn(t, static_cast<double>(v[i]));
  }
  return t;
}

// One search step's decision, by one workgroup per quantisation block z (group
// group + z zgroups, its partials and candidates at z times their strides): the
// candidate with the smallest error (the first one on ties) replaces R_g by P_best R_g
// (double: rd; float32 copy: rf).  n_cand <= 1024.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ part, int nchunk, int n_cand,
                                                     const float* __restrict__ cand_g, int group, int zgroups,
                                                     int cand_zstride, double* rd, float* rf) {
  __shared__ double err_s[1024];
  part += static_cast<size_t>(blockIdx.x) * n_cand * nchunk;
  cand_g += static_cast<size_t>(blockIdx.x) * cand_zstride;
  group += static_cast<int>(blockIdx.x) * zgroups;
  for (int c = threadIdx.x; c < n_cand; c += blockDim.x) err_s[c] = cand_error(part, nchunk, c);
  __syncthreads();
  if (threadIdx.x != 0) return;
  int best = 0;
  for (int c = 1; c < n_cand; ++c) {
    if (err_s[c] < err_s[best]) best = c;
  }
  // the winner is applied even when it is candidate 0: the interface does not require
  // candidate 0 to be the identity (when it is, the double products leave R unchanged)
  const float* P = cand_g + 16 * best;
  double* R = rd + 16 * group;
  double rn[16];
  for (int r = 0; r < 4; ++r)
    for (int c = 0; c < 4; ++c) {
      double a = 0.0;
      for (int k = 0; k < 4; ++k) a = __dadd_rn(a, __dmul_rn(static_cast<double>(P[4 * r + k]), R[4 * k + c]));
      rn[4 * r + c] = a;
    }
  for (int i = 0; i < 16; ++i) {
    R[i] = rn[i];
    rf[16 * group + i] = static_cast<float>(rn[i]);
  }
}

// One thread per calibration vector: the vector's block of H x is read once, the
// outputs of the block's other groups are formed once, and every candidate then
// replaces group g's four outputs (block maximum, then the squared error of the block,
// groups in ascending order).  Partial sums per (candidate, chunk).  Grid z: the z-th
// quantisation block after group g's (group g + z block/4), partials block-major.
template <int NGB>
__global__ __launch_bounds__(kEvalThreads) void eval_kernel(const EvalParams p) {
  constexpr int NCMAX = 64;                // candidates per launch (more: several launches)
  __shared__ float mg[NCMAX][16];          // cand_c R_g
  __shared__ float red[kEvalThreads / 64][NCMAX];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * NCMAX;
  const int group = p.group + static_cast<int>(blockIdx.z) * (p.block / 4);
  float* part = p.part + static_cast<size_t>(blockIdx.z) * p.n_cand * p.nchunk;
  const float* cand = p.cand + static_cast<size_t>(blockIdx.z) * p.cand_zstride;
  const int nc = min(NCMAX, p.n_cand - c0);
  for (int e = tid; e < nc * 16; e += kEvalThreads) {
    const int c = e / 16, r = (e % 16) / 4, col = e % 4;
    const float* P = cand + 16 * (c0 + c);
    const float* R = p.rot + 16 * group;
    mg[c][4 * r + col] = P[4 * r] * R[col] + P[4 * r + 1] * R[4 + col] + P[4 * r + 2] * R[8 + col] +
                         P[4 * r + 3] * R[12 + col];
  }
  __syncthreads();
  const int v = blockIdx.x * kEvalThreads + tid;
  const int g0 = (4 * group) / p.block * (p.block / 4);
  const int gl = group - g0;             // group g inside the block
  float y[NGB][4];                          // outputs of the block's groups (g's: current R_g)
  float4 h[NGB];
  const bool ok = v < p.n;
  {
    const float* row = p.hx + static_cast<size_t>(ok ? v : 0) * p.d;
#pragma unroll
    for (int k = 0; k < NGB; ++k) {
      h[k] = *reinterpret_cast<const float4*>(row + 4 * (g0 + k));
      const float* M = p.rot + 16 * (g0 + k);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        y[k][r] = M[4 * r] * h[k].x + M[4 * r + 1] * h[k].y + M[4 * r + 2] * h[k].z + M[4 * r + 3] * h[k].w;
    }
  }
  // largest |y| over the groups other than g
  float amax_o = 0.0f;
#pragma unroll
  for (int k = 0; k < NGB; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) amax_o = (k == gl) ? amax_o : fmaxf(amax_o, fabsf(y[k][r]));
  const float lev = static_cast<float>(p.lev);
  for (int c = 0; c < nc; ++c) {
    float yg[4];
    const float* M = mg[c];
    float hg[4];
#pragma unroll
    for (int k = 0; k < NGB; ++k)
      if (k == gl) {
        hg[0] = h[k].x; hg[1] = h[k].y; hg[2] = h[k].z; hg[3] = h[k].w;
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) yg[r] = M[4 * r] * hg[0] + M[4 * r + 1] * hg[1] + M[4 * r + 2] * hg[2] + M[4 * r + 3] * hg[3];
    float amax = amax_o;
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(yg[r]));
    const float s = (amax + p.eps) / lev;
    const float rs = s > 0.0f ? 1.0f / s : 0.0f;
    float err = 0.0f;
#pragma unroll
    for (int k = 0; k < NGB; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float yy = (k == gl) ? yg[r] : y[k][r];
        // the error is continuous across rounding thresholds, so the float32 quotient
        // only moves it by rounding noise
        const float q = fminf(fmaxf(__builtin_rintf(yy * rs), -lev), lev);
        const float e = yy - s * q;
        err = __builtin_fmaf(e, e, err);
      }
    err = ok ? err : 0.0f;
    err = wave_sum(err);
    if ((tid & 63) == 0) red[tid >> 6][c] = err;
  }
  __syncthreads();
  for (int c = tid; c < nc; c += kEvalThreads) {
    float t = 0.0f;
    for (int w = 0; w < kEvalThreads / 64; ++w) t += red[w][c];
    part[static_cast<size_t>(c0 + c) * p.nchunk + blockIdx.x] = t;
  }
}

// trace[i] += the errors of nblk blocks (one candidate each, block-major partials),
// block ascending.
__global__ void trace_kernel(const float* __restrict__ part, int nchunk, int nblk, double* trace, int i) {
  if (threadIdx.x != 0) return;
  double t = trace[i];
  for (int b = 0; b < nblk; ++b) t = __dadd_rn(t, cand_error(part + static_cast<size_t>(b) * nchunk, nchunk, 0));
  trace[i] = t;
}

bool hip_ok(hipError_t e) { return e == hipSuccess; }

// Device workspace of one calibration call.
struct Work {
  float* hx = nullptr;
  float* rot = nullptr;
  float* cand = nullptr;
  float* part = nullptr;
  double* rd = nullptr;      // search: B's blocks in double
  double* trace = nullptr;   // search: total error before and after each sweep
  void* pin = nullptr;       // pinned staging of the uploads, read by copy16_kernel (a
                             // DMA copy of the candidates alone takes milliseconds)
  ~Work() {
    if (hx) (void)hipFree(hx);
    if (rot) (void)hipFree(rot);
    if (cand) (void)hipFree(cand);
    if (part) (void)hipFree(part);
    if (rd) (void)hipFree(rd);
    if (trace) (void)hipFree(trace);
    if (pin) (void)hipHostFree(pin);
  }
};

// Launch of eval_kernel for n_cand candidates of group `group` (partials in w.part).
int launch_eval(const Work& w, int32_t n, int32_t d, int32_t block, int32_t bits, float eps, const float* dev_cand,
                int32_t n_cand, int32_t group, hipStream_t s, int nblk = 1, int cand_zstride = 0) {
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
  p.n_cand = n_cand;
  p.cand_zstride = cand_zstride;
  const dim3 grid(p.nchunk, (n_cand + 63) / 64, nblk);
  switch (block / 4) {   // groups per quantisation block
    case 1: hipLaunchKernelGGL(eval_kernel<1>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(eval_kernel<2>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(eval_kernel<4>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(eval_kernel<8>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL(eval_kernel<16>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL(eval_kernel<32>, grid, dim3(kEvalThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL(eval_kernel<64>, grid, dim3(kEvalThreads), 0, s, p); break;
    default: return OKV_E_UNSUPPORTED;
  }
  return hip_ok(hipGetLastError()) ? OKV_OK : OKV_E_HIP;
}

int check_args(const float* x, int32_t n, int32_t d, int32_t block, int32_t bits, float eps, int32_t n_cand) {
  if (x == nullptr || n < 1 || n_cand < 1 || n_cand > 1024) return OKV_E_INVALID;
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return OKV_E_ALIGN;
  if (bits < 2 || bits > 4 || !std::isfinite(eps) || eps < 0.0f) return OKV_E_INVALID;
  if (d != 128 && d != 256) return OKV_E_UNSUPPORTED;
  if (block < 4 || block % 4 != 0 || d % block != 0) return OKV_E_INVALID;
  if (static_cast<int64_t>(n) * d >= (int64_t{1} << 31)) return OKV_E_UNSUPPORTED;
  return OKV_OK;
}

// nz: quantisation blocks evaluated in one launch (partials for n_cand x nz x chunks)
int setup(Work& w, const float* x, int32_t n, int32_t d, int32_t n_cand, int nz, size_t cand_floats,
          hipStream_t s) {
  const int nchunk = (n + kEvalThreads - 1) / kEvalThreads;
  if (!hip_ok(hipMalloc(&w.hx, static_cast<size_t>(n) * d * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.rot, static_cast<size_t>(d) * 4 * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.cand, cand_floats * sizeof(float))) ||
      !hip_ok(hipMalloc(&w.part, static_cast<size_t>(n_cand) * nz * nchunk * sizeof(float)))) {
    return OKV_E_HIP;
  }
  const dim3 grid((n + kVec - 1) / kVec);
  if (d == 128) hipLaunchKernelGGL(hx_kernel<128>, grid, dim3(256), 0, s, x, w.hx, n);
  else hipLaunchKernelGGL(hx_kernel<256>, grid, dim3(256), 0, s, x, w.hx, n);
  return hip_ok(hipGetLastError()) ? OKV_OK : OKV_E_HIP;
}

// Errors of the block holding `group` for n_cand candidates at dev_cand (device), on
// the host (one evaluation: okv_so4_eval).
int evaluate(const Work& w, int32_t n, int32_t d, int32_t block, int32_t bits, float eps, const float* dev_cand,
             int32_t n_cand, int32_t group, std::vector<float>& part, double* err, hipStream_t s) {
  const int st = launch_eval(w, n, d, block, bits, eps, dev_cand, n_cand, group, s);
  if (st != OKV_OK) return st;
  const int nchunk = (n + kEvalThreads - 1) / kEvalThreads;
  part.resize(static_cast<size_t>(n_cand) * nchunk);
  if (!hip_ok(hipMemcpyAsync(part.data(), w.part, part.size() * sizeof(float), hipMemcpyDeviceToHost, s)) ||
      !hip_ok(hipStreamSynchronize(s))) {
    return OKV_E_HIP;
  }
  for (int c = 0; c < n_cand; ++c) {
    double t = 0.0;
    for (int k = 0; k < nchunk; ++k) t += part[static_cast<size_t>(c) * nchunk + k];
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
  st = okv::setup(w, x, n, head_dim, n_cand, 1, static_cast<size_t>(n_cand) * 16, s);
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
  st = okv::setup(w, x, n, head_dim, n_cand, head_dim / block, cand_floats, s);
  if (st != OKV_OK) return st;
  static const float kIdentity[16] = {1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1};
  float* dev_identity = w.cand + cand_floats - 16;
  // the search runs on the device: no host round trip per step.  Uploads, staged in
  // pinned memory: candidates + identity | B's blocks in float32 | in double.
  std::vector<double> R(static_cast<size_t>(ng) * 16);
  const size_t rot_bytes = R.size() * sizeof(float), rd_bytes = R.size() * sizeof(double);
  if (!okv::hip_ok(hipHostMalloc(&w.pin, cand_floats * sizeof(float) + rot_bytes + rd_bytes))) return OKV_E_HIP;
  float* pin_cand = static_cast<float*>(w.pin);
  float* pin_rot = pin_cand + cand_floats;
  double* pin_rd = reinterpret_cast<double*>(pin_rot + R.size());   // cand_floats and R.size() are multiples of 16
  std::memcpy(pin_cand, cand, (cand_floats - 16) * sizeof(float));
  std::memcpy(pin_cand + cand_floats - 16, kIdentity, sizeof(kIdentity));
  std::memcpy(pin_rot, rot, rot_bytes);
  for (size_t i = 0; i < R.size(); ++i) pin_rd[i] = R[i] = rot[i];
  if (!okv::hip_ok(hipMalloc(&w.rd, rd_bytes)) ||
      !okv::hip_ok(hipMalloc(&w.trace, static_cast<size_t>(sweeps + 1) * sizeof(double)))) {
    return OKV_E_HIP;
  }
  void* dpin = nullptr;   // device address of the pinned staging buffer
  if (!okv::hip_ok(hipHostGetDevicePointer(&dpin, w.pin, 0))) return OKV_E_HIP;
  auto upload = [&](void* dst, const void* src, size_t bytes) {   // bytes: a multiple of 16
    const void* dsrc = static_cast<const char*>(dpin) + (static_cast<const char*>(src) - static_cast<char*>(w.pin));
    const size_t n16 = bytes / 16;
    const unsigned nb = static_cast<unsigned>(n16 / 256 + 1 < 1024 ? n16 / 256 + 1 : 1024);
    hipLaunchKernelGGL(okv::copy16_kernel, dim3(nb), dim3(256), 0, s, static_cast<const uint4*>(dsrc),
                       static_cast<uint4*>(dst), n16);
    return okv::hip_ok(hipGetLastError());
  };
  if (!upload(w.cand, pin_cand, cand_floats * sizeof(float)) || !upload(w.rot, pin_rot, rot_bytes) ||
      !upload(w.rd, pin_rd, rd_bytes) ||
      !okv::hip_ok(hipMemsetAsync(w.trace, 0, static_cast<size_t>(sweeps + 1) * sizeof(double), s))) {
    return OKV_E_HIP;
  }
  const int nchunk = (n + okv::kEvalThreads - 1) / okv::kEvalThreads;
  const int nblk = head_dim / block;
  // total error under the current B: every block in one launch, then added up in order
  auto total = [&](int i) {
    const int r = okv::launch_eval(w, n, head_dim, block, bits, eps, dev_identity, 1, 0, s, nblk);
    if (r != OKV_OK) return r;
    hipLaunchKernelGGL(okv::trace_kernel, dim3(1), dim3(64), 0, s, w.part, nchunk, nblk, w.trace, i);
    return okv::hip_ok(hipGetLastError()) ? static_cast<int>(OKV_OK) : static_cast<int>(OKV_E_HIP);
  };
  if (trace != nullptr && (st = total(0)) != OKV_OK) return st;
  for (int sw = 0; sw < sweeps; ++sw) {
    // step k of every block at once: groups k, k + gpb, k + 2 gpb, ...
    const int gpb = block / 4;
    const int zstride = static_cast<int>(gpb * per_group);
    for (int k = 0; k < gpb; ++k) {
      const float* dc = w.cand + (static_cast<size_t>(sw) * ng + k) * per_group;
      st = okv::launch_eval(w, n, head_dim, block, bits, eps, dc, n_cand, k, s, nblk, zstride);
      if (st != OKV_OK) return st;
      hipLaunchKernelGGL(okv::select_kernel, dim3(nblk), dim3(256), 0, s, w.part, nchunk, n_cand, dc, k, gpb,
                         zstride, w.rd, w.rot);
      if (!okv::hip_ok(hipGetLastError())) return OKV_E_HIP;
    }
    if (trace != nullptr && (st = total(sw + 1)) != OKV_OK) return st;
  }
  if (!okv::hip_ok(hipMemcpyAsync(R.data(), w.rd, R.size() * sizeof(double), hipMemcpyDeviceToHost, s)) ||
      (trace != nullptr && !okv::hip_ok(hipMemcpyAsync(trace, w.trace, static_cast<size_t>(sweeps + 1) * sizeof(double),
                                                         hipMemcpyDeviceToHost, s))) ||
      !okv::hip_ok(hipStreamSynchronize(s))) {
    return OKV_E_HIP;
  }
  for (size_t i = 0; i < R.size(); ++i) rot[i] = static_cast<float>(R[i]);
  return OKV_OK;
}

}  // extern "C"
