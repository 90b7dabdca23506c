// Write path: rotate each new key and value head vector with U, quantise it
// blockwise to 3-bit codes and pack the codes.
//
// Pages: "Orthogonally mixed 3-bit KV cache", Implementation notes (k1 = U(k),
// v1 = U(v), one scale per block, signed 3-bit codes, pack, store codes and scales)
// and Key formulas (the quantiser); "Orthogonal Invariance in Activation Space",
// Sections 3.1-3.2 (normalised FWHT after a random sign flip); the news item on
// hardware-fused transforms, third paragraph (asymmetric unsigned 3-bit codes per
// 64-element sub-block with an FP8 scale and zero-point).
//
// Every float32 operation here is rounded on its own, in a fixed order, so the
// result matches the bit specification exactly: contraction into fused
// multiply-adds is disabled for this file.
#pragma clang fp contract(off)

#include "okv_device.hpp"

namespace okv {

namespace {

// One workgroup owns one 32-token tile of one (sequence, KV head): it computes the
// new tokens of the tile, rewrites the key rows of those tokens and the whole value
// tile (old codes kept, unwritten slots zero).  Key and value vectors are spread
// over D/8 lanes, 8 consecutive elements per lane.
template <int D>
__global__ __launch_bounds__(256) void write_kernel(const WriteParams p) {
  constexpr int LPV = D / 8;      // lanes per vector
  constexpr int VPP = 256 / LPV;  // vectors per pass of the workgroup
  __shared__ uint8_t vt[kTile][D];

  const int tile = p.tile0 + static_cast<int>(blockIdx.x);
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int tile_base = tile * kTile;
  const int s_lo = max(p.len - tile_base, 0);
  const int s_hi = min(p.len + p.n_new - tile_base, kTile);
  const int nnew = s_hi - s_lo;
  const size_t unit = static_cast<size_t>(b) * p.hkv + h;
  uint8_t* vtile = p.v_codes + (unit * p.ntile_cap + tile) * static_cast<size_t>(D) * 12;
  const int nblk = D / p.block;

  for (int i = tid; i < kTile * D / 4; i += 256) reinterpret_cast<uint32_t*>(&vt[0][0])[i] = 0u;
  __syncthreads();
  if (s_lo > 0) {
    // tile already holds tokens 0 .. s_lo-1: keep their value codes
    for (int j = tid; j < D; j += 256) {
      const uint32_t* g = reinterpret_cast<const uint32_t*>(vtile + 12 * j);
      const uint32_t w0 = g[0], w1 = g[1], w2 = g[2];
      for (int i = 0; i < s_lo; ++i) vt[i][j] = static_cast<uint8_t>(g32_code(w0, w1, w2, i));
    }
  }

  const int r = tid % LPV;  // lane index inside the vector: elements 8r .. 8r+7
  const float cnorm = (D == 128) ? __uint_as_float(0x3DB504F3u) : 0.0625f;  // RN32(1/sqrt(D))
  const int nvec = 2 * nnew;
  for (int base = 0; base < nvec; base += VPP) {
    const int vi = base + tid / LPV;
    if (vi >= nvec) continue;  // uniform over the LPV lanes of one vector
    const int tensor = vi / nnew;
    const int slot = s_lo + vi % nnew;
    const int pos = tile_base + slot;
    const int t_in = pos - p.len;
    const size_t src = ((static_cast<size_t>(b) * p.n_new + t_in) * p.hkv + h) * D + 8 * r;

    float x[8];
    load8(tensor ? p.v : p.k, src, p.in_bf16, x);

    if (p.rotation == kRotSign) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * p.rot[8 * r + e];
    }
    // butterfly stages of stride 1, 2, 4 inside the lane
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!(e & hs)) {
          const float a = x[e], c = x[e + hs];
          x[e] = a + c;
          x[e + hs] = a - c;
        }
      }
    }
    // stages of stride 8, 16, ... across lanes (partner lane r ^ bit)
#pragma unroll
    for (int bit = 1; bit < LPV; bit <<= 1) {
      const bool upper = (r & bit) != 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o = shfl_xor(x[e], bit);
        x[e] = upper ? (o - x[e]) : (x[e] + o);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * cnorm;

    if (p.rotation == kRotSo4) {
      // y_row = ((R_row0 x0 + R_row1 x1) + R_row2 x2) + R_row3 x3 per 4-block
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const float* R = p.rot + 16 * (2 * r + qd);
        const float x0 = x[4 * qd], x1 = x[4 * qd + 1], x2 = x[4 * qd + 2], x3 = x[4 * qd + 3];
#pragma unroll
        for (int row = 0; row < 4; ++row) {
          float acc = R[4 * row] * x0;
          acc = acc + R[4 * row + 1] * x1;
          acc = acc + R[4 * row + 2] * x2;
          acc = acc + R[4 * row + 3] * x3;
          x[4 * qd + row] = acc;
        }
      }
    }

    // block statistics over the m/8 lanes of a block
    const int lpb = p.block / 8;
    uint32_t u[8];
    const size_t row = unit * p.tcap + pos;
    void* meta = tensor ? p.v_meta : p.k_meta;
    const int blk = (8 * r) / p.block;
    const bool meta_lane = ((8 * r) % p.block) == 0;
    if (p.quant == kQuantSym) {
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
      for (int bit = 1; bit < lpb; bit <<= 1) amax = fmaxf(amax, shfl_xor(amax, bit));
      const float s32 = (amax + p.eps) / 3.0f;
      float s;
      if (p.scale_dtype == kScaleF16) {
        const _Float16 s16 = static_cast<_Float16>(s32);
        s = static_cast<float>(s16);
        if (meta_lane) reinterpret_cast<_Float16*>(meta)[row * nblk + blk] = s16;
      } else {
        s = s32;
        if (meta_lane) reinterpret_cast<float*>(meta)[row * nblk + blk] = s32;
      }
      const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = static_cast<uint32_t>(rne_code(x[e], s, rs, -3, 3) + 4);
    } else {
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) { mn = fminf(mn, x[e]); mx = fmaxf(mx, x[e]); }
      for (int bit = 1; bit < lpb; bit <<= 1) {
        mn = fminf(mn, shfl_xor(mn, bit));
        mx = fmaxf(mx, shfl_xor(mx, bit));
      }
      const float s32 = (mx - mn) / 7.0f;
      const uint32_t sb = e4m3_encode(s32), zb = e4m3_encode(mn);
      const float s = e4m3_decode(sb), z = e4m3_decode(zb);
      if (meta_lane) reinterpret_cast<uint16_t*>(meta)[row * nblk + blk] = static_cast<uint16_t>(sb | (zb << 8));
      const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = static_cast<uint32_t>(rne_code(x[e] - z, s, rs, 0, 7));
    }

    if (tensor == 0) {
      // key row: lane gi (0..3) of a 32-code group holds codes 8gi .. 8gi+7
      const int gi = r & 3;
      uint32_t w = 0, l0 = 0, l1 = 0, l2 = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        w |= (u[bb] | (u[4 + bb] << 3)) << (8 * bb);
        l0 |= (u[bb] & 3u) << (8 * bb + 6);
        l1 |= (u[4 + bb] & 3u) << (8 * bb + 6);
        l2 |= ((u[bb] >> 2) << (8 * bb + 6)) | ((u[4 + bb] >> 2) << (8 * bb + 7));
      }
      // codes 24..31 (lane gi == 3) fill bits 6-7 of every byte of the group
      const int src_lane = lane | 3;
      const uint32_t f0 = __shfl(l0, src_lane, 64);
      const uint32_t f1 = __shfl(l1, src_lane, 64);
      const uint32_t f2 = __shfl(l2, src_lane, 64);
      if (gi < 3) {
        const uint32_t word = w | (gi == 0 ? f0 : (gi == 1 ? f1 : f2));
        uint8_t* dst = p.k_codes + row * (3 * D / 8) + 12 * (r >> 2) + 4 * gi;
        *reinterpret_cast<uint32_t*>(dst) = word;
      }
    } else {
      uint2 packed;
      packed.x = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
      packed.y = u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24);
      *reinterpret_cast<uint2*>(&vt[slot][8 * r]) = packed;
    }
  }
  __syncthreads();

  // value tile: dim j is one group over the tile's 32 tokens; thread idx writes word
  // k = idx % 3 of dim j = idx / 3 (contiguous 4-byte stores)
  for (int idx = tid; idx < 3 * D; idx += 256) {
    const int j = idx / 3;
    const int k = idx - 3 * j;
    uint32_t w = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      w |= (static_cast<uint32_t>(vt[8 * k + bb][j]) | (static_cast<uint32_t>(vt[8 * k + 4 + bb][j]) << 3))
           << (8 * bb);
      const uint32_t a = vt[24 + bb][j], c = vt[28 + bb][j];
      if (k == 0) w |= (a & 3u) << (8 * bb + 6);
      else if (k == 1) w |= (c & 3u) << (8 * bb + 6);
      else w |= ((a >> 2) << (8 * bb + 6)) | ((c >> 2) << (8 * bb + 7));
    }
    reinterpret_cast<uint32_t*>(vtile)[idx] = w;
  }
}

}  // namespace

hipError_t launch_write(const WriteParams& p, int ntiles, int batch, int d, hipStream_t s) {
  const dim3 grid(ntiles, p.hkv, batch);
  if (d == 128) hipLaunchKernelGGL(write_kernel<128>, grid, dim3(256), 0, s, p);
  else if (d == 256) hipLaunchKernelGGL(write_kernel<256>, grid, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace okv
