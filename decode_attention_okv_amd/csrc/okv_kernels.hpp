// Internal interface between the host runtime (okv_host.cpp) and the HIP kernels.
// Not installed; the public interface is include/okv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace okv {

constexpr int kTile = 32;   // tokens per value tile
constexpr int kGroup = 32;  // codes per 12-byte packed group

enum : int { kQuantSym = 0, kQuantAsym = 1 };
enum : int { kScaleF32 = 0, kScaleF16 = 1, kScaleE4M3 = 3 };
enum : int { kRotSign = 0, kRotSo4 = 1, kRotNone = 2 };  // kRotNone: U = I

struct WriteParams {
  const void* k;         // [B][n_new][Hkv][D] input type
  const void* v;
  uint8_t* k_codes;      // [B][Hkv][tcap][b D/8]
  uint8_t* v_codes;      // [B][Hkv][tcap/32][D][4 b]
  void* k_meta;          // [B][Hkv][tcap][D/m] (x2 bytes for E4M3 pairs)
  void* v_meta;
  const float* rot;      // device: D signs or (D/4) 4x4 matrices
  int n_new, len, hkv, tcap, ntile_cap, tile0;
  int block, quant, scale_dtype, rotation, in_bf16, bits;
  float eps;
};

struct DecodeParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const void* k_meta;
  const void* v_meta;
  const void* q;         // [B][Hq][D] input type
  const float* rot;
  float* ws;             // [B][Hq][nsplit][D + 2]: acc[D], m (log2 units), l
  int hq, hkv, tcap, ntile_cap, T, nsplit;   // steps interleave over the nsplit splits
  int block, quant, scale_dtype, rotation, in_bf16, bits;
};

struct ReduceParams {
  const float* ws;
  const float* rot;
  float* out;            // [B][Hq][D] float32
  int hq, nsplit, rotation;
};

struct PrefillParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const void* k_meta;
  const void* v_meta;
  const void* q;         // [B][n_q][Hq][D] input type: the rows of positions pos0 .. len-1
  const float* rot;
  float* out;            // [B][n_q][Hq][D] float32
  int hq, hkv, tcap, ntile_cap, len, n_q, pos0;
  int block, quant, scale_dtype, rotation, in_bf16, bits;
};

hipError_t launch_write(const WriteParams& p, int ntiles, int batch, int d, hipStream_t s);
// Causal attention of the last n_q cached positions over the cache (prefill).
hipError_t launch_prefill(const PrefillParams& p, int batch, int d, hipStream_t s);
// ev0/ev1 (may be null): events recorded at the start and the end of the kernel's
// own dispatch (hipExtLaunchKernelGGL), so their elapsed time is the kernel time.
hipError_t launch_reduce(const ReduceParams& p, int batch, int d, hipStream_t s,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Per-head decode on MFMA (one workgroup per query head): head_dim 128/256, blocks
// of 32 .. head_dim.  Grid (nsplit, hq, batch); writes the split-K workspace.
bool head_decode_supported(int d, int block);
hipError_t launch_decode_head(const DecodeParams& p, int batch, int d, hipStream_t s,
                              hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Grouped decode (one workgroup per KV head serves its whole query group on MFMA):
// built for head_dim 128/256, query groups 2, 4 and 8, blocks of 32, 64 and 128.  Grid
// (nsplit, hkv, batch); writes the same workspace as launch_decode_head.
bool grouped_decode_supported(int d, int block, int group);
hipError_t launch_decode_grouped(const DecodeParams& p, int batch, int d, hipStream_t s,
                                 hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

}  // namespace okv
