// Host runtime of libokv: argument validation, cache layout arithmetic, device
// copies of the rotation parameters, the split-K workspace and kernel launches.
// Implements include/okv.h.
#include "okv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "okv_kernels.hpp"

namespace {

constexpr int kMaxSplits = 256;      // split-K workspace capacity per (sequence, query head)
constexpr int kTargetGroups = 2048;  // workgroups the automatic split count aims for
constexpr int kMinSplitSteps = 8;    // automatic splits keep >= 2 64-token steps per wave
constexpr int kFillGroups = 512;     // workgroups that fill the GPU once (2 per CU)
constexpr int kLongSplitSteps = 64;  // >= 16 steps per wave once the GPU is filled
constexpr int kTimingSlots = 8192;   // event triples kept for okv_timing_read

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// last HIP error that made a call on this thread fail (okv_last_hip_error)
thread_local hipError_t g_last_hip = hipSuccess;

bool hip_ok(hipError_t e) {
  if (e == hipSuccess) return true;
  g_last_hip = e;
  return false;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int meta_entry_bytes(const okv_config& c) {
  if (c.quant == OKV_QUANT_ASYM) return 2;           // E4M3 scale + zero-point
  return c.scale_dtype == OKV_DT_F32 ? 4 : 2;
}

// Shape / enum checks shared by okv_layout and okv_create.
int validate_shape(const okv_config* c) {
  if (c == nullptr) return OKV_E_INVALID;
  if (c->abi_version != OKV_ABI_VERSION) return OKV_E_INVALID;
  if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1) return OKV_E_INVALID;
  if (c->num_q_heads % c->num_kv_heads != 0) return OKV_E_INVALID;
  if (!is_pow2(c->head_dim) || c->head_dim % 4 != 0) return OKV_E_INVALID;
  if (c->block < 8 || c->block % 8 != 0 || c->head_dim % c->block != 0) return OKV_E_INVALID;
  if (c->max_tokens < 1 || c->max_tokens % 32 != 0) return OKV_E_INVALID;
  if (c->quant != OKV_QUANT_SYM && c->quant != OKV_QUANT_ASYM) return OKV_E_INVALID;
  if (c->in_dtype != OKV_DT_F32 && c->in_dtype != OKV_DT_BF16) return OKV_E_INVALID;
  if (c->rotation != OKV_ROT_SIGN && c->rotation != OKV_ROT_SO4 && c->rotation != OKV_ROT_NONE) {
    return OKV_E_INVALID;
  }
  if (c->bits < 2 || c->bits > 4) return OKV_E_INVALID;
  if (c->quant == OKV_QUANT_SYM) {
    if (c->scale_dtype != OKV_DT_F32 && c->scale_dtype != OKV_DT_F16) {
      return c->scale_dtype == OKV_DT_E4M3 ? OKV_E_UNSUPPORTED : OKV_E_INVALID;
    }
    if (!std::isfinite(c->eps) || c->eps < 0.0f) return OKV_E_INVALID;
  } else {
    if (c->scale_dtype != OKV_DT_E4M3) {
      return (c->scale_dtype == OKV_DT_F32 || c->scale_dtype == OKV_DT_F16) ? OKV_E_UNSUPPORTED
                                                                            : OKV_E_INVALID;
    }
  }
  // valid, but only these are built
  if (c->head_dim != 128 && c->head_dim != 256) return OKV_E_UNSUPPORTED;
  // sequences and query heads are launch grid dimensions (y and z) of the kernels
  if (c->batch > 65535 || c->num_q_heads > 65535) return OKV_E_UNSUPPORTED;
  if (c->block % 32 != 0) return OKV_E_UNSUPPORTED;
  // the kernels address one (sequence, KV head) slice of a cache buffer with 32-bit
  // byte offsets (buffer resources), up to 128 tokens past its end: the packed codes
  // of a slice plus that margin stay below 4 GiB
  if ((static_cast<int64_t>(c->max_tokens) + 128) * (c->bits * c->head_dim / 8) >= (int64_t{1} << 32)) {
    return OKV_E_UNSUPPORTED;
  }
  return OKV_OK;
}

void layout_of(const okv_config& c, okv_layout_info* li) {
  const uint64_t units = static_cast<uint64_t>(c.batch) * c.num_kv_heads;
  const uint64_t rows = units * static_cast<uint64_t>(c.max_tokens);
  li->k_codes_bytes = rows * (static_cast<uint64_t>(c.bits) * c.head_dim / 8);
  li->v_codes_bytes = rows * (static_cast<uint64_t>(c.bits) * c.head_dim / 8);
  li->k_meta_bytes = rows * static_cast<uint64_t>(c.head_dim / c.block) * meta_entry_bytes(c);
  li->v_meta_bytes = li->k_meta_bytes;
}

struct TimingSlot {
  hipEvent_t e0, e1, e2, e3;  // attention kernel start/end, reduce kernel start/end
};

}  // namespace

// ---- static split-K scratch of okv_decode_attn_noalloc
//
// A file-scope device array: each GPU the library runs on holds its own copy (from the
// code object's load until the process ends).  In host code `g_scratch` is only a
// host-side stand-in for the symbol, never a device address: the device address of a
// GPU's copy is looked up once per device (scratch_setup, from okv_create with that
// device current) and kept in g_scratch_ptr; kernels receive that pointer.
namespace {
constexpr size_t kScratchBytes = size_t{16} << 20;   // 16 MiB per GPU
constexpr size_t kScratchFloats = kScratchBytes / sizeof(float);
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) float g_scratch[kScratchFloats];

namespace {

std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

// Look up the device address of the scratch on `device` (the current device), once.
void scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::call_once(g_scratch_once[device], [device] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_scratch));
    g_scratch_err[device] = e;
    if (e == hipSuccess) g_scratch_ptr[device] = static_cast<float*>(p);
  });
}

}  // namespace

struct okv_handle {
  okv_config cfg;
  int device = 0;
  float* d_rot = nullptr;
  float* d_ws = nullptr;
  int32_t len = 0;
  int32_t splits = 0;  // 0 = automatic
  int32_t kernel = OKV_DECODE_AUTO;
  bool timing = false;
  std::vector<TimingSlot> slots;
  int recorded = 0;
};

namespace {

bool grouped_built(const okv_config& c) {
  return okv::grouped_decode_supported(c.head_dim, c.block, c.num_q_heads / c.num_kv_heads);
}

// OKV_DECODE_PER_HEAD or OKV_DECODE_GROUPED: the kernel okv_decode_attn launches.
int decode_kernel_of(const okv_handle* h) {
  if (h->kernel == OKV_DECODE_PER_HEAD) return OKV_DECODE_PER_HEAD;
  return grouped_built(h->cfg) ? OKV_DECODE_GROUPED : OKV_DECODE_PER_HEAD;
}

// Split count for a cache of T tokens.  The decode kernels interleave their
// 64-token steps over the splits of a (sequence, head); none is empty.
int choose_splits(const okv_handle* h, int32_t T) {
  const int nsteps = (T + 63) / 64;
  int s = h->splits;
  if (s <= 0) {
    // workgroups per split: one per query head, or one per KV head when grouped
    const int heads = decode_kernel_of(h) == OKV_DECODE_GROUPED ? h->cfg.num_kv_heads : h->cfg.num_q_heads;
    const int units = h->cfg.batch * heads;
    s = (kTargetGroups + units - 1) / units;
    const int cap = nsteps / kMinSplitSteps;   // short caches: fewer, longer splits
    if (s > cap) s = cap;
    // once the grid fills the GPU, longer splits beat more rounds of short ones (each
    // workgroup pays the query prologue and the wave combine once)
    const int fill = (kFillGroups + units - 1) / units;
    if (s > fill) s = std::max(fill, std::min(s, nsteps / kLongSplitSteps));
  }
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > nsteps) s = nsteps;
  if (s < 1) s = 1;
  return s;
}

void free_timing(okv_handle* h) {
  for (auto& t : h->slots) {
    (void)hipEventDestroy(t.e0);
    (void)hipEventDestroy(t.e1);
    (void)hipEventDestroy(t.e2);
    (void)hipEventDestroy(t.e3);
  }
  h->slots.clear();
  h->recorded = 0;
}

// One decode call (attention kernel + split merge) with the split partials in `ws`
// (B x Hq x nsplit x (d + 2) floats); arguments already checked.
int decode_launch(okv_handle* h, const void* q, float* out, hipStream_t s, float* ws) {
  const okv_config& c = h->cfg;
  const int nsplit = choose_splits(h, h->len);
  okv::DecodeParams p{};
  p.k_codes = static_cast<const uint8_t*>(c.k_codes);
  p.v_codes = static_cast<const uint8_t*>(c.v_codes);
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.q = q;
  p.rot = h->d_rot;
  p.ws = ws;
  p.hq = c.num_q_heads;
  p.hkv = c.num_kv_heads;
  p.tcap = c.max_tokens;
  p.ntile_cap = c.max_tokens / okv::kTile;
  p.T = h->len;
  p.nsplit = nsplit;
  p.block = c.block;
  p.quant = c.quant;
  p.scale_dtype = c.scale_dtype;
  p.rotation = c.rotation;
  p.in_bf16 = c.in_dtype == OKV_DT_BF16;
  p.bits = c.bits;
  okv::ReduceParams r{};
  r.ws = ws;
  r.rot = h->d_rot;
  r.out = out;
  r.hq = c.num_q_heads;
  r.nsplit = nsplit;
  r.rotation = c.rotation;
  if (!hip_ok(hipSetDevice(h->device))) return OKV_E_HIP;
  TimingSlot* ts = nullptr;
  if (h->timing && h->recorded < static_cast<int>(h->slots.size())) ts = &h->slots[h->recorded++];
  const hipError_t le = decode_kernel_of(h) == OKV_DECODE_GROUPED
                           ? okv::launch_decode_grouped(p, c.batch, c.head_dim, s, ts ? ts->e0 : nullptr,
                                                        ts ? ts->e1 : nullptr)
                           : okv::launch_decode_head(p, c.batch, c.head_dim, s, ts ? ts->e0 : nullptr,
                                                     ts ? ts->e1 : nullptr);
  if (!hip_ok(le)) return OKV_E_HIP;
  if (!hip_ok(okv::launch_reduce(r, c.batch, c.head_dim, s, ts ? ts->e2 : nullptr, ts ? ts->e3 : nullptr))) {
    return OKV_E_HIP;
  }
  return OKV_OK;
}

}  // namespace

extern "C" {

const char* okv_strerror(int status) {
  switch (status) {
    case OKV_OK: return "ok";
    case OKV_E_INVALID: return "invalid argument or configuration";
    case OKV_E_ALIGN: return "pointer not 16-byte aligned";
    case OKV_E_CAPACITY: return "cache capacity exceeded";
    case OKV_E_UNSUPPORTED: return "configuration not supported by this build";
    case OKV_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int okv_layout(const okv_config* cfg, okv_layout_info* info) {
  if (info == nullptr) return OKV_E_INVALID;
  const int st = validate_shape(cfg);
  if (st != OKV_OK) return st;
  layout_of(*cfg, info);
  return OKV_OK;
}

int okv_create(const okv_config* cfg, okv_handle** out) {
  if (out == nullptr) return OKV_E_INVALID;
  *out = nullptr;
  int st = validate_shape(cfg);
  if (st != OKV_OK) return st;
  if (cfg->rot_params == nullptr && cfg->rotation != OKV_ROT_NONE) return OKV_E_INVALID;
  if (!cfg->k_codes || !cfg->v_codes || !cfg->k_meta || !cfg->v_meta) return OKV_E_INVALID;
  if (!aligned16(cfg->k_codes) || !aligned16(cfg->v_codes) || !aligned16(cfg->k_meta) ||
      !aligned16(cfg->v_meta)) {
    return OKV_E_ALIGN;
  }
  const int d = cfg->head_dim;
  const size_t nrot = cfg->rotation == OKV_ROT_SO4 ? static_cast<size_t>(4) * d : static_cast<size_t>(d);
  // no rotation: the device copy holds d ones (never read by the kernels)
  std::vector<float> ones;
  if (cfg->rotation == OKV_ROT_NONE) ones.assign(d, 1.0f);
  const float* rp = cfg->rotation == OKV_ROT_NONE ? ones.data() : cfg->rot_params;
  if (cfg->rotation == OKV_ROT_SIGN) {
    for (int i = 0; i < d; ++i) {
      if (rp[i] != 1.0f && rp[i] != -1.0f) return OKV_E_INVALID;
    }
  } else if (cfg->rotation == OKV_ROT_SO4) {
    for (int r = 0; r < d / 4; ++r) {
      const float* R = rp + 16 * r;
      for (int a = 0; a < 4; ++a) {
        for (int c = 0; c < 4; ++c) {
          double dot = 0.0;
          for (int k = 0; k < 4; ++k) dot += static_cast<double>(R[4 * k + a]) * R[4 * k + c];
          if (!(std::fabs(dot - (a == c ? 1.0 : 0.0)) <= 1e-3)) return OKV_E_INVALID;
        }
      }
    }
  }

  okv_handle* h = new (std::nothrow) okv_handle();
  if (h == nullptr) return OKV_E_HIP;
  h->cfg = *cfg;
  h->cfg.rot_params = nullptr;  // the host copy is not kept
  if (!hip_ok(hipGetDevice(&h->device))) {
    delete h;
    return OKV_E_HIP;
  }
  // set-up of okv_decode_attn_noalloc: the scratch's address on this device, once per
  // device (a failure is reported by that call, not here)
  scratch_setup(h->device);
  const size_t ws_floats = static_cast<size_t>(cfg->batch) * cfg->num_q_heads * kMaxSplits * (d + 2);
  if (!hip_ok(hipMalloc(&h->d_rot, nrot * sizeof(float))) ||
      !hip_ok(hipMemcpy(h->d_rot, rp, nrot * sizeof(float), hipMemcpyHostToDevice)) ||
      !hip_ok(hipMalloc(&h->d_ws, ws_floats * sizeof(float)))) {
    if (h->d_rot) (void)hipFree(h->d_rot);
    if (h->d_ws) (void)hipFree(h->d_ws);
    delete h;
    return OKV_E_HIP;
  }
  *out = h;
  return OKV_OK;
}

int okv_destroy(okv_handle* h) {
  if (h == nullptr) return OKV_OK;
  int st = OKV_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  free_timing(h);
  if (h->d_rot && !hip_ok(hipFree(h->d_rot))) st = OKV_E_HIP;
  if (h->d_ws && !hip_ok(hipFree(h->d_ws))) st = OKV_E_HIP;
  (void)hipSetDevice(prev);
  delete h;
  return st;
}

int okv_write(okv_handle* h, const void* k, const void* v, int32_t n_new, void* hip_stream) {
  if (h == nullptr || k == nullptr || v == nullptr) return OKV_E_INVALID;
  if (n_new < 1) return OKV_E_INVALID;
  if (!aligned16(k) || !aligned16(v)) return OKV_E_ALIGN;
  const okv_config& c = h->cfg;
  if (static_cast<int64_t>(h->len) + n_new > c.max_tokens) return OKV_E_CAPACITY;
  okv::WriteParams p{};
  p.k = k;
  p.v = v;
  p.k_codes = static_cast<uint8_t*>(c.k_codes);
  p.v_codes = static_cast<uint8_t*>(c.v_codes);
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.rot = h->d_rot;
  p.n_new = n_new;
  p.len = h->len;
  p.hkv = c.num_kv_heads;
  p.tcap = c.max_tokens;
  p.ntile_cap = c.max_tokens / okv::kTile;
  p.tile0 = h->len / okv::kTile;
  p.block = c.block;
  p.quant = c.quant;
  p.scale_dtype = c.scale_dtype;
  p.rotation = c.rotation;
  p.in_bf16 = c.in_dtype == OKV_DT_BF16;
  p.bits = c.bits;
  p.eps = c.eps;
  const int tile1 = (h->len + n_new - 1) / okv::kTile;
  const int ntiles = tile1 - p.tile0 + 1;
  if (!hip_ok(hipSetDevice(h->device))) return OKV_E_HIP;
  if (!hip_ok(okv::launch_write(p, ntiles, c.batch, c.head_dim, static_cast<hipStream_t>(hip_stream)))) {
    return OKV_E_HIP;
  }
  h->len += n_new;
  return OKV_OK;
}

int okv_decode_attn(okv_handle* h, const void* q, float* out, void* hip_stream) {
  if (h == nullptr || q == nullptr || out == nullptr) return OKV_E_INVALID;
  if (!aligned16(q) || !aligned16(out)) return OKV_E_ALIGN;
  if (h->len < 1) return OKV_E_INVALID;
  return decode_launch(h, q, out, static_cast<hipStream_t>(hip_stream), h->d_ws);
}

int okv_decode_attn_noalloc(okv_handle* h, const void* q, float* out, void* hip_stream) {
  if (h == nullptr || q == nullptr || out == nullptr) return OKV_E_INVALID;
  if (!aligned16(q) || !aligned16(out)) return OKV_E_ALIGN;
  if (h->len < 1) return OKV_E_INVALID;
  const okv_config& c = h->cfg;
  const size_t need = static_cast<size_t>(c.batch) * c.num_q_heads * choose_splits(h, h->len) *
                      (static_cast<size_t>(c.head_dim) + 2);
  if (need > kScratchFloats) return OKV_E_CAPACITY;
  if (h->device < 0 || h->device >= kMaxDevices) return OKV_E_UNSUPPORTED;
  float* ws = g_scratch_ptr[h->device];
  if (ws == nullptr) {
    g_last_hip = g_scratch_err[h->device] != hipSuccess ? g_scratch_err[h->device] : hipErrorInvalidSymbol;
    return OKV_E_HIP;
  }
  return decode_launch(h, q, out, static_cast<hipStream_t>(hip_stream), ws);
}

int okv_prefill_attn(okv_handle* h, const void* q, int32_t n_q, float* out, void* hip_stream) {
  if (h == nullptr || q == nullptr || out == nullptr) return OKV_E_INVALID;
  if (!aligned16(q) || !aligned16(out)) return OKV_E_ALIGN;
  if (n_q < 1 || n_q > h->len) return OKV_E_INVALID;
  const okv_config& c = h->cfg;
  okv::PrefillParams p{};
  p.k_codes = static_cast<const uint8_t*>(c.k_codes);
  p.v_codes = static_cast<const uint8_t*>(c.v_codes);
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.q = q;
  p.rot = h->d_rot;
  p.out = out;
  p.hq = c.num_q_heads;
  p.hkv = c.num_kv_heads;
  p.tcap = c.max_tokens;
  p.ntile_cap = c.max_tokens / okv::kTile;
  p.len = h->len;
  p.n_q = n_q;
  p.pos0 = h->len - n_q;
  p.block = c.block;
  p.quant = c.quant;
  p.scale_dtype = c.scale_dtype;
  p.rotation = c.rotation;
  p.in_bf16 = c.in_dtype == OKV_DT_BF16;
  p.bits = c.bits;
  if (!hip_ok(hipSetDevice(h->device))) return OKV_E_HIP;
  if (!hip_ok(okv::launch_prefill(p, c.batch, c.head_dim, static_cast<hipStream_t>(hip_stream)))) {
    return OKV_E_HIP;
  }
  return OKV_OK;
}

int okv_get_len(const okv_handle* h, int32_t* len) {
  if (h == nullptr || len == nullptr) return OKV_E_INVALID;
  *len = h->len;
  return OKV_OK;
}

int okv_set_len(okv_handle* h, int32_t len) {
  if (h == nullptr || len < 0 || len > h->cfg.max_tokens) return OKV_E_INVALID;
  h->len = len;
  return OKV_OK;
}

int okv_set_splits(okv_handle* h, int32_t num_splits) {
  if (h == nullptr || num_splits < 0 || num_splits > kMaxSplits) return OKV_E_INVALID;
  h->splits = num_splits;
  return OKV_OK;
}

int okv_max_splits(const okv_handle* h, int32_t* n) {
  if (h == nullptr || n == nullptr) return OKV_E_INVALID;
  *n = kMaxSplits;
  return OKV_OK;
}

int okv_get_splits(const okv_handle* h, int32_t* n) {
  if (h == nullptr || n == nullptr) return OKV_E_INVALID;
  *n = h->len > 0 ? choose_splits(h, h->len) : 0;
  return OKV_OK;
}

const char* okv_last_hip_error(void) {
  return g_last_hip == hipSuccess ? "none" : hipGetErrorString(g_last_hip);
}

int okv_set_decode_kernel(okv_handle* h, int32_t kind) {
  if (h == nullptr) return OKV_E_INVALID;
  if (kind != OKV_DECODE_AUTO && kind != OKV_DECODE_PER_HEAD && kind != OKV_DECODE_GROUPED) {
    return OKV_E_INVALID;
  }
  if (kind == OKV_DECODE_GROUPED && !grouped_built(h->cfg)) return OKV_E_UNSUPPORTED;
  h->kernel = kind;
  return OKV_OK;
}

int okv_get_decode_kernel(const okv_handle* h, int32_t* kind) {
  if (h == nullptr || kind == nullptr) return OKV_E_INVALID;
  *kind = decode_kernel_of(h);
  return OKV_OK;
}

int okv_timing_enable(okv_handle* h, int32_t enable) {
  if (h == nullptr) return OKV_E_INVALID;
  if (!hip_ok(hipSetDevice(h->device))) return OKV_E_HIP;
  if (enable && h->slots.empty()) {
    h->slots.resize(kTimingSlots);
    for (auto& t : h->slots) {
      if (!hip_ok(hipEventCreate(&t.e0)) || !hip_ok(hipEventCreate(&t.e1)) ||
          !hip_ok(hipEventCreate(&t.e2)) || !hip_ok(hipEventCreate(&t.e3))) {
        return OKV_E_HIP;
      }
    }
  }
  if (!enable) free_timing(h);
  h->timing = enable != 0;
  h->recorded = 0;
  return OKV_OK;
}

int okv_timing_read(okv_handle* h, int32_t* calls, double* attn_ms, double* reduce_ms) {
  if (h == nullptr || calls == nullptr || attn_ms == nullptr || reduce_ms == nullptr) return OKV_E_INVALID;
  double a = 0.0, r = 0.0;
  for (int i = 0; i < h->recorded; ++i) {
    TimingSlot& t = h->slots[i];
    float x = 0.0f, y = 0.0f;
    if (!hip_ok(hipEventSynchronize(t.e3))) return OKV_E_HIP;
    if (!hip_ok(hipEventElapsedTime(&x, t.e0, t.e1))) return OKV_E_HIP;
    if (!hip_ok(hipEventElapsedTime(&y, t.e2, t.e3))) return OKV_E_HIP;
    a += x;
    r += y;
  }
  *calls = h->recorded;
  *attn_ms = a;
  *reduce_ms = r;
  h->recorded = 0;
  return OKV_OK;
}

}  // extern "C"
