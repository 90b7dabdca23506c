// Host-side checks of the C ABI's GPU-free paths (configuration layout and validation,
// argument rejection, null handles, status strings), built together with the library's
// host code under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_sanitize.py.  The kernel launchers are stubs: no path exercised here
// reaches them.  Exit status 0 and the line "ok" on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "okv.h"
#include "okv_kernels.hpp"

namespace okv {
hipError_t launch_write(const WriteParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill(const PrefillParams&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_reduce(const ReduceParams&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorInvalidValue;
}
bool head_decode_supported(int, int) { return false; }
hipError_t launch_decode_head(const DecodeParams&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorInvalidValue;
}
bool grouped_decode_supported(int, int, int) { return false; }
hipError_t launch_decode_grouped(const DecodeParams&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorInvalidValue;
}
}  // namespace okv

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

std::vector<float> signs(int d) { return std::vector<float>(static_cast<size_t>(d), 1.0f); }

okv_config base(const std::vector<float>& rot) {
  okv_config c{};
  c.abi_version = OKV_ABI_VERSION;
  c.batch = 2;
  c.num_q_heads = 8;
  c.num_kv_heads = 2;
  c.head_dim = 128;
  c.max_tokens = 1024;
  c.block = 32;
  c.quant = OKV_QUANT_SYM;
  c.scale_dtype = OKV_DT_F16;
  c.in_dtype = OKV_DT_BF16;
  c.rotation = OKV_ROT_SIGN;
  c.bits = 3;
  c.eps = 1e-6f;
  c.rot_params = rot.data();
  // fake, 16-byte aligned device addresses: never dereferenced on these paths
  c.k_codes = reinterpret_cast<void*>(uintptr_t{0x10000});
  c.v_codes = reinterpret_cast<void*>(uintptr_t{0x20000});
  c.k_meta = reinterpret_cast<void*>(uintptr_t{0x30000});
  c.v_meta = reinterpret_cast<void*>(uintptr_t{0x40000});
  return c;
}

// okv_layout and okv_create both reject cfg with `status`, and leave *out NULL
void rejects(const okv_config& cfg, int status, int line) {
  okv_layout_info info{};
  const int a = okv_layout(&cfg, &info);
  okv_handle* h = reinterpret_cast<okv_handle*>(uintptr_t{1});
  const int b = okv_create(&cfg, &h);
  if (a != status || b != status || h != nullptr) {
    std::printf("FAIL line %d: layout %d create %d (expected %d), handle %p\n", line, a, b, status,
                static_cast<void*>(h));
    ++failures;
  }
}

// okv_create rejects cfg with `status` (okv_layout reads the shape fields only)
void create_rejects(const okv_config& cfg, int status, int line) {
  okv_layout_info info{};
  const int a = okv_layout(&cfg, &info);
  okv_handle* h = reinterpret_cast<okv_handle*>(uintptr_t{1});
  const int b = okv_create(&cfg, &h);
  if (a != OKV_OK || b != status || h != nullptr) {
    std::printf("FAIL line %d: layout %d create %d (expected %d), handle %p\n", line, a, b, status,
                static_cast<void*>(h));
    ++failures;
  }
}

}  // namespace

int main() {
  const std::vector<float> s128 = signs(128), s256 = signs(256);
  {
    // sizes: 2 sequences x 2 KV heads x 1024 rows of 48 code bytes; fp16 scales of 4 blocks
    okv_config c = base(s128);
    okv_layout_info info{};
    EXPECT(okv_layout(&c, &info) == OKV_OK);
    EXPECT(info.k_codes_bytes == 4ull * 1024 * 48 && info.v_codes_bytes == 4ull * 1024 * 48);
    EXPECT(info.k_meta_bytes == 4ull * 1024 * 4 * 2 && info.v_meta_bytes == info.k_meta_bytes);
    c.quant = OKV_QUANT_ASYM;
    c.scale_dtype = OKV_DT_E4M3;
    c.block = 64;
    EXPECT(okv_layout(&c, &info) == OKV_OK && info.k_meta_bytes == 4ull * 1024 * 2 * 2);
    for (int bits = 2; bits <= 4; ++bits) {
      okv_config w = base(s128);
      w.bits = bits;
      EXPECT(okv_layout(&w, &info) == OKV_OK && info.k_codes_bytes == 4ull * 1024 * bits * 16);
    }
    // the largest accepted slices and the first refused ones (the 4 GiB slice limit)
    okv_config big = base(s128);
    big.max_tokens = 89478336;
    EXPECT(okv_layout(&big, &info) == OKV_OK && info.k_codes_bytes == 4ull * 89478336 * 48);
    big.max_tokens = 89478368;
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
    big.bits = 4;
    big.max_tokens = 67108704;
    EXPECT(okv_layout(&big, &info) == OKV_OK);
    big.max_tokens = 67108736;
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
    big = base(s256);
    big.head_dim = 256;
    big.max_tokens = 44739264;
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
    big.max_tokens = 2147483616;   // the largest multiple of 32 in int32
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
    big = base(s128);
    big.batch = 65535;             // the largest grid dimension
    EXPECT(okv_layout(&big, &info) == OKV_OK);
    big.batch = 65536;
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
    big = base(s128);
    big.num_q_heads = 65536;
    rejects(big, OKV_E_UNSUPPORTED, __LINE__);
  }
  {
    // field by field rejections
    struct Case {
      int field, value, status;
    };
    const Case cases[] = {
        {0, 99, OKV_E_INVALID},          // abi_version
        {1, 0, OKV_E_INVALID},           // batch
        {1, -3, OKV_E_INVALID},
        {2, 7, OKV_E_INVALID},           // num_q_heads not a multiple of num_kv_heads
        {3, 0, OKV_E_INVALID},           // num_kv_heads
        {4, 96, OKV_E_INVALID},          // head_dim not a power of two
        {4, 64, OKV_E_UNSUPPORTED},
        {5, 1000, OKV_E_INVALID},        // max_tokens not a multiple of 32
        {5, 0, OKV_E_INVALID},
        {6, 24, OKV_E_INVALID},          // block does not divide d
        {6, 12, OKV_E_INVALID},          // 8 does not divide the block
        {6, 16, OKV_E_UNSUPPORTED},
        {7, 5, OKV_E_INVALID},           // quant
        {8, OKV_DT_BF16, OKV_E_INVALID}, // scale_dtype
        {8, OKV_DT_E4M3, OKV_E_UNSUPPORTED},
        {9, OKV_DT_F16, OKV_E_INVALID},  // in_dtype
        {10, 3, OKV_E_INVALID},          // rotation
        {11, 1, OKV_E_INVALID},          // bits
        {11, 5, OKV_E_INVALID},
        {11, -2147483647 - 1, OKV_E_INVALID},
    };
    for (const Case& k : cases) {
      okv_config c = base(s128);
      int32_t* f[] = {&c.abi_version, &c.batch, &c.num_q_heads, &c.num_kv_heads, &c.head_dim, &c.max_tokens,
                      &c.block, &c.quant, &c.scale_dtype, &c.in_dtype, &c.rotation, &c.bits};
      *f[k.field] = k.value;
      rejects(c, k.status, __LINE__ * 1000 + k.field);
    }
    okv_config c = base(s128);
    c.eps = -1.0f;
    rejects(c, OKV_E_INVALID, __LINE__);
    c.eps = std::nanf("");
    rejects(c, OKV_E_INVALID, __LINE__);
    c.eps = INFINITY;
    rejects(c, OKV_E_INVALID, __LINE__);
    c = base(s128);
    c.quant = OKV_QUANT_ASYM;   // asymmetric codes keep E4M3 pairs only
    rejects(c, OKV_E_UNSUPPORTED, __LINE__);
    c = base(s128);
    c.k_codes = nullptr;
    create_rejects(c, OKV_E_INVALID, __LINE__);
    c = base(s128);
    c.v_meta = reinterpret_cast<void*>(uintptr_t{0x40004});
    create_rejects(c, OKV_E_ALIGN, __LINE__);
    std::vector<float> bad = s128;
    bad[127] = 0.5f;            // a sign that is not +-1
    c = base(bad);
    create_rejects(c, OKV_E_INVALID, __LINE__);
    c = base(s128);
    c.rot_params = nullptr;
    create_rejects(c, OKV_E_INVALID, __LINE__);
    std::vector<float> so4(16 * 32, 0.0f);   // 2 I: not a rotation
    for (int i = 0; i < 32; ++i)
      for (int r = 0; r < 4; ++r) so4[16 * i + 5 * r] = 2.0f;
    c = base(so4);
    c.rotation = OKV_ROT_SO4;
    create_rejects(c, OKV_E_INVALID, __LINE__);
    okv_layout_info info{};
    EXPECT(okv_layout(nullptr, &info) == OKV_E_INVALID);
    EXPECT(okv_layout(&c, nullptr) == OKV_E_INVALID);
    c = base(s128);
    EXPECT(okv_create(&c, nullptr) == OKV_E_INVALID);
    EXPECT(okv_create(nullptr, nullptr) == OKV_E_INVALID);
  }
  {
    // calls on a null handle, and status strings
    int32_t n = 0, calls = 0;
    double a = 0.0, r = 0.0;
    EXPECT(okv_destroy(nullptr) == OKV_OK);
    EXPECT(okv_write(nullptr, nullptr, nullptr, 1, nullptr) == OKV_E_INVALID);
    EXPECT(okv_decode_attn(nullptr, nullptr, nullptr, nullptr) == OKV_E_INVALID);
    EXPECT(okv_decode_attn_noalloc(nullptr, nullptr, nullptr, nullptr) == OKV_E_INVALID);
    EXPECT(okv_prefill_attn(nullptr, nullptr, 1, nullptr, nullptr) == OKV_E_INVALID);
    EXPECT(okv_get_len(nullptr, &n) == OKV_E_INVALID);
    EXPECT(okv_set_len(nullptr, 0) == OKV_E_INVALID);
    EXPECT(okv_set_splits(nullptr, 4) == OKV_E_INVALID);
    EXPECT(okv_get_splits(nullptr, &n) == OKV_E_INVALID);
    EXPECT(okv_max_splits(nullptr, &n) == OKV_E_INVALID);
    EXPECT(okv_timing_enable(nullptr, 1) == OKV_E_INVALID);
    EXPECT(okv_timing_read(nullptr, &calls, &a, &r) == OKV_E_INVALID);
    EXPECT(okv_set_decode_kernel(nullptr, 0) == OKV_E_INVALID);
    EXPECT(okv_get_decode_kernel(nullptr, &n) == OKV_E_INVALID);
    for (int s = -2; s <= 7; ++s) EXPECT(okv_strerror(s) != nullptr && okv_strerror(s)[0] != '\0');
    EXPECT(okv_last_hip_error() != nullptr);
  }
  if (failures) {
    std::printf("%d failure(s)\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
