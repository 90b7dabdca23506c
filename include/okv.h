/*
 * okv -- Hadamard-rotated 3-bit KV cache for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library libokv.so.  Plain pointers and sizes only; every device
 * pointer is memory the caller allocated on the GPU the handle lives on.
 *
 * The method (pages: "Orthogonally mixed 3-bit KV cache", Mathematical statement,
 * Key formulas and Implementation notes; "Orthogonal Invariance in Activation
 * Space: Fast Walsh-Hadamard Transforms for KV Quantization", Sections 2.3, 3.1-3.4
 * and 4.3; "Hardware-Fused Fast Hadamard Transforms Enable Lossless 3-Bit KV-Cache
 * Compression at 128K Context Without Perplexity Drift", third paragraph):
 *
 *   write:  k1 = U k, v1 = U v; one scale per block of m values; b-bit codes
 *           (b = 3 in the pages' method; 2 and 4 are built too); 32 codes in 4 b
 *           bytes; only codes and scales are stored.
 *   decode: q1 = U q; logits from q1 and the dequantised rotated keys, unpacked
 *           and scaled inside the dot product; softmax; weighted sum of the
 *           dequantised rotated values; y = U^T y1.
 *
 *   U = H_d D  (OKV_ROT_SIGN: random signs D, then the normalised Walsh-Hadamard
 *               transform H_d)  or  U = B H_d  (OKV_ROT_SO4: H_d, then the
 *               block-diagonal SO(4) matrix B = diag(R_1 .. R_{d/4})).
 *
 * Quantisers (per block of m rotated values y; code width b, L = 2^(b-1) - 1):
 *   OKV_QUANT_SYM:   s = (max|y| + eps) / L rounded to float32 then to the scale
 *                    type; c = clip(round_half_even(y / s), -L, L); stored code
 *                    u = c + 2^(b-1) (1 .. 2^b - 1); y_hat = s (u - 2^(b-1)).
 *                    For b = 3: s = (max|y| + eps) / 3, u = c + 4.
 *   OKV_QUANT_ASYM:  s = (max - min) / (2^b - 1), z = min, both stored as OCP FP8
 *                    E4M3 (round-half-even, saturating at 448); u = clip(
 *                    round_half_even((y - z) / s), 0, 2^b - 1); y_hat = s u + z.
 * Every float32 step of the write path is rounded to nearest-even in a fixed order
 * (butterfly stages of stride 1, 2, 4, ..., d/2, then one multiply by
 * RN32(1/sqrt d); SO(4) rows as ((R0 x0 + R1 x1) + R2 x2) + R3 x3 without fused
 * multiply-adds), so codes and scales are reproducible bit for bit.
 *
 * Packing: 32 codes e[0..31] form a group of 4 b bytes, b little-endian 32-bit
 * words W0 .. W(b-1).
 *   b = 3: for k = 0,1,2 and byte j = 0..3: bits 0-2 of byte j of W_k hold e[8k+j]
 *          and bits 3-5 hold e[8k+4+j].  Bits 6-7 of byte j of W0 hold the low two
 *          bits of e[24+j], bits 6-7 of byte j of W1 the low two bits of e[28+j];
 *          bit 6 of byte j of W2 holds bit 2 of e[24+j] and bit 7 bit 2 of e[28+j].
 *   b = 4: byte j of W_k holds e[8k+j] in bits 0-3 and e[8k+4+j] in bits 4-7.
 *   b = 2: byte j of W_k holds e[16k+4f+j] in bits 2f, 2f+1 (f = 0..3).
 *
 * Cache layouts (caller-owned device buffers, row-major, contiguous):
 *   k_codes  uint8 [batch][num_kv_heads][max_tokens][b*head_dim/8]
 *            token-major rows; dims 32g..32g+31 are group g (bytes 4bg .. 4bg+4b-1).
 *   v_codes  uint8 [batch][num_kv_heads][max_tokens/32][head_dim][4b]
 *            32-token tiles; in tile t, dim j is one group holding the codes of
 *            tokens 32t .. 32t+31 (token 32t+i is code i).  Token slots of a
 *            tile that are not yet written hold code 0.
 *   k_meta, v_meta  [batch][num_kv_heads][max_tokens][head_dim/block] of the
 *            scale type (float32 or IEEE half) for OKV_QUANT_SYM, and
 *            uint8 [batch][num_kv_heads][max_tokens][head_dim/block][2] holding the
 *            E4M3 (scale, zero-point) pair for OKV_QUANT_ASYM.
 *   k, v     [batch][n_new][num_kv_heads][head_dim] in the input type.
 *   q        [batch][num_q_heads][head_dim] in the input type.
 *   out      float32 [batch][num_q_heads][head_dim].
 *   Query head j attends with key/value head j / (num_q_heads / num_kv_heads).
 *
 * Ownership: the caller owns every tensor buffer (cache, inputs, outputs) and
 * keeps the cache buffers alive until okv_destroy.  The handle owns a device copy
 * of the rotation parameters, the split-K workspace and the host-side sequence
 * length (uniform over the batch).
 *
 * Errors: every call returns an okv_status.  Arguments are checked before any
 * GPU work is queued; on error nothing is launched and no state changes.  No C++
 * exception crosses this interface.  Calls do not synchronise; they queue work on
 * the given HIP stream (NULL = the default stream).  The host side of a handle is
 * not thread-safe: call it from one thread at a time.  On the device, calls with one
 * handle on one stream are ordered; across streams the caller orders them as okv_write
 * states.
 */
#ifndef OKV_H
#define OKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OKV_ABI_VERSION 2

typedef enum okv_status {
  OKV_OK = 0,
  OKV_E_INVALID = 1,      /* bad configuration or argument */
  OKV_E_ALIGN = 2,        /* a pointer is not 16-byte aligned */
  OKV_E_CAPACITY = 3,     /* len + n_new > max_tokens */
  OKV_E_UNSUPPORTED = 4,  /* a valid combination this build does not implement */
  OKV_E_HIP = 5           /* HIP runtime or launch error */
} okv_status;

typedef enum okv_quant {
  OKV_QUANT_SYM = 0,
  OKV_QUANT_ASYM = 1,
  OKV_QUANT_SYM3 = OKV_QUANT_SYM,    /* the names of the 3-bit method */
  OKV_QUANT_ASYM3 = OKV_QUANT_ASYM
} okv_quant;

typedef enum okv_dtype {
  OKV_DT_F32 = 0,
  OKV_DT_F16 = 1,
  OKV_DT_BF16 = 2,
  OKV_DT_E4M3 = 3
} okv_dtype;

/* OKV_ROT_NONE: U = I, the unrotated baseline of the ablations (per-token or
 * per-block 3-bit codes of the raw vectors); rot_params is ignored and may be NULL. */
typedef enum okv_rotation { OKV_ROT_SIGN = 0, OKV_ROT_SO4 = 1, OKV_ROT_NONE = 2 } okv_rotation;

typedef struct okv_config {
  int32_t abi_version;   /* must be OKV_ABI_VERSION */
  int32_t batch;         /* sequences, >= 1; this build: <= 65535 (a launch grid dimension) */
  int32_t num_q_heads;   /* >= 1, multiple of num_kv_heads; this build: <= 65535 */
  int32_t num_kv_heads;  /* >= 1 */
  int32_t head_dim;      /* d: power of two, 4 | d; this build: 128 or 256 */
  int32_t max_tokens;    /* cache capacity per sequence, multiple of 32; this build:
                          * (max_tokens + 128) * bits * head_dim / 8 < 2^32 */
  int32_t block;         /* quantisation block m: m | d, 8 | m; this build: 32 | m */
  int32_t quant;         /* okv_quant */
  int32_t scale_dtype;   /* OKV_DT_F32 or OKV_DT_F16 (SYM); OKV_DT_E4M3 (ASYM) */
  int32_t in_dtype;      /* OKV_DT_F32 or OKV_DT_BF16: type of k, v and q */
  int32_t rotation;      /* okv_rotation */
  int32_t bits;          /* code width b: 2, 3 or 4 */
  float eps;             /* SYM scale offset, finite, >= 0 (1e-6 is usual) */
  /* Host pointer, copied at okv_create.  OKV_ROT_SIGN: head_dim values, each +1
   * or -1 (the diagonal of D; all +1 is the Hadamard-only variant).  OKV_ROT_SO4: (head_dim/4) row-major 4x4 float32
   * matrices R_i (rotation matrices: R^T R = I within 1e-3). */
  const float* rot_params;
  /* Caller-owned device buffers (layouts above), 16-byte aligned. */
  void* k_codes;
  void* v_codes;
  void* k_meta;
  void* v_meta;
} okv_config;

typedef struct okv_handle okv_handle;

/* Sizes in bytes of the four cache buffers a configuration needs (shape fields,
 * quant, scale_dtype are read; the pointers are not).  Returns OKV_E_INVALID or
 * OKV_E_UNSUPPORTED for configurations okv_create would reject. */
typedef struct okv_layout_info {
  uint64_t k_codes_bytes;
  uint64_t v_codes_bytes;
  uint64_t k_meta_bytes;
  uint64_t v_meta_bytes;
} okv_layout_info;

/* Validate cfg (host only, no GPU touched on failure), copy the rotation
 * parameters to the current device, allocate the split-K workspace there and
 * return a handle with sequence length 0.  The current HIP device at this call is
 * the device of the handle.  The handle fixes U once for every head and token, as
 * the idea card's Implementation notes draw the signs or SO(4) blocks once and keep
 * them (and the OIQ report, Section 3.2, generates D once per model); the cache it
 * describes starts empty, as the append-only key and value caches of those notes do.
 * *out is NULL on error. */
int okv_create(const okv_config* cfg, okv_handle** out);

/* Append n_new tokens to every sequence: rotate each new key and value vector by
 * U, quantise it blockwise, pack the codes and store codes and scales at positions
 * len .. len+n_new-1 (the write path of the idea card's Implementation notes).
 * k, v: device, [batch][n_new][kv][d] in the input type, 16-byte aligned.
 * Asynchronous on hip_stream; len advances by n_new at once (host side).
 * Ordering: it writes positions len .. len+n_new-1 and rewrites the earlier codes of
 * the current 32-token value tile unchanged (a read-modify-write of that tile), while
 * okv_decode_attn reads positions below its own len.  So
 *   - write after write: every okv_write must be ordered after the handle's previous
 *     okv_write (same stream, or an event wait): two writes into one value tile are a
 *     read-modify-write race;
 *   - write after decode: a write may run on another stream concurrently with a decode
 *     enqueued before it (the decode never reads the new positions);
 *   - decode after write: the next decode must be ordered after the write. */
int okv_write(okv_handle* h, const void* k, const void* v, int32_t n_new, void* hip_stream);

/* One decode step: for every (sequence, query head) attend over all len cached
 * tokens and write the float32 output (the idea card, Implementation notes: read
 * path).  q: device [batch][num_q_heads][d] in the input type; out: device
 * float32 [batch][num_q_heads][d]; both 16-byte aligned.  OKV_E_INVALID when the
 * cache is empty.  Asynchronous on hip_stream. */
int okv_decode_attn(okv_handle* h, const void* q, float* out, void* hip_stream);

/* okv_decode_attn without any device allocation, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and split count, the same output bit for bit, but the split-K
 * partials go to a static device scratch of 16 MiB (4,194,304 floats) that the library
 * holds on each GPU it runs on until the process ends, instead of the handle's
 * workspace.  It needs batch * num_q_heads * splits * (head_dim + 2) floats (splits:
 * okv_get_splits); beyond 16 MiB it returns OKV_E_CAPACITY and launches nothing.  The
 * scratch's address on a device is looked up by okv_create on that device; OKV_E_HIP if
 * that failed.  Every call on one GPU shares that GPU's scratch and leaves the last
 * call's partials in it: calls of this function that overlap on one GPU (other streams,
 * other handles, other threads) race and must be ordered by the caller.  Arguments and
 * the other errors as okv_decode_attn. */
int okv_decode_attn_noalloc(okv_handle* h, const void* q, float* out, void* hip_stream);

/* Prefill attention: the last n_q cached positions of every sequence (len - n_q ..
 * len - 1, already appended by okv_write) attend causally over the cache: the row at
 * position p sees tokens 0 .. p, its own included.  Each row is the read path of
 * okv_decode_attn over that prefix (the idea card, Implementation notes: read path,
 * and Key formulas, with a causal mask; the OIQ report, Section 2.3).  Keys and
 * values are unpacked from the cache inside the kernel (codes as exact float16
 * integers in LDS, block scales applied in float32; nothing dequantised is written
 * to memory).  q: device [batch][n_q][num_q_heads][d] in the input type; out:
 * device float32 [batch][n_q][num_q_heads][d]; both 16-byte aligned, and out must not
 * overlap q or the cache: on prefixes of more than 65,536 tokens the kernel also keeps
 * partial P.V sums of its rows in out before it writes the result there.  1 <= n_q <=
 * len, else OKV_E_INVALID.  Asynchronous on hip_stream. */
int okv_prefill_attn(okv_handle* h, const void* q, int32_t n_q, float* out, void* hip_stream);

/* SO(4) calibration (the idea card, Implementation notes: start from fixed random
 * rotations and calibrate them on representative vectors by minimising the
 * reconstruction MSE after 3-bit quantisation, each SO(4) block a quaternion pair).
 * Objective: the summed squared error of y = B (H x) after symmetric b-bit
 * quantisation (s = (max|y| + eps) / (2^(b-1) - 1) per block of `block` dims, codes
 * round-half-even, clipped) over the n calibration vectors x.  Search: sweeps over the
 * groups g = 0 .. head_dim/4 - 1 in order; candidate c of (sweep, g) gives
 * R_g' = cand[s][g][c] R_g, and R_g takes the candidate with the smallest error of
 * the quantisation block holding g (the first one on ties; candidate 0 should be the
 * identity, so the error never increases).
 *   x      device float32 [n][head_dim], 16-byte aligned (e.g. keys in input space)
 *   rot    host float32 [head_dim/4][4][4] row-major: in the start, out the result
 *   cand   host float32 [sweeps][head_dim/4][n_cand][4][4]
 *   trace  host double [sweeps + 1] (NULL allowed): total error before and after each
 *          sweep
 * head_dim 128 or 256; 4 | block, block | head_dim; bits 2..4; eps finite >= 0;
 * 1 <= n_cand <= 1024; n * head_dim < 2^31.  Allocates and frees its own device
 * workspace and a pinned host staging buffer for rot and cand; runs on hip_stream and
 * returns when done. */
int okv_so4_calibrate(const float* x, int32_t n, int32_t head_dim, int32_t block, int32_t bits, float eps,
                      float* rot, const float* cand, int32_t sweeps, int32_t n_cand, double* trace,
                      void* hip_stream);

/* One step of that search: err[c] (host double [n_cand]) = error of the quantisation
 * block holding group `group` with R_group replaced by cand[c] R_group (cand: host
 * float32 [n_cand][4][4]; rot as above, not changed).  Synchronous. */
int okv_so4_eval(const float* x, int32_t n, int32_t head_dim, int32_t block, int32_t bits, float eps,
                 const float* rot, const float* cand, int32_t n_cand, int32_t group, double* err,
                 void* hip_stream);

/* Release a handle: free its device copy of U and its split-K workspace (not the
 * caller's cache buffers, which keep the codes written so far).  The end of the
 * append-only cache's life in the idea card's Implementation notes; nothing of the
 * method runs here.  Work already queued with the handle must have finished (the call
 * does not wait for it).  NULL is OK; OKV_E_HIP if a device free fails (the handle is
 * released anyway). */
int okv_destroy(okv_handle* h);

/* ---- auxiliary calls (not part of the method) ---- */

const char* okv_strerror(int status);
/* Text of the HIP runtime error behind the last OKV_E_HIP returned on the calling
 * thread ("none" if there was none).  Static storage; not cleared by later calls. */
const char* okv_last_hip_error(void);
int okv_layout(const okv_config* cfg, okv_layout_info* info);
/* Current sequence length of the handle. */
int okv_get_len(const okv_handle* h, int32_t* len);
/* Set the sequence length to 0..max_tokens (e.g. 0 to reuse the buffers); the
 * cache contents below the new length are taken as written. */
int okv_set_len(okv_handle* h, int32_t len);
/* Split-K count of okv_decode_attn: 0 chooses automatically (default), otherwise
 * 1 .. okv_max_splits. */
int okv_set_splits(okv_handle* h, int32_t num_splits);
int okv_max_splits(const okv_handle* h, int32_t* n);
/* Split count the next okv_decode_attn call will use at the current length. */
int okv_get_splits(const okv_handle* h, int32_t* n);
/* Kernel timing: when enabled, okv_decode_attn records HIP events on its stream
 * attached to the dispatch of its attention kernel and of its reduce kernel (so the
 * elapsed times are the kernels' own).  okv_timing_read waits for the
 * recorded calls, returns how many were recorded since the last read and the
 * summed kernel milliseconds, then clears the record. */
int okv_timing_enable(okv_handle* h, int32_t enable);
int okv_timing_read(okv_handle* h, int32_t* calls, double* attn_ms, double* reduce_ms);

/* Attention kernel of okv_decode_attn.  OKV_DECODE_PER_HEAD: one workgroup per
 * (split, sequence, query head) reads the packed cache of its KV head.
 * OKV_DECODE_GROUPED: one workgroup per (split, sequence, KV head) reads the packed
 * cache once for the whole query group and computes Q.K and P.V on int8 matrix
 * cores; built for query groups of 2, 4 and 8 with blocks of 32, 64 and 128 dims.
 * OKV_DECODE_AUTO (default) takes the grouped kernel where it is built, else the
 * per-head one.  okv_set_decode_kernel returns OKV_E_UNSUPPORTED for
 * OKV_DECODE_GROUPED on other configurations; okv_get_decode_kernel reports the
 * kernel the next call will use (PER_HEAD or GROUPED). */
typedef enum okv_decode_kernel {
  OKV_DECODE_AUTO = 0,
  OKV_DECODE_PER_HEAD = 1,
  OKV_DECODE_GROUPED = 2
} okv_decode_kernel;
int okv_set_decode_kernel(okv_handle* h, int32_t kind);
int okv_get_decode_kernel(const okv_handle* h, int32_t* kind);

/* Streaming-read probe: one pass over `bytes` bytes of the device buffer buf with
 * 16-byte non-temporal loads, eight in flight per lane (grid-stride over 64 workgroups
 * of 256 threads per compute unit), the HBM read rate a plain streaming kernel
 * reaches, for comparison with the decode kernels.  buf:
 * device, 16-byte aligned, bytes >= 16 (the last bytes % 16 are not read); sink:
 * device uint32, written only when the loads' checksum hits a fixed value (it keeps
 * the loads from being removed).  Asynchronous on hip_stream; no handle needed. */
int okv_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* OKV_H */
