// C ABI of the INT4 paged KV-cache library: argument validation and dispatch.
// Every host-checkable problem is reported before anything is enqueued.
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <set>
#include <utility>

#include "../../include/int4kv.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

// Split-K partials of int4_paged_attention_noalloc: a fixed device array,
// one copy per GPU, held until the process ends.  Host code never passes its
// name to a kernel (on the host it is only a stand-in symbol): the device
// address is looked up once per device with hipGetSymbolAddress.
constexpr size_t kNoallocScratchFloats = INT4KV_NOALLOC_SCRATCH_BYTES / sizeof(float);
static __device__ __align__(256) float scratch[kNoallocScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (nullptr and an error on failure).
hipError_t scratch_for_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// floats of each split-K partials array rounded up to 64 (256 bytes)
int64_t round64(int64_t n) { return (n + 63) / 64 * 64; }

int4kv_status_t fail(int4kv_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

int4kv_status_t ok() {
  g_last_error[0] = '\0';
  return INT4KV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Split-count heuristic of the decode path.  A decode workgroup holds a whole
// CU (256 on MI355X), so a grid of W workgroups runs in ceil(W / 256) rounds,
// each as long as one workgroup: a fixed start (the query prologue and the
// ring's first copies, about 3 tiles' time) plus its segment's tiles; a split
// adds the segment reduction (about 3 tiles' time).  The count minimises
//   rounds(ns) * (3 + tiles / ns) + (ns > 1 ? 3 : 0)
// over ns in [1, tiles / 2] (no segment shorter than 2 tiles of 32 keys),
// ties to the smaller count.  It picks the fastest measured counts: 64 for
// the long-context decode, 4 for the Llama-3-shaped one (2 with the INT8
// kernel's 4-head workgroups), 16 for 8 sequences of up to 1024 keys (36.5 us
// at 1 segment, 15 at 8, 14 at 16), and 2 rather than 3 for 100 sequences of
// 512-640 keys (3 segments make 300 workgroups: a second round of 44).
constexpr int64_t kDecodeCUs = 256;
constexpr int64_t kDecodeMinTilesPerSegment = 2;
constexpr double kDecodeStartTiles = 3.0, kDecodeReduceTiles = 3.0;

// the split-count rule for workgroups of up to `hpw_cap` KV heads (8 for the
// INT4 decode kernel, 4 for the INT8 one)
int32_t decode_num_segments(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seqlen_k,
                            int hpw_cap) {
  if (num_seqs < 1 || num_kv_heads < 1 || max_seqlen_k < 1) return 1;
  // KV heads per workgroup of the decode kernels
  int hpw = hpw_cap;
  const int hkv = num_kv_heads;
  if (hkv < hpw_cap && (hkv == 1 || hkv == 2 || hkv == 4))
    hpw = hkv;
  else if (hkv % hpw_cap != 0)
    while (hkv % hpw) hpw >>= 1;
  const int64_t wgs = (int64_t)num_seqs * (hkv / hpw);  // workgroups per segment index
  const int64_t tiles = ((int64_t)max_seqlen_k + 31) / 32;  // 32-key tiles of the longest sequence
  int64_t cap = tiles / kDecodeMinTilesPerSegment;
  if (cap > 256) cap = 256;
  int64_t best = 1;
  double best_cost = 0.0;
  for (int64_t ns = 1; ns <= (cap > 1 ? cap : 1); ++ns) {
    const double rounds = (double)((ns * wgs + kDecodeCUs - 1) / kDecodeCUs);
    const double cost = rounds * (kDecodeStartTiles + (double)tiles / (double)ns) +
                        (ns > 1 ? kDecodeReduceTiles : 0.0);
    if (ns == 1 || cost < best_cost) {
      best = ns;
      best_cost = cost;
    }
  }
  return (int32_t)best;
}

int4kv_status_t check_common(const void* cache, int32_t num_blocks, int32_t block_size,
                             int32_t num_kv_heads, int32_t head_size, const float* signs) {
  if (!cache || !signs) return fail(INT4KV_ERR_INVALID_ARG, "null cache or rht_signs pointer");
  if (num_blocks < 1 || num_kv_heads < 1)
    return fail(INT4KV_ERR_INVALID_ARG, "num_blocks (%d) and num_kv_heads (%d) must be >= 1",
                num_blocks, num_kv_heads);
  if (head_size != 64 && head_size != 128)
    return fail(INT4KV_ERR_UNSUPPORTED, "head_size %d: supported sizes are 64 and 128", head_size);
  if (block_size != 16)
    return fail(INT4KV_ERR_UNSUPPORTED, "block_size %d: only 16 is supported", block_size);
  if (!aligned16(cache) || !aligned16(signs))
    return fail(INT4KV_ERR_INVALID_ARG, "cache and rht_signs must be 16-byte aligned");
  return INT4KV_OK;
}

int4kv_status_t check_write_inputs(const void* key, int64_t key_token_stride, const void* value,
                                   int64_t value_token_stride, const int64_t* slot_mapping,
                                   int32_t num_kv_heads, int32_t head_size) {
  if (!key || !value || !slot_mapping)
    return fail(INT4KV_ERR_INVALID_ARG, "null key, value or slot_mapping pointer");
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_token_stride < row || value_token_stride < row)
    return fail(INT4KV_ERR_INVALID_ARG, "token strides (%lld, %lld) smaller than heads*head_size %lld",
                (long long)key_token_stride, (long long)value_token_stride, (long long)row);
  if ((key_token_stride % 8) || (value_token_stride % 8) || !aligned16(key) || !aligned16(value))
    return fail(INT4KV_ERR_INVALID_ARG,
                "key/value must be 16-byte aligned with token strides a multiple of 8 elements");
  return INT4KV_OK;
}

// Validates the attention arguments (after check_common) and fills `a`.
int4kv_status_t check_attention(const void* q, int64_t q_token_stride, void* out,
                                int4kv_dtype_t dtype, const uint8_t* kv_cache,
                                int32_t num_kv_heads, int32_t head_size, int32_t num_q_heads,
                                const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const int32_t* block_table, int32_t block_table_stride,
                                int32_t block_size, float softmax_scale, int32_t sliding_window,
                                float softcap, const float* rht_signs, int32_t num_segments,
                                float* segm_output, float* segm_max, float* segm_expsum,
                                int4kv::AttnArgs& a, bool internal_workspace = false) {
  if (!q || !out || !cu_seqlens_q || !seqused_k || !block_table)
    return fail(INT4KV_ERR_INVALID_ARG, "null q, out, cu_seqlens_q, seqused_k or block_table");
  if (num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(INT4KV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(INT4KV_ERR_UNSUPPORTED, "query heads per KV head %d: supported 1, 2, 4, 8, 16", G);
  if (q_token_stride < (int64_t)num_q_heads * head_size || (q_token_stride % 8) || !aligned16(q) ||
      !aligned16(out))
    return fail(INT4KV_ERR_INVALID_ARG,
                "q token stride %lld must be >= heads*head_size and a multiple of 8; q and out "
                "16-byte aligned", (long long)q_token_stride);
  if (block_table_stride < (max_seqlen_k + block_size - 1) / block_size)
    return fail(INT4KV_ERR_INVALID_ARG, "block_table_stride %d < ceil(max_seqlen_k / block_size)",
                block_table_stride);
  if (num_segments < 1) return fail(INT4KV_ERR_INVALID_ARG, "num_segments %d < 1", num_segments);
  if (!std::isfinite(softmax_scale))
    return fail(INT4KV_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (std::isnan(softcap) || std::isinf(softcap) ||
      (softcap > 0.f && !std::isfinite(1.0f / (softcap * 1.4426950408889634f))))
    return fail(INT4KV_ERR_INVALID_ARG, "softcap must be finite, and > 0 only with a finite "
                "reciprocal");
  const bool decode = max_seqlen_q == 1;
  if (decode && num_segments > 1 && !internal_workspace &&
      (!segm_output || !segm_max || !segm_expsum))
    return fail(INT4KV_ERR_WORKSPACE, "num_segments %d > 1 needs the three segment buffers",
                num_segments);
  if (num_segments > 65535) return fail(INT4KV_ERR_INVALID_ARG, "num_segments too large");
  if (num_seqs > 65535 || num_kv_heads > 65535)
    return fail(INT4KV_ERR_UNSUPPORTED, "num_seqs and num_kv_heads are limited to 65535");
  a = int4kv::AttnArgs{q, q_token_stride, out, dtype == INT4KV_BF16, kv_cache, num_kv_heads,
                       head_size, num_q_heads, cu_seqlens_q, seqused_k, num_seqs, max_seqlen_q,
                       max_seqlen_k, block_table, block_table_stride, softmax_scale, rht_signs,
                       decode ? num_segments : 1, segm_output, segm_max, segm_expsum};
  a.window = sliding_window > 0 ? sliding_window : 0;
  a.softcap = softcap > 0.f ? softcap : 0.f;
  return INT4KV_OK;
}

}  // namespace

namespace int4kv {

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> raised;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (raised.count({kernel, dev})) return hipSuccess;
  }
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  raised.insert({kernel, dev});
  return hipSuccess;
}

}  // namespace int4kv

extern "C" {

int64_t int4kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size) {
  if (num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_size < 2 || (head_size & 1))
    return -1;
  return (int64_t)num_blocks * 2 * block_size * num_kv_heads * (head_size / 2 + 4);
}

const char* int4kv_status_string(int4kv_status_t s) {
  switch (s) {
    case INT4KV_OK: return "INT4KV_OK";
    case INT4KV_ERR_INVALID_ARG: return "INT4KV_ERR_INVALID_ARG";
    case INT4KV_ERR_UNSUPPORTED: return "INT4KV_ERR_UNSUPPORTED";
    case INT4KV_ERR_WORKSPACE: return "INT4KV_ERR_WORKSPACE";
    case INT4KV_ERR_LAUNCH: return "INT4KV_ERR_LAUNCH";
  }
  return "INT4KV_ERR_UNKNOWN";
}

const char* int4kv_last_error(void) { return g_last_error; }

int32_t int4kv_decode_num_segments(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seqlen_k) {
  return decode_num_segments(num_seqs, num_kv_heads, max_seqlen_k, 8);
}

int32_t int8kv_decode_num_segments(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seqlen_k) {
  return decode_num_segments(num_seqs, num_kv_heads, max_seqlen_k, 4);
}

int4kv_status_t int4_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, const float* rht_signs, void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_tokens < 0) return fail(INT4KV_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  s = check_write_inputs(key, key_token_stride, value, value_token_stride, slot_mapping,
                         num_kv_heads, head_size);
  if (s != INT4KV_OK) return s;
  hipError_t e = int4kv::launch_write(key, key_token_stride, value, value_token_stride,
                                      dtype == INT4KV_BF16, slot_mapping, num_tokens, kv_cache,
                                      (int64_t)num_blocks * block_size, num_kv_heads, head_size,
                                      rht_signs,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "write launch: %s", hipGetErrorString(e));
  return ok();
}

int64_t int8kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size) {
  if (num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_size < 1) return -1;
  return (int64_t)num_blocks * 2 * block_size * num_kv_heads * (head_size + 4);
}

int4kv_status_t int8_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, void* stream) {
  if (!kv_cache) return fail(INT4KV_ERR_INVALID_ARG, "null cache pointer");
  if (num_blocks < 1 || num_kv_heads < 1)
    return fail(INT4KV_ERR_INVALID_ARG, "num_blocks (%d) and num_kv_heads (%d) must be >= 1",
                num_blocks, num_kv_heads);
  if (head_size != 64 && head_size != 128)
    return fail(INT4KV_ERR_UNSUPPORTED, "head_size %d: supported sizes are 64 and 128", head_size);
  if (block_size != 16)
    return fail(INT4KV_ERR_UNSUPPORTED, "block_size %d: only 16 is supported", block_size);
  if (!aligned16(kv_cache)) return fail(INT4KV_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_tokens < 0) return fail(INT4KV_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  int4kv_status_t s = check_write_inputs(key, key_token_stride, value, value_token_stride,
                                         slot_mapping, num_kv_heads, head_size);
  if (s != INT4KV_OK) return s;
  hipError_t e = int4kv::launch_write_int8(key, key_token_stride, value, value_token_stride,
                                           dtype == INT4KV_BF16, slot_mapping, num_tokens,
                                           kv_cache, (int64_t)num_blocks * block_size,
                                           num_kv_heads, head_size,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "write launch: %s", hipGetErrorString(e));
  return ok();
}

int64_t int2kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size) {
  if (num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_size < 4 || head_size % 4)
    return -1;
  return (int64_t)num_blocks * 2 * block_size * num_kv_heads * (head_size / 4 + 4);
}

int4kv_status_t int2_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, const float* rht_signs, void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_tokens < 0) return fail(INT4KV_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  s = check_write_inputs(key, key_token_stride, value, value_token_stride, slot_mapping,
                         num_kv_heads, head_size);
  if (s != INT4KV_OK) return s;
  hipError_t e = int4kv::launch_write_int2(key, key_token_stride, value, value_token_stride,
                                           dtype == INT4KV_BF16, slot_mapping, num_tokens,
                                           kv_cache, (int64_t)num_blocks * block_size,
                                           num_kv_heads, head_size, rht_signs,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "write launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int2_paged_attention(const void* q, int64_t q_token_stride, void* out,
                                     int4kv_dtype_t dtype, const uint8_t* kv_cache,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t num_kv_heads, int32_t head_size,
                                     int32_t num_q_heads, const int32_t* cu_seqlens_q,
                                     const int32_t* seqused_k, int32_t num_seqs,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     const int32_t* block_table, int32_t block_table_stride,
                                     float softmax_scale, int32_t sliding_window, float softcap,
                                     const float* rht_signs, int32_t num_segments,
                                     float* segm_output, float* segm_max, float* segm_expsum,
                                     void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(INT4KV_ERR_INVALID_ARG, "negative num_seqs / max_seqlen_q / max_seqlen_k");
  if (num_seqs == 0 || max_seqlen_q == 0) return ok();
  const bool decode = max_seqlen_q == 1;
  int4kv::AttnArgs a;
  s = check_attention(q, q_token_stride, out, dtype, kv_cache, num_kv_heads, head_size,
                      num_q_heads, cu_seqlens_q, seqused_k, num_seqs, max_seqlen_q, max_seqlen_k,
                      block_table, block_table_stride, block_size, softmax_scale, sliding_window,
                      softcap, rht_signs, num_segments, segm_output, segm_max, segm_expsum, a);
  if (s != INT4KV_OK) return s;
  if (decode && !int4kv::decode_lds_supported(a))
    return fail(INT4KV_ERR_UNSUPPORTED,
                "INT2 decode: num_kv_heads %d must be 1, 2, 4 or a multiple of 8", num_kv_heads);
  a.q2 = true;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = decode ? int4kv::launch_decode_lds(a, st) : int4kv::launch_prefill(a, st);
  if (e != hipSuccess)
    return fail(INT4KV_ERR_LAUNCH, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int8_paged_attention(const void* q, int64_t q_token_stride, void* out,
                                     int4kv_dtype_t dtype, const uint8_t* kv_cache,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t num_kv_heads, int32_t head_size,
                                     int32_t num_q_heads, const int32_t* cu_seqlens_q,
                                     const int32_t* seqused_k, int32_t num_seqs,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     const int32_t* block_table, int32_t block_table_stride,
                                     float softmax_scale, int32_t sliding_window, float softcap,
                                     int32_t num_segments, float* segm_output, float* segm_max,
                                     float* segm_expsum, void* stream) {
  if (!kv_cache) return fail(INT4KV_ERR_INVALID_ARG, "null cache pointer");
  if (num_blocks < 1 || num_kv_heads < 1)
    return fail(INT4KV_ERR_INVALID_ARG, "num_blocks (%d) and num_kv_heads (%d) must be >= 1",
                num_blocks, num_kv_heads);
  if (head_size != 64 && head_size != 128)
    return fail(INT4KV_ERR_UNSUPPORTED, "head_size %d: supported sizes are 64 and 128", head_size);
  if (block_size != 16)
    return fail(INT4KV_ERR_UNSUPPORTED, "block_size %d: only 16 is supported", block_size);
  if (!aligned16(kv_cache)) return fail(INT4KV_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(INT4KV_ERR_INVALID_ARG, "negative num_seqs / max_seqlen_q / max_seqlen_k");
  if (num_seqs == 0 || max_seqlen_q == 0) return ok();
  const bool decode = max_seqlen_q == 1;
  // the decode kernel's workgroups take 1, 2 or 4 KV heads
  if (decode && !(num_kv_heads == 1 || num_kv_heads == 2 || num_kv_heads % 4 == 0))
    return fail(INT4KV_ERR_UNSUPPORTED,
                "INT8 decode: num_kv_heads %d must be 1, 2 or a multiple of 4", num_kv_heads);
  int4kv::AttnArgs a;
  int4kv_status_t s = check_attention(q, q_token_stride, out, dtype, kv_cache, num_kv_heads,
                                      head_size, num_q_heads, cu_seqlens_q, seqused_k, num_seqs,
                                      max_seqlen_q, max_seqlen_k, block_table, block_table_stride,
                                      block_size, softmax_scale, sliding_window, softcap, nullptr,
                                      num_segments, segm_output, segm_max, segm_expsum, a);
  if (s != INT4KV_OK) return s;
  a.q8 = true;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = decode ? int4kv::launch_decode_lds(a, st) : int4kv::launch_prefill(a, st);
  if (e != hipSuccess)
    return fail(INT4KV_ERR_LAUNCH, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int4_paged_attention(const void* q, int64_t q_token_stride, void* out,
                                     int4kv_dtype_t dtype, const uint8_t* kv_cache,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t num_kv_heads, int32_t head_size,
                                     int32_t num_q_heads, const int32_t* cu_seqlens_q,
                                     const int32_t* seqused_k, int32_t num_seqs,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     const int32_t* block_table, int32_t block_table_stride,
                                     float softmax_scale, int32_t sliding_window,
                                     float softcap, const float* rht_signs,
                                     int32_t num_segments,
                                     float* segm_output, float* segm_max, float* segm_expsum,
                                     void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(INT4KV_ERR_INVALID_ARG, "negative num_seqs / max_seqlen_q / max_seqlen_k");
  if (num_seqs == 0 || max_seqlen_q == 0) return ok();
  int4kv::AttnArgs a;
  s = check_attention(q, q_token_stride, out, dtype, kv_cache, num_kv_heads, head_size,
                      num_q_heads, cu_seqlens_q, seqused_k, num_seqs, max_seqlen_q, max_seqlen_k,
                      block_table, block_table_stride, block_size, softmax_scale, sliding_window,
                      softcap, rht_signs, num_segments, segm_output, segm_max, segm_expsum, a);
  if (s != INT4KV_OK) return s;
  const bool decode = max_seqlen_q == 1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = decode ? int4kv::launch_decode(a, st) : int4kv::launch_prefill(a, st);
  if (e != hipSuccess)
    return fail(INT4KV_ERR_LAUNCH, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int4_paged_attention_noalloc(const void* q, int64_t q_token_stride, void* out,
                                             int4kv_dtype_t dtype, const uint8_t* kv_cache,
                                             int32_t num_blocks, int32_t block_size,
                                             int32_t num_kv_heads, int32_t head_size,
                                             int32_t num_q_heads, const int32_t* cu_seqlens_q,
                                             const int32_t* seqused_k, int32_t num_seqs,
                                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                                             const int32_t* block_table,
                                             int32_t block_table_stride, float softmax_scale,
                                             int32_t sliding_window, float softcap,
                                             const float* rht_signs, int32_t num_segments,
                                             void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(INT4KV_ERR_INVALID_ARG, "negative num_seqs / max_seqlen_q / max_seqlen_k");
  if (num_seqs == 0 || max_seqlen_q == 0) return ok();
  int4kv::AttnArgs a;
  s = check_attention(q, q_token_stride, out, dtype, kv_cache, num_kv_heads, head_size,
                      num_q_heads, cu_seqlens_q, seqused_k, num_seqs, max_seqlen_q, max_seqlen_k,
                      block_table, block_table_stride, block_size, softmax_scale, sliding_window,
                      softcap, rht_signs, num_segments, nullptr, nullptr, nullptr, a,
                      /*internal_workspace=*/true);
  if (s != INT4KV_OK) return s;
  const bool split = max_seqlen_q == 1 && num_segments > 1;
  // partials: [S, Hq, NS, d] outputs, then [S, Hq, NS] maxima and exp-sums
  const int64_t rows = (int64_t)num_seqs * num_q_heads * (num_segments > 0 ? num_segments : 1);
  const int64_t need = split ? round64(rows * head_size) + 2 * round64(rows) : 0;
  if (need > (int64_t)kNoallocScratchFloats)
    return fail(INT4KV_ERR_WORKSPACE,
                "split-K partials of %lld bytes exceed the library's fixed %lld-byte buffer "
                "(num_seqs * num_q_heads * num_segments * (head_size + 2) floats); use fewer "
                "segments or int4_paged_attention with caller-owned buffers",
                (long long)(need * 4), (long long)INT4KV_NOALLOC_SCRATCH_BYTES);
  if (split) {
    float* base = nullptr;
    hipError_t e = scratch_for_current_device(&base);
    if (e != hipSuccess)
      return fail(INT4KV_ERR_LAUNCH, "device scratch lookup: %s", hipGetErrorString(e));
    a.segm_out = base;
    a.segm_max = base + round64(rows * head_size);
    a.segm_sum = a.segm_max + round64(rows);
  } else {
    a.segm_out = a.segm_max = a.segm_sum = nullptr;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = max_seqlen_q == 1 ? int4kv::launch_decode(a, st) : int4kv::launch_prefill(a, st);
  if (e != hipSuccess)
    return fail(INT4KV_ERR_LAUNCH, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int4kv_stream_rw(const void* src, int64_t read_bytes, void* dst,
                                 int64_t write_bytes, void* stream) {
  if (read_bytes < 0 || write_bytes < 0 || (read_bytes % 16) || (write_bytes % 16))
    return fail(INT4KV_ERR_INVALID_ARG, "byte counts must be non-negative multiples of 16");
  if ((read_bytes && (!src || !aligned16(src))) || (write_bytes && (!dst || !aligned16(dst))))
    return fail(INT4KV_ERR_INVALID_ARG, "src and dst must be non-null and 16-byte aligned");
  if (read_bytes > 0 && write_bytes == 0)
    return fail(INT4KV_ERR_INVALID_ARG, "reads need at least one written unit to land in");
  if (write_bytes == 0) return ok();
  hipError_t e = int4kv::launch_stream_rw(src, read_bytes, dst, write_bytes,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "stream launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int4kv_stream_blocks(const uint8_t* cache, int64_t block_bytes,
                                     const int32_t* block_ids, int64_t num_ids,
                                     int32_t num_workgroups, void* stream) {
  if (num_ids < 0 || num_workgroups < 1)
    return fail(INT4KV_ERR_INVALID_ARG, "num_ids (%lld) must be >= 0 and num_workgroups (%d) >= 1",
                (long long)num_ids, num_workgroups);
  if (block_bytes < 1024 || block_bytes > 20480 || block_bytes % 1024)
    return fail(INT4KV_ERR_INVALID_ARG,
                "block_bytes %lld must be a multiple of 1024 in [1024, 20480]",
                (long long)block_bytes);
  if (num_ids == 0) return ok();
  if (num_ids % (2 * (int64_t)num_workgroups))
    return fail(INT4KV_ERR_INVALID_ARG,
                "num_ids %lld must be a multiple of 2 * num_workgroups (%d)",
                (long long)num_ids, 2 * num_workgroups);
  if (!cache || !aligned16(cache) || !block_ids)
    return fail(INT4KV_ERR_INVALID_ARG, "cache (16-byte aligned) and block_ids must be non-null");
  hipError_t e = int4kv::launch_stream_blocks(cache, block_bytes, block_ids, num_ids,
                                              num_workgroups, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "stream launch: %s", hipGetErrorString(e));
  return ok();
}

int4kv_status_t int4_decode_step(const void* key_new, int64_t key_token_stride,
                                 const void* value_new, int64_t value_token_stride,
                                 const int64_t* slot_mapping, const void* q,
                                 int64_t q_token_stride, void* out, int4kv_dtype_t dtype,
                                 uint8_t* kv_cache, int32_t num_blocks, int32_t block_size,
                                 int32_t num_kv_heads, int32_t head_size, int32_t num_q_heads,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 const int32_t* block_table, int32_t block_table_stride,
                                 float softmax_scale, int32_t sliding_window, float softcap,
                                 const float* rht_signs, int32_t num_segments,
                                 float* segm_output, float* segm_max, float* segm_expsum,
                                 void* stream) {
  int4kv_status_t s =
      check_common(kv_cache, num_blocks, block_size, num_kv_heads, head_size, rht_signs);
  if (s != INT4KV_OK) return s;
  if (dtype != INT4KV_F16 && dtype != INT4KV_BF16)
    return fail(INT4KV_ERR_INVALID_ARG, "dtype %d is neither F16 nor BF16", (int)dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(INT4KV_ERR_INVALID_ARG, "negative num_seqs / max_seqlen_q / max_seqlen_k");
  if (num_seqs == 0) return ok();
  s = check_write_inputs(key_new, key_token_stride, value_new, value_token_stride, slot_mapping,
                         num_kv_heads, head_size);
  if (s != INT4KV_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = dtype == INT4KV_BF16;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (max_seqlen_q == 0) {  // nothing to attend: the write alone
    hipError_t e = int4kv::launch_write(key_new, key_token_stride, value_new, value_token_stride,
                                        bf16, slot_mapping, num_seqs, kv_cache, num_slots,
                                        num_kv_heads, head_size, rht_signs, st);
    if (e != hipSuccess) return fail(INT4KV_ERR_LAUNCH, "write launch: %s", hipGetErrorString(e));
    return ok();
  }
  int4kv::AttnArgs a;
  s = check_attention(q, q_token_stride, out, dtype, kv_cache, num_kv_heads, head_size,
                      num_q_heads, cu_seqlens_q, seqused_k, num_seqs, max_seqlen_q, max_seqlen_k,
                      block_table, block_table_stride, block_size, softmax_scale, sliding_window,
                      softcap, rht_signs, num_segments, segm_output, segm_max, segm_expsum, a);
  if (s != INT4KV_OK) return s;
  hipError_t e;
  if (max_seqlen_q == 1 && int4kv::decode_lds_supported(a)) {
    a.key_new = key_new;
    a.key_new_stride = key_token_stride;
    a.value_new = value_new;
    a.value_new_stride = value_token_stride;
    a.slot_new = slot_mapping;
    a.num_slots = num_slots;
    e = int4kv::launch_decode_lds(a, st);
  } else {  // the same result as two calls: the write, then the attention
    e = int4kv::launch_write(key_new, key_token_stride, value_new, value_token_stride, bf16,
                             slot_mapping, num_seqs, kv_cache, num_slots, num_kv_heads,
                             head_size, rht_signs, st);
    if (e == hipSuccess)
      e = max_seqlen_q == 1 ? int4kv::launch_decode(a, st) : int4kv::launch_prefill(a, st);
  }
  if (e != hipSuccess)
    return fail(INT4KV_ERR_LAUNCH, "decode step launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
