// Host-side launchers of the INT4 KV-cache kernels (internal to the library).
// The write kernels store a token only when its slot lies in [0, num_slots),
// num_slots = num_blocks * block_size: negative slots are the pages' "skip"
// marker, and larger ones would address memory past the cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int4kv {

hipError_t launch_write(const void* key, int64_t key_stride, const void* value,
                        int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                        int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                        int32_t num_kv_heads, int32_t head_size, const float* signs,
                        hipStream_t stream);

// INT8 per-token-head mode: rows of head_size int8 codes and an fp32 scale
hipError_t launch_write_int8(const void* key, int64_t key_stride, const void* value,
                             int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                             int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                             int32_t num_kv_heads, int32_t head_size, hipStream_t stream);

// INT2 Lloyd-Max mode: rows of head_size / 4 code bytes and an fp32 scale,
// over the INT4 mode's rotation
hipError_t launch_write_int2(const void* key, int64_t key_stride, const void* value,
                             int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                             int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                             int32_t num_kv_heads, int32_t head_size, const float* signs,
                             hipStream_t stream);

struct AttnArgs {
  const void* q;
  int64_t q_stride;
  void* out;
  bool bf16;
  const uint8_t* cache;
  int32_t num_kv_heads, head_size, num_q_heads;
  const int32_t* cu_seqlens_q;
  const int32_t* seqused_k;
  int32_t num_seqs, max_seqlen_q, max_seqlen_k;
  const int32_t* block_table;
  int32_t bt_stride;
  float softmax_scale;
  const float* signs;
  int32_t num_segments;
  float* segm_out;
  float* segm_max;
  float* segm_sum;
  // sliding window: the query at position pos sees keys [pos - window + 1,
  // pos]; <= 0 is no window
  int32_t window = 0;
  // logit soft cap c (natural-log units): scores z become c * tanh(z / c)
  // before the softmax; <= 0 is none
  float softcap = 0.f;
  // INT8 per-token-head cache (rows of head_size int8 codes + fp32 scale, no
  // rotation; signs unused) instead of the INT4 one
  bool q8 = false;
  // INT2 Lloyd-Max cache (rows of head_size / 4 code bytes + fp32 scale, in
  // the rotated domain of the INT4 mode)
  bool q2 = false;
  // fused decode step only: the new token of each sequence (token b belongs to
  // sequence b and is its last key), encoded into the cache by the workgroup
  // that reads its block; null otherwise
  const void* key_new = nullptr;
  int64_t key_new_stride = 0;
  const void* value_new = nullptr;
  int64_t value_new_stride = 0;
  const int64_t* slot_new = nullptr;
  // slots of the cache (num_blocks * block_size): a new token whose slot is
  // outside [0, num_slots) is not stored
  int64_t num_slots = 0;
};

// Raises a kernel's dynamic LDS limit above the 64 KiB default, once per
// (kernel, device): the attribute call is a runtime round trip that a
// launch repeated every decode step should not pay each time.
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream);
hipError_t launch_reduce(const AttnArgs& a, hipStream_t stream);
bool decode_lds_supported(const AttnArgs& a);
hipError_t launch_decode_lds(const AttnArgs& a, hipStream_t stream);
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream);

// plain streaming kernel: reads read_bytes, writes write_bytes (16-byte units)
hipError_t launch_stream_rw(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                            hipStream_t stream);

// The decode path's block gather into LDS without its arithmetic (calibration):
// block_bytes a multiple of 1024 in [1024, 20480], num_ids a multiple of
// 2 * num_workgroups (checked by the caller).
hipError_t launch_stream_blocks(const uint8_t* cache, int64_t block_bytes, const int32_t* ids,
                                int64_t num_ids, int32_t num_workgroups, hipStream_t stream);

}  // namespace int4kv
