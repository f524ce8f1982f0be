/*
 * int4kv: INT4 per-token-head paged KV cache for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Pointers are DEVICE pointers unless marked "host".  `stream`
 * is a hipStream_t passed as void* (NULL = the legacy null stream).  Every call
 * validates its host-side arguments first and returns a status without
 * enqueuing anything when they are invalid; on success the work is enqueued on
 * `stream` and the call returns at once (no synchronisation).  The library
 * allocates no device memory and keeps no global mutable state apart from a
 * thread-local error string, a lock-protected record of the (kernel, device)
 * pairs whose LDS limit it has raised, and the fixed per-device array that
 * int4_paged_attention_noalloc keeps its split-K partials in (with the
 * looked-up address of each device's copy); every other entry point is
 * re-entrant, and its buffers are owned by the caller.  Slot numbers are bounds-checked on the device:
 * every write entry point stores a token only when its slot lies in
 * [0, num_blocks * block_size) and skips it otherwise (negative slots are the
 * pages' skip marker; larger ones would address memory past the cache).  The
 * other device-resident metadata (block ids, lengths) is the caller's
 * contract and is not checked: out-of-range values there are undefined
 * behaviour.
 *
 * Citations name the page and the section that defines each operation:
 *   [report]   PR #40835 report: "[Feature] Triton INT4 per-token-head KV cache
 *              quantization" (prhub.com.cn)
 *   [pr40633]  vLLM Pull Request #40633: "[Feature] Triton INT4 / INT2
 *              per-token-head KV cache quantization"
 *   [testfile] tests/quantization/test_per_token_kv_cache.py (vLLM fork page),
 *              by its numbered sections.
 *
 * Cache layout ([report], key snippets: get_kv_cache_shape):
 *   uint8 [num_blocks][2][block_size][num_kv_heads][R],  R = head_size/2 + 4.
 *   Index 0 of dim 1 holds K rows, index 1 holds V rows.  A row holds the
 *   head_size 4-bit codes of one (token, head), two per byte with the even
 *   element in the low nibble ([testfile] §2 and §6), followed by one
 *   little-endian fp32 scale word whose low 4 mantissa bits carry the zero
 *   point ([pr40633] description; [testfile] §6 steganography step).
 *   Rows are 4-byte aligned; the cache base must be 16-byte aligned.
 */
#ifndef INT4KV_H_
#define INT4KV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INT4KV_OK = 0,
  INT4KV_ERR_INVALID_ARG = 1, /* a host argument is out of range or inconsistent */
  INT4KV_ERR_UNSUPPORTED = 2, /* valid but not implemented (head size, block size, GQA ratio) */
  INT4KV_ERR_WORKSPACE = 3,   /* split-K requested without segment buffers */
  INT4KV_ERR_LAUNCH = 4       /* the HIP runtime reported an error at launch */
} int4kv_status_t;

typedef enum { INT4KV_F16 = 0, INT4KV_BF16 = 1 } int4kv_dtype_t;

/* Bytes of a cache of the given shape, or -1 if a dimension is < 1 or
 * head_size is odd.  R = head_size/2 + 4 bytes per (token, head, K|V) row. */
int64_t int4kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size);

/*
 * int4_kv_write: quantize and store K and V of `num_tokens` tokens.
 * ([report] implementation breakdown, item 2 and item 4: the INT4 write
 *  kernel; [pr40633] description: random Hadamard pre-rotation, asymmetric
 *  16-level quantization with one fp32 scale per (token, head) and the zero
 *  point hidden in the scale; [testfile] §4: negative slots are skipped.)
 *
 * For each token t with slot = slot_mapping[t] >= 0 and each KV head h, for
 * K (kv = 0) and V (kv = 1):
 *   x = input row (converted exactly to fp32); y = H (signs * x), the
 *   unnormalised Walsh-Hadamard transform in natural order, evaluated in fp32
 *   as butterflies of span 1, 2, 4, ..., d/2;
 *   s = max(fl((max y - min y) / 15), 1e-6f); s_t = s with its low 4 bits
 *   cleared; inv = fl(1 / s_t); zp = clamp(rint(-min y * inv), 0, 15);
 *   code_i = clamp(rint(fl(y_i * inv) + zp), 0, 15);
 *   row bytes j = code_{2j} | code_{2j+1} << 4; scale word = bits(s_t) | zp;
 *   the row goes to block slot / block_size, offset slot % block_size.
 * The result is bit-for-bit reproducible (no FMA contraction, no flush to zero).
 *
 *   key, value        [num_tokens, num_kv_heads, head_size] of `dtype`; the
 *                     token stride (in elements) is given; heads are
 *                     contiguous.  Base 16-byte aligned, stride a multiple of 8.
 *   slot_mapping      int64 [num_tokens]; slot < 0 (and slot >=
 *                     num_blocks * block_size) leaves the cache untouched.
 *   kv_cache          the packed cache (layout above), written in place.
 *   rht_signs         fp32 [head_size], each exactly +1.0f or -1.0f.
 * Supported: head_size 64 or 128, block_size 16.  num_tokens == 0 is a no-op.
 * Slots of one call must be distinct (two tokens to one slot race).
 */
int4kv_status_t int4_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, const float* rht_signs, void* stream);

/*
 * int4_paged_attention: causal attention of a varlen batch of queries over
 * the packed cache.
 * ([report] implementation breakdown, item 2 and item 5: the INT4 read
 *  kernel behind unified_attention, and risks: causal attention only;
 *  [pr40633] description: Q split into interleaved streams matching the
 *  nibble order, split-dot score with a sum(Q)*zp correction, per-stream
 *  accumulators, online softmax and segment reduction shared with the common
 *  kernel; [testfile] §6: argument list of unified_attention.)
 *
 * Sequence b has q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] query rows and
 * L_b = seqused_k[b] keys (its new tokens included).  Query row i sits at
 * position L_b - q_len_b + i and attends to keys [0, that position].  Query
 * head g reads KV head g / (num_q_heads / num_kv_heads).  Key j of sequence b
 * is row (j % block_size) of block block_table[b * block_table_stride +
 * j / block_size].  The result equals softmax(softmax_scale * q . k_hat) . v_hat,
 * where k_hat, v_hat are the dequantised, inverse-rotated cache rows
 * (signs * H ((code - zp) * s_t) / head_size); internally the score is taken
 * in the rotated domain and the output rotated back.  fp32 accumulation;
 * `out` has the dtype of q.
 *
 *   q                 [Tq, num_q_heads, head_size], token stride given (elements,
 *                     multiple of 8), heads contiguous, 16-byte aligned base.
 *   out               [Tq, num_q_heads, head_size] contiguous, same dtype as q.
 *   cu_seqlens_q      int32 [num_seqs + 1];  seqused_k int32 [num_seqs].
 *   max_seqlen_q      host: max q_len_b.  1 selects the decode path, which
 *                     may split each sequence's keys into `num_segments`
 *                     segments of whole blocks (ceil(ceil(L_b/16)/NS) blocks
 *                     each) merged by a reduction pass.  > 1 selects the
 *                     prefill/mixed path (no split-K; segments ignored).
 *   max_seqlen_k      host: >= every L_b.
 *   block_table       int32 [num_seqs, block_table_stride], entries < num_blocks.
 *   sliding_window    W > 0: query row i of sequence b (position pos) attends to
 *                     keys [max(0, pos - W + 1), pos] only; <= 0: no window.
 *                     ([pr40633] description: the packed read path shares the
 *                     common kernel's sliding-window masking.)  On the decode
 *                     path the split-K segments divide the blocks from the
 *                     first one the query sees.
 *   softcap           c > 0: each score z = softmax_scale * q . k_hat becomes
 *                     c * tanh(z / c) before the softmax; <= 0: none.
 *                     ([pr40633] description: the packed read path shares the
 *                     common kernel's softcap helper.)  Must be finite, with a
 *                     finite reciprocal when > 0; computed in fp32 from one
 *                     exp2 per score (absolute error a few 2^-24 of c).
 *   rht_signs         fp32 [head_size], the signs used by int4_kv_write.
 *   num_segments      >= 1.  When > 1 on the decode path, segm_output fp32
 *                     [num_seqs, num_q_heads, num_segments, head_size],
 *                     segm_max and segm_expsum fp32 [num_seqs, num_q_heads,
 *                     num_segments] are required scratch (contents on return
 *                     unspecified: per-segment accumulator, running maximum in
 *                     base-2 logit units, and exp-sum).
 * Supported: head_size 64 or 128, block_size 16, num_q_heads / num_kv_heads in
 * {1, 2, 4, 8, 16}.  A sequence with L_b == 0 gets zero output rows.
 */
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
                                     void* stream);

/*
 * int4kv_stream_rw: a plain streaming kernel that reads read_bytes from src and
 * writes write_bytes to dst, for measuring the bandwidth an HBM pass with a
 * given read:write mix attains on the device: the ceiling the cache write
 * (inputs read, packed rows written) is compared against.  Not a step of the
 * method.  In 16-byte units, with nr read and nw written units, written unit w
 * is the XOR of the read units w, w + nw, w + 2 nw, ... below nr (so no read
 * is dead); accesses are coalesced.  Byte counts must be multiples of 16 and
 * pointers 16-byte aligned; reads with write_bytes 0 are rejected
 * (INT4KV_ERR_INVALID_ARG); write_bytes 0 with read_bytes 0 is a no-op.  The
 * launch is asynchronous on the given stream (NULL: the default stream).
 */
int4kv_status_t int4kv_stream_rw(const void* src, int64_t read_bytes, void* dst,
                                 int64_t write_bytes, void* stream);

/*
 * int4kv_stream_blocks: the decode path's block gather on its own, for
 * measuring the rate its access pattern attains: cache blocks listed in
 * `block_ids` (device, int32, num_ids entries) are copied HBM -> LDS with the
 * same instructions and ring discipline as the decode kernel (two blocks per
 * tile, 1 KiB units over 8 waves, a 4-stage ring, a barrier per tile) and
 * nothing is computed or written.  Not a step of the method.  Workgroup g of
 * num_workgroups copies ids [2 g T, 2 (g + 1) T), T = num_ids / (2 *
 * num_workgroups), in order (as a decode workgroup copies its segment's
 * blocks; the decode call's own gather is its block table's rows,
 * concatenated, with one workgroup per segment of each sequence).  Block b
 * occupies bytes [b * block_bytes, (b + 1) * block_bytes) of `cache` (16-byte
 * aligned); block_bytes must be a multiple of 1024 in [1024, 20480] (an INT4
 * block of 8 KV heads: 2 * 16 * 8 * (head_size / 2 + 4) bytes), num_ids a
 * positive multiple of 2 * num_workgroups (INT4KV_ERR_INVALID_ARG otherwise;
 * num_ids 0 is a no-op).  Ids are the caller's contract: each must lie in
 * [0, number of blocks in the cache).  Asynchronous on `stream`.
 */
int4kv_status_t int4kv_stream_blocks(const uint8_t* cache, int64_t block_bytes,
                                     const int32_t* block_ids, int64_t num_ids,
                                     int32_t num_workgroups, void* stream);

/*
 * int4_paged_attention_noalloc: int4_paged_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments minus the three
 * segment buffers, the same kernels and the same result bit for bit.
 *
 * The decode path's split-K partials ([S, Hq, NS, d] outputs, then [S, Hq, NS]
 * maxima and exp-sums, fp32, each rounded up to 256 bytes) live in a fixed
 * device array of INT4KV_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  A call whose partials would not fit
 * returns INT4KV_ERR_WORKSPACE before anything is enqueued; cfg sizes: 64
 * segments of 4 sequences x 64 query heads x 128 take 8.5 MB.  The call makes
 * no hipMalloc or hipFree and uses no allocating library routine; the first
 * call on a device looks up that device's copy of the array once.  Nothing
 * in the array has to start at zero (every partial that the reduction reads
 * is written by the same call).  Calls that overlap on one GPU (different
 * streams, or threads) share the array and race: serialise them.  With
 * max_seqlen_q > 1 or num_segments == 1 no partials are used.
 */
#define INT4KV_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
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
                                             void* stream);

/*
 * int4_decode_step: int4_kv_write of one new token per sequence followed by
 * int4_paged_attention, in one launch on the decode path.
 * (The write half and the read half above, in the order a decode step runs
 *  them: [report] implementation breakdown, items 2 and 5; [testfile] §2 and
 *  §6 call the write, then unified_attention, on the same cache.)
 *
 * The result (cache bytes and `out`) is the same as the two calls in that
 * order.  Token b of key_new / value_new belongs to sequence b and must be its
 * last key: slot_mapping[b] is the cache position of key seqused_k[b] - 1 of
 * sequence b, or < 0 (nothing written for that sequence).  With
 * max_seqlen_q == 1 and a KV-head count that the LDS-staged decode kernel
 * takes (1, 2, 4, 8 or a multiple of 8), the workgroup whose split-K segment
 * holds that key's block encodes and stores the token's rows before copying
 * the block, so no separate write launch is needed; otherwise the library
 * enqueues the write and then the attention.
 *
 *   key_new, value_new  [num_seqs, num_kv_heads, head_size] of `dtype` (the
 *                       dtype of q), token stride given (elements, multiple of
 *                       8), heads contiguous, 16-byte aligned base.
 *   slot_mapping        int64 [num_seqs].
 *   the other arguments as for int4_paged_attention; kv_cache is written.
 * Errors and support as for the two calls.  num_seqs == 0 is a no-op.
 */
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
                                 void* stream);

/*
 * int4kv_decode_num_segments: the split-K segment count the library's decode
 * kernels run best with for a decode batch (max_seqlen_q == 1) of `num_seqs`
 * sequences whose longest has `max_seqlen_k` keys.  A decode workgroup holds
 * a whole CU of MI355X (256), so a grid runs in rounds of 256 workgroups; the
 * count minimises rounds x (a fixed start of about 3 key tiles + the tiles
 * of one segment), plus about 3 tiles for the segment reduction when split,
 * with no segment shorter than 64 keys (2 tiles of 32).  Host only; never
 * fails (returns >= 1).  The caller sizes the segment buffers of
 * int4_paged_attention / int4_decode_step with it and passes it as
 * num_segments.  (The pages' attention test sizes its segment buffers from a
 * segment count chosen by the caller: [testfile] §6.)
 */
int32_t int4kv_decode_num_segments(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seqlen_k);

/* ---------------------------------------------------------------------------
 * INT8 per-token-head mode: the sibling mode on the same cache family
 * ([report] key snippets: get_kv_cache_shape keeps the data dimension at
 * head_size for per-token-head modes other than INT4 and adds a 4-byte scale
 * pad for a 1-byte cache dtype; [pr40633] description and commits: INT8
 * per-token-head scales, its write kernel rounding to nearest).
 *
 * Cache layout: uint8 [num_blocks][2][block_size][num_kv_heads][head_size + 4];
 * index 0 of dim 1 is K, 1 is V; a row holds head_size int8 codes (two's
 * complement) and then the fp32 scale, little-endian.  No rotation.
 * ------------------------------------------------------------------------- */

/* Bytes of an INT8 cache of the given shape, or -1 if a dimension is < 1. */
int64_t int8kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size);

/*
 * int8_kv_write: quantize and store K and V of `num_tokens` tokens.
 * For each token t with slot = slot_mapping[t] >= 0, each KV head, K and V:
 *   x = input row in fp32; s = max(fl(max |x| / 127), 1e-6f); inv = fl(1 / s);
 *   q_i = clamp(trunc(fl(fl(x_i * inv) +- 0.5)), -128, 127), the sign of the
 *   0.5 that of fl(x_i * inv) (round half away from zero: [pr40633] commit on
 *   the INT8 reshape kernel; the quantizer of the [testfile] per-token-head
 *   reference: absmax / 127, clamp(min=1e-6), data * (1 / scale)).
 * Bit-for-bit reproducible.  Arguments as for int4_kv_write (no sign vector).
 */
int4kv_status_t int8_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, void* stream);

/*
 * int8_paged_attention: causal attention over the INT8 per-token-head cache:
 * softmax(softmax_scale * q . k_hat) . v_hat with k_hat, v_hat = codes *
 * scale ([pr40633] description: the INT8 per-token-head read side is the
 * common attention kernel with per-token-head scales).  Arguments, batches
 * (decode and prefill / mixed, as for int4_paged_attention: the segments are
 * used only when max_seqlen_q == 1), window, soft cap and errors as for
 * int4_paged_attention, without the sign vector.  Supported: head_size 64 or
 * 128, block_size 16, query heads per KV head in {1, 2, 4, 8, 16}; decode
 * batches (max_seqlen_q == 1) also need num_kv_heads 1, 2 or a multiple of 4
 * (else INT4KV_ERR_UNSUPPORTED).
 */
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
                                     float* segm_expsum, void* stream);

/* int8kv_decode_num_segments: the split count for int8_paged_attention, by the
 * rule of int4kv_decode_num_segments for its workgroups of up to 4 KV heads. */
int32_t int8kv_decode_num_segments(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seqlen_k);

/* ---------------------------------------------------------------------------
 * INT2 Lloyd-Max mode: the other packed mode of the same family ([pr40633]
 * description and its commit on the packed modes: four 2-bit codes per byte,
 * Hadamard pre-rotation, dequantisation through four centroids fitted over
 * N(0, 1); dropped from the merged PR, [report]).
 *
 * Cache layout: uint8 [num_blocks][2][block_size][num_kv_heads][head_size/4 + 4];
 * index 0 of dim 1 is K, 1 is V; a row holds head_size / 4 code bytes
 * (element 4j + k in bits 2k, 2k+1 of byte j) and then the fp32 scale,
 * little-endian.  Rows live in the rotated domain of the INT4 mode (same
 * sign vector; all signs +1 give the plain Hadamard transform).
 * ------------------------------------------------------------------------- */

/* Bytes of an INT2 cache of the given shape, or -1 if a dimension is < 1 or
 * head_size is not a multiple of 4. */
int64_t int2kv_cache_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_size);

/*
 * int2_kv_write: rotate, quantize and store K and V of `num_tokens` tokens.
 * For each token t with slot = slot_mapping[t] >= 0, each KV head, K and V,
 * in fp32 with each operation rounded once:
 *   y = H (signs * x) (the INT4 mode's rotation and butterfly order);
 *   s = max(sqrt(sum_i y_i^2 / head_size), 1e-6), the squares summed by
 *   halves (pairs, then pairs of pairs, ...); inv = fl(1 / s);
 *   code_i = [v >= -t] + [v >= 0] + [v >= t] with v = fl(y_i * inv) and t =
 *   0.9815988 (as fp32), the threshold of the 4-level Lloyd-Max quantizer of
 *   N(0, 1), whose levels are -b, -a, a, b (a = 0.4527800, b = 1.5104176)
 *   for codes 0..3.  Bit-for-bit reproducible.  Arguments, ownership and
 *   errors as for int4_kv_write.
 */
int4kv_status_t int2_kv_write(const void* key, int64_t key_token_stride, const void* value,
                              int64_t value_token_stride, int4kv_dtype_t dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, uint8_t* kv_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, const float* rht_signs, void* stream);

/*
 * int2_paged_attention: causal attention (decode and prefill / mixed batches)
 * over the INT2 cache: softmax(softmax_scale * q . k_hat) . v_hat with k_hat,
 * v_hat = D H (s * level(code)) / head_size (levels -b, -a, a, b as in
 * int2_kv_write; [pr40633] description: centroid lookup on the read side,
 * scores over the rotated query).  Arguments, window, soft cap, split-K
 * segments (sized with int4kv_decode_num_segments) and errors as for
 * int4_paged_attention (the segments are used only when max_seqlen_q == 1).
 * Supported: head_size 64 or 128, block_size 16, query heads per KV head in
 * {1, 2, 4, 8, 16}; decode batches also need num_kv_heads 1, 2, 4 or a
 * multiple of 8 (else INT4KV_ERR_UNSUPPORTED).
 */
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
                                     void* stream);

/* Human-readable name of a status code (static storage). */
const char* int4kv_status_string(int4kv_status_t s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* int4kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INT4KV_H_ */
