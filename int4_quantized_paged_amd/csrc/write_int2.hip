// INT2 Lloyd-Max cache write (gfx950): four 2-bit codes per byte, after the
// same random Hadamard rotation as the INT4 mode, with one fp32 scale per
// (token, head, K|V) row (PR #40633's description and its commit on the
// packed modes: Hadamard pre-rotation, dequantisation through four centroids
// fitted over N(0, 1)).  Per row, in fp32 with every operation rounded once:
//   y = H (signs * x)          (butterfly spans 1, 2, 4, ..., D/2)
//   s = max(sqrt(sum y_i^2 / D), 1e-6)   (squares summed by halves)
//   v = fl(y * fl(1 / s)),  code = [v >= -t] + [v >= 0] + [v >= t]
// with t the Lloyd-Max threshold of the 4-level quantizer of N(0, 1) (levels
// -b, -a, a, b for codes 0..3).  Element 4j + k of the row sits in bits 2k,
// 2k+1 of byte j; the scale follows the D/4 code bytes.  Slots < 0 write
// nothing.
//
// Work layout: one row = D elements held by D/16 adjacent lanes, 16
// consecutive elements each (two 16-byte loads, one 4-byte store per lane).
// Butterflies of span 1..8 run inside a lane, spans 16.. pair the lanes; the
// sum of squares is a tree over the lane's 16 elements and then over lanes,
// which is the order of halves.
#include "device_common.h"
#include "encode_row.h"
#include "launch.h"

namespace int4kv {

namespace {

// threshold between the levels a and b of the 4-level Lloyd-Max quantizer of
// N(0, 1): (a + b) / 2 with a = 0.45278..., b = 1.51042... (Max, 1960, N = 4)
constexpr float kLloydT = 0.981598821567794f;

template <bool BF16, int D>
__global__ __launch_bounds__(256) void write_int2_kernel(
    const uint16_t* __restrict__ key, int64_t key_stride, const uint16_t* __restrict__ value,
    int64_t value_stride, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    uint8_t* __restrict__ cache, int64_t num_slots, int32_t num_kv_heads,
    const float* __restrict__ signs) {
#pragma clang fp contract(off)
  constexpr int E = 16;
  constexpr int LPR = D / E;        // lanes per row
  constexpr int RPW = kWave / LPR;  // rows per wave
  constexpr int R = D / 4 + 4;      // row bytes
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, rw = lane / LPR;
  const int64_t total_rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  uint32_t flip[E / 2];
  row_flips<E>(signs, sub, flip);
  for (int64_t base = wave_id * RPW; base < total_rows; base += waves_total * RPW) {
    const int64_t row = base + rw;
    const bool ok = row < total_rows;
    const int64_t r = ok ? row : total_rows - 1;  // tail lanes read a valid row, store nothing
    const int h = (int)(r % num_kv_heads);
    const int64_t tk = r / num_kv_heads;
    const int kv = (int)(tk & 1);
    const int64_t t = tk >> 1;
    const uint16_t* src =
        (kv == 0 ? key + t * key_stride : value + t * value_stride) + (int64_t)h * D + E * sub;
    u32x4_t in[2];
    in[0] = reinterpret_cast<const u32x4_t*>(src)[0];
    in[1] = reinterpret_cast<const u32x4_t*>(src)[1];
    float x[E];
    row_inputs<BF16, E>(in, flip, x);
#pragma unroll
    for (int span = 1; span < E; span <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e & span) continue;
        const float u = x[e], w = x[e + span];
        x[e] = __fadd_rn(u, w);
        x[e + span] = __fsub_rn(u, w);
      }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      const bool upper = (sub & m) != 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float p = shfl_xor_rt(x[e], m);
        x[e] = upper ? __fsub_rn(p, x[e]) : __fadd_rn(x[e], p);
      }
    }
    float sq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sq[e] = __fmul_rn(x[e], x[e]);
#pragma unroll
    for (int w = 1; w < E; w <<= 1)
#pragma unroll
      for (int e = 0; e < E; e += 2 * w) sq[e] = __fadd_rn(sq[e], sq[e + w]);
    float ss = sq[0];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss = __fadd_rn(ss, shfl_xor_rt(ss, m));
    // sqrtf is correctly rounded here (the native square root is not)
    float s = sqrtf(__fdiv_rn(ss, (float)D));
    if (!(s > 1e-6f)) s = 1e-6f;
    const float inv = __fdiv_rn(1.0f, s);
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = __fmul_rn(x[e], inv);
      const uint32_t code = (uint32_t)(v >= -kLloydT) + (uint32_t)(v >= 0.f) + (uint32_t)(v >= kLloydT);
      word |= code << (2 * e);
    }
    const int64_t slot = slot_mapping[t];
    if (ok && (uint64_t)slot < (uint64_t)num_slots) {  // skips slot < 0 too
      const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
      uint32_t* dst = reinterpret_cast<uint32_t*>(
          cache + (((blk * 2 + kv) * kBlockSize + off) * num_kv_heads + h) * R);  // 4-byte aligned
      dst[sub] = word;
      if (sub == 0) dst[D / 16] = as_uint(s);
    }
  }
}

}  // namespace

hipError_t launch_write_int2(const void* key, int64_t key_stride, const void* value,
                             int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                             int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                        int32_t num_kv_heads,
                             int32_t head_size, const float* signs, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int rows_per_block = 4 * (kWave / (head_size / 16));
  int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 32;  // grid-stride beyond 32 blocks per CU
  if (blocks > cap) blocks = cap;
  dim3 grid((unsigned)blocks), block(256);
  auto k16 = reinterpret_cast<const uint16_t*>(key);
  auto v16 = reinterpret_cast<const uint16_t*>(value);
#define INT2KV_W(BF, DD)                                                                         \
  hipLaunchKernelGGL((write_int2_kernel<BF, DD>), grid, block, 0, stream, k16, key_stride, v16, \
                     value_stride, slot_mapping, num_tokens, cache, num_slots, num_kv_heads, signs)
  if (bf16) {
    if (head_size == 128) INT2KV_W(true, 128); else INT2KV_W(true, 64);
  } else {
    if (head_size == 128) INT2KV_W(false, 128); else INT2KV_W(false, 64);
  }
#undef INT2KV_W
  return hipGetLastError();
}

}  // namespace int4kv
