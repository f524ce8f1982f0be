// INT8 per-token-head cache write (gfx950): the sibling mode of the INT4 one
// on the same cache family.  One fp32 scale per (token, head, K|V) row, no
// rotation, symmetric int8 codes:
//   s = max(fl(absmax / 127), 1e-6), v = fl(x * fl(1 / s)),
//   q = clamp(trunc(fl(v +- 0.5)), -128, 127)  (round half away from zero),
// the quantizer of the test page's per-token-head reference with the rounding
// of the INT8 write-kernel fix in PR #40633's commits; the row holds the d
// codes and then the scale (the cache-shape snippet of the PR #40835 report:
// data dimension head_size plus a 4-byte scale pad).  Slots < 0 write nothing.
//
// Work layout: one row = D elements held by D/16 adjacent lanes, 16
// consecutive elements each (two 16-byte loads, one 16-byte store per lane);
// the row's absolute maximum is reduced across those lanes.
#include "device_common.h"
#include "launch.h"

namespace int4kv {

namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(256) void write_int8_kernel(
    const uint16_t* __restrict__ key, int64_t key_stride, const uint16_t* __restrict__ value,
    int64_t value_stride, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    uint8_t* __restrict__ cache, int64_t num_slots, int32_t num_kv_heads) {
#pragma clang fp contract(off)
  constexpr int E = 16;
  constexpr int LPR = D / E;        // lanes per row
  constexpr int RPW = kWave / LPR;  // rows per wave
  constexpr int R = D + 4;          // row bytes
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, rw = lane / LPR;
  const int64_t total_rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
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
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = in[k][j];
        if constexpr (BF16) {
          x[8 * k + 2 * j] = as_float(w << 16);
          x[8 * k + 2 * j + 1] = as_float(w & 0xFFFF0000u);
        } else {
          const half2_t hh = __builtin_bit_cast(half2_t, w);
          x[8 * k + 2 * j] = (float)hh[0];
          x[8 * k + 2 * j + 1] = (float)hh[1];
        }
      }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, shfl_xor_rt(amax, m));
    float s = __fdiv_rn(amax, 127.0f);
    if (!(s > 1e-6f)) s = 1e-6f;
    const float inv = __fdiv_rn(1.0f, s);
    uint32_t packed[E / 4];
#pragma unroll
    for (int p = 0; p < E / 4; ++p) {
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = __fmul_rn(x[4 * p + j], inv);
        const float tt = __fadd_rn(v, v >= 0.f ? 0.5f : -0.5f);
        const int q = min(max(__float2int_rz(tt), -128), 127);
        word |= ((uint32_t)q & 0xFFu) << (8 * j);
      }
      packed[p] = word;
    }
    const int64_t slot = slot_mapping[t];
    if (ok && (uint64_t)slot < (uint64_t)num_slots) {  // skips slot < 0 too
      const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
      uint8_t* dst = cache + (((blk * 2 + kv) * kBlockSize + off) * num_kv_heads + h) * R;
      *reinterpret_cast<u32x4a4_t*>(dst + E * sub) =
          u32x4a4_t{packed[0], packed[1], packed[2], packed[3]};  // rows are 4-byte aligned
      if (sub == 0) reinterpret_cast<uint32_t*>(dst)[D / 4] = as_uint(s);
    }
  }
}

}  // namespace

hipError_t launch_write_int8(const void* key, int64_t key_stride, const void* value,
                             int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                             int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                        int32_t num_kv_heads,
                             int32_t head_size, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int rows_per_block = 4 * (kWave / (head_size / 16));
  int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 32;  // grid-stride beyond 32 blocks per CU
  if (blocks > cap) blocks = cap;
  dim3 grid((unsigned)blocks), block(256);
  auto k16 = reinterpret_cast<const uint16_t*>(key);
  auto v16 = reinterpret_cast<const uint16_t*>(value);
#define INT8KV_W(BF, DD)                                                                         \
  hipLaunchKernelGGL((write_int8_kernel<BF, DD>), grid, block, 0, stream, k16, key_stride, v16, \
                     value_stride, slot_mapping, num_tokens, cache, num_slots, num_kv_heads)
  if (bf16) {
    if (head_size == 128) INT8KV_W(true, 128); else INT8KV_W(true, 64);
  } else {
    if (head_size == 128) INT8KV_W(false, 128); else INT8KV_W(false, 64);
  }
#undef INT8KV_W
  return hipGetLastError();
}

}  // namespace int4kv
