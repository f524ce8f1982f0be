// INT4 cache write: rotate, quantize, pack and store K/V rows (gfx950).
//
// Implements the write half described by the PR #40835 report (implementation
// breakdown, item 2: the INT4 write kernel rotates each head vector, derives a
// per (token, head) scale and zero point and packs two codes per byte) and PR
// #40633's description (random Hadamard pre-rotation; asymmetric 16-level
// codes; zero point in the low 4 mantissa bits of the fp32 scale), with the
// quantizer of the test file's section 6 INT4 reference and the skip rule of
// its section 4 (slot < 0 writes nothing).
//
// Work layout: one row = one (token, K|V, head) vector of D elements.  A row
// is owned by D/16 lanes holding 16 consecutive elements each, so a wave owns
// 64/(D/16) rows: 8 rows at D = 128, i.e. all heads of one (token, K|V) when
// there are 8 KV heads, whose packed rows are contiguous in the cache.
// The Walsh-Hadamard butterflies of span 1..8 run inside a lane; spans 16, 32,
// 64 pair lanes (lane ^ 1, ^ 2, ^ 4) through DPP / ds_swizzle.  Every fp32
// operation is a single correctly rounded op in the fixed span order, so the
// packed bytes are reproducible bit for bit (this file is built without FMA
// contraction).
#include "device_common.h"
#include "launch.h"

namespace int4kv {

template <bool BF16, int D>
__global__ __launch_bounds__(256) void write_kernel(
    const uint16_t* __restrict__ key, int64_t key_stride, const uint16_t* __restrict__ value,
    int64_t value_stride, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    uint8_t* __restrict__ cache, int32_t num_kv_heads, const float* __restrict__ signs) {
  constexpr int LPR = D / 16;            // lanes per row
  constexpr int RPW = kWave / LPR;       // rows per wave
  constexpr int R = D / 2 + 4;           // packed row bytes
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  const int rw = lane / LPR;
  const int64_t total_rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);

  float sg[16];
  {
    const float4* sp = reinterpret_cast<const float4*>(signs + 16 * sub);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float4 v = sp[k];
      sg[4 * k + 0] = v.x;
      sg[4 * k + 1] = v.y;
      sg[4 * k + 2] = v.z;
      sg[4 * k + 3] = v.w;
    }
  }

  for (int64_t base = wave_id * RPW; base < total_rows; base += waves_total * RPW) {
    const int64_t row = base + rw;
    const bool in_range = row < total_rows;
    const int64_t r = in_range ? row : total_rows - 1;  // tail lanes compute a valid row, store nothing
    const int h = (int)(r % num_kv_heads);
    const int64_t tk = r / num_kv_heads;
    const int kv = (int)(tk & 1);
    const int64_t t = tk >> 1;

    const uint16_t* src = (kv == 0 ? key + t * key_stride : value + t * value_stride) +
                          (int64_t)h * D + 16 * sub;
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
    u32x4_t a = s4[0], b = s4[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float x[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[2 * k] = to_f32<BF16>((uint16_t)(w[k] & 0xFFFFu));
      x[2 * k + 1] = to_f32<BF16>((uint16_t)(w[k] >> 16));
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = __fmul_rn(x[e], sg[e]);  // exact: signs are +-1

    // butterflies inside the lane: spans 1, 2, 4, 8
#pragma unroll
    for (int span = 1; span < 16; span <<= 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e & span) continue;
        float u = x[e], v = x[e + span];
        x[e] = __fadd_rn(u, v);
        x[e + span] = __fsub_rn(u, v);
      }
    }
    // butterflies across lanes: spans 16, 32, 64.  The lower partner keeps
    // u + v, the upper one u - v, written as partner + (-self).
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      const uint32_t flip = (sub & m) ? 0x80000000u : 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = shfl_xor_rt(x[e], m);
        x[e] = __fadd_rn(p, as_float(as_uint(x[e]) ^ flip));
      }
    }

    // row range
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      mn = fminf(mn, x[e]);
      mx = fmaxf(mx, x[e]);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      mn = fminf(mn, shfl_xor_rt(mn, m));
      mx = fmaxf(mx, shfl_xor_rt(mx, m));
    }
    float s = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
    if (!(s > 1e-6f)) s = 1e-6f;
    const float s_t = as_float(as_uint(s) & 0xFFFFFFF0u);
    const float inv = __fdiv_rn(1.0f, s_t);
    const float zpf = fminf(fmaxf(rintf(__fmul_rn(-mn, inv)), 0.0f), 15.0f);

    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float c = fminf(fmaxf(rintf(__fadd_rn(__fmul_rn(x[e], inv), zpf)), 0.0f), 15.0f);
      packed[e >> 3] |= (uint32_t)c << (4 * (e & 7));
    }

    const int64_t slot = slot_mapping[t];
    if (in_range && slot >= 0) {
      const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
      uint8_t* dst = cache + (((blk * 2 + kv) * kBlockSize + off) * num_kv_heads + h) * R;
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);  // rows are 4-byte aligned
      d32[2 * sub] = packed[0];
      d32[2 * sub + 1] = packed[1];
      if (sub == 0) d32[D / 8] = as_uint(s_t) | (uint32_t)zpf;
    }
  }
}

hipError_t launch_write(const void* key, int64_t key_stride, const void* value,
                        int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                        int32_t num_tokens, uint8_t* cache, int32_t num_kv_heads,
                        int32_t head_size, const float* signs, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int rows_per_block = 4 * (kWave / (head_size / 16));
  int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 32;  // grid-stride beyond 32 blocks per CU
  if (blocks > cap) blocks = cap;
  dim3 grid((unsigned)blocks), block(256);
  auto k16 = reinterpret_cast<const uint16_t*>(key);
  auto v16 = reinterpret_cast<const uint16_t*>(value);
#define INT4KV_W(BF, DD)                                                                  \
  hipLaunchKernelGGL((write_kernel<BF, DD>), grid, block, 0, stream, k16, key_stride, v16, \
                     value_stride, slot_mapping, num_tokens, cache, num_kv_heads, signs)
  if (bf16) {
    if (head_size == 128) INT4KV_W(true, 128); else INT4KV_W(true, 64);
  } else {
    if (head_size == 128) INT4KV_W(false, 128); else INT4KV_W(false, 64);
  }
#undef INT4KV_W
  return hipGetLastError();
}

}  // namespace int4kv
