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
// Work layout: one row = one (token, K|V, head) vector of D elements, held by
// D/E lanes with E consecutive elements each.  Bulk writes use E = 64 (2
// lanes per row at D = 128, 1 at D = 64: the fewest cross-lane steps per
// element); writes of fewer rows than fill the GPU use E = 16 (8 or 4 lanes
// per row: a chain four times shorter per row, four times as many waves).
// The Walsh-Hadamard butterflies of span 1..E/2 run inside a lane and the
// spans E, 2E, ... pair the lanes of a row through DPP, which keeps the spans
// in the increasing order the encoding fixes (encode_row.h).
#include "device_common.h"
#include "encode_row.h"
#include "launch.h"

namespace int4kv {

namespace {

// rows at and above which writes take 64 elements per lane
constexpr int64_t kBulkRows = 65536;

}  // namespace

template <bool BF16, int D, int E>
__global__ __launch_bounds__(256) void write_kernel(
    const uint16_t* __restrict__ key, int64_t key_stride, const uint16_t* __restrict__ value,
    int64_t value_stride, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    uint8_t* __restrict__ cache, int64_t num_slots, int32_t num_kv_heads,
    const float* __restrict__ signs) {
  constexpr int LPR = D / E;             // lanes per row
  constexpr int RPW = kWave / LPR;       // rows per wave
  constexpr int R = D / 2 + 4;           // packed row bytes
  constexpr int NV = E / 8;              // 16-byte input vectors per lane
  constexpr int NP = E / 8;              // packed code dwords per lane
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;            // which E-element piece of the row
  const int rw = lane / LPR;
  const int64_t total_rows = (int64_t)num_tokens * 2 * num_kv_heads;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);

  // sign bits of the lane's E elements, as flips of 16-bit pairs
  uint32_t flip[E / 2];
  row_flips<E>(signs, sub, flip);

  // row coordinates and the raw 16-bit inputs of one row (software-pipelined:
  // the next row's loads are in flight while the current row is encoded)
  struct RowIn {
    int64_t t;
    int h, kv;
    bool ok;
    u32x4_t a[NV];
  };
  auto fetch = [&](int64_t base, RowIn& in) {
    const int64_t row = base + rw;
    in.ok = row < total_rows;
    const int64_t r = in.ok ? row : total_rows - 1;  // tail lanes read a valid row, store nothing
    in.h = (int)(r % num_kv_heads);
    const int64_t tk = r / num_kv_heads;
    in.kv = (int)(tk & 1);
    in.t = tk >> 1;
    const uint16_t* src = (in.kv == 0 ? key + in.t * key_stride : value + in.t * value_stride) +
                          (int64_t)in.h * D + E * sub;
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
    for (int k = 0; k < NV; ++k) in.a[k] = s4[k];
  };
  const int64_t stride = waves_total * RPW;
  int64_t base = wave_id * RPW;
  if (base >= total_rows) return;
  RowIn cur;
  fetch(base, cur);
  for (; base < total_rows; base += stride) {
    RowIn nxt;
    if (base + stride < total_rows) fetch(base + stride, nxt);  // uniform over the wave
    const int64_t t = cur.t;
    const int h = cur.h, kv = cur.kv;
    const bool in_range = cur.ok;
    float x[E];
    row_inputs<BF16, E>(cur.a, flip, x);
    uint32_t packed[NP];
    const uint32_t word = encode_piece<E, LPR>(x, sub, packed);

    const int64_t slot = slot_mapping[t];
    if (in_range && (uint64_t)slot < (uint64_t)num_slots) {  // skips slot < 0 too
      const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
      uint8_t* dst = cache + (((blk * 2 + kv) * kBlockSize + off) * num_kv_heads + h) * R;
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + (E / 2) * sub);  // rows are 4-byte aligned
      if constexpr (E == 64) {
        u32x4a4_t* d16 = reinterpret_cast<u32x4a4_t*>(d32);
        d16[0] = u32x4a4_t{packed[0], packed[1], packed[2], packed[3]};
        d16[1] = u32x4a4_t{packed[4], packed[5], packed[6], packed[7]};
      } else {
#pragma unroll
        for (int q = 0; q < NP; ++q) d32[q] = packed[q];
      }
      if (sub == 0) reinterpret_cast<uint32_t*>(dst)[D / 8] = word;
    }
    cur = nxt;
  }
}

hipError_t launch_write(const void* key, int64_t key_stride, const void* value,
                        int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                        int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                        int32_t num_kv_heads,
                        int32_t head_size, const float* signs, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * 2 * num_kv_heads;
  // 64 elements per lane once there are enough rows for every SIMD to hold
  // several waves of them; 16 below that, where the per-row chain is the cost
  const bool bulk = rows >= kBulkRows;
  const int e = bulk ? 64 : 16;
  const int rows_per_block = 4 * (kWave / (head_size / e));
  int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 32;  // grid-stride beyond 32 blocks per CU
  if (blocks > cap) blocks = cap;
  dim3 grid((unsigned)blocks), block(256);
  auto k16 = reinterpret_cast<const uint16_t*>(key);
  auto v16 = reinterpret_cast<const uint16_t*>(value);
#define INT4KV_W(BF, DD, EE)                                                                  \
  hipLaunchKernelGGL((write_kernel<BF, DD, EE>), grid, block, 0, stream, k16, key_stride, v16, \
                     value_stride, slot_mapping, num_tokens, cache, num_slots, num_kv_heads, signs)
#define INT4KV_WE(BF, DD) \
  do {                    \
    if (bulk)             \
      INT4KV_W(BF, DD, 64); \
    else                  \
      INT4KV_W(BF, DD, 16); \
  } while (0)
  if (bf16) {
    if (head_size == 128) INT4KV_WE(true, 128); else INT4KV_WE(true, 64);
  } else {
    if (head_size == 128) INT4KV_WE(false, 128); else INT4KV_WE(false, 64);
  }
#undef INT4KV_WE
#undef INT4KV_W
  return hipGetLastError();
}

}  // namespace int4kv
