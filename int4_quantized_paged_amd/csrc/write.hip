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
// D/E lanes with E consecutive elements each.  Bulk writes use E = 32 (4
// lanes per row at D = 128, 2 at D = 64): few enough registers for four
// waves per SIMD with two rows' inputs in flight per lane, which hides the
// loads better than E = 64's fewer cross-lane steps save; writes of fewer
// rows than fill the GPU use E = 16 (8 or 4 lanes per row: a shorter chain
// per row, more waves).  The Walsh-Hadamard butterflies of span 1..E/2 run
// inside a lane and the spans E, 2E, ... pair the lanes of a row through
// DPP, which keeps the spans in the increasing order the encoding fixes
// (encode_row.h).  The encoding is VALU-bound: about 17 fp32/int VALU
// instructions per element (7 butterfly adds, the 16-bit to fp32 conversion
// with the sign flip, the range, four per code, the packing and the
// per-row scale), with no packed fp32 math.
#include "device_common.h"
#include "encode_row.h"
#include "launch.h"

namespace int4kv {

namespace {

// rows at and above which writes take 32 elements per lane
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
  // kept in registers: left visible, the compiler re-derives them from the
  // signs inside the row loop (reloading the signs and redoing the sign tests
  // for every pair of rows)
#pragma unroll
  for (int p = 0; p < E / 2; ++p) flip[p] = opaque(flip[p]);

  // Row coordinates, slot and raw 16-bit inputs of one row.  Rows are
  // software-pipelined in two buffers that take turns (the loads of one row
  // are in flight while the other is encoded, and no register copy waits on
  // them); the slot travels with the inputs, as a load issued later would
  // have to wait for them too.  A lane's row advances by the grid's row
  // stride per fetch, so its (token, K|V, head) coordinates advance by the
  // stride's quotient and remainder over the KV heads (no division per row).
  struct RowIn {
    int64_t t, slot;
    int h, kv;
    bool ok;
    u32x4_t a[NV];
  };
  const int64_t stride = waves_total * RPW;
  int64_t row = wave_id * RPW + rw;          // the lane's next row to fetch
  if (wave_id * RPW >= total_rows) return;   // uniform over the wave
  int64_t tk = row / num_kv_heads;           // token * 2 + kv of `row`
  int hh = (int)(row - tk * num_kv_heads);   // head of `row`
  const int64_t s_q = stride / num_kv_heads;
  const int s_r = (int)(stride - s_q * num_kv_heads);
  const int64_t last_tk = (total_rows - 1) / num_kv_heads;
  const int last_h = (int)(total_rows - 1 - last_tk * num_kv_heads);
  auto fetch = [&](RowIn& in) {
    in.ok = row < total_rows;
    const int64_t k2 = in.ok ? tk : last_tk;  // tail lanes read a valid row, store nothing
    in.h = in.ok ? hh : last_h;
    in.kv = (int)(k2 & 1);
    in.t = k2 >> 1;
    const uint16_t* src = (in.kv == 0 ? key + in.t * key_stride : value + in.t * value_stride) +
                          (int64_t)in.h * D + E * sub;
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
    for (int k = 0; k < NV; ++k) in.a[k] = s4[k];
    in.slot = slot_mapping[in.t];
    row += stride;
    tk += s_q;
    hh += s_r;
    if (hh >= num_kv_heads) {
      hh -= num_kv_heads;
      ++tk;
    }
  };
  auto encode_store = [&](const RowIn& in) {
    float x[E];
    row_inputs<BF16, E>(in.a, flip, x);
    uint32_t packed[NP];
    const uint32_t word = encode_piece<E, LPR>(x, sub, packed);
    if (in.ok && (uint64_t)in.slot < (uint64_t)num_slots) {  // skips slot < 0 too
      const int64_t blk = in.slot / kBlockSize, off = in.slot % kBlockSize;
      uint8_t* dst = cache + (((blk * 2 + in.kv) * kBlockSize + off) * num_kv_heads + in.h) * R;
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + (E / 2) * sub);  // rows are 4-byte aligned
      if constexpr (E == 32) {
        *reinterpret_cast<u32x4a4_t*>(d32) = u32x4a4_t{packed[0], packed[1], packed[2], packed[3]};
      } else {
#pragma unroll
        for (int q = 0; q < NP; ++q) d32[q] = packed[q];
      }
      if (sub == 0) reinterpret_cast<uint32_t*>(dst)[D / 8] = word;
    }
  };
  // Fetches are unconditional: past the end every lane is a tail lane and
  // reads the last row again (from the L2), which keeps the count of loads in
  // flight the same on every path, so the wait before an encode covers only
  // that row's loads.  `row - rw` is the wave's next base, uniform over it.
  RowIn A, B;
  fetch(A);
  for (;;) {
    const bool more_b = row - rw < total_rows;
    fetch(B);
    encode_store(A);
    if (!more_b) break;
    const bool more_a = row - rw < total_rows;
    fetch(A);
    encode_store(B);
    if (!more_a) break;
  }
}

hipError_t launch_write(const void* key, int64_t key_stride, const void* value,
                        int64_t value_stride, bool bf16, const int64_t* slot_mapping,
                        int32_t num_tokens, uint8_t* cache, int64_t num_slots,
                        int32_t num_kv_heads,
                        int32_t head_size, const float* signs, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * 2 * num_kv_heads;
  // 32 elements per lane once there are enough rows for every SIMD to hold
  // several waves of them; 16 below that, where the per-row chain is the cost
  const bool bulk = rows >= kBulkRows;
  const int e = bulk ? 32 : 16;
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
      INT4KV_W(BF, DD, 32); \
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
