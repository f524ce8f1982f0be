// INT4 paged decode attention, LDS-staged variant (gfx950).
//
// Same method as decode.hip (rotated Q, split-dot score with the sum(Q)*zp
// correction, online softmax, split-K segments merged by the reduction pass;
// PR #40633's description), with a different data path:
//
//  * The workgroup owns HPW <= 8 KV heads of its (sequence, segment), so the K
//    and V halves of a cache block it reads are 16-byte-aligned runs
//    (16 tokens x HPW x R bytes).  Each 2-block tile is copied HBM -> LDS with
//    global_load_lds_dwordx4 by all waves together (every 128-byte line is
//    fetched once, non-temporal) into a ring of 3 to 6 stages (as deep as the
//    160 KiB of LDS allows).  A tile's words are read one step before its
//    math, so at the barrier of step t the stage of tile t is already free and
//    takes tile t + S: S - 2 to S - 1 tiles stay in flight.  The
//    copies are issued from inline assembly and waited for with explicit
//    vmcnt so the compiler does not drain the ring at every barrier.  When a token's run is
//    a whole number of 16-byte chunks, token rows are re-laid out in LDS with a
//    stride of 12 dwords mod 32 so the per-lane row reads spread over the banks.
//  * Q . K^T runs on the int8 MFMA (v_mfma_i32_16x16x64_i8): K codes become
//    int8 with one mask (low nibbles) and a shift + mask (high nibbles) per
//    dword; the rotated query is held as a fixed-point value below 2^22 in
//    magnitude (23 bits with the sign) split into three int8 planes
//    (p2 * 65536 + p1 * 256 + p0): exact integer products, planes combined in
//    fp32.
//  * P . V runs on the f16 MFMA with the softmax weights W = p * s_V split into
//    f16 hi + lo (22 significant bits; f16 alone leaves an error of 2^-11 of
//    |V| in the output).  V enters as raw bit patterns: a byte of two slot
//    keys' dwords, zero-extended into f16 halves, is the subnormal pair
//    (low + 16 high) * 2^-24, and masked to 0x000F000F the low nibbles alone;
//    per byte one column tile takes the whole bytes and one the low nibbles,
//    the high nibble's column is their difference / 16.  Single products
//    are exact; the matrix cores sum a dot product's products in a window
//    anchored at the largest operand exponents (a subnormal operand's leading
//    zeros spend part of it) and keep only the top bits of an incoming
//    accumulator that the products outweigh, so each tile's products are
//    summed from zero and the tiles are accumulated in fp32 on the vector
//    ALU.  The 2^24 (2^20) is applied per output column at the end.
//  * The next tile's scores are computed on the matrix cores while the
//    current tile's softmax runs; the softmax reference maximum moves only
//    when a logit exceeds it by 4 (base-2 units, a factor 16 in probability),
//    checked per logit, so row maxima are reduced and accumulators rescaled
//    only on the rare tiles that need it.
//  * Fused decode step: given one new token per sequence, the workgroup whose
//    segment holds the sequence's last block encodes and stores that token's
//    rows (the cache write's own encoding, encode_row.h) before its copy of
//    the block, so the write needs no launch of its own.
#include <type_traits>

#include "device_common.h"
#include "encode_row.h"
#include "launch.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace int4kv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 4.0f;  // headroom of the softmax reference maximum (log2 units)

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// 16 bytes per lane from global memory (uniform base + 32-bit lane offset)
// straight into LDS at M0 + lane * 16.  Marked non-temporal: every cache line
// is read once, so it should not displace lines that are reused.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, mask, c, 0xEA);  // (a & mask) | c
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of a DPP row (rotations by 8 and 4, then the quad
// swaps): four v_max_f32 with DPP operands.  Scores are finite or -inf (masked
// keys are selected, never computed), so no NaN handling is needed here.
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  return x;
}

// Compile-time geometry of the LDS image of one tile (two cache blocks).
// INT2 mode: the 4-level Lloyd-Max quantizer of N(0, 1) (Max, 1960, N = 4)
// has levels -b, -a, a, b for codes 0..3.  With the code's bits (hi, lo),
// level + b = (a + b) hi + (b - a) lo (the scores: unsigned bit planes on
// the exact int8 matrix cores, b leaving through the query-sum term), and
// level = u sigma + v tau with the signed planes sigma = 2 hi - 1,
// tau = 2 lo - 1, u = (a + b)/2, v = (b - a)/2 (P.V: centred operands).
constexpr float kLmA = 0.4527800346f, kLmB = 1.5104176085f;
constexpr float kLm2u = kLmA + kLmB, kLm2v = kLmB - kLmA;
constexpr float kLmU = 0.5f * kLm2u, kLmV = 0.5f * kLm2v;

template <int D, int HPW, bool Q8 = false, bool Q2 = false>
struct Geo {
  // row bytes (INT8: d codes + scale; INT2: d/4 code bytes + scale)
  static constexpr uint32_t R = Q8 ? D + 4 : Q2 ? D / 4 + 4 : D / 2 + 4;
  static constexpr uint32_t run = HPW * R;                 // bytes of the group's heads per token
  static constexpr bool kTokenRows = run % 16 == 0;        // token runs are whole chunks
  static constexpr uint32_t TS =                           // LDS token stride
      kTokenRows && ((run / 4) % 8 == 0) ? run + 16 : run;
  static constexpr uint32_t lhalf = 16 * TS;               // one K or V half
  static constexpr uint32_t blk_chunks = 2 * lhalf / 16;   // 16-byte chunks per block image
  static constexpr int UPB = (2 * lhalf + 1023) / 1024;    // 1 KiB DMA units per block
  static constexpr uint32_t BLK = UPB * 1024;              // LDS offset of block 1
  static constexpr int U = 2 * UPB;                        // units per tile
  static constexpr int NI = (U + HPW - 1) / HPW;           // DMA instructions of waves [0, NREM)
  static constexpr int NREM = U % HPW == 0 ? HPW : U % HPW;  // the others issue NI - 1
  static constexpr uint32_t stage = U * 1024;
};

// Per-wave W tile: one 80-byte row per query head of the group (8 rows for
// groups of up to 8 heads, else 16), the weights split into f16 hi rows and
// lo rows (22 significant bits), each half padded to a multiple of 256 bytes
// so the bank pattern is the same for both; then a zero row placed on the
// banks the rows of 4 query heads leave free.
template <int G>
struct WGeo {
  static constexpr uint32_t ROWS = G <= 8 ? 8 : 16;
  static constexpr uint32_t WROW = 80;
  static constexpr uint32_t WLO = (ROWS * WROW + 255) / 256 * 256;
  static constexpr uint32_t WZERO = 2 * WLO + 48;
  static constexpr uint32_t wtile = WZERO + 64;
};

// Whole LDS budget: S ring stages (the last one also holds the staged query in
// the prologue, widened when the query is larger) and the W tiles.  S is the
// deepest ring that fits the 160 KiB of a gfx950 CU, at most 6 for a full
// 8-head workgroup (one per CU) and at most 4 for smaller ones (several per CU
// share the LDS).
template <int D, int G, int HPW, bool Q8 = false, bool Q2 = false>
struct Lay {
  using GG = Geo<D, HPW, Q8, Q2>;
  static constexpr uint32_t qstage = HPW * (G * D * 4 + 2 * G * 4);
  static constexpr uint32_t last = GG::stage > qstage ? GG::stage : qstage;
  static constexpr uint32_t bytes(int s) {
    return (s - 1) * GG::stage + last + HPW * WGeo<G>::wtile;
  }
  static constexpr bool fits(int s) { return s <= (HPW == 8 ? 6 : 4) && bytes(s) <= 160 * 1024; }
  static constexpr int S = fits(6) ? 6 : fits(5) ? 5 : fits(4) ? 4 : 3;
  static constexpr uint32_t qbase = (S - 1) * GG::stage;
  static constexpr uint32_t wbase = qbase + last;
  static constexpr uint32_t total = wbase + HPW * WGeo<G>::wtile;
};

template <bool BF16, int D, int G, int HPW, bool Q8, bool Q2>
__global__ __launch_bounds__(64 * HPW) void decode_lds_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, uint16_t* __restrict__ out,
    const uint8_t* __restrict__ cache, int32_t num_kv_heads, int32_t num_q_heads,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ seqused_k,
    const int32_t* __restrict__ block_table, int32_t bt_stride, float scale_log2,
    const float* __restrict__ signs, int32_t num_segments, float* __restrict__ segm_out,
    float* __restrict__ segm_max, float* __restrict__ segm_sum,
    const uint16_t* __restrict__ key_new, int64_t key_new_stride,
    const uint16_t* __restrict__ value_new, int64_t value_new_stride,
    const int64_t* __restrict__ slot_new, int64_t num_slots, int32_t window, float cap2,
    float inv_cap2) {
  using GG = Geo<D, HPW, Q8, Q2>;
  using WG = WGeo<G>;
  using LY = Lay<D, G, HPW, Q8, Q2>;
  constexpr uint32_t R = GG::R;
  constexpr int DW = Q8 ? D / 4 : Q2 ? D / 16 : D / 8;  // code dwords per row
  constexpr int DWG = DW / 4;    // code dwords per lane group in the score operand
  constexpr int NCK = Q2 ? D / 32 : D / 64;  // int8 MFMA k-chunks (INT2: two bit planes)
  constexpr int NCOL = D / 16;   // P.V column tiles (INT2: elements per lane)
  constexpr int NACC = Q2 ? 2 * NCOL : NCOL;  // P.V accumulators (INT2: sigma and tau sums)
  constexpr int RPG = G <= 4 ? 1 : G / 4;
  constexpr int EPL = G * D / 64;
  constexpr int LPQ = 64 / G;
  constexpr int NI = GG::NI;
  constexpr int S = LY::S;

  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y, seg = blockIdx.x;
  const int h0 = blockIdx.z * HPW;
  const int h = h0 + wave;
  const int col = lane & 15, g = lane >> 4;

  const int q0 = cu_seqlens_q[b];
  const int qlen = cu_seqlens_q[b + 1] - q0;
  const int L = seqused_k[b];
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  // the query sits at L - 1; with a window it sees keys [lo, L) and the
  // segments split the blocks from the first one it sees
  const int lo = (window > 0 && L - window > 0) ? L - window : 0;
  const int blo = lo / kBlockSize;
  const int per = (nblk - blo + num_segments - 1) / num_segments;
  const int b0 = blo + seg * per;
  const int b1 = min(b0 + per, nblk);
  const int ntile = b1 > b0 ? (b1 - b0 + 1) / 2 : 0;

  // ---- fused decode step: the new token of sequence b (its last key, at
  // position L - 1) is encoded exactly as the cache write does and stored by
  // the workgroup whose segment holds that key's block, before any copy of
  // the block is issued.  The writing waves' stores complete before a barrier
  // that precedes that copy: the barrier right here (vmcnt 0) when the
  // block's tile is among the first S - 1 (copied before the loop), else the
  // wait for tile 0 ahead of the loop's first barrier, as vector memory
  // operations retire in issue order and the stores precede tile 0's
  // copies.  The block is read only by this workgroup, through L2.
  if (!Q8 && !Q2 && slot_new != nullptr) {  // (the INT8 and INT2 modes have no fused step)
    const int64_t slot = slot_new[b];
    // (slots outside [0, num_slots) are not stored, as in the cache write)
    if ((uint64_t)slot < (uint64_t)num_slots && L > 0 &&
        ((L - 1) / kBlockSize - blo) / per == seg) {  // uniform over the workgroup
      constexpr int WE = 16, WLPR = D / WE, WRPW = kWave / WLPR;  // rows of 8 or 4 lanes
      if (wave * WRPW < 2 * HPW) {
        const int r = wave * WRPW + lane / WLPR;  // row kv * HPW + head of the group
        const int rr = min(r, 2 * HPW - 1);      // spare lanes encode a valid row, store nothing
        const int sub = lane % WLPR, kv = rr / HPW, hd = h0 + rr % HPW;
        const uint16_t* src = (kv == 0 ? key_new + (int64_t)b * key_new_stride
                                       : value_new + (int64_t)b * value_new_stride) +
                              (int64_t)hd * D + WE * sub;
        u32x4_t in[WE / 8];
#pragma unroll
        for (int k = 0; k < WE / 8; ++k) in[k] = reinterpret_cast<const u32x4_t*>(src)[k];
        uint32_t flip[WE / 2];
        row_flips<WE>(signs, sub, flip);
        float x[WE];
        row_inputs<BF16, WE>(in, flip, x);
        uint32_t packed[WE / 8];
        const uint32_t word = encode_piece<WE, WLPR>(x, sub, packed);
        if (r < 2 * HPW) {
          const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
          uint8_t* dst = const_cast<uint8_t*>(cache) +
                         (((blk * 2 + kv) * kBlockSize + off) * num_kv_heads + hd) * R;
          uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + (WE / 2) * sub);
#pragma unroll
          for (int k = 0; k < WE / 8; ++k) d32[k] = packed[k];
          if (sub == 0) reinterpret_cast<uint32_t*>(dst)[D / 8] = word;
        }
      }
      if (ntile <= S - 1) {
        wait_vmem<0>();  // the stores have reached L2
        __syncthreads();
      }  // else the wait for tile 0 before the loop's first barrier covers them
    }
  }
  if (qlen <= 0) return;  // uniform over the workgroup

  const uint32_t tok_g = (uint32_t)num_kv_heads * R;  // global token stride
  const uint32_t half_g = 16 * tok_g;
  const uint32_t pair_g = 2 * half_g;  // bytes per cache block (K and V halves)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  unsigned char* wt = smem + LY::wbase + wave * WG::wtile;  // this wave's W tile

  // ---- per-lane DMA sources (loop invariant).  Instruction i of wave w copies
  // unit u = i*HPW + w < U; units [0, UPB) hold block 0, [UPB, U) block 1; the
  // padding chunks of token rows and of the last unit re-read valid chunks.
  const bool full = wave < GG::NREM;  // this wave issues NI copies per tile, else NI - 1
  uint32_t goff[NI];
  {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int u = min(i * HPW + wave, GG::U - 1);
      const int blk = u >= GG::UPB ? 1 : 0;
      uint32_t pos = (uint32_t)(u - blk * GG::UPB) * 64 + lane;  // chunk in the block image
      if (pos >= GG::blk_chunks) pos = GG::blk_chunks - 1;
      uint32_t off;
      if constexpr (GG::kTokenRows) {
        constexpr uint32_t TSC = GG::TS / 16, RC = GG::run / 16;
        const uint32_t kv = pos / (16 * TSC), r = pos - kv * 16 * TSC;
        const uint32_t tok = r / TSC;
        uint32_t cc = r - tok * TSC;
        if (cc >= RC) cc = RC - 1;
        off = kv * half_g + tok * tok_g + (uint32_t)h0 * R + 16 * cc;
      } else {  // only when the group holds every head: the half is one slab
        const uint32_t kv = pos / GG::run;
        off = kv * half_g + (pos - kv * GG::run) * 16;
      }
      goff[i] = off;
    }
  }
  // block ids of the next tiles to copy (two slots), read one step before
  // they are needed so the scalar loads never stall the copy issue
  uint32_t nid[2][2] = {{0u, 0u}, {0u, 0u}};
  auto load_ids = [&](int slot, int tile) {
    nid[slot][0] = (uint32_t)bt[min(b0 + 2 * tile, b1 - 1)];
    nid[slot][1] = (uint32_t)bt[min(b0 + 2 * tile + 1, b1 - 1)];
  };
  auto issue = [&](int slot, int tile) {  // nid[slot] holds this tile's block ids
    const uint8_t* p0 = cache + (uint64_t)nid[slot][0] * pair_g;
    const uint8_t* p1 = cache + (uint64_t)nid[slot][1] * pair_g;
    asm volatile("" : "+s"(p0), "+s"(p1));  // keep both bases in SGPRs; select per copy
    const uint32_t sb = lds0 + (uint32_t)(tile % S) * GG::stage + (uint32_t)wave * 1024;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i == NI - 1 && !full) break;
      const int u = i * HPW + wave;
      dma16(u >= GG::UPB ? p1 : p0, goff[i], sb + (uint32_t)(i * HPW) * 1024);
    }
  };
  // wait until at most `ahead` tiles of this wave's copies are in flight
  auto wait_tiles = [&](auto ahead) {
    if (full)
      wait_vmem<decltype(ahead)::value * NI>();
    else
      wait_vmem<decltype(ahead)::value * (NI - 1)>();
  };

  // ---- prologue: q' = H (signs * q) as fixed point below 2^22, staged in the last stage
  int32_t* q24 = reinterpret_cast<int32_t*>(smem + LY::qbase) + wave * G * D;
  float* qinfo =
      reinterpret_cast<float*>(smem + LY::qbase + HPW * G * D * 4) + wave * 2 * G;
  {
    const int i = lane / LPQ, s = lane % LPQ;
    const uint16_t* qp = q + (int64_t)q0 * q_stride + (int64_t)(h * G + i) * D + s * EPL;
    float x[EPL];
    if constexpr (Q8) {  // no rotation: the INT8 rows hold the original domain
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = to_f32<BF16>(qp[e]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = to_f32<BF16>(qp[e]) * signs[s * EPL + e];
#pragma unroll
      for (int span = 1; span < EPL; span <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          if (e & span) continue;
          const float u = x[e], v = x[e + span];
          x[e] = u + v;
          x[e + span] = u - v;
        }
      }
#pragma unroll
      for (int m = 1; m < LPQ; m <<= 1) {
        const bool upper = (s & m) != 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float p = shfl_xor_rt(x[e], m);
          x[e] = upper ? p - x[e] : x[e] + p;
        }
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < LPQ; m <<= 1) mx = fmaxf(mx, shfl_xor_rt(mx, m));
    const int ex = mx > 0.f ? ilogbf(mx) + 1 : 0;  // |q'| * 2^-ex < 1
    // |v| <= 2^22: the centred planes p0, p1 in [-128, 127] then leave the top
    // plane p2 within [-65, 65], so no value is ever clamped.  INT2 stages the
    // unrounded x * 2^(22 - ex) instead: each bit plane's weight (< 1.97) is
    // applied before the one rounding, so weighted values stay below
    // 1.97 * 2^22 < 127 * 65536 + 127 * 257 and p2 within [-127, 127]
    constexpr int QB = 22;
    const float nrm = ldexpf(1.0f, QB - ex);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float xs = x[e] * nrm;  // exact: a power-of-two scaling
      const float v = rintf(xs);
      q24[i * D + s * EPL + e] = Q2 ? __builtin_bit_cast(int, xs) : (int)v;
      sum += v;  // < 2^29 in magnitude; its rounding is far below the score's
    }
#pragma unroll
    for (int m = 1; m < LPQ; m <<= 1) sum += shfl_xor_rt(sum, m);
    if (s == 0) {
      qinfo[2 * i + 0] = sum;
      qinfo[2 * i + 1] = scale_log2 * ldexpf(1.0f, ex - QB);
    }
  }
  // tiles 0 .. S-2 now; tile S-1 goes into the last stage once every wave has
  // read the staged query (the barrier where tile 0 has landed).  Copies past
  // the segment's end re-read its last block, so the vmcnts below are exact.
  if (ntile > 0) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i) {
      load_ids(0, i);
      issue(0, i);
    }
    load_ids(0, S - 1);
  }
  // zero row of the W tile (MFMA rows that carry no query head read it)
  if (lane < 16) reinterpret_cast<uint32_t*>(wt + WG::WZERO)[lane] = 0u;
  __syncthreads();

  // int8 planes of Q in the score MFMA's A layout.  Lane group g reads its K
  // segment dwords in the rotated order j = (q + g) % DWG (spreads LDS banks);
  // slot (rho, beta) of chunk k then holds element
  // 8 * (g*DWG + (2k + rho/2 + g) % DWG) + 2*beta + rho%2 (INT4: low nibbles are
  // the even elements), or 4 * (g*DWG + (4k + rho + g) % DWG) + beta (INT8:
  // byte beta of a dword is its element).
  i32x4_t qa[3][NCK];
  {
    const int r = col, grp = r >> 2, vv = r & 3;
    const int qh = grp * RPG + vv;
    const bool ok = vv < RPG && qh < G;
#pragma unroll
    for (int k = 0; k < NCK; ++k) {
#pragma unroll
      for (int rho = 0; rho < 4; ++rho) {
        uint32_t pw[3] = {0u, 0u, 0u};
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
          int v;
          if constexpr (Q2) {
            // chunk k: code dword k / 2 of the lane group, bit plane k % 2
            // (0: high bits, weight a + b; 1: low bits, weight b - a); slot
            // (rho, beta) is element 4 beta + rho of that dword
            const int j = (k / 2 + g) % DWG;
            const int d = 16 * (g * DWG + j) + 4 * beta + rho;
            v = ok ? (int)rintf(__builtin_bit_cast(float, q24[qh * D + d]) *
                                ((k & 1) ? kLm2v : kLm2u))
                   : 0;
          } else {
            const int j = Q8 ? (4 * k + rho + g) % DWG : (2 * k + (rho >> 1) + g) % DWG;
            const int d = Q8 ? 4 * (g * DWG + j) + beta : 8 * (g * DWG + j) + 2 * beta + (rho & 1);
            v = ok ? q24[qh * D + d] : 0;
          }
          const int p0 = ((v + 128) & 0xFF) - 128, r1 = (v - p0) >> 8;
          const int p1 = ((r1 + 128) & 0xFF) - 128, p2 = (r1 - p1) >> 8;
          pw[0] |= (uint32_t)(p0 & 0xFF) << (8 * beta);
          pw[1] |= (uint32_t)(p1 & 0xFF) << (8 * beta);
          pw[2] |= (uint32_t)(p2 & 0xFF) << (8 * beta);
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) qa[pl][k][rho] = (int)pw[pl];
      }
    }
  }
  float qsf[RPG], c0[RPG];
  bool qok[RPG];
#pragma unroll
  for (int v = 0; v < RPG; ++v) {
    const int qh = g * RPG + v;
    qok[v] = qh < G;
    qsf[v] = qok[v] ? qinfo[2 * qh] : 0.f;
    c0[v] = qok[v] ? qinfo[2 * qh + 1] : 0.f;
  }

  float m_run[RPG], thr[RPG], l_run[RPG], corr[RPG];
  // column tile 2*beta: sum of W * (low nibble of byte beta) in units of 2^-24;
  // tile 2*beta + 1: sum of W * (whole byte beta = low + 16 * high nibble)
  float4_t oacc[NACC];
#pragma unroll
  for (int v = 0; v < RPG; ++v) {
    m_run[v] = -INFINITY;  // an empty segment reports m = -inf, l = 0
    thr[v] = -INFINITY;
    l_run[v] = 0.f;
    corr[v] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NACC; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  // INT4 / INT8: the P.V sums of the last tile, added to oacc at the start
  // of the next step (the matrix cores' latency is then covered)
  float4_t pend[NACC];
#pragma unroll
  for (int c = 0; c < NACC; ++c) pend[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int noff = (D == 64) ? 4 * (col >> 3) : 0;  // nibble offset of this lane's V dword
  // O (rotated domain, zero point not yet removed) of column tile c: the low
  // nibble directly, the high nibble as (byte - low) / 16 (INT4); INT8: every
  // tile holds whole codes offset by 128
  auto o_of = [&](int c, int v) -> float {
    if constexpr (Q8) return oacc[c][v] * 16777216.0f;  // 2^24
    if constexpr (Q2)  // element c: u * sum W sigma + v * sum W tau = sum W level
      return fmaf(kLmU, oacc[2 * c][v], kLmV * oacc[2 * c + 1][v]);
    return (c & 1) ? (oacc[c][v] - oacc[c - 1][v]) * 1048576.0f  // 2^20
                   : oacc[c][v] * 16777216.0f;                   // 2^24
  };
  // INT8 V: the lane's elements NCOL * col .. + NCOL - 1 are NVD dwords of a row
  constexpr int NVD = Q8 ? NCOL / 4 : 1;
  constexpr int NVA = 8 * NVD;  // V dwords per lane per tile
  // v_perm selectors: byte beta (+ noff / 2) of two slot keys' dwords, each
  // zero-extended into one f16 half
  uint32_t vsel[NCOL / 2];
#pragma unroll
  for (int bb = 0; bb < NCOL / 2; ++bb) {
    const uint32_t by = (uint32_t)(bb + noff / 2);
    vsel[bb] = 0x0C000C00u | by | ((4u + by) << 16);
  }

  // INT2: byte bl of the lane's NCOL / 4 V bytes (elements NCOL * col ..),
  // of two slot keys' dwords, each zero-extended into an f16 half
  uint32_t vsel2[Q2 ? NCOL / 4 : 1];
#pragma unroll
  for (int bl = 0; bl < (Q2 ? NCOL / 4 : 1); ++bl) {
    const uint32_t by = (uint32_t)((NCOL / 4) * col + bl) & 3u;
    vsel2[bl] = 0x0C000C00u | by | ((4u + by) << 16);
  }

  // per-lane LDS byte offsets inside a stage (loop invariant)
  const uint32_t hoff = (uint32_t)wave * R;
  const uint32_t row_off = col * GG::TS + hoff;
  uint32_t k_off[DWG];
#pragma unroll
  for (int qq = 0; qq < DWG; ++qq) k_off[qq] = row_off + 4 * (g * DWG + (qq + g) % DWG);
  const uint32_t ks_off = row_off + (Q8 ? D : Q2 ? D / 4 : D / 2);  // + n*BLK (+ lhalf for V)
  uint32_t v_off[NVA];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kk = ((j & 1) << 4) + 4 * g + (j >> 1);  // key of P.V slot j (pairs 4g+i, 16+4g+i)
    const uint32_t kb0 = (kk >> 4) * GG::BLK + GG::lhalf + (kk & 15) * GG::TS + hoff;
#pragma unroll
    for (int w = 0; w < NVD; ++w)
      v_off[j * NVD + w] = kb0 + 4 * (Q8 ? NVD * col + w : Q2 ? NCOL * col / 16 : col % DW);
  }
  // W tile addressing: writer (col, g) -> row qh, dword col; reader (row r, g)
  // -> 16 bytes at dword 4g of its query head's row (or the zero row).  Rows
  // are 80 bytes apart so the 16-byte reads of 8 lanes fall in distinct banks.
  uint32_t wr_off[RPG];
#pragma unroll
  for (int v = 0; v < RPG; ++v) wr_off[v] = (uint32_t)min(g * RPG + v, (int)WG::ROWS - 1) * WG::WROW + 4 * col;
  uint32_t rd_off, rd_lo;
  {
    const int grp = col >> 2, vv = col & 3, qh = grp * RPG + vv;
    const bool valid = vv < RPG && qh < G;
    rd_off = (valid ? (uint32_t)qh * WG::WROW : WG::WZERO) + 16 * g;
    rd_lo = (valid ? WG::WLO + (uint32_t)qh * WG::WROW : WG::WZERO) + 16 * g;
  }

  // ---- int8 K operands of one tile (low nibbles as is, high nibbles shifted)
  auto k_operands = [&](const unsigned char* st, i32x4_t (&kb)[2][NCK]) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      uint32_t segw[DWG];
#pragma unroll
      for (int qq = 0; qq < DWG; ++qq)
        segw[qq] = *reinterpret_cast<const uint32_t*>(st + n * GG::BLK + k_off[qq]);
#pragma unroll
      for (int k = 0; k < NCK; ++k) {
        if constexpr (Q2) {  // one bit plane of a code dword: byte beta, position rho
          const uint32_t w = segw[k / 2];
          const int sh = (k & 1) ? 0 : 1;
#pragma unroll
          for (int rho = 0; rho < 4; ++rho)
            kb[n][k][rho] = (int)((w >> (2 * rho + sh)) & 0x01010101u);
        } else if constexpr (Q8) {  // int8 codes as they are
#pragma unroll
          for (int rho = 0; rho < 4; ++rho) kb[n][k][rho] = (int)segw[4 * k + rho];
        } else {
          const uint32_t w0 = segw[2 * k], w1 = segw[2 * k + 1];
          kb[n][k][0] = (int)(w0 & 0x0F0F0F0Fu);
          kb[n][k][1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
          kb[n][k][2] = (int)(w1 & 0x0F0F0F0Fu);
          kb[n][k][3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
        }
      }
    }
  };
  // score group i (block n = i / NCK, k-chunk k = i % NCK): the three planes
  // S_p += Q_p . K (exact int32)
  auto score_group = [&](int i, const i32x4_t (&kb)[2][NCK], i32x4_t (&acc)[2][3]) {
    const int n = i / NCK, k = i % NCK;
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
      acc[n][pl] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          qa[pl][k], kb[n][k], k == 0 ? i32x4_t{0, 0, 0, 0} : acc[n][pl], 0, 0, 0);
  };
  constexpr int NGROUP = 2 * NCK;
  // emits score group `i` of the next tile if it exists, then fences the phase
  auto phase_end = [&](int i, const i32x4_t (&kb)[2][NCK], i32x4_t (&acc)[2][3]) {
    if (i < NGROUP) {
      score_group(i, kb, acc);
      // one MFMA, then a few vector instructions, so the matrix core works
      // while this wave keeps issuing
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- one pipelined step: the scores of tile t+1 (matrix cores) are
  // interleaved, phase by phase, with the softmax of tile t (vector ALU); then
  // O += W V for tile t.
  // LDS words of a tile needed after its scores: scale words and V bytes
  struct TileWords {
    uint32_t kw[2], vw[2], va[NVA];
  };
  auto tile_words = [&](const unsigned char* st, TileWords& w) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      w.kw[n] = *reinterpret_cast<const uint32_t*>(st + n * GG::BLK + ks_off);
      w.vw[n] = *reinterpret_cast<const uint32_t*>(st + n * GG::BLK + GG::lhalf + ks_off);
    }
#pragma unroll
    for (int j = 0; j < NVA; ++j) w.va[j] = *reinterpret_cast<const uint32_t*>(st + v_off[j]);
  };

  auto step = [&](int t, const i32x4_t (&acc)[2][3], i32x4_t (&nxt)[2][3],
                  const TileWords& cw, TileWords& nw) {
    wait_tiles(std::integral_constant<int, S - 2>());  // this wave's copies of tile t+1
    __syncthreads();  // ... and everyone's.  Every wave read tile t's words in step t-1
                      // (LDS reads complete before the barrier), so its stage is free:
    issue(0, t + S);  // tile t+S (clamped to the segment's last block)
    load_ids(0, t + S + 1);
    const unsigned char* st = smem + (uint32_t)(t % S) * GG::stage;
    const int tb = b0 + 2 * t;

    // phase 0: LDS reads of tile t+1 (K, scale words, V); tile t's words were
    // read one step earlier, so the softmax below starts from registers.
    // After the last tile, tile t+1 is a clamped copy of the last block: its
    // words and scores are never used.
    i32x4_t kb[2][NCK];
    const unsigned char* sn = smem + (uint32_t)((t + 1) % S) * GG::stage;
    k_operands(sn, kb);
    tile_words(sn, nw);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!Q2) {  // tile t-1's P.V sums, under the reference they were taken with
#pragma unroll
      for (int c = 0; c < NACC; c += Q8 ? 1 : 2) oacc[c] += pend[c];
    }

    // phase 1: logits z = c0 sK (S - zK sum(q')) in base-2 units
    bool kval[2];
    float sV[2], zV[2];
    float z[RPG][2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int key = tb * kBlockSize + 16 * n + col;
      kval[n] = (tb + n < b1) & (key < L) & (key >= lo);  // no short circuit: no branch
      // INT4: zero point in the scale word's low 4 bits; INT8: a plain fp32
      // scale, no K zero point, and V codes offset by 128 (see the V operands)
      // INT2: plain fp32 scales; the score planes give sum q (level + b), so
      // b leaves through the query-sum term; the V operands are centred (no
      // V zero point)
      const float sK = as_float((Q8 || Q2) ? cw.kw[n] : cw.kw[n] & 0xFFFFFFF0u);
      const float zK = Q8 ? 0.f : Q2 ? kLmB : (float)(cw.kw[n] & 0xFu);
      sV[n] = kval[n] ? as_float((Q8 || Q2) ? cw.vw[n] : cw.vw[n] & 0xFFFFFFF0u) : 0.f;  // masked: 0
      zV[n] = Q8 ? 128.f : Q2 ? 0.f : (float)(cw.vw[n] & 0xFu);
#pragma unroll
      for (int v = 0; v < RPG; ++v) {
        const float sf = fmaf((float)acc[n][2][v], 65536.0f,
                              (float)((acc[n][1][v] << 8) + acc[n][0][v]));
        const float tt = fmaf(-zK, qsf[v], sf);  // sum_i q_i (code_i - zp)
        z[v][n] = tt * (sK * c0[v]);
      }
    }
    if (cap2 > 0.f) {  // uniform; one branch for the tile
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int v = 0; v < RPG; ++v) z[v][n] = soft_cap(z[v][n], cap2, inv_cap2);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      // masked keys become -inf through a bitwise select (never a branch)
      const uint32_t keep = kval[n] ? 0xFFFFFFFFu : 0u;
      const uint32_t ninf = kval[n] ? 0u : 0xFF800000u;
#pragma unroll
      for (int v = 0; v < RPG; ++v) z[v][n] = as_float(and_or(as_uint(z[v][n]), keep, ninf));
    }
    phase_end(0, kb, nxt);

    // reference maxima.  The reference m of a row only moves when a logit
    // exceeds it by more than kLazy (base-2 units), so p = 2^(z - m) <= 2^kLazy;
    // that is checked per logit against thr = m + kLazy, and the row maxima are
    // reduced and the accumulators rescaled only on the rare tiles where it
    // happens.  m, l and O always share one reference, which is all the merge
    // and the normalisation need.
    bool over = false;
#pragma unroll
    for (int v = 0; v < RPG; ++v) over |= (z[v][0] > thr[v]) | (z[v][1] > thr[v]);
    if (__any(over)) {
#pragma unroll
      for (int v = 0; v < RPG; ++v) {
        const float tmax = max16(fmaxf(z[v][0], z[v][1]));
        const bool up = tmax > thr[v];
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run[v] - tmax) : 1.0f;
        m_run[v] = up ? tmax : m_run[v];
        thr[v] = m_run[v] + kLazy;
        l_run[v] *= alpha;
        if constexpr (!Q2) corr[v] *= alpha;  // INT2 has no V zero-point term
#pragma unroll
        for (int c = 0; c < NACC; ++c) oacc[c][v] *= alpha;
      }
    }

    // phase 2: probabilities, weights W = p sV as f16 hi + lo, sums, zero-point term
#pragma unroll
    for (int v = 0; v < RPG; ++v) {
      const float p0 = __builtin_amdgcn_exp2f(z[v][0] - m_run[v]);
      const float p1 = __builtin_amdgcn_exp2f(z[v][1] - m_run[v]);
      const float w0 = p0 * sV[0], w1 = p1 * sV[1];
      half2_t wh, wl;
      wh[0] = (_Float16)w0;
      wh[1] = (_Float16)w1;
      wh = opaque(wh);  // lo is taken against this hi
      wl[0] = (_Float16)(w0 - (float)wh[0]);
      wl[1] = (_Float16)(w1 - (float)wh[1]);
      l_run[v] += p0 + p1;
      if constexpr (!Q2) corr[v] = fmaf(w1, zV[1], fmaf(w0, zV[0], corr[v]));
      *reinterpret_cast<half2_t*>(wt + wr_off[v]) = wh;
      *reinterpret_cast<half2_t*>(wt + WG::WLO + wr_off[v]) = wl;
    }
    // weights in the A layout, read back from this wave's W tile right away
    // (LDS operations of one wave complete in order); the latency is covered
    // by the work up to the P.V products
    const half8_t wop = *reinterpret_cast<const half8_t*>(wt + rd_off);
    const half8_t wop_lo = *reinterpret_cast<const half8_t*>(wt + rd_lo);
    phase_end(1, kb, nxt);
    // acc += W B for one column tile of subnormal codes (INT4, INT8).  The
    // tile's products are summed on the matrix cores from zero (hi, then lo
    // on top) and tiles are accumulated in fp32 on the vector ALU: the matrix
    // cores cut a dot product off about 24 bits below the largest operand
    // exponents, where a subnormal code counts as 2^-14, so an incoming
    // running sum that a heavier key's products outweigh keeps only about 15
    // bits there.
    auto pv_tile = [&](const half8_t& bop) {
      const float4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          wop, bop, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(wop_lo, bop, t, 0, 0, 0);
    };
    auto pv = [&](float4_t& dst, const half8_t& bop) { dst = pv_tile(bop); };

    if constexpr (Q2) {
      // phase 3 (INT2): byte bl of the lane's dword of two slot keys, zero-
      // extended into f16 halves; element 4 bl + k enters as the signed
      // planes sigma = 2 hi - 1 and tau = 2 lo - 1, each +-1.0 (the bit
      // shifted into the sign position, inverted and merged with the
      // magnitude in one bitop3).  Centred, normal operands: the matrix cores
      // sum a dot product's products in a window anchored at the largest
      // operand exponents and cut off below it, and a subnormal operand's
      // leading zeros spend that window, so 2-bit codes as subnormals would
      // lose the smaller weights' products; and unsigned codes with the
      // offset b taken out in fp32 afterwards would turn such losses into an
      // offset common to every rotated element (output element 0).
      uint32_t vx2[NCOL / 4][4];
#pragma unroll
      for (int bl = 0; bl < NCOL / 4; ++bl)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vx2[bl][i] = __builtin_amdgcn_perm(cw.va[2 * i + 1], cw.va[2 * i], vsel2[bl]);
      phase_end(2, kb, nxt);
#pragma unroll
      for (int bl = 0; bl < NCOL / 4; ++bl)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = 4 * bl + k;
          constexpr uint32_t mag = 0x3C003C00u;  // 1.0 in both halves
          u32x4_t xs, xt;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // (~shifted & sign bits) | magnitude: sign set where the bit is 0
            xs[i] = __builtin_amdgcn_bitop3_b32(vx2[bl][i] << (14 - 2 * k), 0x80008000u, mag, 0xAE);
            xt[i] = __builtin_amdgcn_bitop3_b32(vx2[bl][i] << (15 - 2 * k), 0x80008000u, mag, 0xAE);
          }
          const half8_t sb = __builtin_bit_cast(half8_t, xs);
          const half8_t tb = __builtin_bit_cast(half8_t, xt);
          // the +-1.0 operands are normal numbers, so the matrix cores'
          // running sums keep fp32 precision across tiles: no per-tile flush
          oacc[2 * e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, sb, oacc[2 * e], 0, 0, 0);
          oacc[2 * e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop_lo, sb, oacc[2 * e], 0, 0, 0);
          oacc[2 * e + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, tb, oacc[2 * e + 1], 0, 0, 0);
          oacc[2 * e + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(wop_lo, tb, oacc[2 * e + 1], 0, 0, 0);
        }
    } else if constexpr (Q8) {
      // phase 3 (INT8): column tile c takes byte c % 4 of the lane's dword
      // c / 4 of two slot keys, each zero-extended into an f16 half with its
      // top bit flipped: the subnormal (code + 128) * 2^-24, exact in the
      // products; the 128 leaves through the zero-point term (zV = 128).
      uint32_t vx8[NCOL][4];
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const uint32_t bsel = 0x0C000C00u | (uint32_t)(c & 3) | ((4u + (c & 3)) << 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vx8[c][i] = __builtin_amdgcn_perm(cw.va[(2 * i + 1) * NVD + (c >> 2)],
                                            cw.va[2 * i * NVD + (c >> 2)], bsel) ^ 0x00800080u;
      }
      phase_end(2, kb, nxt);
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        pv(pend[c], __builtin_bit_cast(half8_t, vx8[c]));
      }
    } else {
    // phase 3: V operands.  Byte beta of the lane's dword of two slot keys,
    // each zero-extended into an f16 half: the subnormal (low + 16 * high) *
    // 2^-24; single products are exact.
    uint32_t vx[NCOL / 2][4];
#pragma unroll
    for (int bb = 0; bb < NCOL / 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vx[bb][i] = __builtin_amdgcn_perm(cw.va[2 * i + 1], cw.va[2 * i], vsel[bb]);
    phase_end(2, kb, nxt);

    // O += W V: per byte, one column tile on the low nibbles (masked) and one
    // on the whole bytes; the high nibble's column is their difference / 16.
#pragma unroll
    for (int bb = 0; bb < NCOL / 2; ++bb) {
      u32x4_t vl;
#pragma unroll
      for (int i = 0; i < 4; ++i) vl[i] = vx[bb][i] & 0x000F000Fu;
      // whole bytes straight into the running sums: their columns reach the
      // output only through the high nibble, (bytes - low) / 16, which
      // scales a truncated running sum down by 16; the low nibbles, whose
      // sums are the output as they are, go through the per-tile flush
      {
        const half8_t xb = __builtin_bit_cast(half8_t, vx[bb]);
        float4_t& ox = oacc[2 * bb + 1];
        ox = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, xb, ox, 0, 0, 0);
        ox = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop_lo, xb, ox, 0, 0, 0);
      }
      pv(pend[2 * bb], __builtin_bit_cast(half8_t, vl));
    }
    }
    // the remaining score groups of tile t+1 share this region: one MFMA per
    // vector instruction of the low-nibble masks
#pragma unroll
    for (int i = 3; i < NGROUP; ++i) score_group(i, kb, nxt);
#pragma unroll
    for (int j = 0; j < 2 * NACC + 3 * (NGROUP > 3 ? NGROUP - 3 : 0); ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop.  Tile t+1 must have landed at the top of step t; tiles
  // t+2 .. t+S-1 are in flight, and t+S joins them.  Unrolled by two so the
  // score accumulators alternate without copies.
  i32x4_t accA[2][3], accB[2][3];
  TileWords wA, wB;
  if (ntile > 0) {
    wait_tiles(std::integral_constant<int, S - 2>());  // tile 0
    __syncthreads();
    issue(0, S - 1);  // the staged query has been read by every wave
    load_ids(0, S);
    i32x4_t kb[2][NCK];
    k_operands(smem, kb);
    tile_words(smem, wA);
#pragma unroll
    for (int i = 0; i < NGROUP; ++i) score_group(i, kb, accA);
  }
  int t = 0;
  for (; t + 1 < ntile; t += 2) {
    step(t, accA, accB, wA, wB);
    step(t + 1, accB, accA, wB, wA);
  }
  if (t < ntile) step(t, accA, accB, wA, wB);
  wait_vmem<0>();  // drain the clamped look-ahead copies
  if constexpr (!Q2) {  // the last tile's P.V sums
#pragma unroll
    for (int c = 0; c < NACC; c += Q8 ? 1 : 2) oacc[c] += pend[c];
  }

  // ---- finalise: sums over the 16 lanes of a group
#pragma unroll
  for (int v = 0; v < RPG; ++v) {
    l_run[v] += shfl_xor<1>(l_run[v]);
    l_run[v] += shfl_xor<2>(l_run[v]);
    l_run[v] += shfl_xor<4>(l_run[v]);
    l_run[v] += shfl_xor<8>(l_run[v]);
    if constexpr (!Q2) {
      corr[v] += shfl_xor<1>(corr[v]);
      corr[v] += shfl_xor<2>(corr[v]);
      corr[v] += shfl_xor<4>(corr[v]);
      corr[v] += shfl_xor<8>(corr[v]);
    }
  }
  // column tile c holds element dof(c) of this lane
  auto dof = [&](int c) -> int {
    if constexpr (Q8 || Q2) return NCOL * col + c;  // the V elements the lane read
    return D == 128 ? 8 * col + c : 8 * (col & 7) + 4 * (col >> 3) + c;
  };

  if (num_segments > 1) {
#pragma unroll
    for (int v = 0; v < RPG; ++v) {
      if (!qok[v]) continue;
      const int qg = h * G + g * RPG + v;
      const int64_t base = ((int64_t)b * num_q_heads + qg) * num_segments + seg;
      float* dst = segm_out + base * D;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) dst[dof(c)] = o_of(c, v) - corr[v];
      if (col == 0) {
        segm_max[base] = m_run[v];
        segm_sum[base] = l_run[v];
      }
    }
    return;
  }

#pragma unroll
  for (int v = 0; v < RPG; ++v) {
    const float inv_l = l_run[v] > 0.f ? 1.0f / l_run[v] : 0.f;
    float o[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) o[c] = (o_of(c, v) - corr[v]) * inv_l;
    if constexpr (Q8) {  // the original domain already
      if (!qok[v]) continue;
      const int qg = h * G + g * RPG + v;
      uint16_t* dst = out + ((int64_t)q0 * num_q_heads + qg) * D;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) dst[dof(c)] = from_f32<BF16>(o[c]);
      continue;
    }
#pragma unroll
    for (int span = 1; span < (D == 128 ? 8 : 4); span <<= 1) {
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        if (c & span) continue;
        const float a = o[c], bb = o[c + span];
        o[c] = a + bb;
        o[c + span] = a - bb;
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const bool upper = (col & m) != 0;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const float p = shfl_xor_rt(o[c], m);
        o[c] = upper ? p - o[c] : o[c] + p;
      }
    }
    if (!qok[v]) continue;
    const int qg = h * G + g * RPG + v;
    uint16_t* dst = out + ((int64_t)q0 * num_q_heads + qg) * D;
    const float invD = 1.0f / (float)D;
#pragma unroll
    for (int c = 0; c < NCOL; ++c) dst[dof(c)] = from_f32<BF16>(o[c] * signs[dof(c)] * invD);
  }
}

template <bool BF16, int D, int G, int HPW, bool Q8, bool Q2>
hipError_t launch_h(const AttnArgs& a, hipStream_t stream) {
  using LY = Lay<D, G, HPW, Q8, Q2>;
  constexpr size_t lds = LY::total;
  static_assert(lds <= 160 * 1024, "LDS budget of a gfx950 CU");
  static_assert((LY::S - 2) * Geo<D, HPW, Q8, Q2>::NI <= 63, "vmcnt range");
  auto kern = decode_lds_kernel<BF16, D, G, HPW, Q8, Q2>;
  if (lds > 65536) {  // above the default dynamic LDS limit (gfx950 has 160 KiB per CU)
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.num_segments, a.num_seqs, a.num_kv_heads / HPW), block(64 * HPW);
  // INT4: q . x_hat = q' . y_hat / D in the rotated domain; INT8: no rotation
  const float scale_log2 = a.softmax_scale * kLog2e / (Q8 ? 1.0f : (float)D);
  const float cap2 = a.softcap > 0.f ? a.softcap * kLog2e : 0.f;  // base-2 units
  hipLaunchKernelGGL(kern, grid, block, lds, stream, reinterpret_cast<const uint16_t*>(a.q),
                     a.q_stride, reinterpret_cast<uint16_t*>(a.out), a.cache, a.num_kv_heads,
                     a.num_q_heads, a.cu_seqlens_q, a.seqused_k, a.block_table, a.bt_stride,
                     scale_log2, a.signs, a.num_segments, a.segm_out, a.segm_max, a.segm_sum,
                     reinterpret_cast<const uint16_t*>(a.key_new), a.key_new_stride,
                     reinterpret_cast<const uint16_t*>(a.value_new), a.value_new_stride,
                     a.slot_new, a.num_slots, a.window, cap2, cap2 > 0.f ? 1.0f / cap2 : 0.f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_segments == 1) return e;
  return launch_reduce(a, stream);
}

// KV heads per workgroup: up to 8 for INT4; up to 4 for INT8, whose rows are
// twice as long (a two-block tile of 4 heads is 34 KiB: a four-stage ring)
template <bool BF16, int D, int G, bool Q8, bool Q2>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  // INT2 with 16 query heads per KV head at d = 128 also takes 4: its 8-head
  // instance does not fit in 256 VGPRs (it spills to scratch)
  const int cap = (Q8 || (Q2 && G == 16 && D == 128)) ? 4 : 8;
  switch (a.num_kv_heads >= cap ? cap : a.num_kv_heads) {
    case 1: return launch_h<BF16, D, G, 1, Q8, Q2>(a, stream);
    case 2: return launch_h<BF16, D, G, 2, Q8, Q2>(a, stream);
    case 4: return launch_h<BF16, D, G, 4, Q8, Q2>(a, stream);
    default:
      if constexpr (Q8 || (Q2 && G == 16 && D == 128))
        return hipErrorInvalidValue;  // not reached: cap is 4
      else return launch_h<BF16, D, G, 8, Q8, Q2>(a, stream);
  }
}

template <bool BF16, int D, bool Q8, bool Q2>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_t<BF16, D, 1, Q8, Q2>(a, stream);
    case 2: return launch_t<BF16, D, 2, Q8, Q2>(a, stream);
    case 4: return launch_t<BF16, D, 4, Q8, Q2>(a, stream);
    case 8: return launch_t<BF16, D, 8, Q8, Q2>(a, stream);
    default: return launch_t<BF16, D, 16, Q8, Q2>(a, stream);
  }
}

template <bool Q8, bool Q2>
hipError_t launch_q(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) return a.head_size == 128 ? launch_d<true, 128, Q8, Q2>(a, stream)
                                        : launch_d<true, 64, Q8, Q2>(a, stream);
  return a.head_size == 128 ? launch_d<false, 128, Q8, Q2>(a, stream)
                            : launch_d<false, 64, Q8, Q2>(a, stream);
}

}  // namespace

bool decode_lds_supported(const AttnArgs& a) {
  const int hkv = a.num_kv_heads;
  return hkv == 1 || hkv == 2 || hkv == 4 || hkv == 8 || hkv % 8 == 0;
}

hipError_t launch_decode_lds(const AttnArgs& a, hipStream_t stream) {
  if (a.q8) return launch_q<true, false>(a, stream);
  if (a.q2) return launch_q<false, true>(a, stream);
  return launch_q<false, false>(a, stream);
}

}  // namespace int4kv
