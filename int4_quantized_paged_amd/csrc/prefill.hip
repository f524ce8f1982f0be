// INT4 paged attention for prefill / mixed batches (query lengths > 1), gfx950.
//
// Same method as the decode kernel (PR #40633's description: Q rotated into
// the cache's domain, split-dot score with a sum(Q) * zp correction, online
// softmax, per-stream accumulators; causal only per the PR #40835 report's
// risk list), organised for many query rows per key:
//
//  * One workgroup (8 waves) owns one (sequence, KV head, tile of 128/G query
//    tokens): 128 rows of (token, query head).  Waves 0-3 take the even key
//    tiles and waves 4-7 the odd ones (a split of the key range inside the
//    workgroup, merged through LDS at the end), so the longest contexts run as
//    two chains and every SIMD holds two waves; each wave owns 32 rows as two
//    16-row MFMA tiles, so each K/V tile read from LDS feeds two row tiles.
//  * The K and V rows of the head (R bytes at the cache's token stride) are
//    copied HBM -> LDS with global_load_lds_dword into an 8-stage ring, six
//    tiles ahead of the math; wave q of a group copies (block q/2, K|V q%2)
//    of each of the group's two-block tiles.  Rows land as 17-dword (d =
//    128) or 9-dword (d = 64) records, an odd stride, so the per-key reads of
//    16 lanes hit 16 banks.
//  * Codes enter the f16 MFMAs as raw bit patterns: K as (w & 0x000F000F), a
//    pair of f16 subnormals code * 2^-24, and (w & 0x00F000F0), 16 * code *
//    2^-24; V as whole bytes zero-extended into halves, (low + 16 high) *
//    2^-24, and their low nibbles, the high nibble's column taken as the
//    difference / 16.  Single products are exact; the low-nibble (INT8:
//    code) P . V columns of a tile are summed on the matrix cores from zero
//    and the tiles accumulated in fp32 on the vector ALU (an incoming
//    matrix-core accumulator keeps only its top bits when the products
//    outweigh it).  The 2^24 (and the 16) are folded into per-row and
//    per-column constants.
//  * Q . K^T: Q' as f16 hi + lo (22 significant bits), both against the same
//    K operand.  P . V: softmax weights times the V scale, also as f16 hi +
//    lo, as the A operand through a per-wave LDS tile, against V bytes
//    expanded per lane from one dword of each of 8 keys.
//  * Workgroups are numbered so that the KV heads of one (sequence, tile) run
//    on the same XCD (the heads of a token share 128-byte lines in L2), and
//    the (sequence, tile) groups start in descending order of the key tiles
//    they run (a counting sort each workgroup does at its start): the
//    longest causal chains begin first instead of running alone at the end.
//  * The INT8 per-token-head cache (the same kernel with Q8 set) has no
//    rotation and d + 4 byte rows: K and V codes enter as bytes with the top
//    bit flipped, (code + 128) * 2^-24, the 128 leaving through the same
//    zero-point terms, and Q is staged unrotated.
//  * The INT2 Lloyd-Max cache (Q2 set) keeps the INT4 rotation; its 2-bit
//    codes become their levels as f16 hi + lo pairs through a v_perm table
//    lookup, so K and V enter the same MFMAs as signed values with no
//    zero point (three products where the codes take two).
#include "device_common.h"
#include "launch.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace int4kv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 4.0f;  // headroom of the softmax reference maximum (log2 units)
// the reference of a row that has seen no key: finite, so such a row (or a key
// group that got only masked keys) gives p = 2^(-inf) = 0, never 2^(-inf + inf)
constexpr float kNoRef = -1e30f;
constexpr int kStages = 8;

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// 4 bytes per lane from global memory (uniform base + 32-bit lane offset)
// into LDS at M0 + lane * 4.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// maximum over the 16 lanes of a DPP row (logits are finite or -inf)
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  return x;
}

// INT2 mode: f16 bits of the 4-level Lloyd-Max levels of N(0, 1) (Max, 1960,
// N = 4: -b, -a, a, b for codes 0..3, a = 0.45278003, b = 1.51041761) as
// hi + lo pairs, two codes' levels per dword through one v_perm.
constexpr float kLmA = 0.4527800346f, kLmB = 1.5104176085f;
constexpr _Float16 kLh0 = (_Float16)(-kLmB), kLh1 = (_Float16)(-kLmA), kLh2 = (_Float16)kLmA,
                   kLh3 = (_Float16)kLmB;
constexpr _Float16 kLl0 = (_Float16)(-kLmB - (float)kLh0), kLl1 = (_Float16)(-kLmA - (float)kLh1),
                   kLl2 = (_Float16)(kLmA - (float)kLh2), kLl3 = (_Float16)(kLmB - (float)kLh3);
constexpr uint32_t f16pair(_Float16 x, _Float16 y) {
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
constexpr uint32_t kTh0 = f16pair(kLh0, kLh1), kTh1 = f16pair(kLh2, kLh3);
constexpr uint32_t kTl0 = f16pair(kLl0, kLl1), kTl1 = f16pair(kLl2, kLl3);

// levels of codes c0 (half 0) and c1 (half 1), each 0..3: hi and lo f16 pairs
__device__ __forceinline__ void lm_pair(uint32_t c0, uint32_t c1, uint32_t& hi, uint32_t& lo) {
  const uint32_t sel = 0x01000100u + (c0 | (c1 << 16)) * 0x0202u;  // bytes 2c, 2c + 1
  hi = __builtin_amdgcn_perm(kTh1, kTh0, sel);
  lo = __builtin_amdgcn_perm(kTl1, kTl0, sel);
}

template <int D, int G, bool Q8 = false, bool Q2 = false>
struct PGeo {
  // row bytes (INT8: d codes + scale; INT2: d/4 code bytes + scale)
  static constexpr int R = Q8 ? D + 4 : Q2 ? D / 4 + 4 : D / 2 + 4;
  static constexpr int RW = R / 4;                  // dwords per row
  static constexpr int DW = Q8 ? D / 4 : Q2 ? D / 16 : D / 8;  // code dwords per row
  static constexpr int NIB = (16 * RW + 63) / 64; // copies per (block, K|V) image
  static constexpr uint32_t HALF = NIB * 256;     // LDS bytes of one (block, K|V) image
  static constexpr uint32_t STAGE = 4 * HALF;     // two blocks, K and V
  static constexpr uint32_t RING = kStages * STAGE;
  static constexpr uint32_t QSTAGE = 128 * D * 2 * 2;  // hi and lo, operand order
  static constexpr uint32_t WBASE = RING > QSTAGE ? RING : QSTAGE;
  // per wave: 2 row tiles x 16 rows x 32 keys f16, rows padded to 80 bytes so
  // the 16-byte A-operand reads of 8 lanes cover all 32 banks
  static constexpr uint32_t WROW = 80;
  static constexpr uint32_t WTILE = 2 * 2 * 16 * WROW;  // hi and lo tiles of both row tiles
  // odd-tile group's state for the final merge: per lane 8 m, 8 l, 8 corr, 16*NCOL/2 O
  static constexpr uint32_t MERGE = 4 * 64 * (24 + 8 * (D / 16)) * 4;
  static constexpr uint32_t LOW = WBASE > MERGE ? WBASE : MERGE;
  static constexpr uint32_t TOTAL = LOW + 8 * WTILE;
  static constexpr int TQ = 128 / G;              // query tokens per workgroup
};

// Launch order of the (sequence, query tile) groups: a workgroup holds a
// whole CU, so the launch is a list schedule on the CUs, and starting the
// longest causal chains first keeps them from running alone at the end (the
// chunked-prefill mix: 17% fewer steps on the critical CU in a schedule
// simulation).  Weight of group j (sequence j / T, tile j % T) = key tiles
// its chains run; groups whose tile holds no query token weigh 0 and come
// last.  Rank = descending weight, ties by j, found by a counting sort over
// kRankBuckets buckets of the weight (scaled by max_tiles, the tile count of
// the longest sequence, when that exceeds the buckets).  Every workgroup
// computes the group of its own rank; -1 past the last non-empty group.
// Called by all 512 threads at the start of the kernel; uses the first
// (kRankBuckets + 516) ints of LDS and ends with a barrier.
constexpr int kRankBuckets = 1024;
constexpr int64_t kPrefillCUs = 256;  // MI355X: one prefill workgroup per CU at a time

template <int TQ>
__device__ int ranked_group(int rank, int num_seqs, int tiles_per_seq,
                            const int32_t* __restrict__ cu_seqlens_q,
                            const int32_t* __restrict__ seqused_k, int window, int max_tiles,
                            int* lds) {
  constexpr int NB = kRankBuckets, NT = 512;
  const int tid = threadIdx.x;
  const int ng = num_seqs * tiles_per_seq;
  int* hist = lds;
  int* part = lds + NB;
  int* res = part + NT;
  const int wdiv = max_tiles > NB - 2 ? max_tiles : NB - 2;
  auto bucket_of = [&](int j) -> int {  // 0: empty group; 1 .. NB-1 by weight
    const int b = j / tiles_per_seq, qt = j - b * tiles_per_seq;
    const int qlen = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    if (qt * TQ >= qlen) return 0;
    const int L = seqused_k[b];
    const int t_hi = min((qt + 1) * TQ, qlen) - 1;
    const int nkeys = L - qlen + t_hi + 1;
    const int pos_lo = L - qlen + qt * TQ;
    const int t0 = (window > 0 && pos_lo - window + 1 > 0) ? (pos_lo - window + 1) / 32 : 0;
    const int w = max((nkeys + 31) / 32 - t0, 0);
    return 1 + min((int)((int64_t)w * (NB - 2) / wdiv), NB - 2);
  };
  // inclusive prefix sum over the 512 threads (ascending tid), in `part`
  auto scan = [&](int v) -> int {
    part[tid] = v;
    __syncthreads();
#pragma unroll 1
    for (int off = 1; off < NT; off <<= 1) {
      const int u = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += u;
      __syncthreads();
    }
    return part[tid];
  };
  for (int i = tid; i < NB; i += NT) hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < ng; j += NT) atomicAdd(&hist[bucket_of(j)], 1);
  __syncthreads();
  // descending buckets: thread t owns NB-1-2t and NB-2-2t (thread 511 ends at bucket 0)
  const int bh = NB - 1 - 2 * tid, bl = bh - 1;
  const int mine = hist[bh] + hist[bl];
  const int incl = scan(mine);
  const int nonempty = part[NT - 1] - hist[0];  // (uniform)
  if (rank >= nonempty) {
    __syncthreads();
    return -1;
  }
  const int before = incl - mine;
  if (rank >= before && rank < incl) {  // exactly one thread
    const bool hi = rank < before + hist[bh];
    res[0] = hi ? bh : bl;
    res[1] = rank - (hi ? before : before + hist[bh]);
  }
  __syncthreads();
  const int B = res[0], k = res[1];
  // the k-th group of bucket B in index order
  const int chunk = (ng + NT - 1) / NT;
  const int j0 = tid * chunk, j1 = min(j0 + chunk, ng);
  int c = 0;
  for (int j = j0; j < j1; ++j) c += bucket_of(j) == B ? 1 : 0;
  __syncthreads();  // every thread has read res
  const int ci = scan(c);
  if (k >= ci - c && k < ci) {  // exactly one thread
    int left = k - (ci - c);
    for (int j = j0; j < j1; ++j) {
      if (bucket_of(j) != B) continue;
      if (left == 0) {
        res[2] = j;
        break;
      }
      --left;
    }
  }
  __syncthreads();
  const int gsel = res[2];
  __syncthreads();  // the caller reuses the LDS
  return gsel;
}

template <bool BF16, int D, int G, bool Q8, bool Q2>
__global__ __launch_bounds__(512) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, uint16_t* __restrict__ out,
    const uint8_t* __restrict__ cache, int32_t num_kv_heads, int32_t num_q_heads,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ seqused_k,
    const int32_t* __restrict__ block_table, int32_t bt_stride, float scale_log2,
    const float* __restrict__ signs, int32_t num_seqs, int32_t tiles_per_seq, int32_t window,
    float cap2, float inv_cap2, int32_t max_tiles, int32_t rank_groups) {
  using PG = PGeo<D, G, Q8, Q2>;
  constexpr int R = PG::R, RW = PG::RW, DW = PG::DW, NIB = PG::NIB;
  constexpr int NCH = D / 32;   // f16 MFMA k-chunks of the score
  constexpr int NCOL = D / 16;  // P.V column tiles
  constexpr int TQ = PG::TQ;
  constexpr int EPL = D / 2;    // prologue: elements per lane (2 lanes per row)

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave >> 2;  // key-tile group: 0 takes even tiles, 1 odd tiles
  const int wq = wave & 3;   // row quarter: rows 32 wq .. 32 wq + 31
  const int col = lane & 15, g = lane >> 4;

  // ---- workgroup -> (sequence, query tile, KV head): the heads of one
  // group share the XCD (id % 8); groups start in descending order of the
  // key tiles they run (ranked_group)
  const int id = blockIdx.x;
  const int rr = id >> 3;
  const int h = rr % num_kv_heads;
  const int rank = (rr / num_kv_heads) * 8 + (id & 7);
  if (rank >= num_seqs * tiles_per_seq) return;  // uniform over the workgroup
  // (a launch whose workgroups all fit on the CUs at once needs no order)
  const int grp = rank_groups ? ranked_group<TQ>(rank, num_seqs, tiles_per_seq, cu_seqlens_q,
                                                 seqused_k, window, max_tiles,
                                                 reinterpret_cast<int*>(smem))
                              : rank;
  if (grp < 0) return;  // uniform: past the last non-empty group
  const int b = grp / tiles_per_seq;
  const int qt = grp - b * tiles_per_seq;
  const int q0 = cu_seqlens_q[b];
  const int qlen = cu_seqlens_q[b + 1] - q0;
  if (qt * TQ >= qlen) return;  // uniform over the workgroup
  const int L = seqused_k[b];
  const int t_hi = min((qt + 1) * TQ, qlen) - 1;  // last valid token of this tile
  const int nkeys = L - qlen + t_hi + 1;          // keys the last row sees
  const int ntiles = nkeys > 0 ? (nkeys + 31) / 32 : 0;
  const int nblk = (nkeys + kBlockSize - 1) / kBlockSize;
  const int pos_lo = L - qlen + qt * TQ;          // position of the first row's token
  // sliding window (keys [pos - window + 1, pos] per row): the first row's
  // window start bounds the key range from below; tiles before it are skipped
  const int last_lo = L - qlen + t_hi - window + 1;  // the last row's window start
  const int t0 = (window > 0 && pos_lo - window + 1 > 0) ? (pos_lo - window + 1) / 32 : 0;

  // ---- prologue: q' = H (signs * q), normalised per row to |q'| < 2^10, split
  // into f16 hi + lo and staged in LDS in the MFMA operand order
  _Float16* sq = reinterpret_cast<_Float16*>(smem);  // [128 rows][2][NCH][4][8]
  float* sinfo = reinterpret_cast<float*>(smem + PG::LOW);  // [128 + 4], reuses the W tiles
  if (kg == 0) {  // the even group rotates Q; both groups read it
    const int row = 32 * wq + (lane >> 1), s = lane & 1;
    const int tq = min(qt * TQ + row / G, qlen - 1);  // rows past the end repeat the last token
    const int qh = row % G;
    const uint16_t* qp = q + (int64_t)(q0 + tq) * q_stride + (int64_t)(h * G + qh) * D + s * EPL;
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
      for (int e = 0; e < EPL; ++e) {
        const float p = shfl_xor<1>(x[e]);
        x[e] = s ? p - x[e] : x[e] + p;
      }
    }
    // one exponent for the wave's 32 rows, so the logit scale is one constant
    // per wave (a row far below the wave's maximum keeps fewer significant
    // bits, but its logits, and their absolute error, are as small)
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mx = fmaxf(mx, shfl_xor_rt(mx, m));
    const int ex = mx > 0.f ? ilogbf(mx) + 1 : 0;  // |q'| * 2^(10-ex) < 2^10
    const float nrm = ldexpf(1.0f, 10 - ex);
    float sum = 0.f;
#pragma unroll
    for (int e8 = 0; e8 < EPL / 8; ++e8) {
      // elements el = s*EPL + 8*e8 + j sit in chunk el/32, lane group (el%32)/8
      // and slot {0,2,4,6,1,3,5,7}[j]; slots of odd j meet codes scaled by 16
      half8_t hi8, lo8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[8 * e8 + j] * nrm;
        const _Float16 hv = (_Float16)v;
        const _Float16 lv = (_Float16)(v - (float)hv);
        sum += (float)hv + (float)lv;
        // INT4 operand order [e0 e4 e1 e5 e2 e6 e3 e7], odd elements against
        // codes scaled by 16; INT8 [e0 e2 e1 e3 e4 e6 e5 e7], codes as they are
        // (INT2: natural order, against the levels of 8 consecutive codes)
        const int slot = Q2 ? j : Q8 ? (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1)
                                     : ((j & 3) << 1) | (j >> 2);
        hi8[slot] = (!Q8 && !Q2 && (j & 1)) ? (_Float16)((float)hv * 0.0625f) : hv;
        lo8[slot] = (!Q8 && !Q2 && (j & 1)) ? (_Float16)((float)lv * 0.0625f) : lv;
      }
      const int el = s * EPL + 8 * e8;
      const int off = ((row * 2 + 0) * NCH + el / 32) * 32 + ((el % 32) / 8) * 8;
      *reinterpret_cast<half8_t*>(sq + off) = hi8;
      *reinterpret_cast<half8_t*>(sq + off + NCH * 32) = lo8;
    }
    sum += shfl_xor<1>(sum);
    if (s == 0) sinfo[row] = sum * 5.9604644775390625e-08f;  // sum(q') in 2^-24 code units
    // codes enter as 2^-24 units, INT2 levels as themselves
    if (lane == 0) sinfo[128 + wq] = scale_log2 * ldexpf(1.0f, ex - 10 + (Q2 ? 0 : 24));
  }
  __syncthreads();

  // A operands of the score: row tile i = rows 32w + 16i + col
  half8_t qa_hi[2][NCH], qa_lo[2][NCH];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * wq + 16 * i + col;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qa_hi[i][c] = *reinterpret_cast<const half8_t*>(sq + ((row * 2 + 0) * NCH + c) * 32 + g * 8);
      qa_lo[i][c] = *reinterpret_cast<const half8_t*>(sq + ((row * 2 + 1) * NCH + c) * 32 + g * 8);
    }
  }
  // per-row constants in the accumulator layout: register v of row tile i is
  // row 32w + 16i + 4g + v
  float qsum[2][4];
  int pos[2][4];
  const float c0 = sinfo[128 + wq];  // logit units (base 2) per unit of S
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * wq + 16 * i + 4 * g + v;
      qsum[i][v] = sinfo[row];
      pos[i][v] = L - qlen + min(qt * TQ + row / G, qlen - 1);
    }
  __syncthreads();  // the staged Q and the row constants are consumed; the ring may start

  // ---- K/V copies: wave q of group k copies (block q/2, K|V q%2) of tiles
  // 2s + k
  const uint32_t tok_g = (uint32_t)num_kv_heads * R;
  const uint32_t half_g = 16 * tok_g;
  const uint32_t pair_g = 2 * half_g;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  const int my_blk = wq >> 1;
  const uint32_t my_half = (uint32_t)(wq & 1) * half_g + (uint32_t)h * R;
  uint32_t goff[NIB];
#pragma unroll
  for (int i = 0; i < NIB; ++i) {
    const int idx = min(i * 64 + lane, 16 * RW - 1);  // padding lanes re-read the last dword
    goff[i] = (uint32_t)(idx / RW) * tok_g + (uint32_t)(idx % RW) * 4;
  }
  uint32_t nid = 0;  // block id of the next tile to copy, read one step ahead
  auto load_id = [&](int tile) { nid = (uint32_t)bt[min(2 * tile + my_blk, nblk - 1)]; };
  auto issue = [&](int tile) {  // nid holds this tile's block id for this wave
    const uint8_t* p = cache + (uint64_t)nid * pair_g + my_half;
    const uint32_t sb = lds0 + (uint32_t)(tile % kStages) * PG::STAGE + (uint32_t)wq * PG::HALF;
#pragma unroll
    for (int i = 0; i < NIB; ++i) dma4(p, goff[i], sb + (uint32_t)i * 256);
  };

  float m_run[2][4], l_run[2][4], corr[2][4];
  bool all_ref = false;  // every row of the wave holds a reference (uniform)
  float4_t oacc[2][NCOL];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m_run[i][v] = kNoRef;
      l_run[i][v] = 0.f;
      corr[i][v] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < NCOL; ++c) oacc[i][c] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS byte offsets inside a stage (loop invariant)
  const uint32_t krow = (uint32_t)col * RW * 4;  // key col's record in a (block, K) image
  uint32_t k_off[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)  // INT8: two dwords (8 codes) per lane group and chunk;
    // INT2: half a dword (8 codes), dword 2c + g/2
    k_off[c] = krow + (Q2 ? (uint32_t)(2 * c + g / 2) * 4 : (uint32_t)(4 * c + g) * (Q8 ? 8 : 4));
  const uint32_t s_off = krow + (uint32_t)(RW - 1) * 4;  // scale word
  // INT8 V: the lane's elements NCOL * col .. + NCOL - 1 are NVD dwords of a row
  constexpr int NVD = Q8 ? NCOL / 4 : 1;
  uint32_t v_off[8 * NVD];  // slot j = 2i + n <-> key 16n + g + 4i
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = j & 1, t = g + 4 * (j >> 1);
#pragma unroll
    for (int w = 0; w < NVD; ++w)
      v_off[j * NVD + w] = (uint32_t)(2 * n + 1) * PG::HALF + (uint32_t)t * RW * 4 +
                           (uint32_t)(Q8 ? NVD * col + w : Q2 ? NCOL * col / 16 : col % DW) * 4;
  }
  unsigned char* wt = smem + PG::LOW + wave * PG::WTILE;
  // W tile: the f16 pair of key col (blocks 0 and 1) of row r sits at dword
  // 4 (col % 4) + col / 4, so reader group g (dwords 4g..4g+3) gets keys g + 4i
  uint32_t wr_off[4];  // writer: rows 4g + v
#pragma unroll
  for (int v = 0; v < 4; ++v)
    wr_off[v] = (uint32_t)(4 * g + v) * PG::WROW + 4 * (4 * (col % 4) + col / 4);
  const uint32_t rd_off = (uint32_t)col * PG::WROW + 16 * g;  // reader: row col
  const int noff = (D == 64) ? 4 * (col >> 3) : 0;      // nibble offset of this lane's V dword
  // v_perm selectors: byte bb (+ noff / 2) of two slot keys' dwords, each
  // zero-extended into one f16 half
  uint32_t vsel[NCOL / 2];
#pragma unroll
  for (int bb = 0; bb < NCOL / 2; ++bb) {
    const uint32_t by = (uint32_t)(bb + noff / 2);
    vsel[bb] = 0x0C000C00u | by | ((4u + by) << 16);
  }

  // steps s = 0 .. nsteps-1 process tiles t0 + 2s (even group) and t0 + 2s + 1
  // (odd group); each group keeps kPairs - 1 of its own tiles in flight.  A
  // tile past the last one (odd count) is a clamped copy whose keys are all
  // masked.
  constexpr int kPairs = kStages / 2;
  const int nsteps = (ntiles - t0 + 1) / 2;
  if (nsteps > 0) {
#pragma unroll
    for (int i = 0; i < kPairs - 1; ++i) {
      load_id(t0 + 2 * i + kg);
      issue(t0 + 2 * i + kg);
    }
    load_id(t0 + 2 * (kPairs - 1) + kg);
  }

  // One step of the key group.  `fastc`: every row of the wave holds a
  // reference maximum and there is no soft cap, so the logits enter the
  // softmax in one fused step; the steps before that (the rows' first keys)
  // and all steps under a soft cap take the general path.  The two kinds of
  // step are separate loops, so neither carries the other's registers.
  auto step = [&](const int sidx, auto fastc) {
    constexpr bool kFast = decltype(fastc)::value;
    const int t = t0 + 2 * sidx + kg;
    wait_vmem<(kPairs - 2) * NIB>();  // this wave's copies of tile t have landed
    __syncthreads();                  // ... and everyone's; everyone is done with step s-1
    issue(t + 2 * (kPairs - 1));      // into the stage of tile t-2 (clamped to the last block)
    load_id(t + 2 * kPairs);
    const unsigned char* st = smem + (uint32_t)(t % kStages) * PG::STAGE;

    // K operands: raw code dword (block n, chunk c) -> 4 dwords of f16 subnormals
    uint32_t va[8 * NVD];
#pragma unroll
    for (int j = 0; j < 8 * NVD; ++j) va[j] = *reinterpret_cast<const uint32_t*>(st + v_off[j]);
    half8_t kb[2][Q2 ? 1 : NCH];
    uint32_t kw[2], vw[2];
    float4_t sacc[2][2];
    if constexpr (Q2) {
      // INT2: each chunk's level operands (hi, lo) feed the score MFMAs at
      // once: S = q_hi L_hi + q_lo L_hi + q_hi L_lo (L_lo q_lo is 2^-22 below)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int n = 0; n < 2; ++n) sacc[i][n] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 2; ++n) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(st + 2 * n * PG::HALF + k_off[c]);
          const uint32_t u = w >> (16 * (g & 1));
          u32x4_t lh, ll;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uint32_t h2, l2;
            lm_pair((u >> (4 * m)) & 3u, (u >> (4 * m + 2)) & 3u, h2, l2);
            lh[m] = h2;
            ll[m] = l2;
          }
          const half8_t kh = __builtin_bit_cast(half8_t, lh);
          const half8_t kl = __builtin_bit_cast(half8_t, ll);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            sacc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[i][c], kh, sacc[i][n], 0, 0, 0);
            sacc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[i][c], kh, sacc[i][n], 0, 0, 0);
            sacc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[i][c], kl, sacc[i][n], 0, 0, 0);
          }
        }
        kw[n] = *reinterpret_cast<const uint32_t*>(st + 2 * n * PG::HALF + s_off);
        vw[n] = *reinterpret_cast<const uint32_t*>(st + (2 * n + 1) * PG::HALF + s_off);
      }
    } else {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(st + 2 * n * PG::HALF + k_off[c]);
        const uint32_t w8 = w >> 8;
        u32x4_t r;
        if constexpr (Q8) {  // bytes zero-extended with the top bit flipped: code + 128
          const uint32_t x = *reinterpret_cast<const uint32_t*>(st + 2 * n * PG::HALF + k_off[c] + 4);
          r[0] = (w & 0x00FF00FFu) ^ 0x00800080u;
          r[1] = (w8 & 0x00FF00FFu) ^ 0x00800080u;
          r[2] = (x & 0x00FF00FFu) ^ 0x00800080u;
          r[3] = ((x >> 8) & 0x00FF00FFu) ^ 0x00800080u;
        } else {
          r[0] = w & 0x000F000Fu;
          r[1] = w & 0x00F000F0u;
          r[2] = w8 & 0x000F000Fu;
          r[3] = w8 & 0x00F000F0u;
        }
        kb[n][c] = __builtin_bit_cast(half8_t, r);
      }
      kw[n] = *reinterpret_cast<const uint32_t*>(st + 2 * n * PG::HALF + s_off);
      vw[n] = *reinterpret_cast<const uint32_t*>(st + (2 * n + 1) * PG::HALF + s_off);
    }

    // scores: S[i][n] for row tile i, keys 16n + col (sum of q' * code * 2^-24)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        float4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          a = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[i][c], kb[n][c], a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[i][c], kb[n][c], a, 0, 0, 0);
        }
        sacc[i][n] = a;
      }
    }

    // online softmax (base 2) per row; keys past a row's position are masked
    // uniform: only tiles near the diagonal, or near a row's window start
    const bool masked = 32 * t + 31 > pos_lo || (window > 0 && 32 * t < last_lo);
    float sKc[2], zK[2], sV[2], zV[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      // INT4: zero points in the scale words' low 4 bits; INT8: plain fp32
      // scales, and the codes enter offset by 128 (K and V alike)
      // (INT2: plain scales and signed levels, no zero point)
      sKc[n] = as_float((Q8 || Q2) ? kw[n] : kw[n] & 0xFFFFFFF0u) * c0;
      zK[n] = Q8 ? 128.f : Q2 ? 0.f : (float)(kw[n] & 0xFu);
      sV[n] = as_float((Q8 || Q2) ? vw[n] : vw[n] & 0xFFFFFFF0u);
      zV[n] = Q8 ? 128.f : Q2 ? 0.f : (float)(vw[n] & 0xFu);
    }
    // logits in base-2 units, kept relative to the row's reference m:
    // d = z - m.  m only moves when a logit exceeds it by more than kLazy (so
    // p = 2^d <= 2^kLazy), and the row maxima are only reduced on the rare
    // tiles where that happens.  Once every row holds a reference, d is one
    // fma per logit from the score; while some row has none yet (its first
    // keys) and under a soft cap, the logit is formed first.
    float z[2][4][2];
    auto mask_all = [&]() {  // the causal / window mask
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int key = 32 * t + 16 * n + col;
            const bool in = key <= pos[i][v] && (window <= 0 || key > pos[i][v] - window);
            z[i][v][n] = in ? z[i][v][n] : -INFINITY;
          }
    };
    if constexpr (!kFast) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int n = 0; n < 2; ++n) z[i][v][n] = fmaf(-zK[n], qsum[i][v], sacc[i][n][v]) * sKc[n];
      if (cap2 > 0.f) {  // soft cap before the mask, so masked keys stay -inf
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int n = 0; n < 2; ++n) z[i][v][n] = soft_cap(z[i][v][n], cap2, inv_cap2);
      }
      if (masked) mask_all();
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // a row without a reference takes its maximum as one (its l, corr
          // and O are still zero); one whose keys are all masked keeps none
          const float tmax = max16(fmaxf(z[i][v][0], z[i][v][1]));
          if (m_run[i][v] == kNoRef && tmax > kNoRef) m_run[i][v] = tmax;
          z[i][v][0] -= m_run[i][v];
          z[i][v][1] -= m_run[i][v];
        }
      bool none = false;  // a row of this wave still without a reference
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) none |= m_run[i][v] == kNoRef;
      all_ref = !__any(none);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            z[i][v][n] = fmaf(fmaf(-zK[n], qsum[i][v], sacc[i][n][v]), sKc[n], -m_run[i][v]);
      if (masked) mask_all();
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fmaxf(z[i][v][0], z[i][v][1]));
    if (__any(mx > kLazy)) {  // move the references of the rows that outgrew theirs
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float dmax = max16(fmaxf(z[i][v][0], z[i][v][1]));
          const float mnew = dmax > kLazy ? m_run[i][v] + dmax : m_run[i][v];
          const float shift = mnew - m_run[i][v];  // 0 for a row that keeps its reference
          const float alpha = __builtin_amdgcn_exp2f(-shift);
          m_run[i][v] = mnew;
          l_run[i][v] *= alpha;
          corr[i][v] *= alpha;
#pragma unroll
          for (int c = 0; c < NCOL; ++c) oacc[i][c][v] *= alpha;
          z[i][v][0] -= shift;
          z[i][v][1] -= shift;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p0 = __builtin_amdgcn_exp2f(z[i][v][0]);
        const float p1 = __builtin_amdgcn_exp2f(z[i][v][1]);
        const float w0 = p0 * sV[0], w1 = p1 * sV[1];
        half2_t wh, wl;  // W = p sV as f16 hi + lo (22 significant bits)
        wh[0] = (_Float16)w0;
        wh[1] = (_Float16)w1;
        wh = opaque(wh);  // lo is taken against this hi
        wl[0] = (_Float16)(w0 - (float)wh[0]);
        wl[1] = (_Float16)(w1 - (float)wh[1]);
        l_run[i][v] += p0 + p1;
        corr[i][v] = fmaf(w1, zV[1], fmaf(w0, zV[0], corr[i][v]));
        *reinterpret_cast<half2_t*>(wt + (2 * i) * 16 * PG::WROW + wr_off[v]) = wh;
        *reinterpret_cast<half2_t*>(wt + (2 * i + 1) * 16 * PG::WROW + wr_off[v]) = wl;
      }
    // weights in the A layout, read back from this wave's W tiles (LDS
    // operations of one wave complete in order)
    half8_t wop[2], wlo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      wop[i] = *reinterpret_cast<const half8_t*>(wt + (2 * i) * 16 * PG::WROW + rd_off);
      wlo[i] = *reinterpret_cast<const half8_t*>(wt + (2 * i + 1) * 16 * PG::WROW + rd_off);
    }

    // Columns of subnormal codes whose sums reach the output directly (INT4
    // low nibbles, INT8 codes) are summed on the matrix cores from zero per
    // tile and accumulated in fp32 on the vector ALU: the matrix cores cut a
    // dot product off about 24 bits below the largest operand exponents,
    // where a subnormal code counts as 2^-14, so a running sum that a
    // heavier key's products outweigh keeps only its top bits.  INT2 levels
    // are normal f16 values and accumulate on the matrix cores.
    constexpr float4_t kZero4 = {0.f, 0.f, 0.f, 0.f};
    // V operands (shared by both row tiles) and O += W V.  Byte bb (+ noff/2)
    // of the lane's dword of two slot keys, zero-extended into f16 halves, is
    // the subnormal (low + 16 high) * 2^-24; masked, the low nibble alone.
    // Column tile 2bb takes the low nibbles, 2bb + 1 the whole bytes; the
    // high nibble's column is their difference / 16.  INT8: column tile c
    // takes byte c % 4 of the lane's dword c / 4 of two slot keys, top bit
    // flipped: the subnormal (code + 128) * 2^-24 (the 128 leaves through the
    // zero-point term, zV = 128).
    if constexpr (Q2) {
      // INT2: column tile c is element NCOL col + c of 8 slot keys; their
      // levels as hi + lo f16 pairs: O += W_hi L_hi + W_lo L_hi + W_hi L_lo
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const int sh = 2 * ((NCOL * col + c) & 15);
        u32x4_t lh, ll;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t h2, l2;
          lm_pair((va[2 * k] >> sh) & 3u, (va[2 * k + 1] >> sh) & 3u, h2, l2);
          lh[k] = h2;
          ll[k] = l2;
        }
        const half8_t vh = __builtin_bit_cast(half8_t, lh);
        const half8_t vl = __builtin_bit_cast(half8_t, ll);
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // normal operands: running sums on the matrix cores
          oacc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop[i], vh, oacc[i][c], 0, 0, 0);
          oacc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo[i], vh, oacc[i][c], 0, 0, 0);
          oacc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop[i], vl, oacc[i][c], 0, 0, 0);
        }
      }
    } else if constexpr (Q8) {
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const uint32_t bsel = 0x0C000C00u | (uint32_t)(c & 3) | ((4u + (c & 3)) << 16);
        u32x4_t vx;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          vx[k] = __builtin_amdgcn_perm(va[(2 * k + 1) * NVD + (c >> 2)],
                                        va[2 * k * NVD + (c >> 2)], bsel) ^ 0x00800080u;
        const half8_t xb = __builtin_bit_cast(half8_t, vx);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop[i], xb, kZero4, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo[i], xb, t, 0, 0, 0);
          oacc[i][c] += t;
        }
      }
    } else
#pragma unroll
    for (int bb = 0; bb < NCOL / 2; ++bb) {
      u32x4_t vx, vl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vx[k] = __builtin_amdgcn_perm(va[2 * k + 1], va[2 * k], vsel[bb]);
        vl[k] = vx[k] & 0x000F000Fu;
      }
      const half8_t xb = __builtin_bit_cast(half8_t, vx);
      const half8_t lb = __builtin_bit_cast(half8_t, vl);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // whole bytes straight into the running sums (they reach the output
        // only through the high nibble, (bytes - low) / 16); the low nibbles
        // from zero per tile, accumulated on the vector ALU
        float4_t& ox = oacc[i][2 * bb + 1];
        float4_t tl = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop[i], lb, kZero4, 0, 0, 0);
        ox = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop[i], xb, ox, 0, 0, 0);
        tl = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo[i], lb, tl, 0, 0, 0);
        ox = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo[i], xb, ox, 0, 0, 0);
        oacc[i][2 * bb] += tl;
      }
    }
  };
  int sidx = 0;
  for (; sidx < nsteps && (!all_ref || cap2 > 0.f); ++sidx) step(sidx, std::false_type{});
  for (; sidx < nsteps; ++sidx) step(sidx, std::true_type{});
  wait_vmem<0>();  // drain the clamped look-ahead copies

  // ---- merge the odd-tile group into the even one (same rows, wave q + 4 ->
  // wave q), through LDS; per-lane partial sums are merged before reduction
  __syncthreads();  // the ring is no longer read
  {
    float* mg = reinterpret_cast<float*>(smem) + (size_t)(wq * 64 + lane) * (24 + 8 * NCOL);
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          mg[(i * 4 + v) * 3 + 0] = m_run[i][v];
          mg[(i * 4 + v) * 3 + 1] = l_run[i][v];
          mg[(i * 4 + v) * 3 + 2] = corr[i][v];
#pragma unroll
          for (int c = 0; c < NCOL; ++c) mg[24 + (i * NCOL + c) * 4 + v] = oacc[i][c][v];
        }
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float m1 = mg[(i * 4 + v) * 3 + 0];
        const float mm = fmaxf(m_run[i][v], m1);
        // factors are 1 for a reference equal to the maximum (also when both
        // groups saw no key: m = -inf)
        const float f0 = m_run[i][v] == mm ? 1.0f : __builtin_amdgcn_exp2f(m_run[i][v] - mm);
        const float f1 = m1 == mm ? 1.0f : __builtin_amdgcn_exp2f(m1 - mm);
        l_run[i][v] = l_run[i][v] * f0 + mg[(i * 4 + v) * 3 + 1] * f1;
        corr[i][v] = corr[i][v] * f0 + mg[(i * 4 + v) * 3 + 2] * f1;
#pragma unroll
        for (int c = 0; c < NCOL; ++c)
          oacc[i][c][v] = oacc[i][c][v] * f0 + mg[24 + (i * NCOL + c) * 4 + v] * f1;
      }
  }

  // ---- finalise and rotate back.  Column tile c holds element dof(c) of this
  // lane: even tiles directly in units of 2^-24, odd ones as (bytes - low) in
  // units of 2^-20.
  auto dof = [&](int c) -> int {
    if constexpr (Q8 || Q2) return NCOL * col + c;  // the V elements the lane read
    return D == 128 ? 8 * col + c : 8 * (col & 7) + 4 * (col >> 3) + c;
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float lv = l_run[i][v], cv = corr[i][v];
      lv += shfl_xor<1>(lv);
      lv += shfl_xor<2>(lv);
      lv += shfl_xor<4>(lv);
      lv += shfl_xor<8>(lv);
      cv += shfl_xor<1>(cv);
      cv += shfl_xor<2>(cv);
      cv += shfl_xor<4>(cv);
      cv += shfl_xor<8>(cv);
      const float inv_l = lv > 0.f ? 1.0f / lv : 0.f;
      float o[NCOL];
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const float oc = Q2 ? oacc[i][c][v]  // levels as themselves
                         : (!Q8 && (c & 1)) ? (oacc[i][c][v] - oacc[i][c - 1][v]) * 1048576.0f
                                            : oacc[i][c][v] * 16777216.0f;  // 2^20 / 2^24
        o[c] = (oc - cv) * inv_l;
      }
      if constexpr (Q8) {  // the original domain already
        const int row = 32 * wq + 16 * i + 4 * g + v;
        const int tq = qt * TQ + row / G;
        if (tq < qlen) {
          const int qg = h * G + row % G;
          uint16_t* dst = out + ((int64_t)(q0 + tq) * num_q_heads + qg) * D;
#pragma unroll
          for (int c = 0; c < NCOL; ++c) dst[dof(c)] = from_f32<BF16>(o[c]);
        }
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
      const int row = 32 * wq + 16 * i + 4 * g + v;
      const int tq = qt * TQ + row / G;
      if (tq < qlen) {
        const int qg = h * G + row % G;
        uint16_t* dst = out + ((int64_t)(q0 + tq) * num_q_heads + qg) * D;
        const float invD = 1.0f / (float)D;
#pragma unroll
        for (int c = 0; c < NCOL; ++c) dst[dof(c)] = from_f32<BF16>(o[c] * signs[dof(c)] * invD);
      }
    }
}

template <bool BF16, int D, int G, bool Q8, bool Q2>
hipError_t launch_prefill_t(const AttnArgs& a, hipStream_t stream) {
  using PG = PGeo<D, G, Q8, Q2>;
  static_assert(PG::TOTAL <= 160 * 1024, "LDS of a gfx950 CU");
  auto kern = prefill_kernel<BF16, D, G, Q8, Q2>;
  if (PG::TOTAL > 65536) {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)PG::TOTAL);
    if (e != hipSuccess) return e;
  }
  const int tiles_per_seq = (a.max_seqlen_q + PG::TQ - 1) / PG::TQ;
  const int64_t groups = (int64_t)a.num_seqs * tiles_per_seq;
  const int64_t nwg = (groups + 7) / 8 * 8 * a.num_kv_heads;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // INT4: the rotation is an unnormalised Hadamard transform on both sides,
  // so q' . k' carries a factor D
  const float scale_log2 = a.softmax_scale * kLog2e / (Q8 ? 1.0f : (float)D);
  const float cap2 = a.softcap > 0.f ? a.softcap * kLog2e : 0.f;  // base-2 units
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(512), PG::TOTAL, stream,
                     reinterpret_cast<const uint16_t*>(a.q), a.q_stride,
                     reinterpret_cast<uint16_t*>(a.out), a.cache, a.num_kv_heads, a.num_q_heads,
                     a.cu_seqlens_q, a.seqused_k, a.block_table, a.bt_stride, scale_log2, a.signs,
                     a.num_seqs, tiles_per_seq, a.window, cap2, cap2 > 0.f ? 1.0f / cap2 : 0.f,
                     (a.max_seqlen_k + 31) / 32, nwg > kPrefillCUs ? 1 : 0);
  return hipGetLastError();
}

template <bool BF16, int D, bool Q8, bool Q2>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_t<BF16, D, 1, Q8, Q2>(a, stream);
    case 2: return launch_prefill_t<BF16, D, 2, Q8, Q2>(a, stream);
    case 4: return launch_prefill_t<BF16, D, 4, Q8, Q2>(a, stream);
    case 8: return launch_prefill_t<BF16, D, 8, Q8, Q2>(a, stream);
    default: return launch_prefill_t<BF16, D, 16, Q8, Q2>(a, stream);
  }
}

template <bool Q8, bool Q2>
hipError_t launch_prefill_q(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) return a.head_size == 128 ? launch_prefill_d<true, 128, Q8, Q2>(a, stream)
                                        : launch_prefill_d<true, 64, Q8, Q2>(a, stream);
  return a.head_size == 128 ? launch_prefill_d<false, 128, Q8, Q2>(a, stream)
                            : launch_prefill_d<false, 64, Q8, Q2>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  if (a.q8) return launch_prefill_q<true, false>(a, stream);
  if (a.q2) return launch_prefill_q<false, true>(a, stream);
  return launch_prefill_q<false, false>(a, stream);
}

}  // namespace int4kv
