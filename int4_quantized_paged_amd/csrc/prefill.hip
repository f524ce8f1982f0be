// INT4 paged attention for prefill / mixed batches (query lengths > 1), gfx950.
//
// Same method as the decode kernel (PR #40633's description: Q rotated into
// the cache's domain and split to match the nibble order, split-dot score with
// a sum(Q) * zp correction, online softmax, per-stream accumulators; causal
// only per the PR #40835 report's risk list), organised for many query rows:
//
// One workgroup (4 waves) owns one (sequence, KV head, tile of 64/G query
// tokens); its 64 rows are (token, query head) pairs, 16 per wave, so every
// 16x16x32 f16 MFMA tile is fully used.  Key tiles of 32 keys (2 cache blocks)
// are fetched once per workgroup (prefetched into registers one tile ahead),
// expanded from nibbles to f16 and stored in LDS:
//   K as [key][d] in the operand order of the score MFMA (padded rows),
//   V transposed as [d][key slot] for the P.V MFMA (xor-swizzled 16-byte chunks),
// so all four waves read their MFMA operands from LDS.  Softmax weights go
// back through a small per-wave LDS tile to become the A operand of P.V.
#include "device_common.h"
#include "launch.h"

namespace int4kv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8_t unpack8(uint32_t w) {
  u32x4_t r;
  r.x = nib_pair_f16(w);
  r.y = nib_pair_f16(w >> 4);
  r.z = nib_pair_f16(w >> 8);
  r.w = nib_pair_f16(w >> 12);
  return __builtin_bit_cast(half8_t, r);
}

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// Slot of tile-local key kk (0..31) in the P.V contraction: slots 8g..8g+7
// hold keys 4g + i (even slots) and 16 + 4g + i (odd slots), i = 0..3.
__device__ __forceinline__ int key_slot(int kk) {
  return 8 * ((kk & 15) >> 2) + 2 * (kk & 3) + (kk >> 4);
}

// Byte offset of (row d, slot chunk ch) in the transposed V tile: 64-byte rows,
// the 16-byte chunk index xor-swizzled by bits 3..4 of d.
__device__ __forceinline__ int vt_off(int d, int ch) { return d * 64 + 16 * (ch ^ ((d >> 3) & 3)); }

template <int D>
struct KVRegs {
  uint32_t k0, k1, v0, v1;  // dword w of keys kk and kk + 16 (K and V)
  uint32_t sw;              // a scale word (K or V) of one key, for threads that own one
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, uint16_t* __restrict__ out,
    const uint8_t* __restrict__ cache, int32_t num_kv_heads, int32_t num_q_heads,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ seqused_k,
    const int32_t* __restrict__ block_table, int32_t bt_stride, float scale_log2,
    const float* __restrict__ signs) {
  constexpr int NCH = D / 32;
  constexpr int NCOL = D / 16;
  constexpr int DW = D / 8;
  constexpr int R = D / 2 + 4;
  constexpr int TQ = 64 / G;        // query tokens per workgroup
  constexpr int KROW = D * 2 + 16;  // padded bytes per key row of the K tile
  constexpr int EPL = D / 4;        // prologue: elements per lane (4 lanes per row)

  __shared__ __align__(16) _Float16 s_qhi[64 * D];
  __shared__ __align__(16) _Float16 s_qlo[64 * D];
  __shared__ float s_qinfo[64 * 2];
  __shared__ __align__(16) unsigned char s_k[32 * KROW];
  __shared__ __align__(16) unsigned char s_vt[D * 64];
  __shared__ uint32_t s_kw[32], s_vw[32];
  __shared__ __align__(16) uint32_t s_w[4][16 * 16];  // per wave: W [16 rows][32 slots] f16

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qt = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int q0 = cu_seqlens_q[b];
  const int qlen = cu_seqlens_q[b + 1] - q0;
  if (qt * TQ >= qlen) return;  // uniform over the workgroup
  const int L = seqused_k[b];
  const int t_hi = min((qt + 1) * TQ, qlen) - 1;  // last valid token of this tile
  const int pos_max = L - qlen + t_hi;
  const int nkeys = pos_max + 1;
  const int ntiles = nkeys > 0 ? (nkeys + 31) / 32 : 0;
  const int nblk = (nkeys + kBlockSize - 1) / kBlockSize;

  // ---- prologue: rotate the 64 rows of Q (4 lanes per row), split into f16 hi + lo
  {
    const int row = 16 * wave + (lane >> 2), s = lane & 3;
    const int tq = min(qt * TQ + row / G, qlen - 1);  // rows past the end repeat the last token
    const int qh = row % G;
    const uint16_t* qp = q + (int64_t)(q0 + tq) * q_stride + (int64_t)(h * G + qh) * D + s * EPL;
    float x[EPL];
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
    for (int m = 1; m < 4; m <<= 1) {
      const bool upper = (s & m) != 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float p = shfl_xor_rt(x[e], m);
        x[e] = upper ? p - x[e] : x[e] + p;
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(x[e]));
    mx = fmaxf(mx, shfl_xor<1>(mx));
    mx = fmaxf(mx, shfl_xor<2>(mx));
    const int ex = mx > 0.f ? ilogbf(mx) + 1 : 0;
    const float nrm = ldexpf(1.0f, -ex);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float v = x[e] * nrm;
      const _Float16 hv = (_Float16)v;
      const _Float16 lv = (_Float16)(v - (float)hv);
      s_qhi[row * D + s * EPL + e] = hv;
      s_qlo[row * D + s * EPL + e] = lv;
      sum += (float)hv + (float)lv;
    }
    sum += shfl_xor<1>(sum);
    sum += shfl_xor<2>(sum);
    if (s == 0) {
      s_qinfo[2 * row] = sum;
      s_qinfo[2 * row + 1] = scale_log2 * ldexpf(1.0f, ex);
    }
  }
  __syncthreads();

  const int col = lane & 15, g = lane >> 4;
  half8_t qa_hi[NCH], qa_lo[NCH];
  {
    const int row = 16 * wave + col;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 8 * (g * NCH + c) + (j >> 1) + 4 * (j & 1);
        qa_hi[c][j] = s_qhi[row * D + d];
        qa_lo[c][j] = s_qlo[row * D + d];
      }
    }
  }
  // per-row constants in the accumulator layout: register v <-> row 16*wave + 4g + v
  float qsum[4], c0[4];
  int pos[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 16 * wave + 4 * g + v;
    qsum[v] = s_qinfo[2 * row];
    c0[v] = s_qinfo[2 * row + 1];
    const int tq = min(qt * TQ + row / G, qlen - 1);
    pos[v] = L - qlen + tq;
  }

  float m_run[4], l_run[4], corr[4];
  float4_t oacc[NCOL];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    m_run[v] = -INFINITY;
    l_run[v] = 0.f;
    corr[v] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NCOL; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- cooperative tile loads: thread -> (key pair kk / kk + 16, dword w)
  const int64_t tok_stride = (int64_t)num_kv_heads * R;
  const int64_t blk_bytes = (int64_t)kBlockSize * tok_stride;
  const int64_t head_off = (int64_t)h * R;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  const bool has_item = tid < 16 * DW;
  const int it_kk = tid & 15, it_w = (tid >> 4) % DW;
  // scale words: threads [0, 32) take K of key tid, [32, 64) V of key tid - 32
  // when D == 128; with D == 64 the idle threads [128, 192) do it instead.
  const int sw_base = (D == 128) ? 0 : 128;
  const bool has_sw = tid >= sw_base && tid < sw_base + 64;
  const int sw_key = (tid - sw_base) & 31, sw_v = ((tid - sw_base) >> 5) & 1;

  auto load = [&](int tile, KVRegs<D>& r) {
    const int bi0 = 2 * tile, bi1 = min(2 * tile + 1, nblk - 1);
    const int64_t p0 = bt[bi0], p1 = bt[bi1];
    if (has_item) {
      const uint8_t* r0 = cache + p0 * 2 * blk_bytes + it_kk * tok_stride + head_off + 4 * it_w;
      const uint8_t* r1 = cache + p1 * 2 * blk_bytes + it_kk * tok_stride + head_off + 4 * it_w;
      r.k0 = ld32(r0);
      r.k1 = ld32(r1);
      r.v0 = ld32(r0 + blk_bytes);
      r.v1 = ld32(r1 + blk_bytes);
    }
    if (has_sw) {
      const int64_t p = (sw_key >> 4) ? p1 : p0;
      r.sw = ld32(cache + p * 2 * blk_bytes + sw_v * blk_bytes + (sw_key & 15) * tok_stride +
                  head_off + D / 2);
    }
  };
  auto store = [&](const KVRegs<D>& r) {
    if (has_item) {
      *reinterpret_cast<half8_t*>(s_k + it_kk * KROW + 16 * it_w) = unpack8(r.k0);
      *reinterpret_cast<half8_t*>(s_k + (it_kk + 16) * KROW + 16 * it_w) = unpack8(r.k1);
      const uint32_t ylo = (r.v0 & 0xFFFFu) | (r.v1 << 16);
      const uint32_t yhi = (r.v0 >> 16) | (r.v1 & 0xFFFF0000u);
      const int sl = key_slot(it_kk);  // even; key it_kk + 16 takes sl + 1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * it_w + e;
        const uint32_t y = e < 4 ? ylo : yhi;
        *reinterpret_cast<uint32_t*>(s_vt + vt_off(d, sl >> 3) + 2 * (sl & 7)) =
            nib_pair_f16(y >> (4 * (e & 3)));
      }
    }
    if (has_sw) (sw_v ? s_vw : s_kw)[sw_key] = r.sw;
  };

  KVRegs<D> regs;
  if (ntiles > 0) load(0, regs);
  uint32_t* wl = s_w[wave];
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // previous tile's readers are done
    store(regs);
    __syncthreads();
    if (t + 1 < ntiles) load(t + 1, regs);

    // scores for keys 16n + col of this tile
    float4_t sacc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const half8_t kb =
            *reinterpret_cast<const half8_t*>(s_k + (16 * n + col) * KROW + 16 * (g * NCH + c));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[c], kb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[c], kb, acc, 0, 0, 0);
      }
      sacc[n] = acc;
    }
    float sK[2], zK[2], sV[2], zV[2];
    int key[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const uint32_t kw = s_kw[16 * n + col], vw = s_vw[16 * n + col];
      sK[n] = as_float(kw & 0xFFFFFFF0u);
      zK[n] = (float)(kw & 0xFu);
      sV[n] = as_float(vw & 0xFFFFFFF0u);
      zV[n] = (float)(vw & 0xFu);
      key[n] = 32 * t + 16 * n + col;
    }
    uint32_t wpk[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float z[2];
      bool ok[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        ok[n] = key[n] <= pos[v];
        const float tt = sacc[n][v] - zK[n] * qsum[v];
        z[n] = ok[n] ? tt * (sK[n] * c0[v]) : -INFINITY;
      }
      float tmax = fmaxf(z[0], z[1]);
      tmax = fmaxf(tmax, shfl_xor<1>(tmax));
      tmax = fmaxf(tmax, shfl_xor<2>(tmax));
      tmax = fmaxf(tmax, shfl_xor<4>(tmax));
      tmax = fmaxf(tmax, shfl_xor<8>(tmax));
      const float mnew = fmaxf(m_run[v], tmax);
      const bool none = mnew == -INFINITY;  // row sees no key yet
      const float alpha = none ? 1.0f : exp2f(m_run[v] - mnew);
      m_run[v] = mnew;
      const float p0 = ok[0] ? exp2f(z[0] - mnew) : 0.f;
      const float p1 = ok[1] ? exp2f(z[1] - mnew) : 0.f;
      const _Float16 w0 = (_Float16)(p0 * sV[0]);
      const _Float16 w1 = (_Float16)(p1 * sV[1]);
      l_run[v] = l_run[v] * alpha + (p0 + p1);
      corr[v] = corr[v] * alpha + ((float)w0 * zV[0] + (float)w1 * zV[1]);
#pragma unroll
      for (int c = 0; c < NCOL; ++c) oacc[c][v] *= alpha;
      wpk[v] = (uint32_t)__builtin_bit_cast(uint16_t, w0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, w1) << 16);
    }
    // W [row 4g + v][slot of key col, slot + 1 for key 16 + col] through LDS
    {
      const int sl = key_slot(col);
#pragma unroll
      for (int v = 0; v < 4; ++v) wl[(4 * g + v) * 16 + (sl >> 1)] = wpk[v];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const half8_t wop = *reinterpret_cast<const half8_t*>(&wl[col * 16 + 4 * g]);
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
      const half8_t vb = *reinterpret_cast<const half8_t*>(s_vt + vt_off(16 * c + col, g));
      oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, vb, oacc[c], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // W tile is rewritten next iteration
  }

  // ---- finalise and rotate back; register v of column tile c holds row
  // 16*wave + 4g + v, d = 16c + col
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float lv = l_run[v], cv = corr[v];
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
    for (int c = 0; c < NCOL; ++c) o[c] = (oacc[c][v] - cv) * inv_l;
#pragma unroll
    for (int span = 1; span < NCOL; span <<= 1) {  // d spans 16, 32, 64 over c
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        if (c & span) continue;
        const float a = o[c], bb = o[c + span];
        o[c] = a + bb;
        o[c + span] = a - bb;
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {  // d spans 1, 2, 4, 8 over col
      const bool upper = (col & m) != 0;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const float p = shfl_xor_rt(o[c], m);
        o[c] = upper ? p - o[c] : o[c] + p;
      }
    }
    const int row = 16 * wave + 4 * g + v;
    const int tq = qt * TQ + row / G;
    if (tq < qlen) {
      const int qg = h * G + row % G;
      uint16_t* dst = out + ((int64_t)(q0 + tq) * num_q_heads + qg) * D;
      const float invD = 1.0f / (float)D;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const int d = 16 * c + col;
        dst[d] = from_f32<BF16>(o[c] * signs[d] * invD);
      }
    }
  }
}

template <bool BF16, int D, int G>
hipError_t launch_prefill_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int TQ = 64 / G;
  dim3 grid((a.max_seqlen_q + TQ - 1) / TQ, a.num_seqs, a.num_kv_heads), block(256);
  const float scale_log2 = a.softmax_scale * kLog2e / (float)D;
  hipLaunchKernelGGL((prefill_kernel<BF16, D, G>), grid, block, 0, stream,
                     reinterpret_cast<const uint16_t*>(a.q), a.q_stride,
                     reinterpret_cast<uint16_t*>(a.out), a.cache, a.num_kv_heads, a.num_q_heads,
                     a.cu_seqlens_q, a.seqused_k, a.block_table, a.bt_stride, scale_log2, a.signs);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_t<BF16, D, 1>(a, stream);
    case 2: return launch_prefill_t<BF16, D, 2>(a, stream);
    case 4: return launch_prefill_t<BF16, D, 4>(a, stream);
    case 8: return launch_prefill_t<BF16, D, 8>(a, stream);
    default: return launch_prefill_t<BF16, D, 16>(a, stream);
  }
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) return a.head_size == 128 ? launch_prefill_d<true, 128>(a, stream)
                                        : launch_prefill_d<true, 64>(a, stream);
  return a.head_size == 128 ? launch_prefill_d<false, 128>(a, stream)
                            : launch_prefill_d<false, 64>(a, stream);
}

}  // namespace int4kv
