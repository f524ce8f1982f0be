// Calibration kernels, no method arithmetic: a plain streaming kernel with a
// chosen read:write mix (the attainable bandwidth that the cache write, which
// reads K and V and writes packed rows, is compared against; the written
// words are XORs of the read ones, so no load is dead), and the decode
// path's block gather into LDS on its own (the attainable rate of that
// access pattern, which the decode kernel is compared against).
#include "device_common.h"
#include "launch.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace int4kv {

namespace {

// Written unit w (16 bytes) is the XOR of the read units w, w + nw, w + 2 nw,
// ... below nr, so every read unit reaches exactly one written unit (nw > 0)
// and no load is dead; a wave reads and writes consecutive units, four
// independent loads in flight per thread, with non-temporal loads and
// stores (the data is touched once).  One written unit per thread, grid-
// stride only past the grid's size limit.
__global__ __launch_bounds__(256) void stream_rw_kernel(const u32x4_t* __restrict__ src,
                                                        int64_t nr, u32x4_t* __restrict__ dst,
                                                        int64_t nw) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nw; w += T) {
    u32x4_t a = {0u, 0u, 0u, 0u};
    for (int64_t r0 = w; r0 < nr; r0 += 4 * nw) {
      u32x4_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t r = r0 + j * nw;
        v[j] = r < nr ? __builtin_nontemporal_load(src + r) : u32x4_t{0u, 0u, 0u, 0u};
      }
      a ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __builtin_nontemporal_store(a, dst + w);
  }
}

// Copy-only pass over cache blocks listed in a table: the decode path's
// gather (HBM -> LDS with global_load_lds_dwordx4, non-temporal, two blocks
// per tile, 1 KiB units spread over 8 waves, a ring of kCopyStages stages
// with a barrier per tile) without any of its arithmetic.  Workgroup g
// copies the 2 * tiles_per_wg blocks ids[2 g tiles_per_wg ..] in order;
// copies past its last tile re-read that tile (as the decode ring does), so
// the vmcnt waits are exact.  Nothing is written.
constexpr int kCopyStages = 4;

__device__ __forceinline__ void copy16_lds(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// NI = ceil(units per tile / 8): copies per wave per tile (waves whose last
// unit would be past the tile issue NI - 1)
template <int NI>
__global__ __launch_bounds__(512) void stream_blocks_kernel(const uint8_t* __restrict__ cache,
                                                            int32_t units_per_block,
                                                            const int32_t* __restrict__ ids,
                                                            int32_t tiles_per_wg) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int S = kCopyStages;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const int upb = units_per_block, U = 2 * upb;
  const bool full = (NI - 1) * 8 + wave < U;
  const uint64_t block_bytes = (uint64_t)upb * 1024;
  const int32_t* my = ids + (int64_t)blockIdx.x * 2 * tiles_per_wg;
  // block ids of the next tile to copy, read one tile ahead (as the decode
  // ring does) so the scalar loads never hold up the copies
  uint32_t nid[2];
  auto load_ids = [&](int t) {
    const int tt = t < tiles_per_wg ? t : tiles_per_wg - 1;
    nid[0] = (uint32_t)my[2 * tt];
    nid[1] = (uint32_t)my[2 * tt + 1];
  };
  auto issue = [&](int t) {  // nid holds tile t's block ids
    const uint8_t* p0 = cache + (uint64_t)nid[0] * block_bytes;
    const uint8_t* p1 = cache + (uint64_t)nid[1] * block_bytes;
    asm volatile("" : "+s"(p0), "+s"(p1));
    const uint32_t sb = lds0 + (uint32_t)(t % S) * (uint32_t)U * 1024u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i == NI - 1 && !full) break;
      const int u = i * 8 + wave;
      const int blk = u >= upb ? 1 : 0;
      copy16_lds(blk ? p1 : p0, (uint32_t)(u - blk * upb) * 1024u + (uint32_t)lane * 16u,
                 sb + (uint32_t)u * 1024u);
    }
  };
  for (int t = 0; t < S - 1; ++t) {
    load_ids(t);
    issue(t);
  }
  load_ids(S - 1);
  for (int t = 0; t < tiles_per_wg; ++t) {
    // tile t has landed once at most S - 2 younger tiles are in flight
    if (full)
      wait_vmem_n<(S - 2) * NI>();
    else
      wait_vmem_n<(S - 2) * (NI - 1)>();
    __syncthreads();  // ... in every wave: its stage (that of tile t - 1 + S) is free
    issue(t + S - 1);
    load_ids(t + S);
  }
  wait_vmem_n<0>();
}

template <int NI>
hipError_t launch_blocks_t(const uint8_t* cache, int upb, const int32_t* ids, int tiles,
                           int num_wg, hipStream_t stream) {
  const int lds = kCopyStages * 2 * upb * 1024;
  auto kern = stream_blocks_kernel<NI>;
  if (lds > 65536) {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(num_wg), dim3(512), lds, stream, cache, upb, ids, tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_blocks(const uint8_t* cache, int64_t block_bytes, const int32_t* ids,
                                int64_t num_ids, int32_t num_workgroups, hipStream_t stream) {
  const int upb = (int)(block_bytes / 1024);
  const int tiles = (int)(num_ids / (2 * (int64_t)num_workgroups));
  switch ((2 * upb + 7) / 8) {
    case 1: return launch_blocks_t<1>(cache, upb, ids, tiles, num_workgroups, stream);
    case 2: return launch_blocks_t<2>(cache, upb, ids, tiles, num_workgroups, stream);
    case 3: return launch_blocks_t<3>(cache, upb, ids, tiles, num_workgroups, stream);
    case 4: return launch_blocks_t<4>(cache, upb, ids, tiles, num_workgroups, stream);
    default: return launch_blocks_t<5>(cache, upb, ids, tiles, num_workgroups, stream);
  }
}

hipError_t launch_stream_rw(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                            hipStream_t stream) {
  const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
  const int64_t need = (nw + 255) / 256;
  const int64_t blocks = need < (int64_t(1) << 30) ? need : (int64_t(1) << 30);
  hipLaunchKernelGGL(stream_rw_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), nr, reinterpret_cast<u32x4_t*>(dst),
                     nw);
  return hipGetLastError();
}

}  // namespace int4kv
