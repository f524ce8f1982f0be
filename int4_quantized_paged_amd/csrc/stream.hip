// A plain streaming kernel with a chosen read:write mix, the attainable
// bandwidth that the cache write (which reads K and V and writes packed rows)
// is compared against.  No method arithmetic: the written words are XORs of
// the read ones, so no load is dead.
#include "device_common.h"
#include "launch.h"

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

}  // namespace

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
