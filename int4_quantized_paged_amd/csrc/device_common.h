// Device-side helpers shared by the INT4 KV-cache kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int4kv {

constexpr int kWave = 64;
constexpr int kBlockSize = 16;  // tokens per cache block (the only supported value)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16- and 8-byte vectors with 4-byte alignment: packed cache rows are only
// dword aligned; global_load_dwordx4/x2 accept dword-aligned addresses.
typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4_t __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ float as_float(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __float_as_uint(f); }

// Value of `v` held by lane (lane ^ mask).  xor 1 and 2 use DPP quad
// permutes; 4, 8 and 16 use ds_swizzle in bit mode (32-lane groups); 32 uses
// ds_bpermute.  Every lane of the wave must be active.
template <int MASK>
__device__ __forceinline__ float shfl_xor(float v) {
  int x = __float_as_int(v);
  int r;
  if constexpr (MASK == 1) {
    r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (MASK == 4 || MASK == 8 || MASK == 16) {
    r = __builtin_amdgcn_ds_swizzle(x, 0x1F | (MASK << 10));  // and 0x1F, xor MASK
  } else {
    static_assert(MASK == 32, "xor mask");
    int lane = __lane_id();
    r = __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, x);
  }
  return __int_as_float(r);
}

__device__ __forceinline__ float shfl_xor_rt(float v, int mask) {
  switch (mask) {
    case 1: return shfl_xor<1>(v);
    case 2: return shfl_xor<2>(v);
    case 4: return shfl_xor<4>(v);
    case 8: return shfl_xor<8>(v);
    case 16: return shfl_xor<16>(v);
    default: return shfl_xor<32>(v);
  }
}

// Value of `v` held by lane `src` (any lane of the wave).
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

// 16-bit input element (raw bits) to fp32; exact for both formats.
template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (BF16) {
    return __uint_as_float((uint32_t)bits << 16);
  } else {
    _Float16 h = __builtin_bit_cast(_Float16, bits);
    return (float)h;
  }
}

// fp32 to 16-bit output (round to nearest even), raw bits.
template <bool BF16>
__device__ __forceinline__ uint16_t from_f32(float f) {
  if constexpr (BF16) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  } else {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
  }
}

// Four nibbles n0..n3 of a 16-bit field expanded to two f16 pairs.
// (w & 0x000F000F) | 0x64006400 is the f16 pair (1024 + nib0, 1024 + nib4) of
// the dword; subtracting 1024 in f16 is exact and leaves the codes 0..15.
__device__ __forceinline__ uint32_t nib_pair_f16(uint32_t w) {
  uint32_t t = (w & 0x000F000Fu) | 0x64006400u;
  half2_t h = __builtin_bit_cast(half2_t, t);
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  h = h - k1024;
  return __builtin_bit_cast(uint32_t, h);
}

// Logit soft cap in base-2 logit units: c * tanh(x / c), given c and 1 / c
// (c > 0).  tanh(a) = 1 - 2 / (e^{2a} + 1) from one exp2 and one reciprocal;
// large |x| gives exactly +-c, and the absolute error is a few 2^-24 of c.
__device__ __forceinline__ float soft_cap(float x, float c, float inv_c) {
  const float a = fabsf(x) * inv_c;
  const float e = __builtin_amdgcn_exp2f(a * 2.8853900817779268f);  // e^(2a)
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return copysignf(c * t, x);
}

// A value the compiler cannot trace back to the expression that made it.
// The f16 hi + lo split of a softmax weight w = p * s needs lo computed
// against the hi that is stored.  Left visible, hi = f16(p * s) may be formed
// twice: once from the fp32 product for the stored copy and once by rounding
// the exact product straight to f16 (v_fma_mix with a zero addend) for lo's
// subtrahend.  The two differ at fp32 ties, and hi + lo is then off by an f16
// ulp.  Pinning hi leaves lo = f16(w - hi) free to use the exact product.
template <typename T>
__device__ __forceinline__ T opaque(T x) {
  asm("" : "+v"(x));
  return x;
}
}  // namespace int4kv
