// Encoding of one (token, K|V, head) row into its packed INT4 form, shared by
// the cache write and the fused decode step so both store the same bytes.
//
// PR #40633's description and the PR #40835 report (implementation breakdown,
// item 2): random Hadamard rotation, asymmetric 16-level codes, one fp32 scale
// per row with the zero point in its low 4 mantissa bits; the quantizer is the
// test file's section 6 INT4 reference.  A row of D elements is held by
// LPR = D / E lanes (adjacent lanes, piece `sub` = lane % LPR) with E
// consecutive elements each.  Every fp32 operation is one correctly rounded op
// in a fixed order (spans 1, 2, 4, ..., D/2; contraction is switched off
// here), so the bytes are reproducible bit for bit:
//   * the signs are applied as bit flips of the 16-bit inputs (exact),
//   * clamp-then-round equals round-then-clamp for the integer bounds 0 and
//     15, and the rounding to nearest even is the float-to-byte conversion
//     (v_cvt_pk_u8_f32, round-to-nearest-even mode), which also places the
//     code in its byte.
#pragma once

#include "device_common.h"

namespace int4kv {

__device__ __forceinline__ float enc_med3(float x, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(x, lo, hi);
}

// element i of a 16-bit pair dword (i = 0: low half)
template <bool BF16>
__device__ __forceinline__ float half_of(uint32_t w, int i) {
  if constexpr (BF16) {
    return as_float(i == 0 ? (w << 16) : (w & 0xFFFF0000u));
  } else {
    const half2_t hh = __builtin_bit_cast(half2_t, w);
    return (float)hh[i];
  }
}

// sign bits of elements [E * sub, E * sub + E) as flips of 16-bit pairs
template <int E>
__device__ __forceinline__ void row_flips(const float* __restrict__ signs, int sub,
                                          uint32_t (&flip)[E / 2]) {
#pragma unroll
  for (int p = 0; p < E / 2; ++p) {
    const float s0 = signs[E * sub + 2 * p], s1 = signs[E * sub + 2 * p + 1];
    flip[p] = (s0 < 0.f ? 0x8000u : 0u) | (s1 < 0.f ? 0x80000000u : 0u);
  }
}

// the lane's E inputs (E / 8 vectors of 8 16-bit values) times the signs, in fp32
template <bool BF16, int E>
__device__ __forceinline__ void row_inputs(const u32x4_t (&a)[E / 8], const uint32_t (&flip)[E / 2],
                                           float (&x)[E]) {
#pragma unroll
  for (int k = 0; k < E / 8; ++k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = a[k][j] ^ flip[4 * k + j];  // x * sign, exactly
      x[8 * k + 2 * j] = half_of<BF16>(w, 0);
      x[8 * k + 2 * j + 1] = half_of<BF16>(w, 1);
    }
  }
}

// x[e + i] = partner(x[e + i]) * c + x[e + i] for i < 8, the partner being
// lane ^ m (m = 1 or 2) read through a DPP quad permute of the fmac's first
// operand.  The leading s_nop gives the two wait states a DPP read needs after
// the VALU writes of these registers, which all precede the block.
template <int E>
__device__ __forceinline__ void cross_fmac8(int m, float (&x)[E], int e, float c) {
  if (m == 1) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(x[e]), "+v"(x[e + 1]), "+v"(x[e + 2]), "+v"(x[e + 3]), "+v"(x[e + 4]),
          "+v"(x[e + 5]), "+v"(x[e + 6]), "+v"(x[e + 7])
        : "v"(c));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(x[e]), "+v"(x[e + 1]), "+v"(x[e + 2]), "+v"(x[e + 3]), "+v"(x[e + 4]),
          "+v"(x[e + 5]), "+v"(x[e + 6]), "+v"(x[e + 7])
        : "v"(c));
  }
}

// Rotation, range, scale, zero point and codes of one row: the lane's E / 8
// packed code dwords (bytes j = code_{2j} | code_{2j+1} << 4) and the row's
// scale word bits(s_t) | zp.
//
// The spans that pair lanes (E, 2E, ...) take one fused multiply-add per
// element, new = partner * c + self with c = +1 in the lower lane of a pair
// and -1 in the upper one: the product is exact, so the sum is rounded once
// and the lower lane holds u + v while the upper one holds v - u = -(u - v)
// (round-to-nearest-even is symmetric).  A lane's values are therefore its
// row elements times sigma = (-1)^popcount(sub); the range and the codes
// undo that exactly (min and max swap under negation, and the codes are
// fl(stored * (sigma * inv)) = fl(y * inv)).
//
// Codes: t = fl(fl(y * inv) + zp) is clamped to [0, 15] and rounded to
// nearest even by the float-to-byte conversion; two codes share a byte.
template <int E, int LPR>
__device__ __forceinline__ uint32_t encode_piece(float (&x)[E], int sub,
                                                 uint32_t (&packed)[E / 8]) {
#pragma clang fp contract(off)
  // butterflies inside the lane: spans 1 .. E/2
#pragma unroll
  for (int span = 1; span < E; span <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e & span) continue;
      const float u = x[e], v = x[e + span];
      x[e] = __fadd_rn(u, v);
      x[e + span] = __fsub_rn(u, v);
    }
  }
  // spans E, 2E, ... across the lanes of a row
  float sigma = 1.0f;
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    const float c = (sub & m) ? -1.0f : 1.0f;
    sigma *= c;
    if (m <= 2) {
#pragma unroll
      for (int e = 0; e < E; e += 8) cross_fmac8(m, x, e, c);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __builtin_fmaf(shfl_xor_rt(x[e], m), c, x[e]);
    }
  }

  // row range of the stored values (one min3 / max3 per two elements), then
  // of the row's elements, then over the row's lanes
  float mn = __builtin_fminf(x[0], x[1]), mx = __builtin_fmaxf(x[0], x[1]);
#pragma unroll
  for (int e = 2; e < E; e += 2) {
    mn = __builtin_fminf(__builtin_fminf(mn, x[e]), x[e + 1]);
    mx = __builtin_fmaxf(__builtin_fmaxf(mx, x[e]), x[e + 1]);
  }
  if (LPR > 1 && sigma < 0.0f) {
    const float t = mn;
    mn = -mx;
    mx = -t;
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    mn = fminf(mn, shfl_xor_rt(mn, m));
    mx = fmaxf(mx, shfl_xor_rt(mx, m));
  }
  float sc = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
  if (!(sc > 1e-6f)) sc = 1e-6f;
  const float s_t = as_float(as_uint(sc) & 0xFFFFFFF0u);
  const float inv = __fdiv_rn(1.0f, s_t);
  const float zpf = fminf(fmaxf(rintf(__fmul_rn(-mn, inv)), 0.0f), 15.0f);
  const float invs = LPR > 1 ? sigma * inv : inv;  // exact

#pragma unroll
  for (int q = 0; q < E / 8; ++q) {
    // codes 8q .. 8q+7 as bytes [c1 c0 c3 c2] of w[0] and [c5 c4 c7 c6] of
    // w[1] (each code < 16), so that (w << 12) | w holds c0 | c1 << 4 in byte
    // 1 and c2 | c3 << 4 in byte 3
    uint32_t w[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint32_t acc = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 8 * q + 4 * hf + j;
        const float t = enc_med3(__fadd_rn(__fmul_rn(x[e], invs), zpf), 0.0f, 15.0f);
        acc = __builtin_amdgcn_cvt_pk_u8_f32(t, j ^ 1, acc);  // round to nearest even
      }
      w[hf] = (acc << 12) | acc;
    }
    packed[q] = __builtin_amdgcn_perm(w[1], w[0], 0x07050301u);  // bytes 1, 3 of w[0], w[1]
  }
  return as_uint(s_t) | (uint32_t)zpf;
}

}  // namespace int4kv
