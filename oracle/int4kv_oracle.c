/*
 * CPU oracle for the INT4 per-token-head paged KV cache: TEST INFRASTRUCTURE.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or call this library.  The product path (the HIP library) never does;
 * the two share no source, header, table or helper.
 *
 * Plain, slow, obviously correct.  Every step cites the passage it follows.
 * Page names used in citations:
 *   [report]    "PR #40835 report: [Feature] Triton INT4 per-token-head KV cache
 *               quantization" (prhub.com.cn)
 *   [pr40633]   "[Feature] Triton INT4 / INT2 per-token-head KV cache
 *               quantization, Pull Request #40633, vllm-project/vllm"
 *   [testfile]  "tests/quantization/test_per_token_kv_cache.py" (vLLM fork page),
 *               cited by the numbered section of that file.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * fp32 steps are single correctly-rounded IEEE operations (x86-64 SSE,
 * FLT_EVAL_METHOD == 0, no FMA contraction, no DAZ/FTZ, rint = round half to
 * even in the default rounding mode).  Attention is computed in fp64.
 *
 * Readings of the pages that this file fixes (each one is listed in the design
 * notes with its justification):
 *   R-rht   forward y = H (D x), unnormalised Sylvester H, signs applied first;
 *           inverse x = D (H y) / d.                     ([testfile] §2, §3
 *           dequant divides the inverse transform by head_size; [pr40633] commit
 *           caching the "D1" sign vector)
 *   R-fwht  butterfly stages with span 1, 2, 4, ..., d/2; pair (i, i+span)
 *           becomes (u_i + u_{i+span}, u_i - u_{i+span}).
 *   R-range codes are unsigned 0..15 with a zero point.   ([testfile] §6 INT4
 *           reference quantizer)
 *   R-trunc zero point and codes use the truncated scale s_t.  ([pr40633]
 *           gemini-code-assist review asking the write path to match the read)
 *   R-recip one correctly rounded reciprocal per row, codes from y * (1/s_t).
 *   R-rint  round half to even.                          ([testfile] §6 uses
 *           torch.round; INT4 config comment speaks of a rint path)
 *   R-kv    cache dim 1: index 0 = K, index 1 = V; scale word at the row tail.
 *           ([report] key snippets, get_kv_cache_shape)
 *   R-pos   query i of a sequence with q_len new tokens and seqused_k keys sits
 *           at position seqused_k - q_len + i and sees keys [0, pos].
 *   R-gqa   query head g reads KV head g / (Hq / Hkv).
 *   R-seg   split-K segment k of a sequence with nb blocks covers blocks
 *           [k*c, min((k+1)*c, nb)), c = ceil(nb / NS); with a window, the
 *           segments split the blocks from the first one any query row of
 *           the sequence can see, b_lo, in the same way: [b_lo + k*c, ...),
 *           c = ceil((nb - b_lo) / NS).
 *   R-win   sliding window W > 0: the query at position pos sees keys
 *           [max(0, pos - W + 1), pos], W keys counting its own; W <= 0 is no
 *           window.  ([pr40633] description: the packed read path shares the
 *           common kernel's sliding-window masking helper.)
 *   R-cap   logit soft-capping c > 0: each scaled score z becomes
 *           c * tanh(z / c) before the softmax; c <= 0 is no capping.
 *           ([pr40633] description: the packed read path shares the common
 *           kernel's softcap helper; the pages do not restate its formula,
 *           and this is the usual tanh soft cap.)
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F16 0
#define OR_BF16 1

/* ---------- 16-bit float decoders, written from the IEEE-754 definitions. */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float or_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return (float)(sign ? -v : v); /* exact: every binary16 value fits fp32 */
}

/* bfloat16: the upper 16 bits of a binary32. */
static float or_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

static float or_load(const uint16_t* p, int dtype) {
  return dtype == OR_BF16 ? or_bf16_to_f32(*p) : or_f16_to_f32(*p);
}

static uint32_t or_f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}
static float or_bits_f32(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}

/* ---------- Random Hadamard transform (R-rht, R-fwht). */

/* In-place forward transform of one fp32 vector: multiply by the sign vector
 * (exact for +-1), then the fast Walsh-Hadamard butterflies in span order
 * 1, 2, 4, ...  Each output of a butterfly is one rounded fp32 add or sub. */
void oracle_rht_forward_f32(float* u, int d, const float* signs) {
  for (int i = 0; i < d; ++i) u[i] = u[i] * signs[i];
  for (int span = 1; span < d; span <<= 1) {
    for (int i = 0; i < d; ++i) {
      if (i & span) continue;
      float a = u[i], b = u[i + span];
      u[i] = a + b;
      u[i + span] = a - b;
    }
  }
}

/* fp64 Walsh-Hadamard (unnormalised), same stage order, for the read side. */
static void or_fwht_f64(double* u, int d) {
  for (int span = 1; span < d; span <<= 1) {
    for (int i = 0; i < d; ++i) {
      if (i & span) continue;
      double a = u[i], b = u[i + span];
      u[i] = a + b;
      u[i + span] = a - b;
    }
  }
}

/* Inverse rotation in fp64: x = D (H y) / d.  ([testfile] §2/§3 dequant:
 * inverse transform, then divide by head_size.) */
void oracle_rht_inverse_f64(double* y, int d, const float* signs) {
  or_fwht_f64(y, d);
  for (int i = 0; i < d; ++i) y[i] = (double)signs[i] * y[i] / (double)d;
}

/* ---------- Nibble packing ([testfile] §2 dequant and §6 _pack_int4: even
 * element in the low nibble, odd element in the high nibble). */
void oracle_pack_nibbles(const uint8_t* q, int n, uint8_t* out) {
  for (int j = 0; j < n / 2; ++j)
    out[j] = (uint8_t)((q[2 * j] & 0xF) | ((q[2 * j + 1] & 0xF) << 4));
}
void oracle_unpack_nibbles(const uint8_t* bytes, int n, uint8_t* q) {
  for (int j = 0; j < n / 2; ++j) {
    q[2 * j] = bytes[j] & 0xF;
    q[2 * j + 1] = (bytes[j] >> 4) & 0xF;
  }
}

/* ---------- Zero-point steganography ([pr40633] description: zero point in
 * the low 4 mantissa bits of the fp32 scale; [testfile] §6: bits & -16 | zp,
 * and §2: zp = bits & 0xF, clean scale = bits & -16). */
uint32_t oracle_stego_encode(float s, int zp) {
  return (or_f32_bits(s) & 0xFFFFFFF0u) | ((uint32_t)zp & 0xFu);
}
void oracle_stego_decode(uint32_t word, float* s_t, int* zp) {
  *zp = (int)(word & 0xFu);
  *s_t = or_bits_f32(word & 0xFFFFFFF0u);
}

/* clamp(rint(v), 0, 15), clamped in float before the integer conversion. */
static int or_code(float v) {
  float r = rintf(v);
  if (!(r > 0.0f)) return 0;
  if (r > 15.0f) return 15;
  return (int)r;
}

/* ---------- Asymmetric per-row quantizer ([testfile] §6 INT4 reference:
 * scale = (max - min) / 15 clamped at 1e-6, zp = round(-min / scale) in
 * [0, 15], q = round(x / scale + zp) in [0, 15]; R-trunc, R-recip, R-rint).
 * y: d rotated fp32 values.  Writes d/2 packed bytes and the scale word. */
void oracle_quantize_row(const float* y, int d, uint8_t* bytes, uint32_t* word_out) {
  float mn = y[0], mx = y[0];
  for (int i = 1; i < d; ++i) {
    if (y[i] < mn) mn = y[i];
    if (y[i] > mx) mx = y[i];
  }
  float s = (mx - mn) / 15.0f;
  if (!(s > 1e-6f)) s = 1e-6f;
  float s_t = or_bits_f32(or_f32_bits(s) & 0xFFFFFFF0u);
  float inv = 1.0f / s_t;
  float zpf = (float)or_code(-mn * inv);
  uint8_t* q = (uint8_t*)malloc((size_t)d);
  for (int i = 0; i < d; ++i) {
    float t = y[i] * inv;
    q[i] = (uint8_t)or_code(t + zpf);
  }
  oracle_pack_nibbles(q, d, bytes);
  free(q);
  *word_out = oracle_stego_encode(s_t, (int)zpf);
}

/* Byte offset of the packed row for (slot's block, slot's offset, kv, head)
 * in the cache [num_blocks, 2, block_size, num_kv_heads, d/2 + 4] ([report]
 * key snippets, get_kv_cache_shape; R-kv). */
static int64_t or_row_offset(int64_t blk, int kv, int64_t off, int h, int block_size,
                             int num_kv_heads, int d) {
  int64_t R = d / 2 + 4;
  return (((blk * 2 + kv) * block_size + off) * num_kv_heads + h) * R;
}

/* ---------- Cache write ([report] implementation breakdown item 2: the write
 * kernel rotates, computes a per (token, head) scale and zero point and packs;
 * [testfile] §4: a negative slot leaves the cache untouched; slot decode
 * blk = slot / block_size, off = slot % block_size as in §2).
 * key/value: raw 16-bit words, element (t, h, i) at t*stride + h*d + i. */
void oracle_kv_write(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                     int64_t value_stride, int dtype, const int64_t* slot_mapping,
                     int num_tokens, uint8_t* cache, int num_blocks, int block_size,
                     int num_kv_heads, int d, const float* signs) {
  (void)num_blocks;
  /* tokens are independent (each writes its own rows), so OpenMP threads may
   * take them in any order; every row is computed exactly as with one thread */
#pragma omp parallel
  {
  float* y = (float*)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(static)
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = kv == 0 ? key + (int64_t)t * key_stride
                                    : value + (int64_t)t * value_stride;
      for (int h = 0; h < num_kv_heads; ++h) {
        for (int i = 0; i < d; ++i) y[i] = or_load(src + (int64_t)h * d + i, dtype);
        oracle_rht_forward_f32(y, d, signs);
        uint8_t* row = cache + or_row_offset(blk, kv, off, h, block_size, num_kv_heads, d);
        uint32_t word;
        oracle_quantize_row(y, d, row, &word);
        /* little-endian scale word at bytes [d/2, d/2 + 4) */
        row[d / 2 + 0] = (uint8_t)(word & 0xFF);
        row[d / 2 + 1] = (uint8_t)((word >> 8) & 0xFF);
        row[d / 2 + 2] = (uint8_t)((word >> 16) & 0xFF);
        row[d / 2 + 3] = (uint8_t)((word >> 24) & 0xFF);
      }
    }
  }
  free(y);
  }
}

static uint32_t or_row_word(const uint8_t* row, int d) {
  return (uint32_t)row[d / 2] | ((uint32_t)row[d / 2 + 1] << 8) |
         ((uint32_t)row[d / 2 + 2] << 16) | ((uint32_t)row[d / 2 + 3] << 24);
}

/* Rotated-domain dequantised row y_hat_i = (n_i - zp) * s_t, fp64
 * ([testfile] §2 dequant in the RHT domain). */
static void or_row_dequant_rotated(const uint8_t* row, int d, double* yhat) {
  float s_t;
  int zp;
  oracle_stego_decode(or_row_word(row, d), &s_t, &zp);
  for (int j = 0; j < d / 2; ++j) {
    yhat[2 * j] = (double)((int)(row[j] & 0xF) - zp) * (double)s_t;
    yhat[2 * j + 1] = (double)((int)((row[j] >> 4) & 0xF) - zp) * (double)s_t;
  }
}

/* Original-domain dequantised row x_hat = D (H y_hat) / d, fp64. */
void oracle_decode_row(const uint8_t* row, int d, const float* signs, double* out) {
  or_row_dequant_rotated(row, d, out);
  oracle_rht_inverse_f64(out, d, signs);
}

/* Pointer to the row of key j of sequence b (block table, R-kv). */
static const uint8_t* or_key_row(const uint8_t* cache, const int32_t* block_table,
                                 int bt_stride, int b, int64_t j, int kv, int h,
                                 int block_size, int num_kv_heads, int d) {
  int64_t blk = block_table[(int64_t)b * bt_stride + j / block_size];
  return cache + or_row_offset(blk, kv, j % block_size, h, block_size, num_kv_heads, d);
}

/* ---------- Attention, plain definition (fp64).  Causal softmax attention of
 * the query rows over the decoded K/V of the paged cache ([testfile] §6: the
 * packed kernel is compared with ordinary attention over the dequantised
 * cache; [report] risks: causal only; R-pos, R-gqa).
 * q: raw 16-bit, row t head g at t*q_stride + g*d.  out: fp64 [Tq, Hq, d]. */
void oracle_attention_plain(const uint16_t* q, int64_t q_stride, int dtype,
                            const uint8_t* cache, int num_blocks, int block_size,
                            int num_kv_heads, int d, int num_q_heads,
                            const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                            int num_seqs, const int32_t* block_table, int bt_stride,
                            double softmax_scale, const float* signs, int window,
                            double softcap, double* out) {
  (void)num_blocks;
  int G = num_q_heads / num_kv_heads;
  /* (sequence, kv head) pairs are independent (each writes its own output
   * rows), so OpenMP threads may take them in any order; every output is
   * computed exactly as with one thread */
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < num_seqs * num_kv_heads; ++bh) {
    const int b = bh / num_kv_heads, h = bh % num_kv_heads;
    int q0 = cu_seqlens_q[b], qlen = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int64_t L = seqused_k[b];
    if (qlen <= 0 || L <= 0) continue;
    {
      /* decode every key and value of this (sequence, kv head) once */
      double* K = (double*)malloc(sizeof(double) * (size_t)(L * d));
      double* V = (double*)malloc(sizeof(double) * (size_t)(L * d));
      for (int64_t j = 0; j < L; ++j) {
        oracle_decode_row(or_key_row(cache, block_table, bt_stride, b, j, 0, h, block_size,
                                     num_kv_heads, d), d, signs, K + j * d);
        oracle_decode_row(or_key_row(cache, block_table, bt_stride, b, j, 1, h, block_size,
                                     num_kv_heads, d), d, signs, V + j * d);
      }
      double* z = (double*)malloc(sizeof(double) * (size_t)L);
      double* qv = (double*)malloc(sizeof(double) * (size_t)d);
      for (int i = 0; i < qlen; ++i) {
        int64_t pos = L - qlen + i;
        for (int gg = 0; gg < G; ++gg) {
          int g = h * G + gg;
          const uint16_t* qrow = q + (int64_t)(q0 + i) * q_stride + (int64_t)g * d;
          for (int k = 0; k < d; ++k) qv[k] = (double)or_load(qrow + k, dtype);
          double* o = out + ((int64_t)(q0 + i) * num_q_heads + g) * d;
          for (int k = 0; k < d; ++k) o[k] = 0.0;
          if (pos < 0) continue;
          int64_t jlo = 0; /* R-win */
          if (window > 0 && pos - window + 1 > 0) jlo = pos - window + 1;
          double zmax = -INFINITY;
          for (int64_t j = jlo; j <= pos; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += qv[k] * K[j * d + k];
            z[j] = softmax_scale * acc;
            if (softcap > 0.0) z[j] = softcap * tanh(z[j] / softcap); /* R-cap */
            if (z[j] > zmax) zmax = z[j];
          }
          double den = 0.0;
          for (int64_t j = jlo; j <= pos; ++j) {
            z[j] = exp(z[j] - zmax);
            den += z[j];
          }
          for (int64_t j = jlo; j <= pos; ++j) {
            double w = z[j] / den;
            for (int k = 0; k < d; ++k) o[k] += w * V[j * d + k];
          }
        }
      }
      free(qv);
      free(z);
      free(K);
      free(V);
    }
  }
}

/* ---------- Attention, method formulation (fp64).  Follows the read path the
 * pages describe: rotate Q into the cache's domain, score each packed key with
 * a dot product over the codes plus a sum(Q) * zero-point correction ([pr40633]
 * description), keep an online softmax per block ([pr40633]: softmax
 * bookkeeping shared with the common kernel), split the key range into
 * segments merged by a segment reduction ([pr40633]: reduce_segments; [testfile]
 * §6 segment buffers), and rotate the result back (R-rht inverse).
 * Agrees with oracle_attention_plain up to fp64 rounding, because H is
 * symmetric with H H = d I, so q . x_hat = (H D q) . y_hat / d. */
void oracle_attention_method(const uint16_t* q, int64_t q_stride, int dtype,
                             const uint8_t* cache, int num_blocks, int block_size,
                             int num_kv_heads, int d, int num_q_heads,
                             const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                             int num_seqs, const int32_t* block_table, int bt_stride,
                             double softmax_scale, const float* signs, int num_segments,
                             int window, double softcap, double* out) {
  (void)num_blocks;
  int G = num_q_heads / num_kv_heads;
  if (num_segments < 1) num_segments = 1;
  double* qr = (double*)malloc(sizeof(double) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* seg_acc = (double*)malloc(sizeof(double) * (size_t)(num_segments * d));
  double* seg_m = (double*)malloc(sizeof(double) * (size_t)num_segments);
  double* seg_l = (double*)malloc(sizeof(double) * (size_t)num_segments);
  for (int b = 0; b < num_seqs; ++b) {
    int q0 = cu_seqlens_q[b], qlen = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int64_t L = seqused_k[b];
    if (qlen <= 0 || L <= 0) continue;
    int64_t nblk = (L + block_size - 1) / block_size;
    int64_t blo = 0; /* first block any row of the sequence sees (R-win, R-seg) */
    if (window > 0 && L - qlen - window + 1 > 0) blo = (L - qlen - window + 1) / block_size;
    int64_t per = (nblk - blo + num_segments - 1) / num_segments; /* R-seg */
    for (int i = 0; i < qlen; ++i) {
      int64_t pos = L - qlen + i;
      int64_t jlo = 0; /* R-win */
      if (window > 0 && pos - window + 1 > 0) jlo = pos - window + 1;
      for (int g = 0; g < num_q_heads; ++g) {
        int h = g / G;
        double* o = out + ((int64_t)(q0 + i) * num_q_heads + g) * d;
        for (int k = 0; k < d; ++k) o[k] = 0.0;
        if (pos < 0) continue;
        /* prologue: q' = H (D q), and sum(q') */
        const uint16_t* qrow = q + (int64_t)(q0 + i) * q_stride + (int64_t)g * d;
        for (int k = 0; k < d; ++k) qr[k] = (double)or_load(qrow + k, dtype) * (double)signs[k];
        or_fwht_f64(qr, d);
        double qsum = 0.0;
        for (int k = 0; k < d; ++k) qsum += qr[k];
        double c = softmax_scale / (double)d;
        for (int sgi = 0; sgi < num_segments; ++sgi) {
          double m = -INFINITY, l = 0.0;
          for (int k = 0; k < d; ++k) acc[k] = 0.0;
          int64_t b0 = blo + (int64_t)sgi * per, b1 = b0 + per;
          if (b1 > nblk) b1 = nblk;
          for (int64_t blk = b0; blk < b1; ++blk) {
            /* scores of this block's keys that the query may see */
            double zb[1024]; /* block_size <= 1024 (checked by the Python wrapper) */
            int64_t j0 = blk * block_size, j1 = j0 + block_size;
            if (j0 < jlo) j0 = jlo;
            if (j1 > pos + 1) j1 = pos + 1;
            if (j0 >= j1) continue;
            double bmax = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
              const uint8_t* row = or_key_row(cache, block_table, bt_stride, b, j, 0, h,
                                              block_size, num_kv_heads, d);
              float s_t;
              int zp;
              oracle_stego_decode(or_row_word(row, d), &s_t, &zp);
              double dot_even = 0.0, dot_odd = 0.0; /* two interleaved streams */
              for (int jj = 0; jj < d / 2; ++jj) {
                dot_even += qr[2 * jj] * (double)(row[jj] & 0xF);
                dot_odd += qr[2 * jj + 1] * (double)((row[jj] >> 4) & 0xF);
              }
              zb[j - j0] = c * (double)s_t * (dot_even + dot_odd - (double)zp * qsum);
              if (softcap > 0.0) zb[j - j0] = softcap * tanh(zb[j - j0] / softcap); /* R-cap */
              if (zb[j - j0] > bmax) bmax = zb[j - j0];
            }
            /* online softmax: rescale the running state to the new maximum */
            double mnew = m > bmax ? m : bmax;
            double alpha = exp(m - mnew); /* exp(-inf) = 0 on the first block */
            l *= alpha;
            for (int k = 0; k < d; ++k) acc[k] *= alpha;
            m = mnew;
            for (int64_t j = j0; j < j1; ++j) {
              double p = exp(zb[j - j0] - m);
              l += p;
              const uint8_t* row = or_key_row(cache, block_table, bt_stride, b, j, 1, h,
                                              block_size, num_kv_heads, d);
              float s_t;
              int zp;
              oracle_stego_decode(or_row_word(row, d), &s_t, &zp);
              double w = p * (double)s_t;
              for (int jj = 0; jj < d / 2; ++jj) { /* per-stream accumulators */
                acc[2 * jj] += w * (double)((int)(row[jj] & 0xF) - zp);
                acc[2 * jj + 1] += w * (double)((int)((row[jj] >> 4) & 0xF) - zp);
              }
            }
          }
          seg_m[sgi] = m;
          seg_l[sgi] = l;
          memcpy(seg_acc + (int64_t)sgi * d, acc, sizeof(double) * (size_t)d);
        }
        /* segment reduction: M = max m_k, L = sum l_k e^(m_k - M),
         * O = sum acc_k e^(m_k - M) / L; an empty segment has m = -inf, l = 0 */
        double M = -INFINITY;
        for (int sgi = 0; sgi < num_segments; ++sgi)
          if (seg_m[sgi] > M) M = seg_m[sgi];
        double Lsum = 0.0;
        for (int k = 0; k < d; ++k) acc[k] = 0.0;
        for (int sgi = 0; sgi < num_segments; ++sgi) {
          if (seg_m[sgi] == -INFINITY) continue;
          double f = exp(seg_m[sgi] - M);
          Lsum += seg_l[sgi] * f;
          for (int k = 0; k < d; ++k) acc[k] += seg_acc[(int64_t)sgi * d + k] * f;
        }
        for (int k = 0; k < d; ++k) acc[k] /= Lsum;
        /* epilogue: back from the rotated domain */
        oracle_rht_inverse_f64(acc, d, signs);
        memcpy(o, acc, sizeof(double) * (size_t)d);
      }
    }
  }
  free(qr);
  free(acc);
  free(seg_acc);
  free(seg_m);
  free(seg_l);
}

/* ==========================================================================
 * INT8 per-token-head mode (the sibling mode on the same cache family).
 *
 * Readings (listed with the INT4 ones in the design notes):
 *   R8-layout cache uint8 [num_blocks][2][block_size][num_kv_heads][d + 4]:
 *             d int8 codes (two's complement bytes), then the fp32 scale,
 *             little-endian.  ([report] key snippets: get_kv_cache_shape keeps
 *             data_head_size = head_size for modes other than INT4 and adds a
 *             scale pad of 4 bytes for a 1-byte cache dtype.)
 *   R8-quant  no rotation; s = max(fl(absmax / 127), 1e-6f); inv = fl(1 / s);
 *             v = fl(x * inv).  ([testfile] helpers: per-token-head
 *             reference quantizer, data * (1.0 / scales), quant_max 127.)
 *   R8-round  q = trunc(fl(v + 0.5)) for v >= 0, trunc(fl(v - 0.5)) for
 *             v < 0, then clamped to [-128, 127]: round half away from zero
 *             the way the INT8 write-kernel fix describes it ([pr40633]
 *             commit on the INT8 reshape kernel: +0.5 / -0.5, then to int32).
 *             The test reference's torch.round (half to even) differs only at
 *             exact .5 ties and where fl(v + 0.5) rounds up to an integer.
 *   R8-deq    x_hat = q * s.
 * ========================================================================== */

static int64_t or8_row_offset(int64_t blk, int kv, int64_t off, int h, int block_size,
                              int num_kv_heads, int d) {
  int64_t R = d + 4;
  return (((blk * 2 + kv) * block_size + off) * num_kv_heads + h) * R;
}

/* Quantizes one row of d fp32 values: d codes and the scale. */
void oracle_quantize_row_int8(const float* x, int d, int8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < d; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float s = amax / 127.0f;
  if (!(s > 1e-6f)) s = 1e-6f; /* clamp(min=1e-6) */
  float inv = 1.0f / s;
  for (int i = 0; i < d; ++i) {
    float v = x[i] * inv;
    float t = v >= 0.0f ? v + 0.5f : v - 0.5f; /* one rounded fp32 add */
    long q = (long)t;                          /* C conversion truncates toward zero */
    if (q < -128) q = -128;
    if (q > 127) q = 127;
    codes[i] = (int8_t)q;
  }
  *scale = s;
}

/* The INT8 write: every (token, head, K|V) row with slot >= 0 goes to block
 * slot / block_size, offset slot % block_size; other rows are untouched. */
void oracle_kv_write_int8(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                          int64_t value_stride, int dtype, const int64_t* slot_mapping,
                          int num_tokens, uint8_t* cache, int num_blocks, int block_size,
                          int num_kv_heads, int d) {
  (void)num_blocks;
  float* x = (float*)malloc(sizeof(float) * (size_t)d);
  int8_t* codes = (int8_t*)malloc((size_t)d);
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = kv == 0 ? key + (int64_t)t * key_stride
                                    : value + (int64_t)t * value_stride;
      for (int h = 0; h < num_kv_heads; ++h) {
        for (int i = 0; i < d; ++i) x[i] = or_load(src + (int64_t)h * d + i, dtype);
        float s;
        oracle_quantize_row_int8(x, d, codes, &s);
        uint8_t* row = cache + or8_row_offset(blk, kv, off, h, block_size, num_kv_heads, d);
        memcpy(row, codes, (size_t)d);
        uint32_t w = or_f32_bits(s);
        row[d + 0] = (uint8_t)(w & 0xFF);
        row[d + 1] = (uint8_t)((w >> 8) & 0xFF);
        row[d + 2] = (uint8_t)((w >> 16) & 0xFF);
        row[d + 3] = (uint8_t)((w >> 24) & 0xFF);
      }
    }
  }
  free(codes);
  free(x);
}

/* Dequantised row x_hat_i = q_i * s (R8-deq), fp64. */
void oracle_decode_row_int8(const uint8_t* row, int d, double* out) {
  uint32_t w = (uint32_t)row[d] | ((uint32_t)row[d + 1] << 8) | ((uint32_t)row[d + 2] << 16) |
               ((uint32_t)row[d + 3] << 24);
  double s = (double)or_bits_f32(w);
  for (int i = 0; i < d; ++i) out[i] = (double)(int8_t)row[i] * s;
}

/* Plain causal softmax attention over the dequantised INT8 cache (fp64), with
 * the same positions, GQA mapping, window and soft cap as the INT4 oracle
 * (R-pos, R-gqa, R-win, R-cap). */
void oracle_attention_plain_int8(const uint16_t* q, int64_t q_stride, int dtype,
                                 const uint8_t* cache, int num_blocks, int block_size,
                                 int num_kv_heads, int d, int num_q_heads,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                 int num_seqs, const int32_t* block_table, int bt_stride,
                                 double softmax_scale, int window, double softcap, double* out) {
  (void)num_blocks;
  int G = num_q_heads / num_kv_heads;
  for (int b = 0; b < num_seqs; ++b) {
    int q0 = cu_seqlens_q[b], qlen = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int64_t L = seqused_k[b];
    if (qlen <= 0 || L <= 0) continue;
    for (int h = 0; h < num_kv_heads; ++h) {
      double* K = (double*)malloc(sizeof(double) * (size_t)(L * d));
      double* V = (double*)malloc(sizeof(double) * (size_t)(L * d));
      for (int64_t j = 0; j < L; ++j) {
        int64_t blk = block_table[(int64_t)b * bt_stride + j / block_size];
        oracle_decode_row_int8(
            cache + or8_row_offset(blk, 0, j % block_size, h, block_size, num_kv_heads, d), d,
            K + j * d);
        oracle_decode_row_int8(
            cache + or8_row_offset(blk, 1, j % block_size, h, block_size, num_kv_heads, d), d,
            V + j * d);
      }
      double* z = (double*)malloc(sizeof(double) * (size_t)L);
      double* qv = (double*)malloc(sizeof(double) * (size_t)d);
      for (int i = 0; i < qlen; ++i) {
        int64_t pos = L - qlen + i;
        for (int gg = 0; gg < G; ++gg) {
          int g = h * G + gg;
          const uint16_t* qrow = q + (int64_t)(q0 + i) * q_stride + (int64_t)g * d;
          for (int k = 0; k < d; ++k) qv[k] = (double)or_load(qrow + k, dtype);
          double* o = out + ((int64_t)(q0 + i) * num_q_heads + g) * d;
          for (int k = 0; k < d; ++k) o[k] = 0.0;
          if (pos < 0) continue;
          int64_t jlo = 0;
          if (window > 0 && pos - window + 1 > 0) jlo = pos - window + 1;
          double zmax = -INFINITY;
          for (int64_t j = jlo; j <= pos; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += qv[k] * K[j * d + k];
            z[j] = softmax_scale * acc;
            if (softcap > 0.0) z[j] = softcap * tanh(z[j] / softcap);
            if (z[j] > zmax) zmax = z[j];
          }
          double den = 0.0;
          for (int64_t j = jlo; j <= pos; ++j) {
            z[j] = exp(z[j] - zmax);
            den += z[j];
          }
          for (int64_t j = jlo; j <= pos; ++j) {
            double w = z[j] / den;
            for (int k = 0; k < d; ++k) o[k] += w * V[j * d + k];
          }
        }
      }
      free(qv);
      free(z);
      free(K);
      free(V);
    }
  }
}

/* ==========================================================================
 * INT2 Lloyd-Max mode ([pr40633] description and its commit on the packed
 * modes: four 2-bit codes per byte, Hadamard pre-rotation, dequantisation by
 * a lookup into four centroids fitted over N(0, 1); the mode was dropped from
 * the merged PR, [report]).
 *
 * Readings (listed with the others in the design notes):
 *   R2-layout cache uint8 [num_blocks][2][block_size][num_kv_heads][d/4 + 4]:
 *             d/4 code bytes, element 4j + k in bits 2k, 2k+1 of byte j,
 *             then the fp32 scale, little-endian.
 *   R2-rot    the INT4 mode's rotation y = H (D x) (R-rht, R-fwht) with the
 *             caller's signs; the pages' unrandomised "full" Hadamard is the
 *             case D = I (all signs +1).
 *   R2-lm     the 4-level Lloyd-Max quantizer of N(0, 1): levels -b, -a, a, b
 *             for codes 0..3, thresholds -t, 0, t with t = (a + b) / 2
 *             (nearest level; a value on a threshold takes the upper code).
 *   R2-scale  s = max(sqrt(sum y_i^2 / d), 1e-6): the row's RMS in the
 *             rotated domain, which brings a Gaussian-like row to N(0, 1).
 *             fp32, squares summed pairwise (halves, recursively), then one
 *             correctly rounded sqrt; inv = fl(1 / s), v = fl(y * inv).  The
 *             pages' "d1.5 scale factor" is garbled: nothing else is folded
 *             into the stored scale (parity unpinned for that phrase).
 *   R2-deq    y_hat_i = s * level(code_i), then x_hat = D (H y_hat) / d.
 * ========================================================================== */

static double or_npdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }
static double or_ncdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Lloyd's iteration for four levels over N(0, 1), kept symmetric (the density
 * is): with thresholds 0 and +-t, the levels are the conditional means of
 * their cells, a = E[X | 0 <= X < t] and b = E[X | X >= t]; then t moves to
 * the midpoint (a + b) / 2.  Repeated until t stops changing in fp64. */
void oracle_lloyd_max4(double* a_out, double* b_out, double* t_out) {
  static int done = 0; /* computed once per process */
  static double a = 0.0, b = 0.0, t = 1.0;
  if (!done) {
    for (int it = 0; it < 100000; ++it) {
      a = (or_npdf(0.0) - or_npdf(t)) / (or_ncdf(t) - 0.5);
      b = or_npdf(t) / (1.0 - or_ncdf(t));
      double tn = 0.5 * (a + b);
      double step = fabs(tn - t);
      t = tn;
      if (step <= 1e-15) break; /* converged to fp64 resolution */
    }
    done = 1;
  }
  *a_out = a;
  *b_out = b;
  *t_out = t;
}

static int64_t or2_row_offset(int64_t blk, int kv, int64_t off, int h, int block_size,
                              int num_kv_heads, int d) {
  int64_t R = d / 4 + 4;
  return (((blk * 2 + kv) * block_size + off) * num_kv_heads + h) * R;
}

/* fp32 sum of y_i^2 over [lo, lo + n), n a power of two, by halves. */
static float or_pairwise_sq(const float* y, int lo, int n) {
  if (n == 1) return y[lo] * y[lo];
  return or_pairwise_sq(y, lo, n / 2) + or_pairwise_sq(y, lo + n / 2, n / 2);
}

/* Quantizes one rotated row: d/4 code bytes and the scale (R2-lm, R2-scale). */
void oracle_quantize_row_int2(const float* y, int d, uint8_t* bytes, float* scale) {
  double a, b, t;
  oracle_lloyd_max4(&a, &b, &t);
  const float tf = (float)t;
  float s = sqrtf(or_pairwise_sq(y, 0, d) / (float)d);
  if (!(s > 1e-6f)) s = 1e-6f;
  float inv = 1.0f / s;
  memset(bytes, 0, (size_t)(d / 4));
  for (int i = 0; i < d; ++i) {
    float v = y[i] * inv;
    int code = (v >= -tf) + (v >= 0.0f) + (v >= tf);
    bytes[i / 4] |= (uint8_t)(code << (2 * (i % 4)));
  }
  *scale = s;
}

/* The INT2 write: rotate (R2-rot) and quantize every (token, head, K|V) row
 * with slot >= 0; rows of negative slots are untouched. */
void oracle_kv_write_int2(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                          int64_t value_stride, int dtype, const int64_t* slot_mapping,
                          int num_tokens, uint8_t* cache, int num_blocks, int block_size,
                          int num_kv_heads, int d, const float* signs) {
  (void)num_blocks;
  float* y = (float*)malloc(sizeof(float) * (size_t)d);
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = kv == 0 ? key + (int64_t)t * key_stride
                                    : value + (int64_t)t * value_stride;
      for (int h = 0; h < num_kv_heads; ++h) {
        for (int i = 0; i < d; ++i) y[i] = or_load(src + (int64_t)h * d + i, dtype);
        oracle_rht_forward_f32(y, d, signs);
        uint8_t* row = cache + or2_row_offset(blk, kv, off, h, block_size, num_kv_heads, d);
        float s;
        oracle_quantize_row_int2(y, d, row, &s);
        uint32_t w = or_f32_bits(s);
        row[d / 4 + 0] = (uint8_t)(w & 0xFF);
        row[d / 4 + 1] = (uint8_t)((w >> 8) & 0xFF);
        row[d / 4 + 2] = (uint8_t)((w >> 16) & 0xFF);
        row[d / 4 + 3] = (uint8_t)((w >> 24) & 0xFF);
      }
    }
  }
  free(y);
}

/* Original-domain dequantised row (R2-deq), fp64. */
void oracle_decode_row_int2(const uint8_t* row, int d, const float* signs, double* out) {
  double a, b, t;
  oracle_lloyd_max4(&a, &b, &t);
  const double level[4] = {-b, -a, a, b};
  uint32_t w = (uint32_t)row[d / 4] | ((uint32_t)row[d / 4 + 1] << 8) |
               ((uint32_t)row[d / 4 + 2] << 16) | ((uint32_t)row[d / 4 + 3] << 24);
  double s = (double)or_bits_f32(w);
  for (int i = 0; i < d; ++i) out[i] = s * level[(row[i / 4] >> (2 * (i % 4))) & 3];
  oracle_rht_inverse_f64(out, d, signs);
}

/* Plain causal softmax attention over the dequantised INT2 cache (fp64), with
 * the positions, GQA mapping, window and soft cap of the INT4 oracle. */
void oracle_attention_plain_int2(const uint16_t* q, int64_t q_stride, int dtype,
                                 const uint8_t* cache, int num_blocks, int block_size,
                                 int num_kv_heads, int d, int num_q_heads,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                 int num_seqs, const int32_t* block_table, int bt_stride,
                                 double softmax_scale, const float* signs, int window,
                                 double softcap, double* out) {
  (void)num_blocks;
  int G = num_q_heads / num_kv_heads;
  for (int bq = 0; bq < num_seqs; ++bq) {
    int q0 = cu_seqlens_q[bq], qlen = cu_seqlens_q[bq + 1] - cu_seqlens_q[bq];
    int64_t L = seqused_k[bq];
    if (qlen <= 0 || L <= 0) continue;
    for (int h = 0; h < num_kv_heads; ++h) {
      double* K = (double*)malloc(sizeof(double) * (size_t)(L * d));
      double* V = (double*)malloc(sizeof(double) * (size_t)(L * d));
      for (int64_t j = 0; j < L; ++j) {
        int64_t blk = block_table[(int64_t)bq * bt_stride + j / block_size];
        oracle_decode_row_int2(
            cache + or2_row_offset(blk, 0, j % block_size, h, block_size, num_kv_heads, d), d,
            signs, K + j * d);
        oracle_decode_row_int2(
            cache + or2_row_offset(blk, 1, j % block_size, h, block_size, num_kv_heads, d), d,
            signs, V + j * d);
      }
      double* z = (double*)malloc(sizeof(double) * (size_t)L);
      double* qv = (double*)malloc(sizeof(double) * (size_t)d);
      for (int i = 0; i < qlen; ++i) {
        int64_t pos = L - qlen + i;
        for (int gg = 0; gg < G; ++gg) {
          int g = h * G + gg;
          const uint16_t* qrow = q + (int64_t)(q0 + i) * q_stride + (int64_t)g * d;
          for (int k = 0; k < d; ++k) qv[k] = (double)or_load(qrow + k, dtype);
          double* o = out + ((int64_t)(q0 + i) * num_q_heads + g) * d;
          for (int k = 0; k < d; ++k) o[k] = 0.0;
          if (pos < 0) continue;
          int64_t jlo = 0;
          if (window > 0 && pos - window + 1 > 0) jlo = pos - window + 1;
          double zmax = -INFINITY;
          for (int64_t j = jlo; j <= pos; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += qv[k] * K[j * d + k];
            z[j] = softmax_scale * acc;
            if (softcap > 0.0) z[j] = softcap * tanh(z[j] / softcap);
            if (z[j] > zmax) zmax = z[j];
          }
          double den = 0.0;
          for (int64_t j = jlo; j <= pos; ++j) {
            z[j] = exp(z[j] - zmax);
            den += z[j];
          }
          for (int64_t j = jlo; j <= pos; ++j) {
            double w = z[j] / den;
            for (int k = 0; k < d; ++k) o[k] += w * V[j * d + k];
          }
        }
      }
      free(qv);
      free(z);
      free(K);
      free(V);
    }
  }
}

/* Threads the OpenMP loops above use (the timing harness only; results do not
 * depend on it).  Without OpenMP everything runs on one thread. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
