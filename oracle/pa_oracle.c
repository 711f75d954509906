/*
 * pa_oracle.c -- CPU oracle for decode-time paged attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  Built with
 * gcc -O2 -ffp-contract=off (no fast-math, no fused multiply-add), so each
 * operation rounds exactly once, in the precision of its instantiation.
 *
 * ORACLE_MUTATION (default 0) plants one known mistake for the tests that
 * prove the pins can fail; the shipped build has none:
 *   1 window one key short          6 merge weight without l_j
 *   2 interleaved GQA head map      7 softmax scale dropped
 *   3 slot mirrored inside a page   8 MLA value row shifted by d_rope
 *   4 W_UK read as [j][d]           9 MLA rope term dropped
 *   5 lse without the max          10 split partitions counted from key 0
 *  11 KV insert: page and in-page offset of a slot swapped
 *  12 MLA insert: rope part written first, latent after it
 *  13 multi-query decode: causal limit one key too far
 *  14 FP8 decode: e4m3 exponent bias read as 8 instead of 7
 *  15 FP8 decode: the K and V scales swapped
 *  16 f32 decode: V rows read one token after K's
 *  17 FP8 MLA insert: block exponent floor(log2(absmax / 448)) instead of ceil
 *  18 FP8 MLA decode: block scale 2^(byte - 128) instead of 2^(byte - 127)
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "pa_oracle.h"

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

/* bf16 -> float is exact: the 16 stored bits are the top half of an IEEE
 * binary32 pattern. */
static float bf16_to_float(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return f;
}

#define REAL double
#define EXPR exp
#define LOGR log
#define NAME(x) x##_f64
#define BF(x) ((REAL)bf16_to_float(x))
#include "pa_oracle_body.h"
#undef REAL
#undef EXPR
#undef LOGR
#undef NAME
#undef BF

#define REAL float
#define EXPR expf
#define LOGR logf
#define NAME(x) x##_f32
#define BF(x) ((REAL)bf16_to_float(x))
#include "pa_oracle_body.h"
#undef REAL
#undef EXPR
#undef LOGR
#undef NAME
#undef BF

void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

int32_t oracle_mutation(void) { return ORACLE_MUTATION; }

/* KV insert ("reshape and cache"): token i of the source goes to the flat
 * slot s = slots[i] = page * page_size + offset of the pool, every KV head,
 * as a plain copy of the bf16 bits [vllm.cpp kernel matrix, row
 * KERNEL-KV-CACHE: KV insert into the paged cache, checked exactly since a
 * copy does not round].  Slots outside [0, num_pages * page_size) -- negative
 * ones mark padding -- are skipped. */
int oracle_kv_insert(const uint16_t* k_new, const uint16_t* v_new, int64_t src_token_stride,
                     int64_t src_head_stride, uint16_t* k_pool, uint16_t* v_pool,
                     const oracle_pool* pool, const int64_t* slots, int32_t num_tokens) {
  if (!k_new || !v_new || !k_pool || !v_pool || !pool || !slots || num_tokens < 0 ||
      pool->num_pages <= 0 || pool->page_size <= 0 || pool->num_kv_heads <= 0 ||
      pool->head_dim <= 0)
    return ORACLE_ERR_ARGS;
  const int64_t total = (int64_t)pool->num_pages * pool->page_size;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slots[i];
    if (s < 0 || s >= total) continue;
#if ORACLE_MUTATION == 11
    const int64_t page = s % pool->page_size, off = s / pool->page_size; /* planted */
    if (page >= pool->num_pages || off >= pool->page_size) continue;
#else
    const int64_t page = s / pool->page_size, off = s % pool->page_size;
#endif
    for (int32_t h = 0; h < pool->num_kv_heads; ++h) {
      const int64_t dst = page * pool->page_stride + h * pool->head_stride + off * pool->token_stride;
      const int64_t src = i * src_token_stride + h * src_head_stride;
      for (int32_t d = 0; d < pool->head_dim; ++d) {
        k_pool[dst + d] = k_new[src + d];
        v_pool[dst + d] = v_new[src + d];
      }
    }
  }
  return ORACLE_OK;
}

/* MLA cache write: row s of the latent cache becomes the latent part kv_c
 * (d_lat values) followed by the rope part k_pe (d_rope values), copied bit
 * for bit [vllm.cpp kernel matrix, row KERNEL-KV-CACHE: the MLA cache write
 * concatenates the two projections into the 576-wide row, exact, with
 * strided sources].  Slots outside the pool are skipped. */
int oracle_mla_cache_insert(const uint16_t* kv_c, int64_t c_stride, const uint16_t* k_pe,
                            int64_t pe_stride, uint16_t* cache, const oracle_pool* pool,
                            const int64_t* slots, int32_t num_tokens, int32_t d_lat,
                            int32_t d_rope) {
  if (!kv_c || !k_pe || !cache || !pool || !slots || num_tokens < 0 || d_lat <= 0 ||
      d_rope < 0 || pool->num_kv_heads != 1 || pool->head_dim != d_lat + d_rope ||
      pool->num_pages <= 0 || pool->page_size <= 0)
    return ORACLE_ERR_ARGS;
  const int64_t total = (int64_t)pool->num_pages * pool->page_size;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slots[i];
    if (s < 0 || s >= total) continue;
    uint16_t* row = cache + (s / pool->page_size) * pool->page_stride +
                    (s % pool->page_size) * pool->token_stride;
#if ORACLE_MUTATION == 12
    for (int32_t r = 0; r < d_rope; ++r) row[r] = k_pe[i * pe_stride + r]; /* planted */
    for (int32_t j = 0; j < d_lat; ++j) row[d_rope + j] = kv_c[i * c_stride + j];
#else
    for (int32_t j = 0; j < d_lat; ++j) row[j] = kv_c[i * c_stride + j];
    for (int32_t r = 0; r < d_rope; ++r) row[d_lat + r] = k_pe[i * pe_stride + r];
#endif
  }
  return ORACLE_OK;
}

/* ---- FP8 (OCP E4M3) KV cache ------------------------------------------------
 *
 * A quantized pool stores one byte per element; the real value is the byte's
 * E4M3 value times the pool's scale [vllm.cpp kernel matrix, inventory row
 * "Quantized KV cache, including FP8 and NVFP4" (the paged path there admits
 * F32/BF16 only); row KERNEL-KV-CACHE-DSA, the fp8_ds_mla dequant read: an
 * e4m3 element times its scale].  The pages fix no scale granularity for a
 * GQA pool; the reading taken is one scale per K pool and one per V pool. */

/* OCP FP8 E4M3 ("e4m3fn"): sign = bit 7, exponent E = bits 6..3 with bias 7,
 * mantissa M = bits 2..0.  E = 0 is subnormal, M * 2^-9; otherwise
 * (1 + M/8) * 2^(E-7), except S.1111.111, which is NaN.  There are no
 * infinities; the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t byte) {
  const int sign = byte >> 7;
  const int e = (byte >> 3) & 15;
  const int m = byte & 7;
#if ORACLE_MUTATION == 14
  const int bias = 8; /* planted */
#else
  const int bias = 7;
#endif
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, 1 - bias - 3);
  else
    v = ldexp(1.0 + m / 8.0, e - bias);
  return sign ? -v : v;
}

/* Decode with FP8 pools, float64: K_t = e4m3(k byte) * k_scale, V_t =
 * e4m3(v byte) * v_scale, then the same two-pass softmax attention as
 * oracle_pa_decode over keys [lo, n) in ascending order. */
int oracle_pa_decode_fp8(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                         const oracle_pool* pool, const int32_t* block_table, int32_t bt_stride,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                         double scale, double k_scale, double v_scale, int32_t window,
                         double* out, double* lse) {
  if (!q || !k_pool || !v_pool || !pool || !block_table || !context_lens || !out || !lse ||
      batch < 0 || num_q_heads <= 0 || pool->num_pages <= 0 || pool->page_size <= 0 ||
      pool->num_kv_heads <= 0 || pool->head_dim <= 0 || num_q_heads % pool->num_kv_heads)
    return ORACLE_ERR_ARGS;
#if ORACLE_MUTATION == 15
  { const double t = k_scale; k_scale = v_scale; v_scale = t; } /* planted */
#endif
  const int32_t D = pool->head_dim;
  const int32_t G = num_q_heads / pool->num_kv_heads;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_q_heads; ++h) {
      const int32_t n = context_lens[b];
      const int32_t lo = (window > 0 && n - window > 0) ? n - window : 0;
      const int32_t g = h / G;
      const uint16_t* qr = q + ((int64_t)b * num_q_heads + h) * D;
      const int32_t* bt = block_table + (int64_t)b * bt_stride;
      double* o = out + ((int64_t)b * num_q_heads + h) * D;
      for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
      const int32_t cnt = n > lo ? n - lo : 0;
      double* sc = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
      if (!sc) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
        continue;
      }
      int bad = 0;
      double m = -INFINITY;
      for (int32_t i = 0; i < cnt && !bad; ++i) {          /* pass 1: scores, max */
        const int32_t t = lo + i;
        const int32_t page = bt[t / pool->page_size];
        if (page < 0 || page >= pool->num_pages) { bad = 1; break; }
        const uint8_t* k = k_pool + (int64_t)page * pool->page_stride +
                           (int64_t)g * pool->head_stride +
                           (int64_t)(t % pool->page_size) * pool->token_stride;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
          dot += (double)bf16_to_float(qr[d]) * (oracle_e4m3_value(k[d]) * k_scale);
        sc[i] = scale * dot;
        if (sc[i] > m) m = sc[i];
      }
      double l = 0.0;
      for (int32_t i = 0; i < cnt && !bad; ++i) {          /* pass 2: sums */
        const int32_t t = lo + i;
        const int32_t page = bt[t / pool->page_size];
        const uint8_t* v = v_pool + (int64_t)page * pool->page_stride +
                           (int64_t)g * pool->head_stride +
                           (int64_t)(t % pool->page_size) * pool->token_stride;
        const double e = exp(sc[i] - m);
        l += e;
        for (int32_t d = 0; d < D; ++d) o[d] += e * (oracle_e4m3_value(v[d]) * v_scale);
      }
      free(sc);
      if (bad) {
#pragma omp atomic write
        err = ORACLE_ERR_PAGE;
        continue;
      }
      if (cnt > 0)
        for (int32_t d = 0; d < D; ++d) o[d] /= l;
      lse[(int64_t)b * num_q_heads + h] = cnt > 0 ? m + log(l) : -INFINITY;
    }
  }
  return err;
}

/* ---- f32 KV cache -----------------------------------------------------------
 *
 * Pools of IEEE binary32 elements, read as they are [vllm.cpp PR #425, the
 * row loader's float instantiation next to the bf16 one; vllm.cpp kernel
 * matrix, inventory row: the paged path admits F32/BF16].  float64
 * arithmetic, the same two-pass softmax attention as oracle_pa_decode. */
int oracle_pa_decode_f32pool(const uint16_t* q, const float* k_pool, const float* v_pool,
                             const oracle_pool* pool, const int32_t* block_table,
                             int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, double scale, int32_t window, double* out,
                             double* lse) {
  if (!q || !k_pool || !v_pool || !pool || !block_table || !context_lens || !out || !lse ||
      batch < 0 || num_q_heads <= 0 || pool->num_pages <= 0 || pool->page_size <= 0 ||
      pool->num_kv_heads <= 0 || pool->head_dim <= 0 || num_q_heads % pool->num_kv_heads)
    return ORACLE_ERR_ARGS;
  const int32_t D = pool->head_dim;
  const int32_t G = num_q_heads / pool->num_kv_heads;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_q_heads; ++h) {
      const int32_t n = context_lens[b];
      const int32_t lo = (window > 0 && n - window > 0) ? n - window : 0;
      const int32_t g = h / G;
      const uint16_t* qr = q + ((int64_t)b * num_q_heads + h) * D;
      const int32_t* bt = block_table + (int64_t)b * bt_stride;
      double* o = out + ((int64_t)b * num_q_heads + h) * D;
      for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
      const int32_t cnt = n > lo ? n - lo : 0;
      double* sc = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
      if (!sc) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
        continue;
      }
      int bad = 0;
      double m = -INFINITY;
      for (int32_t i = 0; i < cnt; ++i) {                  /* pass 1: scores, max */
        const int32_t t = lo + i;
        const int32_t page = bt[t / pool->page_size];
        if (page < 0 || page >= pool->num_pages) { bad = 1; break; }
        const float* k = k_pool + (int64_t)page * pool->page_stride +
                         (int64_t)g * pool->head_stride +
                         (int64_t)(t % pool->page_size) * pool->token_stride;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += (double)bf16_to_float(qr[d]) * (double)k[d];
        sc[i] = scale * dot;
        if (sc[i] > m) m = sc[i];
      }
      double l = 0.0;
      for (int32_t i = 0; i < cnt && !bad; ++i) {          /* pass 2: sums */
        const int32_t t = lo + i;
        const int32_t page = bt[t / pool->page_size];
#if ORACLE_MUTATION == 16
        const int32_t slot = (t + 1) % pool->page_size; /* planted */
#else
        const int32_t slot = t % pool->page_size;
#endif
        const float* v = v_pool + (int64_t)page * pool->page_stride +
                         (int64_t)g * pool->head_stride + (int64_t)slot * pool->token_stride;
        const double e = exp(sc[i] - m);
        l += e;
        for (int32_t d = 0; d < D; ++d) o[d] += e * (double)v[d];
      }
      free(sc);
      if (bad) {
#pragma omp atomic write
        err = ORACLE_ERR_PAGE;
        continue;
      }
      if (cnt > 0)
        for (int32_t d = 0; d < D; ++d) o[d] /= l;
      lse[(int64_t)b * num_q_heads + h] = cnt > 0 ? m + log(l) : -INFINITY;
    }
  }
  return err;
}

/* ---- FP8 MLA latent cache ----------------------------------------------------
 *
 * The fp8_ds_mla cache state of the pages [vllm.cpp kernel matrix, row
 * KERNEL-KV-CACHE-DSA]: the latent is quantized to E4M3 in blocks of 64
 * elements, each block with one UE8M0 power-of-two scale whose exponent is
 * ceil(log2(absmax / 448)) (stored as exponent + 127); the rope part stays
 * bf16; the dequant read is e4m3(byte) * 2^(scale byte - 127).  The pages
 * apply it to a 448 + 64 latent; here it is applied to the d_lat + d_rope
 * latent of the MLA path (all d_lat values in blocks of 64), with this row
 * layout, in bytes:
 *   [0, d_lat)                        E4M3 latent
 *   [d_lat, d_lat + 2 d_rope)         rope, bf16 little-endian
 *   [d_lat + 2 d_rope, + d_lat / 64)  scale bytes, block j at offset j
 *   then zero bytes up to the row size (pool->head_dim bytes).
 * Readings where the pages are silent: an all-zero block (absmax 0) and any
 * block whose exponent falls outside [-126, 127] take the nearest end of that
 * range, so every scale is a normal float32; the element byte is the E4M3
 * value nearest x / 2^exponent (|x / 2^exponent| <= 448 by the choice of the
 * exponent), ties to the even code, sign bit = the sign bit of x. */

#define ORACLE_FP8_BLOCK 64

/* Block exponent: the smallest e with 448 * 2^e >= absmax, clamped. */
static int fp8_block_exponent(double absmax) {
  if (absmax == 0.0) return -126;
#if ORACLE_MUTATION == 17
  double e = floor(log2(absmax / 448.0)); /* planted */
#else
  double e = ceil(log2(absmax / 448.0));
#endif
  if (e < -126) e = -126;
  if (e > 127) e = 127;
  return (int)e;
}

/* E4M3 byte nearest to v (|v| <= 448), ties to the even code, by comparing
 * v with the value of every finite non-negative code. */
uint8_t oracle_e4m3_encode(double v) {
  const double a = fabs(v);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 127; ++c) {   /* 0x7F is NaN */
    const double d = fabs(oracle_e4m3_value((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(signbit(v) ? (best | 0x80) : best);
}

static int mla_fp8_row_ok(const oracle_pool* pool, int32_t d_lat, int32_t d_rope) {
  return pool && pool->num_kv_heads == 1 && pool->num_pages > 0 && pool->page_size > 0 &&
         d_lat > 0 && d_lat % ORACLE_FP8_BLOCK == 0 && d_rope >= 0 &&
         pool->head_dim >= d_lat + 2 * d_rope + d_lat / ORACLE_FP8_BLOCK &&
         pool->token_stride >= pool->head_dim;
}

int oracle_mla_cache_insert_fp8(const uint16_t* kv_c, int64_t c_stride, const uint16_t* k_pe,
                                int64_t pe_stride, uint8_t* cache, const oracle_pool* pool,
                                const int64_t* slots, int32_t num_tokens, int32_t d_lat,
                                int32_t d_rope) {
  if (!kv_c || !k_pe || !cache || !slots || num_tokens < 0 || !mla_fp8_row_ok(pool, d_lat, d_rope))
    return ORACLE_ERR_ARGS;
  const int64_t total = (int64_t)pool->num_pages * pool->page_size;
  const int32_t nblk = d_lat / ORACLE_FP8_BLOCK;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slots[i];
    if (s < 0 || s >= total) continue;
    uint8_t* row = cache + (s / pool->page_size) * pool->page_stride +
                   (s % pool->page_size) * pool->token_stride;
    const uint16_t* x = kv_c + i * c_stride;
    for (int32_t j = 0; j < nblk; ++j) {
      double absmax = 0.0;
      for (int32_t k = 0; k < ORACLE_FP8_BLOCK; ++k) {
        const double a = fabs((double)bf16_to_float(x[j * ORACLE_FP8_BLOCK + k]));
        if (a > absmax) absmax = a;
      }
      const int e = fp8_block_exponent(absmax);
      for (int32_t k = 0; k < ORACLE_FP8_BLOCK; ++k) {
        const int32_t d = j * ORACLE_FP8_BLOCK + k;
        double q = ldexp((double)bf16_to_float(x[d]), -e);
        if (q > 448.0) q = 448.0;   /* only reachable with the planted floor */
        if (q < -448.0) q = -448.0;
        row[d] = oracle_e4m3_encode(q);
      }
      row[d_lat + 2 * d_rope + j] = (uint8_t)(e + 127);
    }
    for (int32_t r = 0; r < d_rope; ++r) {
      const uint16_t v = k_pe[i * pe_stride + r];
      row[d_lat + 2 * r] = (uint8_t)(v & 0xff);
      row[d_lat + 2 * r + 1] = (uint8_t)(v >> 8);
    }
    for (int32_t o = d_lat + 2 * d_rope + nblk; o < pool->head_dim; ++o) row[o] = 0;
  }
  return ORACLE_OK;
}

/* Value of element d of a row: the dequantized latent (d < d_lat) or the
 * bf16 rope part. */
static double mla_fp8_elem(const uint8_t* row, int32_t d, int32_t d_lat, int32_t d_rope) {
  if (d < d_lat) {
    const int sb = row[d_lat + 2 * d_rope + d / ORACLE_FP8_BLOCK];
#if ORACLE_MUTATION == 18
    return ldexp(oracle_e4m3_value(row[d]), sb - 128); /* planted */
#else
    return ldexp(oracle_e4m3_value(row[d]), sb - 127);
#endif
  }
  const int32_t r = d - d_lat;
  return (double)bf16_to_float((uint16_t)(row[d_lat + 2 * r] | (row[d_lat + 2 * r + 1] << 8)));
}

/* Absorbed MLA decode over an FP8 latent cache, float64: every row of a
 * sequence is dequantized, then the steps of oracle_mla_decode_f64 follow on
 * the dequantized rows (q_abs, scores over the d_lat + d_rope values, two-pass
 * softmax, o_lat over the latent values, W_UV). */
int oracle_mla_decode_fp8(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* cache,
                          const oracle_pool* pool, const uint16_t* w_uk, const uint16_t* w_uv,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* context_lens, int32_t batch, int32_t num_heads,
                          int32_t d_nope, int32_t d_rope, int32_t d_lat, int32_t d_v,
                          double scale, double* out, double* lse) {
  if (!q_nope || !q_rope || !cache || !w_uk || !w_uv || !block_table || !context_lens || !out ||
      batch < 0 || num_heads <= 0 || d_nope <= 0 || d_v <= 0 || !mla_fp8_row_ok(pool, d_lat, d_rope))
    return ORACLE_ERR_ARGS;
  const int32_t R = d_lat + d_rope;
  int err = ORACLE_OK;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = context_lens[b];
    const int32_t* bt = block_table + (int64_t)b * bt_stride;
    double* rows = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)R);
    if (!rows) return ORACLE_ERR_ARGS;
    int bad = 0;
    for (int32_t t = 0; t < n && !bad; ++t) {
      const int32_t page = bt[t / pool->page_size];
      if (page < 0 || page >= pool->num_pages) { bad = 1; break; }
      const uint8_t* row = cache + (int64_t)page * pool->page_stride +
                           (int64_t)(t % pool->page_size) * pool->token_stride;
      for (int32_t d = 0; d < R; ++d) rows[(int64_t)t * R + d] = mla_fp8_elem(row, d, d_lat, d_rope);
    }
    if (bad) { free(rows); err = ORACLE_ERR_PAGE; continue; }
#pragma omp parallel for schedule(dynamic)
    for (int32_t h = 0; h < num_heads; ++h) {
      const int64_t hr = (int64_t)b * num_heads + h;
      const uint16_t* qn = q_nope + hr * d_nope;
      const uint16_t* qr = q_rope + hr * d_rope;
      double* q_abs = (double*)malloc(sizeof(double) * (size_t)d_lat);
      double* o_lat = (double*)calloc((size_t)d_lat, sizeof(double));
      double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
      if (!q_abs || !o_lat || !s) { free(q_abs); free(o_lat); free(s); continue; }
      for (int32_t j = 0; j < d_lat; ++j) {
        double acc = 0.0;
        for (int32_t d = 0; d < d_nope; ++d)
          acc += (double)bf16_to_float(qn[d]) *
                 (double)bf16_to_float(w_uk[((int64_t)h * d_nope + d) * d_lat + j]);
        q_abs[j] = acc;
      }
      double m = -INFINITY;
      for (int32_t t = 0; t < n; ++t) {
        const double* c = rows + (int64_t)t * R;
        double dot = 0.0;
        for (int32_t j = 0; j < d_lat; ++j) dot += q_abs[j] * c[j];
        for (int32_t r = 0; r < d_rope; ++r) dot += (double)bf16_to_float(qr[r]) * c[d_lat + r];
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
      }
      double l = 0.0;
      for (int32_t t = 0; t < n; ++t) {
        const double e = exp(s[t] - m);
        l += e;
        for (int32_t j = 0; j < d_lat; ++j) o_lat[j] += e * rows[(int64_t)t * R + j];
      }
      for (int32_t j = 0; j < d_lat; ++j) o_lat[j] = (n > 0) ? o_lat[j] / l : 0.0;
      for (int32_t dv = 0; dv < d_v; ++dv) {
        double acc = 0.0;
        for (int32_t j = 0; j < d_lat; ++j)
          acc += (double)bf16_to_float(w_uv[((int64_t)h * d_v + dv) * d_lat + j]) * o_lat[j];
        out[hr * d_v + dv] = acc;
      }
      if (lse) lse[hr] = (n > 0) ? m + log(l) : -INFINITY;
      free(q_abs); free(o_lat); free(s);
    }
    free(rows);
  }
  return err;
}
