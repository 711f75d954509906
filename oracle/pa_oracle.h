/*
 * pa_oracle.h -- the CPU oracle for decode-time paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no source with the GPU path.
 *
 * Every routine exists twice, with suffix _f64 (all arithmetic in double) and
 * _f32 (all arithmetic in float).  _f64 is the parity gate; _f32 is the plain
 * fp32 formulation and is checked against _f64.  Inputs are raw bf16 bit
 * patterns (uint16_t); outputs are double arrays holding the value the
 * routine computed (an f32 result is widened exactly).
 *
 * Definitions followed (sources are cited by page title and section):
 *  - Paged gather: token t of a sequence lives in page block_table[t / ps],
 *    slot t % ps; a block table and per-request lengths are device metadata
 *    read in place [vllm.cpp kernel matrix, row KERNEL-ATTN-DFLASH-PAGED-BLOCK].
 *  - Softmax attention of one query over the gathered keys, computed two-pass
 *    (max, then sums) in ascending token order; the online (streamed) softmax
 *    that the decode kernels use reaches the same value up to rounding order
 *    [vllm.cpp PR #425, commit message: the warp-strided online softmax and
 *    the per-tile loop differ only in reduction order].
 *  - GQA: q head h reads KV head h / (Hq / Hkv) [vllm.cpp PR #49, commit body:
 *    the q heads of one KV group form one work item].
 *  - Split-KV partials (max, sum, normalised partial out) and their merge with
 *    both -inf edge cases, ascending split order, no atomics [vllm.cpp kernel
 *    matrix, row KERNEL-ATTN-MLA-SPARSE, W4/W5].
 *  - Absorbed MLA: q_abs = q_nope . W_UK[h] (W_UK indexed [d][j]); score over
 *    the 576-wide latent row (512 latent ++ 64 rope); V is the latent itself;
 *    out = W_UV[h] . o_lat (W_UV indexed [dv][j]) [pegainfer PR #938, review
 *    quote of the kernel's "Schedule" comment, steps 1-7; vllm.cpp kernel
 *    matrix, row KERNEL-ATTN-MLA-SPARSE, W6 absorption and W4 "v is the
 *    transposed k"].
 *
 * Return codes: 0 on success, ORACLE_ERR_ARGS for bad sizes or pointers,
 * ORACLE_ERR_PAGE when a block-table entry needed for a live token lies
 * outside [0, num_pages).
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_PAGE (-2)

/* Geometry of one KV page pool (all strides in elements). */
typedef struct oracle_pool {
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
} oracle_pool;

/* Full decode: out[b,h,:] (unrounded), lse[b,h] (natural log).  window <= 0
 * means no window; otherwise only keys t >= ctx - window are attended. */
#define ORACLE_DECL_DECODE(SFX)                                                 \
  int oracle_pa_decode##SFX(                                                   \
      const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,       \
      const oracle_pool* pool, const int32_t* block_table, int32_t bt_stride,  \
      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,         \
      double scale, int32_t window, double* out, double* lse);

/* Split-KV partials: partition j of sequence b covers
 * [lo + j*P, min(lo + (j+1)*P, ctx)); empty -> max=-inf, sum=0, out=0.
 * part_out [B,Hq,max_parts,D], part_max/part_sum [B,Hq,max_parts]. */
#define ORACLE_DECL_PARTIALS(SFX)                                               \
  int oracle_pa_partials##SFX(                                                 \
      const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,       \
      const oracle_pool* pool, const int32_t* block_table, int32_t bt_stride,  \
      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,         \
      double scale, int32_t window, int32_t partition_size,                    \
      int32_t max_parts, double* part_out, double* part_max,                   \
      double* part_sum);

/* LSE merge of partials (inputs as double, read at the routine's precision). */
#define ORACLE_DECL_MERGE(SFX)                                                  \
  int oracle_pa_merge##SFX(                                                    \
      const double* part_out, const double* part_max, const double* part_sum,  \
      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,         \
      int32_t head_dim, int32_t partition_size, int32_t max_parts,             \
      int32_t window, double* out, double* lse);

/* Absorbed MLA decode over a single-head latent cache whose rows hold
 * d_lat latent values followed by d_rope rope values.
 * q_nope [B,H,d_nope], q_rope [B,H,d_rope], w_uk [H,d_nope,d_lat],
 * w_uv [H,d_v,d_lat]; out [B,H,d_v]; q_abs_out [B,H,d_lat] may be NULL;
 * lse [B,H] may be NULL. */
#define ORACLE_DECL_MLA(SFX)                                                    \
  int oracle_mla_decode##SFX(                                                  \
      const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* cache,   \
      const oracle_pool* pool, const uint16_t* w_uk, const uint16_t* w_uv,     \
      const int32_t* block_table, int32_t bt_stride,                           \
      const int32_t* context_lens, int32_t batch, int32_t num_heads,           \
      int32_t d_nope, int32_t d_rope, int32_t d_lat, int32_t d_v,              \
      double scale, double* out, double* q_abs_out, double* lse);

ORACLE_DECL_DECODE(_f64)
ORACLE_DECL_DECODE(_f32)
ORACLE_DECL_PARTIALS(_f64)
ORACLE_DECL_PARTIALS(_f32)
ORACLE_DECL_MERGE(_f64)
ORACLE_DECL_MERGE(_f32)
/* Multi-query decode: q [B][S][Hq][D], out [B][S][Hq][D], lse [B][S][Hq];
 * query s sees keys t <= n - S + s (causal) or t < n (not causal), and with
 * a window only the last `window` of those. */
#define ORACLE_DECL_MULTI(SFX)                                                  \
  int oracle_pa_decode_multi##SFX(                                             \
      const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,       \
      const oracle_pool* pool, const int32_t* block_table, int32_t bt_stride,  \
      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,         \
      int32_t num_queries, int32_t causal, double scale, int32_t window,       \
      double* out, double* lse);

ORACLE_DECL_MULTI(_f64)
ORACLE_DECL_MULTI(_f32)
ORACLE_DECL_MLA(_f64)
ORACLE_DECL_MLA(_f32)

/* FP8 KV cache (OCP E4M3 bytes, one scale per pool), float64 only.
 * oracle_e4m3_value decodes one byte (NaN for S.1111.111).
 * oracle_pa_decode_fp8: as oracle_pa_decode_f64 with K = e4m3(k) * k_scale
 * and V = e4m3(v) * v_scale; pool strides are in bytes (= elements). */
double oracle_e4m3_value(uint8_t byte);
int oracle_pa_decode_fp8(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                         const oracle_pool* pool, const int32_t* block_table, int32_t bt_stride,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                         double scale, double k_scale, double v_scale, int32_t window,
                         double* out, double* lse);

/* f32 KV cache: as oracle_pa_decode_f64 over pools of binary32 elements
 * (strides in elements). */
int oracle_pa_decode_f32pool(const uint16_t* q, const float* k_pool, const float* v_pool,
                             const oracle_pool* pool, const int32_t* block_table,
                             int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, double scale, int32_t window, double* out,
                             double* lse);

/* Thread control for the (b, h) loop; results do not depend on it. */
void oracle_set_num_threads(int32_t n);
int32_t oracle_max_threads(void);
/* Which planted mistake (0 = none) this build carries; see pa_oracle.c. */
int32_t oracle_mutation(void);

/* KV insert: token i of k_new / v_new ([token][kv head][dim] with the given
 * element strides) is copied to flat slot slots[i] = page * page_size + offset
 * of both pools; slots outside the pool are skipped. */
int oracle_kv_insert(const uint16_t* k_new, const uint16_t* v_new, int64_t src_token_stride,
                     int64_t src_head_stride, uint16_t* k_pool, uint16_t* v_pool,
                     const oracle_pool* pool, const int64_t* slots, int32_t num_tokens);

/* MLA cache write: row slots[i] becomes kv_c[i][0:d_lat] ++ k_pe[i][0:d_rope]. */
int oracle_mla_cache_insert(const uint16_t* kv_c, int64_t c_stride, const uint16_t* k_pe,
                            int64_t pe_stride, uint16_t* cache, const oracle_pool* pool,
                            const int64_t* slots, int32_t num_tokens, int32_t d_lat,
                            int32_t d_rope);

/* FP8 MLA latent cache (E4M3 latent in blocks of 64 with one UE8M0 scale
 * byte each, bf16 rope); row layout in bytes: [d_lat E4M3][2 d_rope rope]
 * [d_lat / 64 scale bytes][zeros up to pool->head_dim].  pool strides and
 * head_dim count bytes; num_kv_heads = 1.
 * oracle_e4m3_encode: the E4M3 byte nearest to v (|v| <= 448), ties to even.
 * oracle_mla_cache_insert_fp8: quantizes kv_c rows and copies k_pe into the
 * rows at the slots (slots outside the pool are skipped).
 * oracle_mla_decode_fp8: absorbed MLA over the dequantized rows, float64. */
uint8_t oracle_e4m3_encode(double v);
int oracle_mla_cache_insert_fp8(const uint16_t* kv_c, int64_t c_stride, const uint16_t* k_pe,
                                int64_t pe_stride, uint8_t* cache, const oracle_pool* pool,
                                const int64_t* slots, int32_t num_tokens, int32_t d_lat,
                                int32_t d_rope);
int oracle_mla_decode_fp8(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* cache,
                          const oracle_pool* pool, const uint16_t* w_uk, const uint16_t* w_uv,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* context_lens, int32_t batch, int32_t num_heads,
                          int32_t d_nope, int32_t d_rope, int32_t d_lat, int32_t d_v,
                          double scale, double* out, double* lse);

#ifdef __cplusplus
}
#endif
#endif /* PA_ORACLE_H */
