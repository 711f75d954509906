/*
 * pa_decode.h -- C ABI of the MI355X (gfx950) decode-time paged-attention
 * library (libpa_decode.so).
 *
 * One new query token per sequence attends over that sequence's KV cache,
 * which lives in fixed-size pages of a shared pool and is found through a
 * per-sequence block table: logical token t sits in page block_table[b][t /
 * page_size] at slot t % page_size.  The block table and the context lengths
 * are device arrays read in place, so every entry point is safe to record in
 * a HIP graph [vllm.cpp kernel matrix, row KERNEL-ATTN-DFLASH-PAGED-BLOCK:
 * paged K/V with per-request lengths and block table as persistent device
 * tensors, static grid].
 *
 * Conventions for every entry point:
 *  - Pointers named as tensors are DEVICE pointers owned by the caller; the
 *    library never allocates, frees, copies between host and device, or
 *    synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and the call returns before it finishes.
 *  - bf16 is IEEE-754 binary32 truncated to its upper 16 bits; every bf16
 *    output is rounded to nearest, ties to even.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    non-zero status nothing was launched and pa_last_error() describes why.
 *  - Device-side contract, not checked: 0 <= context_lens[b] <=
 *    max_pages_per_seq * page_size, and block_table[b][i] lies in
 *    [0, num_pages) for every page i that holds a live key.  Block-table
 *    entries past a sequence's last live page are never read.
 *  - Results are bitwise reproducible run to run and independent of which
 *    physical pages hold the keys: every reduction runs in a fixed order
 *    over logical token positions and there are no floating-point atomics.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the entry points below are exported from the shared library. */
#ifndef PA_API
#define PA_API __attribute__((visibility("default")))
#endif

/* Status codes. */
#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* sizes inconsistent or out of range */
#define PA_ERR_UNSUPPORTED (-3) /* head_dim / group / page size not built */
#define PA_ERR_ALIGN (-4)       /* stride not a multiple of 8 elements or pointer not 16-byte aligned */
#define PA_ERR_WORKSPACE (-5)   /* workspace missing or too small */
#define PA_ERR_LAUNCH (-6)      /* the HIP runtime refused a launch */

/* Geometry of a K or V page pool of bf16 elements.  Strides are in ELEMENTS;
 * the innermost (head_dim) axis is contiguous.  The layout [page][kv head]
 * [slot][dim] (head_stride = page_size*head_dim, token_stride = head_dim)
 * makes each (page, KV head) tile one contiguous block and is the layout this
 * library is tuned for; the layout [page][slot][kv head][dim] works through
 * the same code.  All three strides must be multiples of 8 and the pool
 * 16-byte aligned.  For the MLA latent cache num_kv_heads = 1, head_dim = 576
 * and head_stride is ignored. */
typedef struct pa_kv_layout {
  int32_t num_pages;
  int32_t page_size;    /* 16, 32 or 64 */
  int32_t num_kv_heads;
  int32_t head_dim;     /* 64, 128, 256 or 512 (576 for the MLA cache); 512 is the
                           global-layer head size of a model that mixes 256 and 512
                           per layer [vllm.cpp kernel matrix, row KERNEL-ATTN-PAGED] */
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
} pa_kv_layout;

/* ---------------------------------------------------------------------------
 * pa_decode_splitkv -- stage 1 of split-KV decode.
 *
 * Softmax attention of q head h of sequence b over keys of KV head
 * g = h / (num_q_heads / num_kv_heads) (contiguous groups; each KV page tile
 * is read once per KV head and serves all of its q heads) [vllm.cpp PR #49,
 * commit body: the decode grid over batch x KV heads with the q heads of a
 * group processed together].  Scores s_t = scale * q . k_t in fp32.
 * With window > 0 only keys t >= ctx - window are attended (the newest
 * `window` keys); window <= 0 attends every key [vllm.cpp PR #425,
 * LIMITATIONS: windowed instantiation].
 *
 * The attended range [lo, ctx) is cut into partitions of partition_size
 * keys counted from lo: partition j = [lo + j*P, min(lo + (j+1)*P, ctx)).
 * For every b, h and j < max_partitions it writes, in fp32,
 *   part_max[b][h][j] = m_j = max_t s_t          (natural-log domain)
 *   part_sum[b][h][j] = l_j = sum_t exp(s_t - m_j)
 *   part_out[b][h][j][:] = sum_t exp(s_t - m_j) v_t / l_j
 * and for an empty partition m_j = -inf, l_j = 0, part_out = 0
 * [vllm.cpp kernel matrix, row KERNEL-ATTN-MLA-SPARSE, W4: per-split partial
 * results and a second merge stage; row KERNEL-ATTN-FA2: split-KV decode].
 *
 * q            [batch][num_q_heads][head_dim] bf16, contiguous
 * k_pool/v_pool  pools described by *kv (host pointer to the descriptor)
 * block_table  [batch][block_table_stride] int32, device
 * context_lens [batch] int32, device
 * part_out     [batch][num_q_heads][max_partitions][head_dim] fp32
 * part_max, part_sum [batch][num_q_heads][max_partitions] fp32
 * Requires partition_size >= 1 and max_partitions * partition_size >= the
 * largest possible attended range (min(window, max_pages_per_seq *
 * page_size) with a window, else max_pages_per_seq * page_size); supported
 * head_dim 64, 128, 256 or 512 with 1 to 16 q heads per KV head (a group
 * that is not a power of two runs on the kernel built for the next one,
 * its padding heads masked); page_size 16/32/64.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode_splitkv(const void* q, const void* k_pool, const void* v_pool,
                      const pa_kv_layout* kv, const int32_t* block_table,
                      int32_t block_table_stride, const int32_t* context_lens,
                      int32_t batch, int32_t num_q_heads,
                      int32_t max_pages_per_seq, float scale, int32_t window,
                      int32_t partition_size, int32_t max_partitions,
                      float* part_out, float* part_max, float* part_sum,
                      void* stream);

/* ---------------------------------------------------------------------------
 * pa_merge_lse -- stage 2: log-sum-exp merge of split partials.
 *
 * For each (b, h), over the live partitions j < ceil((ctx - lo) / P):
 *   M = max_j m_j,  w_j = l_j exp(m_j - M),  W = sum_j w_j,
 *   out[b][h][:] = bf16( sum_j (w_j / W) part_out[j][:] ),
 *   lse_out[b][h] = M + ln W.
 * The weighted sum is taken in one fixed order (for each g < 32 the
 * partitions j = g, g + 32, ... in ascending j, then the 32 group sums in
 * ascending g), so the result is the same on every call.
 * Empty partitions (m_j = -inf) weigh nothing; no live partition, or all
 * empty, gives out = 0 and lse = -inf [vllm.cpp kernel matrix, row
 * KERNEL-ATTN-MLA-SPARSE, W5: merge of attention states with both -inf edge
 * cases; W4: fixed ascending split order, no atomics].
 *
 * Arguments as written by pa_decode_splitkv with the same partition_size,
 * max_partitions and window; max_partitions must cover every sequence's live
 * partitions (not checked: the context lengths live on the device).  A row
 * with more live partitions than that (outside the contract) merges its
 * first max_partitions and reads nothing past its own partials.
 * out [batch][num_q_heads][head_dim] bf16; lse_out [batch][num_q_heads]
 * fp32 or NULL.  head_dim 64, 128, 256 or 512.
 * ------------------------------------------------------------------------- */
PA_API int pa_merge_lse(const float* part_out, const float* part_max,
                 const float* part_sum, const int32_t* context_lens,
                 int32_t batch, int32_t num_q_heads, int32_t head_dim,
                 int32_t partition_size, int32_t max_partitions,
                 int32_t window, void* out, float* lse_out, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode -- complete decode attention: the result pa_decode_splitkv +
 * pa_merge_lse define, with a balanced split instead of fixed partitions.
 *
 * The attended keys of the whole batch, counted once per KV head (rows
 * (b, kv head) laid end to end, each preceded by a fixed number of units
 * that stand for the cost of starting it), are cut into equal contiguous
 * ranges, one per workgroup, so every workgroup has the same work whatever
 * the length mix [vllm.cpp kernel matrix, row
 * KERNEL-ATTN-MLA-SPARSE, W4: split-KV with a fixed, ordered merge].  A row
 * that one range covers is written directly; a row cut by range boundaries
 * gets one partial per piece, merged in ascending order as in pa_merge_lse.
 * The cut points are computed on the device from context_lens and a block
 * count fixed by the build (resident blocks per compute unit x 256), not by
 * the device: a row's result may differ in the last bits when other
 * sequences' lengths change; for fixed inputs the result is deterministic
 * run to run, the same on every gfx950 device, and does not depend on where
 * the pages sit in the pool.
 *
 * Any 1 to 16 q heads per KV head, at head_dim 64, 128, 256 or 512.
 * out [batch][num_q_heads][head_dim] bf16; lse_out [batch][num_q_heads] fp32
 * (natural log of the softmax denominator, -inf for an empty row) or NULL.
 * workspace: device memory of at least pa_decode_workspace_size(...) bytes,
 * 256-byte aligned, owned by the caller and clobbered by the call; it needs
 * no initialisation (every call rewrites what it later reads) and keeps no
 * state between calls.  Two calls must not share a workspace while both run.
 * workspace NULL (workspace_bytes ignored): no split -- one workgroup per
 * (sequence, KV head) row writes that row's bf16 output directly, so the
 * call needs no memory beyond its arguments, at the price of balance: the
 * longest row sets the time.  Its bits are fixed by the row alone.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode(const void* q, const void* k_pool, const void* v_pool,
              const pa_kv_layout* kv, const int32_t* block_table,
              int32_t block_table_stride, const int32_t* context_lens,
              int32_t batch, int32_t num_q_heads, int32_t max_pages_per_seq,
              float scale, int32_t window, void* out, float* lse_out,
              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_multiquery -- decode with S query tokens per sequence (the verify
 * step of speculative decoding, or a block of draft queries).
 *
 * The S queries of sequence b stand at the last S positions of its context
 * (context_lens[b] counts them; their K/V rows are already in the pools).
 * Query s attends to keys t <= context_lens[b] - S + s when causal != 0, to
 * all keys t < context_lens[b] otherwise; with window > 0 only to the last
 * `window` of those [pegainfer PR #938, commit message: the b=8 and b=16
 * verify steps; vllm.cpp kernel matrix, row KERNEL-ATTN-DFLASH-PAGED-BLOCK:
 * the (1+k) block queries attend over the paged context holding their own
 * block, under a causal or a non-causal in-block mask].  All S queries of a
 * KV group share one pass over its K/V rows, as S * (Hq / Hkv) heads.  A
 * query with no key gives out = 0 and lse = -inf.
 *
 * q [batch][S][num_q_heads][head_dim] bf16; out the same shape; lse_out
 * [batch][S][num_q_heads] fp32 or NULL.  1 <= S <= 16, and S times
 * num_q_heads / num_kv_heads must be at most 16.  workspace: at least
 * pa_decode_multiquery_workspace_size(...) bytes, 256-byte aligned,
 * clobbered, or NULL as for pa_decode.  S = 1 gives exactly pa_decode.
 * Other arguments as pa_decode.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode_multiquery(const void* q, const void* k_pool, const void* v_pool,
                                const pa_kv_layout* kv, const int32_t* block_table,
                                int32_t block_table_stride, const int32_t* context_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_queries,
                                int32_t causal, int32_t max_pages_per_seq, float scale,
                                int32_t window, void* out, float* lse_out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_fp8 -- pa_decode over an FP8 KV cache.
 *
 * k_pool and v_pool hold one OCP FP8 E4M3 byte per element (sign, 4-bit
 * exponent with bias 7, 3-bit mantissa; S.1111.111 is NaN; largest finite
 * magnitude 448).  The value of a K element is e4m3(byte) * k_scale, of a V
 * element e4m3(byte) * v_scale: one scale per pool [vllm.cpp kernel matrix,
 * inventory row "Quantized KV cache, including FP8 and NVFP4"; row
 * KERNEL-KV-CACHE-DSA, the fp8_ds_mla dequant read: the e4m3 element times
 * its scale; the per-pool granularity is this library's reading, the pages
 * fix none for a GQA pool].  The bytes are widened to bf16 in registers
 * (exact), k_scale is folded into the softmax scale and v_scale into the
 * output, so the result is attention over the dequantized values, computed
 * as in pa_decode.  K/V bytes read per call are half those of bf16 pools.
 *
 * kv: strides and sizes in elements (= bytes); every K/V row must start on
 * a 16-byte boundary (strides multiples of 16).  k_scale, v_scale: finite,
 * > 0.  Every group size pa_decode takes is supported.  workspace: at least
 * pa_decode_workspace_size(...) bytes for the same shapes, 256-byte aligned,
 * needs no initialisation.  Other arguments, the split, determinism and
 * the error codes as pa_decode.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                         const pa_kv_layout* kv, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens,
                         int32_t batch, int32_t num_q_heads, int32_t max_pages_per_seq,
                         float scale, float k_scale, float v_scale, int32_t window, void* out,
                         float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_f32 -- pa_decode over f32 K/V pools.
 *
 * k_pool and v_pool hold IEEE binary32 elements [vllm.cpp PR #425, the row
 * loader's float instantiation beside the bf16 one; vllm.cpp kernel matrix,
 * inventory row: the paged path admits F32/BF16].  Every element is split
 * exactly into three bf16 terms on the matrix cores, so the score and P.V
 * products are exact and the sums fp32, as in pa_decode.  head_dim 64, 128,
 * 256 or 512; strides in elements, rows on 16-byte
 * boundaries (strides multiples of 4).  workspace: at least
 * pa_decode_workspace_size(...) bytes for the same shapes.  Other arguments,
 * the split, determinism and the error codes as pa_decode.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode_f32(const void* q, const void* k_pool, const void* v_pool,
                         const pa_kv_layout* kv, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens,
                         int32_t batch, int32_t num_q_heads, int32_t max_pages_per_seq,
                         float scale, int32_t window, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same arguments and results as pa_decode (bit for bit) without the
 * workspace: the balanced split's partials and row records live in a
 * 32 MiB array of the library's own device memory, one per device, set up
 * on the first call on that device and held until the process ends.  Shapes
 * whose pa_decode_workspace_size(...) exceeds 32 MiB return
 * PA_ERR_WORKSPACE (nothing launched).  The call allocates nothing.  Every
 * call on one device shares that device's array: calls that may overlap in
 * time on one device (other streams, other threads) race and must be
 * serialised by the caller.  The array needs no initialisation: each call
 * rewrites what it later reads.
 * ------------------------------------------------------------------------- */
PA_API int pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                             const pa_kv_layout* kv, const int32_t* block_table,
                             int32_t block_table_stride, const int32_t* context_lens,
                             int32_t batch, int32_t num_q_heads, int32_t max_pages_per_seq,
                             float scale, int32_t window, void* out, float* lse_out,
                             void* stream);

/* Bytes of workspace pa_decode_multiquery needs (0 on invalid shapes). */
PA_API size_t pa_decode_multiquery_workspace_size(int32_t batch, int32_t num_q_heads,
                                                  int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t max_pages_per_seq, int32_t page_size,
                                                  int32_t window, int32_t num_queries);

/* Bytes of workspace pa_decode needs for these shapes (0 on invalid shapes). */
PA_API size_t pa_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_pages_per_seq, int32_t page_size,
                                int32_t window);

/* Partition size suggested for pa_decode_splitkv / pa_merge_lse with these
 * shapes (0 on invalid shapes); pa_decode itself splits by balanced ranges. */
PA_API int32_t pa_decode_partition_size(int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_pages_per_seq, int32_t page_size,
                                 int32_t window);

/* ---------------------------------------------------------------------------
 * mla_absorbed_decode -- absorbed multi-head latent attention decode.
 *
 * The cache holds one 576-wide bf16 row per token: 512 latent values c[0:512]
 * followed by 64 rope values c[512:576], shared by all heads.  For sequence b
 * and head h [pegainfer PR #938, review quote of the kernel's "Schedule"
 * comment, steps 1-7; vllm.cpp kernel matrix, row KERNEL-ATTN-MLA-SPARSE:
 * absorption as a load-time weight transform plus two batched products, and
 * V equal to the latent part of the cache]:
 *   q_abs[j]  = sum_d q_nope[b][h][d] * w_uk[h][d][j]          (d < 128, j < 512)
 *   s_t       = scale * (q_abs . c_t[0:512] + q_rope[b][h] . c_t[512:576])
 *   o_lat[j]  = sum_t softmax(s)_t * c_t[j]
 *   out[b][h][dv] = bf16( sum_j w_uv[h][dv][j] * o_lat[j] )    (dv < 128)
 * q_abs, the probabilities and o_lat are fp32; they enter the bf16 matrix
 * products as three bf16 terms that sum to the fp32 value exactly, so only
 * fp32 accumulation rounds.  Each (64-head group, sequence) row is cut into
 * pieces of whole 32-key tiles, one per workgroup, in one of two ways chosen
 * from the context lengths alone: every row into its own near-equal pieces,
 * the fewest tiles per piece that fit the grid (at most partition_size keys
 * each when that is given), or, when rows are too few for even pieces, the
 * keys of all rows laid end to end (each after a fixed number of units for
 * the cost of starting it) and cut into equal contiguous ranges (the
 * library's choice only; a grid fixed by the shapes and the build rather
 * than the device).  The pieces of a row are merged by log-sum-exp in
 * ascending order; an empty context gives 0.
 * Deterministic run to run, the same on every gfx950 device, and
 * independent of page placement.  The pieces are cut from the context
 * lengths of the whole batch, so a row's result may differ in the last bits
 * when other sequences' lengths change.
 *
 * q_nope [batch][num_heads][128] bf16; q_rope [batch][num_heads][64] bf16;
 * kv_cache: pool described by *cache (num_kv_heads 1, head_dim 576,
 * page_size 16/32/64, token_stride >= 576 and a multiple of 8);
 * w_uk, w_uv [num_heads][128][512] bf16; out [batch][num_heads][128] bf16.
 * Any num_heads >= 1 (heads past the last 32-head tile are masked).
 * partition_size: most keys per piece of a row (multiple of 64; pieces grow
 * when a call would need more than 16384 of them), or 0 to let the library
 * choose.
 * workspace: at least mla_absorbed_decode_workspace_size(...) bytes,
 * 256-byte aligned, clobbered by the call.  Device-side contract as for
 * pa_decode: 0 <= context_lens[b] <= max_pages_per_seq * page_size and the
 * block_table entries a sequence uses lie in [0, num_pages).
 * Returns PA_OK, or an error code with pa_last_error() set; nothing is
 * launched on error.
 * ------------------------------------------------------------------------- */
PA_API int mla_absorbed_decode(const void* q_nope, const void* q_rope,
                        const void* kv_cache, const pa_kv_layout* cache,
                        const void* w_uk, const void* w_uv,
                        const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* context_lens, int32_t batch,
                        int32_t num_heads, int32_t max_pages_per_seq,
                        float scale, int32_t partition_size, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_absorbed_decode needs (0 on invalid shapes). */
PA_API size_t mla_absorbed_decode_workspace_size(int32_t batch, int32_t num_heads,
                                          int32_t max_pages_per_seq,
                                          int32_t page_size,
                                          int32_t partition_size);

/* ---------------------------------------------------------------------------
 * pa_kv_insert -- write new tokens' K and V rows into the paged pools.
 *
 * Token i of k_new / v_new ([token][kv head][head_dim] bf16, element strides
 * src_token_stride and src_head_stride, head_dim contiguous) is copied bit
 * for bit to flat slot s = slots[i] = page * page_size + offset of k_pool /
 * v_pool (layout *kv), for every KV head [vllm.cpp kernel matrix, row
 * KERNEL-KV-CACHE: KV insert into the paged cache, an exact copy].  This is
 * the step before decode: the new token of sequence b goes to slot
 * block_table[b][t / page_size] * page_size + t % page_size with
 * t = context_lens[b] - 1.
 *
 * slots: num_tokens int64, device.  Slots outside [0, num_pages *
 * page_size) are skipped (negative marks padding).  Two tokens with the same
 * slot race.  head_dim any multiple of 8; strides multiples of 8 elements
 * (a head stride may be 0 for a one-head pool); pointers 16-byte aligned.
 * num_tokens 0 is a no-op.  Returns PA_OK or an error code (nothing launched).
 * ------------------------------------------------------------------------- */
PA_API int pa_kv_insert(const void* k_new, const void* v_new, int64_t src_token_stride,
                        int64_t src_head_stride, void* k_pool, void* v_pool,
                        const pa_kv_layout* kv, const int64_t* slots,
                        int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * mla_cache_insert -- write new tokens' rows into the MLA latent cache.
 *
 * Row slots[i] of the cache (layout *cache: num_kv_heads 1, head_dim 576)
 * becomes kv_c[i][0:512] followed by k_pe[i][0:64], copied bit for bit
 * [vllm.cpp kernel matrix, row KERNEL-KV-CACHE: the MLA cache write
 * concatenates the latent and rope projections into the 576-wide row, from
 * strided sources].  kv_c rows c_stride elements apart, k_pe rows pe_stride
 * apart (multiples of 8; c_stride >= 512, pe_stride >= 64), bf16, 16-byte
 * aligned.  Slots outside the cache are skipped.  Returns PA_OK or an error
 * code (nothing launched).
 * ------------------------------------------------------------------------- */
PA_API int mla_cache_insert(const void* kv_c, int64_t c_stride, const void* k_pe,
                            int64_t pe_stride, void* kv_cache, const pa_kv_layout* cache,
                            const int64_t* slots, int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 MLA latent cache.
 *
 * The fp8_ds_mla quantization of the pages [vllm.cpp kernel matrix, row
 * KERNEL-KV-CACHE-DSA: E4M3 elements in blocks of 64, one UE8M0 power-of-two
 * scale per block, exponent ceil(log2(absmax / 448)) stored as exponent +
 * 127, rope in bf16; dequant read e4m3 * 2^(byte - 127)], applied to the
 * 512 + 64 latent of this library's MLA.  One row per token, 656 bytes:
 *   [0, 512)    the latent as E4M3 (OCP e4m3fn), block j = elements 64j..64j+63
 *   [512, 640)  the rope part, 64 bf16
 *   [640, 648)  scale byte of block j at 640 + j
 *   [648, 656)  zero
 * The cache layout has num_kv_heads 1 and head_dim 656, with page_stride and
 * token_stride in BYTES (positive multiples of 16, token_stride >= 656).
 * Element value: e4m3(byte) * 2^(scale byte - 127).  Scale bytes are 1..254
 * as written by mla_cache_insert_fp8; other values are outside the contract.
 * ------------------------------------------------------------------------- */

/* mla_cache_insert_fp8 -- quantize new tokens' latent rows into the FP8
 * cache.  Per 64-block of kv_c[i][0:512]: exponent e = the smallest integer
 * with 448 * 2^e >= max |x| over the block (computed exactly), clamped to
 * [-126, 127] (an all-zero block takes -126); element byte = the E4M3 value
 * nearest x * 2^-e, ties to the even code, sign bit from x.  k_pe[i][0:64]
 * is copied bit for bit.  Sources as for mla_cache_insert (bf16, strides in
 * elements, multiples of 8, 16-byte aligned); non-finite inputs give
 * unspecified bytes.  Slots outside the cache are skipped.  Returns PA_OK or
 * an error code (nothing launched). */
PA_API int mla_cache_insert_fp8(const void* kv_c, int64_t c_stride, const void* k_pe,
                                int64_t pe_stride, void* kv_cache, const pa_kv_layout* cache,
                                const int64_t* slots, int32_t num_tokens, void* stream);

/* mla_absorbed_decode_fp8 -- mla_absorbed_decode over the FP8 latent cache.
 * Each row is widened to bf16 on the way into the workgroup's shared tile
 * (exact for every value in bf16's normal range), then the computation is
 * mla_absorbed_decode's over the dequantized latent and rope.  Latent bytes
 * read per key: 656 instead of 1152.  Workspace as mla_absorbed_decode
 * (mla_absorbed_decode_workspace_size with the same shapes); other arguments,
 * determinism and error codes as mla_absorbed_decode. */
PA_API int mla_absorbed_decode_fp8(const void* q_nope, const void* q_rope, const void* kv_cache,
                                   const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                                   const int32_t* block_table, int32_t block_table_stride,
                                   const int32_t* context_lens, int32_t batch, int32_t num_heads,
                                   int32_t max_pages_per_seq, float scale,
                                   int32_t partition_size, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mla_absorbed_decode_multiquery -- absorbed MLA with S queries per sequence
 * (the verify step of speculative decoding).
 *
 * The S queries of sequence b stand at the last S positions of its context
 * (context_lens[b] counts them; their rows are already in the cache).  Query
 * s attends to keys t <= context_lens[b] - S + s when causal != 0, to all keys
 * t < context_lens[b] otherwise [pegainfer PR #938: plain decode and the
 * speculative verify step (the b=8 and b=16 verify launches) run through the
 * same absorbed-MLA kernel; vllm.cpp kernel matrix, row
 * KERNEL-ATTN-DFLASH-PAGED-BLOCK: the (1+k) block queries attend over the
 * paged context holding their own block, under a causal or a non-causal
 * in-block mask].  Each query is mla_absorbed_decode of its own q_nope and
 * q_rope; a query with no key gives 0.  The S * num_heads query heads of a
 * sequence share one pass over its cache rows (head s*num_heads + h uses
 * W_UK[h] and W_UV[h]), so the cache is read from HBM about once however
 * large S is.
 *
 * q_nope [batch][S][num_heads][128] bf16; q_rope [batch][S][num_heads][64];
 * out [batch][S][num_heads][128] bf16.  1 <= num_queries = S <= 16.
 * workspace: at least mla_absorbed_decode_workspace_size(batch,
 * S * num_heads, max_pages_per_seq, page_size, partition_size) bytes.
 * S = 1 gives exactly mla_absorbed_decode (causal or not).  Other arguments,
 * determinism and error codes as mla_absorbed_decode; the _fp8 variant reads
 * the FP8 latent cache as mla_absorbed_decode_fp8 does.
 * ------------------------------------------------------------------------- */
PA_API int mla_absorbed_decode_multiquery(const void* q_nope, const void* q_rope,
                                          const void* kv_cache, const pa_kv_layout* cache,
                                          const void* w_uk, const void* w_uv,
                                          const int32_t* block_table,
                                          int32_t block_table_stride,
                                          const int32_t* context_lens, int32_t batch,
                                          int32_t num_heads, int32_t num_queries, int32_t causal,
                                          int32_t max_pages_per_seq, float scale,
                                          int32_t partition_size, void* out, void* workspace,
                                          size_t workspace_bytes, void* stream);
PA_API int mla_absorbed_decode_multiquery_fp8(const void* q_nope, const void* q_rope,
                                              const void* kv_cache, const pa_kv_layout* cache,
                                              const void* w_uk, const void* w_uv,
                                              const int32_t* block_table,
                                              int32_t block_table_stride,
                                              const int32_t* context_lens, int32_t batch,
                                              int32_t num_heads, int32_t num_queries,
                                              int32_t causal, int32_t max_pages_per_seq,
                                              float scale, int32_t partition_size, void* out,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

/* Measurement hook.  Arms the calling thread so that its next entry-point
 * call launches that call's dominant kernel with start_event and stop_event
 * attached to the launch itself (hipExtLaunchKernelGGL), so that they are
 * stamped on its stream when the kernel starts and when it ends: the split
 * kernel of the pa_decode family and of pa_decode_splitkv, the merge kernel
 * of pa_merge_lse, the split kernel of the absorbed-MLA entry points, the
 * copy kernel of pa_kv_insert.  The hook is then disarmed; a call that fails
 * validation launches nothing and leaves it armed.  The events are
 * hipEvent_t values owned by the caller, created with timing enabled (NULL
 * cancels).  Nothing else about the call changes; it exists so a benchmark
 * can time that kernel alone, live, on the stream it runs on [measurement of
 * a kernel against its roofline: the duration of its own launches]. */
PA_API void pa_profile_next(void* start_event, void* stop_event);

/* Text describing the last non-zero status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on that thread. */
PA_API const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_DECODE_H */
