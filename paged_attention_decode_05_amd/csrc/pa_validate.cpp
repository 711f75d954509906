// pa_validate.cpp -- host-side checks and launch planning (no HIP).
#include "pa_validate.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace pa {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult8(int64_t s) { return s > 0 && (s % 8) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}
void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }

bool head_dim_supported(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// Heads per KV group: one 16-column matrix tile holds up to 16 of them at
// every head_dim.
bool group_supported(int32_t head_dim, int32_t group) {
  return head_dim_supported(head_dim) && group >= 1 && group <= 16;
}

int32_t group_padded(int32_t heads) {
  if (heads < 1 || heads > 16) return 0;
  int32_t g = 1;
  while (g < heads) g *= 2;
  return g;
}

bool page_size_supported(int32_t ps) { return ps == 16 || ps == 32 || ps == 64; }

int64_t max_keys(int32_t max_pages_per_seq, int32_t page_size, int32_t window) {
  int64_t k = static_cast<int64_t>(max_pages_per_seq) * page_size;
  if (window > 0 && window < k) k = window;
  return k;
}

int check_gqa(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
              int32_t max_pages_per_seq, float scale, int32_t elem_bytes) {
  if (!q || !k_pool || !v_pool || !kv || !block_table || !context_lens)
    return fail(PA_ERR_NULL, "a required pointer (q, k_pool, v_pool, kv, block_table, "
                             "context_lens) is NULL");
  if (batch < 1 || num_q_heads < 1 || max_pages_per_seq < 1)
    return fail(PA_ERR_SHAPE, "batch, num_q_heads and max_pages_per_seq must be >= 1");
  if (batch > 65535 || num_q_heads > 65535)
    return fail(PA_ERR_SHAPE, "batch and num_q_heads must be <= 65535 (grid limits)");
  if (kv->num_pages < 1 || kv->num_kv_heads < 1 || kv->page_size < 1 || kv->head_dim < 1)
    return fail(PA_ERR_SHAPE, "kv layout: num_pages, num_kv_heads, page_size, head_dim must be >= 1");
  if (num_q_heads % kv->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (block_table_stride < max_pages_per_seq)
    return fail(PA_ERR_SHAPE, "block_table_stride must be >= max_pages_per_seq");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PA_ERR_SHAPE, "scale must be finite and > 0");
  if (static_cast<int64_t>(max_pages_per_seq) * kv->page_size > INT32_MAX / 2)
    return fail(PA_ERR_SHAPE, "max_pages_per_seq * page_size is too large");
  if (!head_dim_supported(kv->head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512");
  const int32_t group = num_q_heads / kv->num_kv_heads;
  if (!group_supported(kv->head_dim, group))
    return fail(PA_ERR_UNSUPPORTED, "q heads per KV head must be 1 .. 16");
  if (!page_size_supported(kv->page_size))
    return fail(PA_ERR_UNSUPPORTED, "page_size must be 16, 32 or 64");
  const int64_t row_align = 16 / elem_bytes;   // elements per 16 bytes
  auto mult = [&](int64_t v) { return v > 0 && v % row_align == 0; };
  if (!mult(kv->page_stride) || !mult(kv->head_stride) || !mult(kv->token_stride))
    return fail(PA_ERR_ALIGN, "kv strides must be positive multiples of " +
                                  std::to_string(row_align) + " elements (16 bytes)");
  if (kv->token_stride < kv->head_dim)
    return fail(PA_ERR_SHAPE, "token_stride must be >= head_dim");
  if (static_cast<int64_t>(kv->page_size - 1) * kv->token_stride + kv->head_dim > INT32_MAX / 4)
    return fail(PA_ERR_SHAPE, "token_stride too large");
  if (static_cast<double>(batch) * kv->num_kv_heads *
          static_cast<double>(max_keys(max_pages_per_seq, kv->page_size, 0)) > 1e15)
    return fail(PA_ERR_SHAPE, "batch * num_kv_heads * max keys is too large");
  // the kernels hold one page's size in bytes in 32 bits
  if (kv->page_stride * elem_bytes > static_cast<int64_t>(UINT32_MAX) ||
      kv->head_stride > static_cast<int64_t>(UINT32_MAX / 2))
    return fail(PA_ERR_SHAPE, "page_stride must stay below 2^32 bytes and head_stride below "
                              "2^31 elements");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_ALIGN, "q, k_pool and v_pool must be 16-byte aligned");
  return PA_OK;
}

int check_split(int32_t partition_size, int32_t max_partitions, int32_t max_pages_per_seq,
                int32_t page_size, int32_t window, const float* part_out, const float* part_max,
                const float* part_sum) {
  if (!part_out || !part_max || !part_sum)
    return fail(PA_ERR_NULL, "part_out, part_max and part_sum must not be NULL");
  if (partition_size < 1 || max_partitions < 1)
    return fail(PA_ERR_SHAPE, "partition_size and max_partitions must be >= 1");
  const int64_t need = ceil_div(max_keys(max_pages_per_seq, page_size, window), partition_size);
  if (max_partitions < need) {
    char buf[160];
    std::snprintf(buf, sizeof buf,
                  "max_partitions %d cannot cover %lld keys in partitions of %d (need %lld)",
                  max_partitions, (long long)max_keys(max_pages_per_seq, page_size, window),
                  partition_size, (long long)need);
    return fail(PA_ERR_SHAPE, buf);
  }
  if (!aligned16(part_out) || !aligned16(part_max) || !aligned16(part_sum))
    return fail(PA_ERR_ALIGN, "partial buffers must be 16-byte aligned");
  return PA_OK;
}

int check_merge(const float* part_out, const float* part_max, const float* part_sum,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t head_dim, int32_t partition_size, int32_t max_partitions, const void* out) {
  if (!part_out || !part_max || !part_sum || !context_lens || !out)
    return fail(PA_ERR_NULL, "part_out, part_max, part_sum, context_lens and out must not be NULL");
  if (batch < 1 || num_q_heads < 1 || partition_size < 1 || max_partitions < 1)
    return fail(PA_ERR_SHAPE, "batch, num_q_heads, partition_size, max_partitions must be >= 1");
  if (batch > 65535 || num_q_heads > 65535)
    return fail(PA_ERR_SHAPE, "batch and num_q_heads must be <= 65535 (grid limits)");
  if (!head_dim_supported(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512");
  if (!aligned16(part_out) || !aligned16(out))
    return fail(PA_ERR_ALIGN, "part_out and out must be 16-byte aligned");
  return PA_OK;
}

// Partition size suggested for the two-stage API: about 4096 work items of
// (sequence, KV head, partition) when contexts average half the maximum, at
// least 256 keys for head_dim 128 (128 for 256) so a partition's fp32 partial
// output stays small next to the K/V bytes it summarises.
int32_t suggest_partition(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_pages_per_seq, int32_t page_size, int32_t window) {
  if (batch < 1 || num_kv_heads < 1 || max_pages_per_seq < 1 || page_size < 1 ||
      !head_dim_supported(head_dim))
    return 0;
  const int64_t keys = max_keys(max_pages_per_seq, page_size, window);
  const int64_t work = static_cast<int64_t>(batch) * num_kv_heads * keys;
  int64_t p = 1;
  while (p * 2 * 4096 < work) p *= 2;
  const int64_t pmin = head_dim == 128 ? 256 : 128;
  if (p < pmin) p = pmin;
  if (p > 4096) p = 4096;
  return static_cast<int32_t>(p);
}

bool plan_decode(int32_t batch, int32_t num_kv_heads, int32_t vheads, int32_t head_dim,
                 int32_t max_pages_per_seq, int32_t page_size, int32_t window, DecodePlan* plan) {
  if (batch < 1 || num_kv_heads < 1 || max_pages_per_seq < 1 || page_size < 1 ||
      !head_dim_supported(head_dim) || group_padded(vheads) == 0)
    return false;
  if (static_cast<int64_t>(batch) * num_kv_heads > (int64_t{1} << 30)) return false;
  plan->rows = batch * num_kv_heads;
  plan->group = group_padded(vheads);
  const size_t slots = static_cast<size_t>(plan->rows) + kMaxBalancedBlocks;
  size_t o = 0;
  plan->off_seg_out = o;    o += round_up(slots * plan->group * head_dim * sizeof(float), 256);
  plan->off_seg_max = o;    o += round_up(slots * plan->group * sizeof(float), 256);
  plan->off_seg_sum = o;    o += round_up(slots * plan->group * sizeof(float), 256);
  plan->off_row_info = o;   o += round_up(static_cast<size_t>(plan->rows) * sizeof(int32_t), 256);
  plan->bytes = o;
  return true;
}

// MLA split plan.  Heads form groups of 64; the keys of all (group,
// sequence) rows are cut into at most max_blocks equal ranges, one per split
// block, and every block writes one partial per row piece it covers, so
// groups * batch + max_blocks partial slots bound the workspace.  An explicit
// partition size P asks for about P keys per block (ceil(T / P) blocks for T
// keys in all, capped); 0 leaves it to the library (one block per CU).
bool plan_mla(int32_t batch, int32_t num_heads, int32_t max_pages_per_seq, int32_t page_size,
              int32_t partition_size, MlaPlan* plan) {
  if (batch < 1 || num_heads < 1 || max_pages_per_seq < 1 ||
      !page_size_supported(page_size) || partition_size < 0 || partition_size % kMlaKeyTile)
    return false;
  const int64_t keys = static_cast<int64_t>(max_pages_per_seq) * page_size;
  plan->groups = static_cast<int32_t>(ceil_div(num_heads, kMlaBlockHeads));
  // every (group, sequence) row needs a block of its own (rows of a group
  // padded to a multiple of 8)
  const int64_t rows8 = plan->groups * round_up(static_cast<size_t>(batch), 8);
  const int64_t most = partition_size > 0 ? rows8 * ceil_div(keys, partition_size) : kSplitCUs;
  const int64_t cap = partition_size > 0 ? kMlaMaxExplicitBlocks : kSplitCUs;
  if (rows8 > (int64_t{1} << 30)) return false;
  plan->max_blocks = static_cast<int32_t>(std::max<int64_t>(rows8, std::min<int64_t>(most, cap)));
  // q_abs in 32-head tiles (the split kernel's operand layout), heads padded
  const size_t bh = static_cast<size_t>(batch) * round_up(static_cast<size_t>(num_heads), 32);
  // one partial per block, or per (row, block) segment of the key line
  const size_t slots = static_cast<size_t>(plan->groups) * batch + plan->max_blocks;
  size_t o = 0;
  plan->off_qhi = o;      o += round_up(bh * kMlaRow * sizeof(uint16_t), 256);   // q_abs|q_rope, hi
  plan->off_qmid = o;     o += round_up(bh * kMlaLat * sizeof(uint16_t), 256);   // q_abs, mid
  plan->off_qlo = o;      o += round_up(bh * kMlaLat * sizeof(uint16_t), 256);   // q_abs, lo
  plan->off_seg_out = o;  o += round_up(slots * kMlaBlockHeads * kMlaLat * sizeof(float), 256);
  plan->off_seg_max = o;  o += round_up(slots * kMlaBlockHeads * sizeof(float), 256);
  plan->off_seg_sum = o;  o += round_up(slots * kMlaBlockHeads * sizeof(float), 256);
  plan->off_split_plan = o;  o += 256;   // the split plan, computed once per call
  plan->off_row_slots = o;   o += round_up(static_cast<size_t>(plan->groups) * batch * 16, 256);   // per row: first slot, pieces
  plan->bytes = o;
  return true;
}

int check_mla(const void* q_nope, const void* q_rope, const void* kv_cache,
              const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_heads,
              int32_t max_pages_per_seq, float scale, int32_t partition_size, const void* out,
              bool fp8, int32_t num_queries) {
  if (!q_nope || !q_rope || !kv_cache || !cache || !w_uk || !w_uv || !block_table ||
      !context_lens || !out)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (batch < 1 || num_heads < 1 || max_pages_per_seq < 1)
    return fail(PA_ERR_SHAPE, "batch, num_heads and max_pages_per_seq must be >= 1");
  if (num_queries < 1 || num_queries > 16)
    return fail(PA_ERR_SHAPE, "num_queries must be in 1..16");
  if (batch > 65535 || static_cast<int64_t>(num_heads) * num_queries > 65535)
    return fail(PA_ERR_SHAPE, "batch and num_heads * num_queries must be <= 65535 (grid limits)");
  if (cache->num_pages < 1 || cache->page_size < 1)
    return fail(PA_ERR_SHAPE, "cache: num_pages and page_size must be >= 1");
  if (block_table_stride < max_pages_per_seq)
    return fail(PA_ERR_SHAPE, "block_table_stride must be >= max_pages_per_seq");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PA_ERR_SHAPE, "scale must be finite and > 0");
  if (static_cast<int64_t>(max_pages_per_seq) * cache->page_size > INT32_MAX / 2)
    return fail(PA_ERR_SHAPE, "max_pages_per_seq * page_size is too large");
  const int32_t row = fp8 ? kMlaFp8Row : kMlaRow;
  if (cache->num_kv_heads != 1 || cache->head_dim != row)
    return fail(PA_ERR_UNSUPPORTED, fp8 ? "FP8 MLA cache must have num_kv_heads 1 and head_dim 656 (bytes)"
                                        : "MLA cache must have num_kv_heads 1 and head_dim 576");
  if (!page_size_supported(cache->page_size))
    return fail(PA_ERR_UNSUPPORTED, "page_size must be 16, 32 or 64");
  if (partition_size < 0 || partition_size % kMlaKeyTile)
    return fail(PA_ERR_SHAPE, "partition_size must be 0 or a positive multiple of 64");
  const int64_t smul = fp8 ? 16 : 8;   // 16 bytes either way
  if (cache->page_stride <= 0 || cache->page_stride % smul || cache->token_stride <= 0 ||
      cache->token_stride % smul)
    return fail(PA_ERR_ALIGN, fp8 ? "FP8 cache strides must be positive multiples of 16 bytes"
                                  : "cache strides must be positive multiples of 8 elements");
  if (cache->token_stride < row)
    return fail(PA_ERR_SHAPE, fp8 ? "FP8 cache token_stride must be >= 656"
                                  : "cache token_stride must be >= 576");
  if (static_cast<int64_t>(cache->page_size) * cache->token_stride > INT32_MAX / 4)
    return fail(PA_ERR_SHAPE, "cache token_stride too large");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(out))
    return fail(PA_ERR_ALIGN, "q_nope, q_rope, kv_cache, w_uk, w_uv and out must be 16-byte aligned");
  return PA_OK;
}

// Checks of the cache writes.  A stride of 0 is allowed for the head axis of
// a one-head pool; every other stride is a positive multiple of 8 elements.
static bool stride_ok(int64_t s, bool may_be_zero) { return (may_be_zero && s == 0) || mult8(s); }

int check_kv_insert(const void* k_new, const void* v_new, int64_t src_token_stride,
                    int64_t src_head_stride, const void* k_pool, const void* v_pool,
                    const pa_kv_layout* kv, const int64_t* slots, int32_t num_tokens) {
  if (!k_new || !v_new || !k_pool || !v_pool || !kv || !slots)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens must be >= 0");
  if (kv->num_pages < 1 || kv->page_size < 1 || kv->num_kv_heads < 1 || kv->head_dim < 8)
    return fail(PA_ERR_SHAPE, "pool: num_pages, page_size, num_kv_heads >= 1, head_dim >= 8");
  if (kv->head_dim % 8) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  const bool one_head = kv->num_kv_heads == 1;
  if (!mult8(kv->page_stride) || !stride_ok(kv->head_stride, one_head) || !mult8(kv->token_stride) ||
      !mult8(src_token_stride) || !stride_ok(src_head_stride, one_head))
    return fail(PA_ERR_ALIGN, "strides must be positive multiples of 8 elements");
  if (kv->token_stride < kv->head_dim || (!one_head && src_head_stride < kv->head_dim))
    return fail(PA_ERR_SHAPE, "rows of one token and head must not overlap");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_ALIGN, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
  const int64_t blocks = ceil_div(static_cast<int64_t>(num_tokens) * 2 * kv->num_kv_heads *
                                      (kv->head_dim / 8), 256);
  if (blocks > INT32_MAX) return fail(PA_ERR_SHAPE, "too many tokens for one launch");
  return PA_OK;
}

int check_mla_insert(const void* kv_c, int64_t c_stride, const void* k_pe, int64_t pe_stride,
                     const void* kv_cache, const pa_kv_layout* cache, const int64_t* slots,
                     int32_t num_tokens, bool fp8) {
  if (!kv_c || !k_pe || !kv_cache || !cache || !slots)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens must be >= 0");
  if (cache->num_pages < 1 || cache->page_size < 1)
    return fail(PA_ERR_SHAPE, "cache: num_pages and page_size must be >= 1");
  const int32_t row = fp8 ? kMlaFp8Row : kMlaRow;
  if (cache->num_kv_heads != 1 || cache->head_dim != row)
    return fail(PA_ERR_UNSUPPORTED, fp8 ? "FP8 MLA cache must have num_kv_heads 1 and head_dim 656 (bytes)"
                                        : "MLA cache must have num_kv_heads 1 and head_dim 576");
  const int64_t smul = fp8 ? 16 : 8;   // cache strides: 16 bytes either way
  if (cache->page_stride <= 0 || cache->page_stride % smul || cache->token_stride <= 0 ||
      cache->token_stride % smul || !mult8(c_stride) || !mult8(pe_stride))
    return fail(PA_ERR_ALIGN, fp8 ? "FP8 cache strides must be positive multiples of 16 bytes, "
                                    "source strides multiples of 8 elements"
                                  : "strides must be positive multiples of 8 elements");
  if (cache->token_stride < row || c_stride < kMlaLat || pe_stride < kMlaRope)
    return fail(PA_ERR_SHAPE, fp8 ? "token_stride >= 656, c_stride >= 512 and pe_stride >= 64 required"
                                  : "token_stride >= 576, c_stride >= 512 and pe_stride >= 64 required");
  if (!aligned16(kv_c) || !aligned16(k_pe) || !aligned16(kv_cache))
    return fail(PA_ERR_ALIGN, "kv_c, k_pe and kv_cache must be 16-byte aligned");
  return PA_OK;
}

}  // namespace pa
