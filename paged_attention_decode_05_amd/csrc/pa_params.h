// pa_params.h -- kernel parameter blocks shared by the launchers and the
// C-ABI entry points (passed to the kernels by value).
#pragma once

#include <stdint.h>

namespace pa {

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* part_out;
  float* part_max;
  float* part_sum;
  int64_t page_stride;
  int64_t head_stride;
  int32_t token_stride;
  int32_t tile_bytes;   // bytes spanned by one (page, KV head) tile: ((ps-1)*token_stride + D)*2
  int32_t token_bytes;  // token_stride * 2
  uint32_t page_bytes;  // page_stride * 2
  int32_t bt_stride;
  int32_t num_q_heads;  // rows of q and out per sequence: Hq * num_queries
  int32_t kv_heads;     // Hkv
  int32_t page_size;
  int32_t page_shift;   // log2(page_size)
  int32_t window;
  // Virtual heads of a KV group: S query tokens per sequence (q [b][s][Hq][D])
  // times Gq = Hq / Hkv q heads give vheads = S * Gq live heads, virtual head
  // h being query h / Gq, q head h % Gq of the group.  The kernel's group G
  // (a template argument: 1, 2, 4, 8 or 16) is vheads rounded up; heads
  // vheads .. G-1 are padding, see no key and write nothing.  Query s sees
  // keys up to n - S + s when causal; `reach` is the window of the union of
  // the queries' key ranges (window + S - 1 when causal, else window).
  int32_t num_queries;
  int32_t q_heads;      // Hq
  int32_t gq;           // Gq, q heads per KV head
  int32_t vheads;       // S * Gq
  int32_t causal;
  int32_t reach;
  int32_t partition_size;
  int32_t max_parts;
  int32_t write_empty;
  float scale_log2;     // softmax scale * log2(e) (times the K pool scale for FP8 pools)
  float out_scale;      // factor on every output and partial: the V pool scale (1 for bf16)
};

struct MergeParams {
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  uint16_t* out;
  float* lse;
  int32_t num_q_heads;
  int32_t partition_size;
  int32_t max_parts;
  int32_t window;
};

// Device buffers of the balanced split and its merge.
struct BalancedLayout {
  const int32_t* context_lens;
  uint16_t* out;         // [batch][num_q_heads][D] bf16
  float* lse;            // [batch][num_q_heads] or NULL
  float* seg_out;        // [(rows + grid) * G][D]  partial of segment slot s, head h at s*G + h
  float* seg_max;        // [(rows + grid) * G]
  float* seg_sum;
  // Record of row r, rewritten by every call: (first block << 12) | pieces,
  // the pieces sitting in slots r + first .. r + first + pieces - 1.
  int32_t* row_info;     // [rows]
  int64_t min_units;     // a block owns at least this many units (keys of one KV head)
  int32_t row_cost;      // units charged to a row's start (its prologue), before its keys
  int32_t rows;          // batch * num_kv_heads
  int32_t batch;
  int32_t q_heads;       // Hq (out rows are [b][s][Hq])
  int32_t gq;            // Gq; virtual head h -> query h / Gq, head h % Gq
  int32_t vheads;        // S * Gq; padding heads h >= vheads write nothing
};

}  // namespace pa
