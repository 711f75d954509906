// pa_validate.h -- host-side argument checks and launch planning for the
// paged-decode C ABI.  Pure C++ (no HIP headers), so the checks build and
// run on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "pa_decode.h"

namespace pa {

// Records `msg` as the calling thread's last error and returns `status`.
int fail(int status, const std::string& msg);
void clear_error();
const char* last_error();

// Supported shapes.  Any 1..16 heads per KV group (q heads per KV head,
// times the queries per sequence for multi-query decode) run on a kernel
// built for 1, 2, 4, 8 or 16: group_padded() rounds up (0 if out of range).
bool head_dim_supported(int32_t d);
bool group_supported(int32_t head_dim, int32_t group);
bool page_size_supported(int32_t ps);
int32_t group_padded(int32_t heads);

// Compute units the balanced split is sized for (MI355X has 256): a fixed
// count, so the cut points, and with them an output's last bits, do not
// depend on the device the call runs on.
constexpr int32_t kSplitCUs = 256;

// Largest number of keys one sequence can attend to.
int64_t max_keys(int32_t max_pages_per_seq, int32_t page_size, int32_t window);

// Checks shared by pa_decode and pa_decode_splitkv.
// elem_bytes: 2 for bf16 pools, 1 for FP8 (E4M3) pools; pool strides count
// elements, and every K/V row must start on a 16-byte boundary.
int check_gqa(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
              int32_t max_pages_per_seq, float scale, int32_t elem_bytes = 2);

// Checks for explicit split parameters.
int check_split(int32_t partition_size, int32_t max_partitions, int32_t max_pages_per_seq,
                int32_t page_size, int32_t window, const float* part_out, const float* part_max,
                const float* part_sum);

int check_merge(const float* part_out, const float* part_max, const float* part_sum,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t head_dim, int32_t partition_size, int32_t max_partitions, const void* out);

// Workspace carve-up of pa_decode (balanced split): the segment partials,
// one slot per (row, block) segment, rows + kMaxBalancedBlocks slots in all.
constexpr int32_t kMaxBalancedBlocks = 2048;
// Keys (of one KV head) below which a block is not worth it.  32 measured best
// on the tiny decode (8 sequences, 1 to 1000 keys): 23.9 us at 128, 19.3 at
// 64, 17.8 at 32, 21.5 at 16 (more pieces to merge); larger calls fill every
// block well above it.
constexpr int64_t kMinUnitsPerBlock = 32;
// Units of the balanced key line that stand for a row's prologue, charged
// before its keys, so a block whose share starts several rows gets fewer keys
// (for 4-wave blocks over FP8 and f32 pools; balanced_row_cost halves it for
// bf16 pools and doubles it for a block of all the waves of a CU, which
// streams its keys faster).
constexpr int32_t kRowCostUnits = 128;

struct DecodePlan {
  int32_t rows = 0;          // batch * num_kv_heads
  int32_t group = 0;         // padded heads per KV group (the kernel's tile)
  size_t off_seg_out = 0, off_seg_max = 0, off_seg_sum = 0;
  size_t off_row_info = 0;   // one 32-bit record per row
  size_t bytes = 0;
};
// vheads: live heads per KV group (q heads per KV head x queries per sequence).
bool plan_decode(int32_t batch, int32_t num_kv_heads, int32_t vheads, int32_t head_dim,
                 int32_t max_pages_per_seq, int32_t page_size, int32_t window, DecodePlan* plan);

// Fixed partition size used by pa_decode_partition_size (the two-stage API's
// suggestion for these shapes).
int32_t suggest_partition(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_pages_per_seq, int32_t page_size, int32_t window);

// MLA geometry fixed by the absorbed-MLA entry point.
constexpr int32_t kMlaNope = 128;
constexpr int32_t kMlaRope = 64;
constexpr int32_t kMlaLat = 512;
constexpr int32_t kMlaRow = kMlaLat + kMlaRope;  // 576
constexpr int32_t kMlaDv = 128;
constexpr int32_t kMlaKeyTile = 64;              // partition sizes are multiples of this
constexpr int32_t kMlaTileKeys = 32;             // keys per LDS tile of the split kernel
constexpr int32_t kMlaBlockHeads = 64;           // heads per split-kernel block (a head group)
constexpr int32_t kMlaMaxExplicitBlocks = 16384; // cap for an explicit partition size
constexpr int32_t kMlaMinKeys = 128;             // fewest keys per piece at the library's choice
// FP8 latent-cache row, in bytes: E4M3 latent (blocks of 64, one scale byte
// each), bf16 rope, the scale bytes, zero padding to a 16-byte multiple.
constexpr int32_t kMlaFp8Block = 64;
constexpr int32_t kMlaFp8Rope = kMlaLat;                        // 512
constexpr int32_t kMlaFp8Scales = kMlaLat + 2 * kMlaRope;       // 640
constexpr int32_t kMlaFp8Row = kMlaFp8Scales + 16;              // 656

struct MlaPlan {
  int32_t groups = 0;        // ceil(num_heads / 64)
  int32_t max_blocks = 0;    // split-kernel blocks launched, one partial slot each
  size_t off_qhi = 0, off_qmid = 0, off_qlo = 0;
  size_t off_seg_out = 0, off_seg_max = 0, off_seg_sum = 0, off_split_plan = 0, off_row_slots = 0;
  size_t bytes = 0;
};
bool plan_mla(int32_t batch, int32_t num_heads, int32_t max_pages_per_seq, int32_t page_size,
              int32_t partition_size, MlaPlan* plan);

// fp8: the cache holds FP8 rows (head_dim kMlaFp8Row, strides in bytes,
// multiples of 16) instead of bf16 576-wide rows.  num_queries: queries per
// sequence (1..16), each with num_heads heads.
int check_mla(const void* q_nope, const void* q_rope, const void* kv_cache,
              const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_heads,
              int32_t max_pages_per_seq, float scale, int32_t partition_size, const void* out,
              bool fp8 = false, int32_t num_queries = 1);

int check_kv_insert(const void* k_new, const void* v_new, int64_t src_token_stride,
                    int64_t src_head_stride, const void* k_pool, const void* v_pool,
                    const pa_kv_layout* kv, const int64_t* slots, int32_t num_tokens);

int check_mla_insert(const void* kv_c, int64_t c_stride, const void* k_pe, int64_t pe_stride,
                     const void* kv_cache, const pa_kv_layout* cache, const int64_t* slots,
                     int32_t num_tokens, bool fp8 = false);

}  // namespace pa
