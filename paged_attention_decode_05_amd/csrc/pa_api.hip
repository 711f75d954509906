// pa_api.hip -- extern "C" entry points of libpa_decode.so.  Each one checks
// its arguments on the host (pa_validate.cpp), fills a parameter block and
// enqueues kernels on the caller's stream.  Nothing here allocates, copies or
// synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

#include "pa_decode.h"
#include "pa_validate.h"

#include "pa_params.h"
#include "pa_profile.h"

namespace pa {

thread_local ProfileHook g_profile;

hipError_t launch_split(const SplitParams& p, int head_dim, int group, int batch,
                        int num_kv_heads, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int head_dim, int batch, hipStream_t stream);
// kv: pool element type, 0 bf16, 1 FP8 (E4M3), 2 f32
hipError_t launch_balanced(const SplitParams& sp, const BalancedLayout& bl, int head_dim, int group,
                           int grid, hipStream_t stream, int kv);
int balanced_grid(int head_dim, int group, int num_cus, int max_blocks, int kv);
int balanced_row_cost(int head_dim, int group, int kv);

}  // namespace pa

namespace {

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return pa::fail(PA_ERR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

int ilog2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

pa::SplitParams split_params(const void* q, const void* k_pool, const void* v_pool,
                             const pa_kv_layout* kv, const int32_t* block_table,
                             int32_t block_table_stride, const int32_t* context_lens,
                             int32_t num_q_heads, float scale, int32_t window,
                             int32_t partition_size, int32_t max_partitions, float* part_out,
                             float* part_max, float* part_sum, int32_t write_empty,
                             int32_t elem_bytes = 2) {
  pa::SplitParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_pool);
  p.v = static_cast<const uint16_t*>(v_pool);
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.page_stride = kv->page_stride;
  p.head_stride = kv->head_stride;
  p.token_stride = static_cast<int32_t>(kv->token_stride);
  p.tile_bytes =
      static_cast<int32_t>(((kv->page_size - 1) * kv->token_stride + kv->head_dim) * elem_bytes);
  p.token_bytes = static_cast<int32_t>(kv->token_stride * elem_bytes);
  p.page_bytes = static_cast<uint32_t>(kv->page_stride * elem_bytes);
  p.bt_stride = block_table_stride;
  p.num_q_heads = num_q_heads;
  p.kv_heads = kv->num_kv_heads;
  p.page_size = kv->page_size;
  p.page_shift = ilog2(kv->page_size);
  p.window = window;
  p.num_queries = 1;
  p.q_heads = num_q_heads;
  p.gq = num_q_heads / kv->num_kv_heads;
  p.vheads = p.gq;
  p.causal = 1;
  p.reach = window;
  p.partition_size = partition_size;
  p.max_parts = max_partitions;
  p.write_empty = write_empty;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.out_scale = 1.0f;
  return p;
}

}  // namespace

extern "C" {

int pa_decode_splitkv(const void* q, const void* k_pool, const void* v_pool,
                      const pa_kv_layout* kv, const int32_t* block_table,
                      int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                      int32_t num_q_heads, int32_t max_pages_per_seq, float scale,
                      int32_t window, int32_t partition_size, int32_t max_partitions,
                      float* part_out, float* part_max, float* part_sum, void* stream) {
  int rc = pa::check_gqa(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens,
                         batch, num_q_heads, max_pages_per_seq, scale);
  if (rc) return rc;
  rc = pa::check_split(partition_size, max_partitions, max_pages_per_seq, kv->page_size, window,
                       part_out, part_max, part_sum);
  if (rc) return rc;
  const pa::SplitParams p = split_params(q, k_pool, v_pool, kv, block_table, block_table_stride,
                                         context_lens, num_q_heads, scale, window, partition_size,
                                         max_partitions, part_out, part_max, part_sum, 1);
  pa::clear_error();
  return launch_status(pa::launch_split(p, kv->head_dim, pa::group_padded(p.gq), batch,
                                        kv->num_kv_heads, static_cast<hipStream_t>(stream)),
                       "split kernel");
}

int pa_merge_lse(const float* part_out, const float* part_max, const float* part_sum,
                 const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                 int32_t head_dim, int32_t partition_size, int32_t max_partitions,
                 int32_t window, void* out, float* lse_out, void* stream) {
  int rc = pa::check_merge(part_out, part_max, part_sum, context_lens, batch, num_q_heads,
                           head_dim, partition_size, max_partitions, out);
  if (rc) return rc;
  pa::MergeParams p{};
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.context_lens = context_lens;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse_out;
  p.num_q_heads = num_q_heads;
  p.partition_size = partition_size;
  p.max_parts = max_partitions;
  p.window = window;
  pa::clear_error();
  return launch_status(pa::launch_merge(p, head_dim, batch, static_cast<hipStream_t>(stream)),
                       "merge kernel");
}

size_t pa_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_pages_per_seq, int32_t page_size,
                                int32_t window) {
  pa::DecodePlan plan;
  if (num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads ||
      !pa::plan_decode(batch, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                       max_pages_per_seq, page_size, window, &plan))
    return 0;
  return plan.bytes;
}

int32_t pa_decode_partition_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_pages_per_seq, int32_t page_size,
                                 int32_t window) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads) return 0;
  return pa::suggest_partition(batch, num_kv_heads, head_dim, max_pages_per_seq, page_size, window);
}

}  // extern "C"

namespace {

// pa_decode with S query tokens per sequence (S = 1: plain decode).
// kv_type: 0 bf16 pools; 1 FP8, OCP E4M3 bytes with values e4m3 * k_scale /
// v_scale; 2 f32 pools.
int decode_impl(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
                const int32_t* block_table, int32_t block_table_stride,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t num_queries, int32_t causal, int32_t max_pages_per_seq, float scale,
                int32_t window, void* out, float* lse_out, void* workspace,
                size_t workspace_bytes, void* stream, int kv_type = 0, float k_scale = 1.0f,
                float v_scale = 1.0f) {
  const bool fp8 = kv_type == 1;
  const int elem_bytes = kv_type == 1 ? 1 : kv_type == 2 ? 4 : 2;
  int rc = pa::check_gqa(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens,
                         batch, num_q_heads, max_pages_per_seq, scale, elem_bytes);
  if (rc) return rc;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
               v_scale > 0.0f))
    return pa::fail(PA_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  if (fp8 && !(std::isfinite(scale * k_scale) && scale * k_scale > 0.0f))
    return pa::fail(PA_ERR_SHAPE, "scale * k_scale must be a finite positive float");
  if (!out) return pa::fail(PA_ERR_NULL, "out must not be NULL");
  if (reinterpret_cast<uintptr_t>(out) & 15u)
    return pa::fail(PA_ERR_ALIGN, "out must be 16-byte aligned");
  const int group = num_q_heads / kv->num_kv_heads;
  const int vheads = num_queries * group;   // live heads of one KV group
  if (vheads > 16)
    return pa::fail(PA_ERR_UNSUPPORTED, "num_queries times the q heads per KV head must be <= 16");
  pa::DecodePlan plan;
  if (!pa::plan_decode(batch, kv->num_kv_heads, vheads, kv->head_dim, max_pages_per_seq,
                       kv->page_size, window, &plan))
    return pa::fail(PA_ERR_SHAPE, "no launch plan for these shapes");
  // No workspace: one block per (sequence, KV head) row, outputs written
  // directly.  With one: the balanced split and the merge of cut rows.
  if (workspace && workspace_bytes < plan.bytes)
    return pa::fail(PA_ERR_WORKSPACE, "workspace must hold " + std::to_string(plan.bytes) +
                                          " bytes (or be NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return pa::fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const int vgroup = plan.group;
  int nbmax = pa::balanced_grid(kv->head_dim, vgroup, pa::kSplitCUs, pa::kMaxBalancedBlocks, kv_type);
  if (nbmax < 1) return pa::fail(PA_ERR_UNSUPPORTED, "no balanced-split kernel for these shapes");

  pa::BalancedLayout bl{};
  bl.context_lens = context_lens;
  bl.out = static_cast<uint16_t*>(out);
  bl.lse = lse_out;
  if (ws) {
    bl.seg_out = reinterpret_cast<float*>(ws + plan.off_seg_out);
    bl.seg_max = reinterpret_cast<float*>(ws + plan.off_seg_max);
    bl.seg_sum = reinterpret_cast<float*>(ws + plan.off_seg_sum);
    bl.row_info = reinterpret_cast<int32_t*>(ws + plan.off_row_info);
  } else {
    nbmax = plan.rows < (1 << 20) ? plan.rows : (1 << 20);   // one block per row
  }
  bl.min_units = pa::kMinUnitsPerBlock;
  bl.row_cost = pa::balanced_row_cost(kv->head_dim, vgroup, kv_type);
  bl.rows = plan.rows;
  bl.batch = batch;
  bl.q_heads = num_q_heads;
  bl.gq = group;
  bl.vheads = vheads;

  pa::SplitParams sp = split_params(q, k_pool, v_pool, kv, block_table, block_table_stride,
                                    context_lens, num_q_heads, fp8 ? scale * k_scale : scale,
                                    window, 1, 1, nullptr, nullptr, nullptr, 0, elem_bytes);
  if (fp8) sp.out_scale = v_scale;
  sp.num_q_heads = num_q_heads * num_queries;   // rows of q and out per sequence
  sp.num_queries = num_queries;
  sp.vheads = vheads;
  sp.causal = causal ? 1 : 0;
  sp.reach = (window > 0 && causal) ? window + num_queries - 1 : window;
  pa::clear_error();
  return launch_status(pa::launch_balanced(sp, bl, kv->head_dim, vgroup, nbmax,
                                           static_cast<hipStream_t>(stream), kv_type),
                       "balanced decode");
}

}  // namespace

extern "C" {

int pa_decode(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
              int32_t max_pages_per_seq, float scale, int32_t window, void* out,
              float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens, batch,
                     num_q_heads, 1, 1, max_pages_per_seq, scale, window, out, lse_out,
                     workspace, workspace_bytes, stream);
}

int pa_decode_multiquery(const void* q, const void* k_pool, const void* v_pool,
                         const pa_kv_layout* kv, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                         int32_t num_q_heads, int32_t num_queries, int32_t causal,
                         int32_t max_pages_per_seq, float scale, int32_t window, void* out,
                         float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_queries < 1 || num_queries > 16)
    return pa::fail(PA_ERR_SHAPE, "num_queries must be in 1..16");
  return decode_impl(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens, batch,
                     num_q_heads, num_queries, causal, max_pages_per_seq, scale, window, out,
                     lse_out, workspace, workspace_bytes, stream);
}

int pa_decode_fp8(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
                  const int32_t* block_table, int32_t block_table_stride,
                  const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                  int32_t max_pages_per_seq, float scale, float k_scale, float v_scale,
                  int32_t window, void* out, float* lse_out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens, batch,
                     num_q_heads, 1, 1, max_pages_per_seq, scale, window, out, lse_out,
                     workspace, workspace_bytes, stream, 1, k_scale, v_scale);
}

int pa_decode_f32(const void* q, const void* k_pool, const void* v_pool, const pa_kv_layout* kv,
                  const int32_t* block_table, int32_t block_table_stride,
                  const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                  int32_t max_pages_per_seq, float scale, int32_t window, void* out,
                  float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens, batch,
                     num_q_heads, 1, 1, max_pages_per_seq, scale, window, out, lse_out,
                     workspace, workspace_bytes, stream, 2);
}

size_t pa_decode_multiquery_workspace_size(int32_t batch, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_pages_per_seq, int32_t page_size,
                                           int32_t window, int32_t num_queries) {
  if (num_queries < 1 || num_queries > 16 || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads)
    return 0;
  pa::DecodePlan plan;
  if (!pa::plan_decode(batch, num_kv_heads, num_queries * (num_q_heads / num_kv_heads), head_dim,
                       max_pages_per_seq, page_size, window, &plan))
    return 0;
  return plan.bytes;
}

const char* pa_last_error(void) { return pa::last_error(); }

void pa_profile_next(void* start_event, void* stop_event) {
  pa::g_profile.start = static_cast<hipEvent_t>(start_event);
  pa::g_profile.stop = static_cast<hipEvent_t>(stop_event);
}

}  // extern "C"

// ---- pa_decode_noalloc: the workspace in a library-owned device array ------------
//
// For callers that cannot allocate.  `scratch` holds pa_decode's partials
// and row records; every gfx950 device the library runs on gets its own copy
// when the code object loads there, kept until the process ends.  Host code
// never uses the array's name as an address: its device address is looked up
// once per device with hipGetSymbolAddress and kept in scratch_dev[].
namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;   // 32 MiB per device
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device (nullptr and an error
// message on failure).
void* scratch_address(std::string& err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    err = std::string("hipGetDevice: ") + (e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return nullptr;
    }
    scratch_dev[dev] = ptr;
  }
  return scratch_dev[dev];
}

}  // namespace

extern "C" {

int pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                      const pa_kv_layout* kv, const int32_t* block_table,
                      int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                      int32_t num_q_heads, int32_t max_pages_per_seq, float scale, int32_t window,
                      void* out, float* lse_out, void* stream) {
  int rc = pa::check_gqa(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens,
                         batch, num_q_heads, max_pages_per_seq, scale);
  if (rc) return rc;
  const size_t need = pa_decode_workspace_size(batch, num_q_heads, kv->num_kv_heads, kv->head_dim,
                                               max_pages_per_seq, kv->page_size, window);
  if (need == 0) return pa::fail(PA_ERR_SHAPE, "no launch plan for these shapes");
  if (need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE, "these shapes need " + std::to_string(need) +
                                          " bytes of scratch; pa_decode_noalloc holds " +
                                          std::to_string(kScratchBytes));
  std::string err;
  void* ws = scratch_address(err);
  if (!ws) return pa::fail(PA_ERR_LAUNCH, err);
  return decode_impl(q, k_pool, v_pool, kv, block_table, block_table_stride, context_lens, batch,
                     num_q_heads, 1, 1, max_pages_per_seq, scale, window, out, lse_out, ws,
                     kScratchBytes, stream);
}

}  // extern "C"
