// pa_mla.hip -- absorbed MLA decode (entry points; kernels follow).
#include <hip/hip_runtime.h>

#include "pa_decode.h"
#include "pa_validate.h"

extern "C" {

size_t mla_absorbed_decode_workspace_size(int32_t batch, int32_t num_heads,
                                          int32_t max_pages_per_seq, int32_t page_size,
                                          int32_t partition_size) {
  pa::MlaPlan plan;
  if (!pa::plan_mla(batch, num_heads, max_pages_per_seq, page_size, partition_size, &plan))
    return 0;
  return plan.bytes;
}

int mla_absorbed_decode(const void* q_nope, const void* q_rope, const void* kv_cache,
                        const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                        const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* context_lens, int32_t batch, int32_t num_heads,
                        int32_t max_pages_per_seq, float scale, int32_t partition_size, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int rc = pa::check_mla(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out);
  if (rc) return rc;
  pa::MlaPlan plan;
  if (!pa::plan_mla(batch, num_heads, max_pages_per_seq, cache->page_size, partition_size, &plan))
    return pa::fail(PA_ERR_SHAPE, "no launch plan for these shapes");
  if (!workspace || workspace_bytes < plan.bytes)
    return pa::fail(PA_ERR_WORKSPACE, "workspace too small");
  return pa::fail(PA_ERR_UNSUPPORTED, "absorbed MLA kernels are not in this build yet");
}

}  // extern "C"
