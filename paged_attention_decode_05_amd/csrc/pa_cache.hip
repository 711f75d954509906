// pa_cache.hip -- writes into the paged caches: K/V insert and the MLA
// latent-cache write.
//
// Token i goes to the flat slot s = slots[i] = page * page_size + offset
// [vllm.cpp kernel matrix, row KERNEL-KV-CACHE: KV insert into the paged
// cache; the MLA cache write concatenates the latent and rope projections
// into the 576-wide row; both are exact copies].  The copies move 16-byte
// chunks (8 bf16) from the source row to the cache row, indexed by a flat
// (token, chunk) item number, so a launch covers any number of tokens with
// full 16-byte accesses (the K/V insert moves four items per thread, the
// latent write one).  Slots outside [0, num_pages *
// page_size) -- negative ones mark padding -- are skipped, so no slot value
// can make the kernel write outside the pool.
#include <hip/hip_runtime.h>

#include <string>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_profile.h"
#include "pa_validate.h"

namespace pa {

constexpr int kCopyThreads = 256;

struct KvInsertParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int64_t* slots;
  int64_t src_token_stride, src_head_stride;
  int64_t page_stride, head_stride, token_stride;
  int64_t total_slots;
  int64_t num_tokens;
  int32_t page_size;
  int32_t chunks_per_head;    // head_dim / 8
  int32_t chunks_per_tensor;  // num_kv_heads * head_dim / 8
};

// Item x: token x / (2 * chunks_per_tensor); within it, K chunks first,
// then V chunks; chunk c of a tensor is head c / chunks_per_head, dims
// 8 * (c % chunks_per_head) .. +8.  A thread moves the kInsertItems items
// t, t + T, t + 2T, ... (T threads in the grid): their slot reads, then their
// row loads, then their stores, so each thread has that many copies in
// flight while consecutive threads still touch consecutive chunks.
constexpr int kInsertItems = 4;

__global__ __launch_bounds__(kCopyThreads) void kv_insert_kernel(const KvInsertParams p) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  const int64_t T = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  const int64_t per_token = 2 * static_cast<int64_t>(p.chunks_per_tensor);
  const int64_t items = p.num_tokens * per_token;
  int64_t dst[kInsertItems];
  bool to_v[kInsertItems], live[kInsertItems];
  uint4 v[kInsertItems];
#pragma unroll
  for (int k = 0; k < kInsertItems; ++k) {
    const int64_t x = t + k * T;
    const int64_t i = x / per_token;
    int c = static_cast<int>(x - i * per_token);
    const bool is_v = c >= p.chunks_per_tensor;
    if (is_v) c -= p.chunks_per_tensor;
    const int64_t s = x < items ? p.slots[i] : -1;
    live[k] = s >= 0 && s < p.total_slots;
    to_v[k] = is_v;
    const int h = c / p.chunks_per_head;
    const int d = 8 * (c - h * p.chunks_per_head);
    const int64_t page = s / p.page_size, off = s - page * p.page_size;
    dst[k] = page * p.page_stride + h * p.head_stride + off * p.token_stride + d;
    const int64_t src = i * p.src_token_stride + h * p.src_head_stride + d;
    v[k] = live[k] ? load16((is_v ? p.v_new : p.k_new) + src) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < kInsertItems; ++k)
    if (live[k]) *reinterpret_cast<uint4*>((to_v[k] ? p.v_pool : p.k_pool) + dst[k]) = v[k];
}

struct MlaInsertParams {
  const uint16_t* kv_c;
  const uint16_t* k_pe;
  uint16_t* cache;
  const int64_t* slots;
  int64_t c_stride, pe_stride;
  int64_t page_stride, token_stride;
  int64_t total_slots;
  int64_t num_tokens;
  int32_t page_size;
};

// Thread x: token x / 72, chunk x % 72 of the 576-wide row: chunks 0..63 come
// from the latent source, 64..71 from the rope source.
__global__ __launch_bounds__(kCopyThreads) void mla_insert_kernel(const MlaInsertParams p) {
  constexpr int kLatChunks = kMlaLat / 8, kRowChunks = kMlaRow / 8;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (x >= p.num_tokens * kRowChunks) return;
  const int64_t i = x / kRowChunks;
  const int c = static_cast<int>(x - i * kRowChunks);
  const int64_t s = p.slots[i];
  if (s < 0 || s >= p.total_slots) return;
  const int64_t page = s / p.page_size, off = s - page * p.page_size;
  const uint4 v = c < kLatChunks ? load16(p.kv_c + i * p.c_stride + 8 * c)
                                 : load16(p.k_pe + i * p.pe_stride + 8 * (c - kLatChunks));
  *reinterpret_cast<uint4*>(p.cache + page * p.page_stride + off * p.token_stride + 8 * c) = v;
}

// ---- FP8 latent cache write ----------------------------------------------------
//
// The fp8_ds_mla quantization of the pages [vllm.cpp kernel matrix, row
// KERNEL-KV-CACHE-DSA: E4M3 elements in blocks of 64, one UE8M0 power-of-two
// scale per block with exponent ceil(log2(absmax / 448)), stored as
// exponent + 127; the rope part stays bf16], applied to the 512-wide latent
// of the MLA cache row.  Row layout in bytes: [0, 512) E4M3 latent, [512, 640)
// bf16 rope, [640, 648) the 8 block-scale bytes, [648, 656) zero.  An
// all-zero block, or one whose exponent would fall below -126, takes -126, so
// every scale 2^e is a normal float32.

// Smallest e with 448 * 2^e >= a (a >= 0 finite), clamped to [-126, 127]:
// with a = m * 2^E, m in [1, 2), and 448 = 1.75 * 2^8, e = E - 8 when
// m <= 1.75 (mantissa field <= 0x600000), else E - 7.
__device__ __forceinline__ int fp8_block_exponent(float a) {
  if (a == 0.0f) return -126;
  uint32_t u = f2u(a);
  int E;
  if (u < 0x00800000u) {              // subnormal: scale up by 2^32 (exact)
    u = f2u(a * 4294967296.0f);
    E = static_cast<int>(u >> 23) - 127 - 32;
  } else {
    E = static_cast<int>(u >> 23) - 127;
  }
  const int e = (u & 0x7fffffu) <= 0x600000u ? E - 8 : E - 7;
  return min(max(e, -126), 127);
}

// E4M3 byte nearest to q (|q| <= 448), ties to the even code, sign bit = the
// sign bit of q.  Normal range (|q| >= 2^-6): round the float32 mantissa to 3
// bits to nearest even (a carry moves into the exponent), then rebias the
// exponent from 127 to 7.  Below 2^-6 the codes are the multiples of 2^-9:
// the code is |q| * 2^9 rounded to nearest even (8 is the smallest normal).
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = f2u(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {              // |q| < 2^-6
    code = static_cast<uint32_t>(__builtin_rintf(u2f(a) * 512.0f));
  } else {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

struct MlaInsertFp8Params {
  const uint16_t* kv_c;
  const uint16_t* k_pe;
  uint8_t* cache;
  const int64_t* slots;
  int64_t c_stride, pe_stride;      // elements
  int64_t page_stride, token_stride;  // bytes
  int64_t total_slots;
  int64_t num_tokens;
  int32_t page_size;
};

constexpr int kFp8InsertTokens = kCopyThreads / 64;   // one wave per token

// Wave w of block x writes token 4x + w.  Lane l quantizes latent values
// 8l .. 8l+7 (block l / 8; the block's 8 lanes share its absmax), lanes 0..7
// copy the rope part, lane 0 writes the scale bytes and the padding.
__global__ __launch_bounds__(kCopyThreads) void mla_insert_fp8_kernel(const MlaInsertFp8Params p) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kFp8InsertTokens + (threadIdx.x >> 6);
  if (i >= p.num_tokens) return;
  const int64_t s = p.slots[i];
  if (s < 0 || s >= p.total_slots) return;
  const int64_t page = s / p.page_size, off = s - page * p.page_size;
  uint8_t* row = p.cache + page * p.page_stride + off * p.token_stride;

  const uint4 x = load16(p.kv_c + i * p.c_stride + 8 * lane);
  float v[8];
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = u2f(w[k] << 16);
    v[2 * k + 1] = u2f(w[k] & 0xffff0000u);
  }
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  a = fmaxf(a, __shfl_xor(a, 4));
  const int e = fp8_block_exponent(a);
  // 2^-e is a normal float32 for e in [-126, 126]; e = 127 needs
  // absmax > 448 * 2^126, beyond any bf16 value, so it never occurs
  const float inv = u2f(static_cast<uint32_t>(127 - e) << 23);
  uint32_t b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) b[k] = e4m3_encode(v[k] * inv);
  *reinterpret_cast<uint2*>(row + 8 * lane) =
      make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                 b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
  if (lane < kMlaRope / 8)
    *reinterpret_cast<uint4*>(row + kMlaFp8Rope + 16 * lane) = load16(p.k_pe + i * p.pe_stride + 8 * lane);
  // scale byte of block j sits on lane 8j
  uint32_t sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sc[j] = static_cast<uint32_t>(__shfl(e + 127, 8 * j));
  if (lane == 0)
    *reinterpret_cast<uint4*>(row + kMlaFp8Scales) =
        make_uint4(sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24),
                   sc[4] | (sc[5] << 8) | (sc[6] << 16) | (sc[7] << 24), 0u, 0u);
}

}  // namespace pa

extern "C" {

int pa_kv_insert(const void* k_new, const void* v_new, int64_t src_token_stride,
                 int64_t src_head_stride, void* k_pool, void* v_pool, const pa_kv_layout* kv,
                 const int64_t* slots, int32_t num_tokens, void* stream) {
  const int rc = pa::check_kv_insert(k_new, v_new, src_token_stride, src_head_stride, k_pool,
                                     v_pool, kv, slots, num_tokens);
  if (rc) return rc;
  if (num_tokens == 0) return PA_OK;
  pa::KvInsertParams p{};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_pool = static_cast<uint16_t*>(k_pool);
  p.v_pool = static_cast<uint16_t*>(v_pool);
  p.slots = slots;
  p.src_token_stride = src_token_stride;
  p.src_head_stride = src_head_stride;
  p.page_stride = kv->page_stride;
  p.head_stride = kv->head_stride;
  p.token_stride = kv->token_stride;
  p.total_slots = static_cast<int64_t>(kv->num_pages) * kv->page_size;
  p.num_tokens = num_tokens;
  p.page_size = kv->page_size;
  p.chunks_per_head = kv->head_dim / 8;
  p.chunks_per_tensor = kv->num_kv_heads * (kv->head_dim / 8);
  const int64_t items = static_cast<int64_t>(num_tokens) * 2 * p.chunks_per_tensor;
  const int64_t per_block = static_cast<int64_t>(pa::kCopyThreads) * pa::kInsertItems;
  const int64_t blocks = (items + per_block - 1) / per_block;
  pa::clear_error();
  pa::launch_profiled(pa::kv_insert_kernel, dim3(static_cast<unsigned>(blocks)),
                      dim3(pa::kCopyThreads), 0, static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("kv insert: ") + hipGetErrorString(e));
  return PA_OK;
}

int mla_cache_insert(const void* kv_c, int64_t c_stride, const void* k_pe, int64_t pe_stride,
                     void* kv_cache, const pa_kv_layout* cache, const int64_t* slots,
                     int32_t num_tokens, void* stream) {
  const int rc = pa::check_mla_insert(kv_c, c_stride, k_pe, pe_stride, kv_cache, cache, slots,
                                      num_tokens);
  if (rc) return rc;
  if (num_tokens == 0) return PA_OK;
  pa::MlaInsertParams p{};
  p.kv_c = static_cast<const uint16_t*>(kv_c);
  p.k_pe = static_cast<const uint16_t*>(k_pe);
  p.cache = static_cast<uint16_t*>(kv_cache);
  p.slots = slots;
  p.c_stride = c_stride;
  p.pe_stride = pe_stride;
  p.page_stride = cache->page_stride;
  p.token_stride = cache->token_stride;
  p.total_slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  p.num_tokens = num_tokens;
  p.page_size = cache->page_size;
  const int64_t threads = static_cast<int64_t>(num_tokens) * (pa::kMlaRow / 8);
  const int64_t blocks = (threads + pa::kCopyThreads - 1) / pa::kCopyThreads;
  pa::clear_error();
  hipLaunchKernelGGL(pa::mla_insert_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(pa::kCopyThreads), 0, static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("mla insert: ") + hipGetErrorString(e));
  return PA_OK;
}

int mla_cache_insert_fp8(const void* kv_c, int64_t c_stride, const void* k_pe, int64_t pe_stride,
                         void* kv_cache, const pa_kv_layout* cache, const int64_t* slots,
                         int32_t num_tokens, void* stream) {
  const int rc = pa::check_mla_insert(kv_c, c_stride, k_pe, pe_stride, kv_cache, cache, slots,
                                      num_tokens, true);
  if (rc) return rc;
  if (num_tokens == 0) return PA_OK;
  pa::MlaInsertFp8Params p{};
  p.kv_c = static_cast<const uint16_t*>(kv_c);
  p.k_pe = static_cast<const uint16_t*>(k_pe);
  p.cache = static_cast<uint8_t*>(kv_cache);
  p.slots = slots;
  p.c_stride = c_stride;
  p.pe_stride = pe_stride;
  p.page_stride = cache->page_stride;
  p.token_stride = cache->token_stride;
  p.total_slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  p.num_tokens = num_tokens;
  p.page_size = cache->page_size;
  const int64_t blocks = (static_cast<int64_t>(num_tokens) + pa::kFp8InsertTokens - 1) /
                         pa::kFp8InsertTokens;
  pa::clear_error();
  hipLaunchKernelGGL(pa::mla_insert_fp8_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(pa::kCopyThreads), 0, static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return pa::fail(PA_ERR_LAUNCH, std::string("mla fp8 insert: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
