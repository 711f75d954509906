// pa_mla.hip -- absorbed multi-head latent attention (MLA) decode for gfx950.
//
// Per sequence b and head h [pegainfer PR #938, review quote of the kernel's
// "Schedule" comment, steps 1-7; vllm.cpp kernel matrix, row
// KERNEL-ATTN-MLA-SPARSE: absorption as a weight transform plus two batched
// products, V = the latent part of the cache, split-KV with a merge]:
//   q_abs[j]  = sum_d q_nope[d] W_UK[h][d][j]                     (absorb kernel)
//   s_t       = scale * (q_abs . c_t[0:512] + q_rope . c_t[512:576])
//   o_lat[j]  = sum_t softmax(s)_t c_t[j]                          (split kernel)
//   out[dv]   = sum_j W_UV[h][dv][j] o_lat[j]                      (merge + W_UV kernel)
//
// The two 576/512-deep contractions over the latent cache run on MFMA
// (v_mfma_f32_16x16x32_bf16): per 32-key tile, S^T[32 keys x 16 heads] =
// C[32 x 576] . Q^T, and O[16 heads x 512] += P[16 x 32 keys] . C[32 x 512].
// The cache and W_UV are exact bf16; each fp32 operand (q_abs, P, o_lat)
// enters as three bf16 terms hi + mid + lo, which represent an fp32 value
// exactly (3 x 8 significant bits), so the MFMAs multiply the fp32 operands
// exactly and only the fp32 accumulation rounds, at three MFMAs instead of one.
#include <hip/hip_runtime.h>

#include <string>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_validate.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kLat = kMlaLat;      // 512
constexpr int kRow = kMlaRow;      // 576
constexpr int kNope = kMlaNope;    // 128
constexpr int kRope = kMlaRope;    // 64
constexpr int kDv = kMlaDv;        // 128
constexpr int kKS = kRow / 32;     // 18 k-steps of the score MFMA
constexpr int kKSL = kLat / 32;    // 16 of them over the latent part
constexpr int kTileKeys = 32;      // keys per LDS tile
constexpr int kHeadsPerWave = 16;
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kRowPad = kRow + 8;          // LDS row stride (elements) of the key-major copy
constexpr int kTPad = kTileKeys + 8;       // LDS row stride of the latent-major copy

struct MlaParams {
  const uint16_t* q_nope;
  const uint16_t* q_rope;
  const uint16_t* cache;
  const uint16_t* w_uk;
  const uint16_t* w_uv;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* q_hi;          // [B][H][576]  q_abs | q_rope
  uint16_t* q_mid;         // [B][H][512]  second and third terms of q_abs
  uint16_t* q_lo;
  float* part_out;         // [B][H][max_parts][512]
  float* part_max;         // [B][H][max_parts]  (natural-log domain)
  float* part_sum;
  uint16_t* out;           // [B][H][128]
  int64_t page_stride;
  int32_t token_stride;
  int32_t bt_stride;
  int32_t batch;
  int32_t num_heads;
  int32_t page_size;
  int32_t page_shift;
  int32_t partition_size;
  int32_t max_parts;
  float scale_log2;
};

__device__ __forceinline__ uint32_t pack_bf16(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

__device__ __forceinline__ float bf16_val(uint16_t b) { return u2f(static_cast<uint32_t>(b) << 16); }

// x = hi + mid + lo exactly: hi = bf16(x), mid = bf16(x - hi), lo = x - hi - mid
// (round to nearest even; each residual is exact in fp32 and the last one
// has at most 8 significant bits left).
__device__ __forceinline__ void split3_bf16(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16_rne(x);
  const float r = x - bf16_val(hi);
  mid = f32_to_bf16_rne(r);
  lo = f32_to_bf16_rne(r - bf16_val(mid));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---- 1. absorption: q_abs = q_nope . W_UK[h], split in three; rope copied ----------
//
// Block (h, jc) computes q_abs[b][h][jc*128 .. +128) for every b: thread t
// owns column j = jc*128 + t%128 and rows b = t/128, t/128 + 2, ...; the
// q_nope rows of a 16-row batch tile sit in LDS.  fp32 FMAs in ascending d.
__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p) {
  __shared__ float qs[16][kNope];
  const int h = blockIdx.x;
  const int jc = blockIdx.y;
  const int t = threadIdx.x;
  const int j = jc * 128 + (t & 127);
  const int par = t >> 7;
  const uint16_t* wcol = p.w_uk + static_cast<int64_t>(h) * kNope * kLat + j;
  for (int b0 = 0; b0 < p.batch; b0 += 16) {
    const int nb = min(16, p.batch - b0);
    __syncthreads();
    for (int i = t; i < nb * kNope; i += 256) {
      const int bb = i / kNope, d = i % kNope;
      qs[bb][d] = u2f(static_cast<uint32_t>(
                          p.q_nope[(static_cast<int64_t>(b0 + bb) * p.num_heads + h) * kNope + d])
                      << 16);
    }
    __syncthreads();
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    for (int d = 0; d < kNope; ++d) {
      const float w = u2f(static_cast<uint32_t>(wcol[static_cast<int64_t>(d) * kLat]) << 16);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(qs[par + 2 * k][d], w, acc[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int bb = par + 2 * k;
      if (bb < nb) {
        uint16_t hi, mid, lo;
        split3_bf16(acc[k], hi, mid, lo);
        const int64_t row = static_cast<int64_t>(b0 + bb) * p.num_heads + h;
        p.q_hi[row * kRow + j] = hi;
        p.q_mid[row * kLat + j] = mid;
        p.q_lo[row * kLat + j] = lo;
      }
    }
    if (jc == 0) {   // rope part: exact bf16, one term
      for (int i = t; i < nb * kRope; i += 256) {
        const int bb = i / kRope, r = i % kRope;
        const int64_t row = static_cast<int64_t>(b0 + bb) * p.num_heads + h;
        p.q_hi[row * kRow + kLat + r] = p.q_rope[row * kRope + r];
      }
    }
  }
}

// ---- 2. split attention over the latent cache ----------------------------------------
//
// Block (part, hg, b): keys [part*P, min(part*P + P, ctx)) of sequence b for
// heads hg*64 .. hg*64+63, wave w taking 16 of them.  Per 32-key tile the
// block stages the cache rows in LDS twice: key-major (A operand of the
// score MFMA) and latent-major (B operand of P.V, whose contraction runs over
// keys).  Score D layout: lane l holds S^T[key 4*(l/16)+i (+16)][head l%16];
// those 8 values are exactly the A operand of P.V for head l%16 when the P.V
// k-slots 8g..8g+7 are taken as keys {4g..4g+3, 16+4g..16+4g+3}, which is
// also the order the latent-major reads use.  The softmax keeps a per-head
// reference max and rescales the accumulators only when a score exceeds it
// by more than 2^8 (log2 domain), so P stays below 2^8 and rescaling is rare.
__global__ __launch_bounds__(kMlaThreads) void mla_split_kernel(const MlaParams p) {
  __shared__ __align__(16) uint16_t crow[kTileKeys][kRowPad];
  __shared__ __align__(16) uint16_t ct[kLat][kTPad];
  __shared__ __align__(16) uint16_t qlo_s[kHeadsPerWave * kMlaWaves][kLat + 8];   // third q term

  const int part = blockIdx.x;
  const int hg = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = p.context_lens[b];
  const int begin = part * p.partition_size;
  if (begin >= n) return;
  const int end = min(begin + p.partition_size, n);
  const int h0 = hg * (kHeadsPerWave * kMlaWaves) + wave * kHeadsPerWave;
  const bool active = h0 < p.num_heads;       // waves past the last head only load tiles
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;

  // Q^T operand for all 18 k-steps: head h0 + c16, dims 32*ks + 8g .. +8;
  // hi (18 steps) and mid (16 latent steps) in registers, lo in LDS (read
  // once per tile); the rope steps have one term.
  uint4 qh[kKS], qm[kKSL];
  if (active) {
    const int64_t hrow = static_cast<int64_t>(b) * p.num_heads + h0 + c16;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qh[ks] = load16(p.q_hi + hrow * kRow + 32 * ks + 8 * g);
#pragma unroll
    for (int ks = 0; ks < kKSL; ++ks) qm[ks] = load16(p.q_mid + hrow * kLat + 32 * ks + 8 * g);
  }
  {
    const int hb = hg * (kHeadsPerWave * kMlaWaves);
    const int nh = min(kHeadsPerWave * kMlaWaves, p.num_heads - hb);
    for (int c = tid; c < nh * (kLat / 8); c += kMlaThreads) {
      const int r = c / (kLat / 8), cc = c % (kLat / 8);
      *reinterpret_cast<uint4*>(&qlo_s[r][cc * 8]) =
          load16(p.q_lo + (static_cast<int64_t>(b) * p.num_heads + hb + r) * kLat + cc * 8);
    }
  }

  f32x4_t acc[kLat / 16];
#pragma unroll
  for (int jt = 0; jt < kLat / 16; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;     // per head c16 (same on the 4 lanes of the head)
  float l_sum = 0.0f;          // this lane's share of the head's denominator

  // Staging of one tile: 32 keys x 72 chunks of 16 B, 9 chunks per thread.
  constexpr int kChunks = kTileKeys * (kRow / 8) / kMlaThreads;   // 9
  uint4 stage[kChunks];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int c = tid + kMlaThreads * k;
      const int key = c / (kRow / 8);
      const int cc = c % (kRow / 8);
      const int t = t0 + key;
      if (t >= begin && t < end) {
        const int page = bt[t >> p.page_shift];
        stage[k] = load16(p.cache + static_cast<int64_t>(page) * p.page_stride +
                          static_cast<int64_t>(t & (p.page_size - 1)) * p.token_stride + cc * 8);
      } else {
        stage[k] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int c = tid + kMlaThreads * k;
      const int key = c / (kRow / 8);
      const int cc = c % (kRow / 8);
      *reinterpret_cast<uint4*>(&crow[key][cc * 8]) = stage[k];
      if (cc < kLat / 8) {
        const uint32_t w[4] = {stage[k].x, stage[k].y, stage[k].z, stage[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ct[cc * 8 + 2 * e][key] = static_cast<uint16_t>(w[e] & 0xffffu);
          ct[cc * 8 + 2 * e + 1][key] = static_cast<uint16_t>(w[e] >> 16);
        }
      }
    }
  };

  const int first_tile = begin / kTileKeys;
  const int last_tile = (end - 1) / kTileKeys;
  load_tile(first_tile * kTileKeys);
  for (int tile = first_tile; tile <= last_tile; ++tile) {
    const int t0 = tile * kTileKeys;
    __syncthreads();                 // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (tile < last_tile) load_tile(t0 + kTileKeys);   // next tile streams during the math
    if (!active) continue;

    // scores S^T for keys t0 .. t0+31 (two 16-key M tiles), heads h0 .. h0+15.
    // The LDS operands of step ks+1 are read while the MFMAs of step ks run;
    // the scheduling barriers keep the compiler from hoisting all 18 steps'
    // reads (which would need ~200 more registers).
    f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const uint16_t* arow0 = &crow[c16][8 * g];
    const uint16_t* arow1 = &crow[16 + c16][8 * g];
    const uint16_t* lrow = &qlo_s[wave * kHeadsPerWave + c16][8 * g];
    uint4 a0 = *reinterpret_cast<const uint4*>(arow0);
    uint4 a1 = *reinterpret_cast<const uint4*>(arow1);
    uint4 qlv = *reinterpret_cast<const uint4*>(lrow);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      uint4 n0 = a0, n1 = a1, nl = qlv;
      if (ks + 1 < kKS) {
        n0 = *reinterpret_cast<const uint4*>(arow0 + 32 * (ks + 1));
        n1 = *reinterpret_cast<const uint4*>(arow1 + 32 * (ks + 1));
        if (ks + 1 < kKSL) nl = *reinterpret_cast<const uint4*>(lrow + 32 * (ks + 1));
      }
      if (ks < kKSL) {
        sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qlv), sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qlv), sc[1], 0, 0, 0);
        sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qm[ks]), sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qm[ks]), sc[1], 0, 0, 0);
      }
      sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qh[ks]), sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qh[ks]), sc[1], 0, 0, 0);
      a0 = n0;
      a1 = n1;
      qlv = nl;
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds keys t0 + 16*mt + 4g + i for head c16
    float pv[8];
    float cm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * mt + 4 * g + i;
        const float v = (t >= begin && t < end) ? sc[mt][i] * p.scale_log2 : -INFINITY;
        pv[4 * mt + i] = v;
        cm = fmaxf(cm, v);
      }
    cm = fmaxf(cm, xor16(cm));
    cm = fmaxf(cm, xor32(cm));
    // move the reference max when a score passes it by more than 2^8
    const bool bump = cm > m_ref + 8.0f;
    if (__builtin_amdgcn_read_exec() & __ballot(bump)) {
      const float nref = bump ? cm : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.0f : fast_exp2(m_ref - nref);
      m_ref = nref;
      l_sum *= alpha;
      // accumulator rows are heads 4g + i: fetch their factors
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int jt = 0; jt < kLat / 16; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[jt][i] *= ar[i];
    }
    const float base = (m_ref == -INFINITY) ? 0.0f : m_ref;
    uint16_t ph[8], pm[8], pl[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float e = fast_exp2(pv[k] - base);
      l_sum += e;
      split3_bf16(e, ph[k], pm[k], pl[k]);
    }
    const uint4 pa_hi = make_uint4(pack_bf16(ph[0], ph[1]), pack_bf16(ph[2], ph[3]),
                                   pack_bf16(ph[4], ph[5]), pack_bf16(ph[6], ph[7]));
    const uint4 pa_mid = make_uint4(pack_bf16(pm[0], pm[1]), pack_bf16(pm[2], pm[3]),
                                    pack_bf16(pm[4], pm[5]), pack_bf16(pm[6], pm[7]));
    const uint4 pa_lo = make_uint4(pack_bf16(pl[0], pl[1]), pack_bf16(pl[2], pl[3]),
                                   pack_bf16(pl[4], pl[5]), pack_bf16(pl[6], pl[7]));
    // O[heads][latent] += P . C over the 32 keys of the tile
#pragma unroll
    for (int jt = 0; jt < kLat / 16; ++jt) {
      const int jrow = 16 * jt + c16;
      const uint2 lo4 = *reinterpret_cast<const uint2*>(&ct[jrow][4 * g]);
      const uint2 hi4 = *reinterpret_cast<const uint2*>(&ct[jrow][16 + 4 * g]);
      const uint4 bop = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa_lo), as_bf16x8(bop), acc[jt], 0, 0, 0);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa_mid), as_bf16x8(bop), acc[jt], 0, 0, 0);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa_hi), as_bf16x8(bop), acc[jt], 0, 0, 0);
    }
  }
  if (!active) return;

  // denominators: lanes of one head (c16) across the 4 key groups
  l_sum += xor16(l_sum);
  l_sum += xor32(l_sum);
  float lr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lr[i] = __shfl(l_sum, 4 * g + i);
  const int64_t rows = static_cast<int64_t>(b) * p.num_heads + h0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = p.part_out + ((rows + 4 * g + i) * p.max_parts + part) * kLat;
    const float inv = 1.0f / lr[i];
#pragma unroll
    for (int jt = 0; jt < kLat / 16; ++jt) dst[16 * jt + c16] = acc[jt][i] * inv;
  }
  if (g == 0) {
    const int64_t idx = (rows + c16) * p.max_parts + part;
    p.part_max[idx] = m_ref * kLn2;
    p.part_sum[idx] = l_sum;
  }
}

// ---- 3. merge of the partitions, then out = W_UV[h] . o_lat on MFMA ------------------
//
// Block h handles all sequences in tiles of 16: o_lat[b][:] is the
// l_j e^(m_j - M)/W -weighted sum of the live partials (ascending j), written
// to LDS as three bf16 terms; then out[b][dv] = sum_j o_lat[b][j] W_UV[h][dv][j] with
// A = o_lat (16 sequences x 32 latent dims per step) and B = W_UV rows, whose
// 8 consecutive latent dims per lane are contiguous in memory.
__global__ __launch_bounds__(kMlaThreads) void mla_merge_uv_kernel(const MlaParams p) {
  __shared__ __align__(16) uint16_t ohi[16][kLat + 8];
  __shared__ __align__(16) uint16_t omid[16][kLat + 8];
  __shared__ __align__(16) uint16_t olo[16][kLat + 8];
  __shared__ float mx[16], wsum[16];
  __shared__ int cnt[16];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  for (int b0 = 0; b0 < p.batch; b0 += 16) {
    const int nb = min(16, p.batch - b0);
    __syncthreads();
    // per sequence: live partitions, max and total weight
    if (tid < 16) {
      const int bb = tid;
      int live = 0;
      float M = -INFINITY, W = 0.0f;
      if (bb < nb) {
        const int nctx = p.context_lens[b0 + bb];
        live = min((nctx + p.partition_size - 1) / p.partition_size, p.max_parts);
        const int64_t row = (static_cast<int64_t>(b0 + bb) * p.num_heads + h) * p.max_parts;
        for (int k = 0; k < live; ++k) M = fmaxf(M, p.part_max[row + k]);
        for (int k = 0; k < live; ++k) W += p.part_sum[row + k] * __expf(p.part_max[row + k] - M);
      }
      cnt[bb] = live;
      mx[bb] = M;
      wsum[bb] = W;
    }
    __syncthreads();
    // o_lat for 16 sequences x 512 dims: thread owns dims (tid % 128) * 4 .. +4 of rows tid / 128 + 2r
    for (int rr = 0; rr < 8; ++rr) {
      const int bb = (tid >> 7) + 2 * rr;
      const int d0 = (tid & 127) * 4;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bb < nb && cnt[bb] > 0 && mx[bb] != -INFINITY) {
        const int64_t row = (static_cast<int64_t>(b0 + bb) * p.num_heads + h) * p.max_parts;
        for (int k = 0; k < cnt[bb]; ++k) {
          const float w = p.part_sum[row + k] * __expf(p.part_max[row + k] - mx[bb]) / wsum[bb];
          const float4 v = *reinterpret_cast<const float4*>(p.part_out + (row + k) * kLat + d0);
          o.x = fmaf(w, v.x, o.x);
          o.y = fmaf(w, v.y, o.y);
          o.z = fmaf(w, v.z, o.z);
          o.w = fmaf(w, v.w, o.w);
        }
      }
      uint16_t h4[4], m4[4], l4[4];
      split3_bf16(o.x, h4[0], m4[0], l4[0]);
      split3_bf16(o.y, h4[1], m4[1], l4[1]);
      split3_bf16(o.z, h4[2], m4[2], l4[2]);
      split3_bf16(o.w, h4[3], m4[3], l4[3]);
      *reinterpret_cast<uint2*>(&ohi[bb][d0]) = make_uint2(pack_bf16(h4[0], h4[1]), pack_bf16(h4[2], h4[3]));
      *reinterpret_cast<uint2*>(&omid[bb][d0]) = make_uint2(pack_bf16(m4[0], m4[1]), pack_bf16(m4[2], m4[3]));
      *reinterpret_cast<uint2*>(&olo[bb][d0]) = make_uint2(pack_bf16(l4[0], l4[1]), pack_bf16(l4[2], l4[3]));
    }
    __syncthreads();
    // out[b][dv]: wave w takes dv tiles 2w, 2w+1
    const uint16_t* wuv = p.w_uv + static_cast<int64_t>(h) * kDv * kLat;
#pragma unroll
    for (int nt2 = 0; nt2 < 2; ++nt2) {
      const int nt = 2 * wave + nt2;
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ks = 0; ks < kLat / 32; ++ks) {
        const uint4 a_hi = *reinterpret_cast<const uint4*>(&ohi[c16][32 * ks + 8 * g]);
        const uint4 a_mid = *reinterpret_cast<const uint4*>(&omid[c16][32 * ks + 8 * g]);
        const uint4 a_lo = *reinterpret_cast<const uint4*>(&olo[c16][32 * ks + 8 * g]);
        const uint4 bw = load16(wuv + static_cast<int64_t>(16 * nt + c16) * kLat + 32 * ks + 8 * g);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_lo), as_bf16x8(bw), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_mid), as_bf16x8(bw), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_hi), as_bf16x8(bw), c, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bb = 4 * g + i;
        if (bb < nb)
          p.out[(static_cast<int64_t>(b0 + bb) * p.num_heads + h) * kDv + 16 * nt + c16] =
              f32_to_bf16_rne(c[i]);
      }
    }
  }
}

}  // namespace pa

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
    return pa::fail(PA_ERR_WORKSPACE, "workspace must hold mla_absorbed_decode_workspace_size() = " +
                                          std::to_string(plan.bytes) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return pa::fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  pa::MlaParams p{};
  p.q_nope = static_cast<const uint16_t*>(q_nope);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.cache = static_cast<const uint16_t*>(kv_cache);
  p.w_uk = static_cast<const uint16_t*>(w_uk);
  p.w_uv = static_cast<const uint16_t*>(w_uv);
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.q_hi = reinterpret_cast<uint16_t*>(ws + plan.off_qhi);
  p.q_mid = reinterpret_cast<uint16_t*>(ws + plan.off_qmid);
  p.q_lo = reinterpret_cast<uint16_t*>(ws + plan.off_qlo);
  p.part_out = reinterpret_cast<float*>(ws + plan.off_out);
  p.part_max = reinterpret_cast<float*>(ws + plan.off_max);
  p.part_sum = reinterpret_cast<float*>(ws + plan.off_sum);
  p.out = static_cast<uint16_t*>(out);
  p.page_stride = cache->page_stride;
  p.token_stride = static_cast<int32_t>(cache->token_stride);
  p.bt_stride = block_table_stride;
  p.batch = batch;
  p.num_heads = num_heads;
  p.page_size = cache->page_size;
  int shift = 0;
  while ((1 << shift) < cache->page_size) ++shift;
  p.page_shift = shift;
  p.partition_size = plan.partition_size;
  p.max_parts = plan.max_partitions;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::clear_error();
  hipLaunchKernelGGL(pa::mla_absorb_kernel, dim3(num_heads, pa::kMlaLat / 128), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("absorb: ") + hipGetErrorString(e));
  const int head_groups = (num_heads + 63) / 64;
  hipLaunchKernelGGL(pa::mla_split_kernel, dim3(plan.max_partitions, head_groups, batch),
                     dim3(pa::kMlaThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("split: ") + hipGetErrorString(e));
  hipLaunchKernelGGL(pa::mla_merge_uv_kernel, dim3(num_heads), dim3(pa::kMlaThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("merge: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
