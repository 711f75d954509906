// pa_gqa.hip -- GQA paged decode for gfx950: split-KV partial kernel and
// log-sum-exp merge kernel.
//
// Work item = (sequence b, KV head g, key partition j), one 256-thread block
// (4 waves).  All G = Hq/Hkv query heads of the group are computed in the
// same pass, so every K/V row of KV head g is read from HBM once per call
// [vllm.cpp PR #49, commit body: grid over batch x KV heads instead of batch x
// q heads; vllm.cpp kernel matrix, row KERNEL-ATTN-FA2: a split axis across
// the context fills the machine when batch x heads alone does not].
//
// Lane layout (wave64): a K or V row of D bf16 is read as D/8 lanes x 16
// bytes, so one wave load instruction covers 64*16 B = 1 KB = 64/(D/8)
// consecutive keys of a contiguous (page, head) tile.  A wave walks aligned
// chunks of NI such loads (NI*64/(D/8) keys), the four waves of the block
// taking every fourth chunk of the partition.
//
// Per chunk:  q.k partial dots with v_dot2_f32_bf16 (bf16 products exact,
// fp32 sums), summed over the D/8 lanes of a row with DPP; online softmax in
// the log2 domain (scale*log2(e) folded into the score); P stays fp32 and
// multiplies V widened to fp32.  Each group of D/8 lanes that shares a key
// slot keeps its own running (max, sum, accumulator); the groups and the four
// waves are merged once at the end, in a fixed order.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_params.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;

// Loads per lane per chunk: fewer for wide groups to bound registers.
template <int G>
constexpr int chunk_loads() { return G <= 4 ? 8 : (G == 8 ? 4 : 2); }

template <int D, int G>
__global__ __launch_bounds__(kBlock) void split_kernel(const SplitParams p) {
  constexpr int LPT = D / 8;         // lanes per key row
  constexpr int TPI = 64 / LPT;      // keys per wave load
  constexpr int NI = chunk_loads<G>();
  constexpr int CH = TPI * NI;       // keys per chunk

  __shared__ float red_acc[kWaves][G][D];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];

  const int j = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPT;          // key slot within a wave load
  const int e0 = (lane % LPT) * 8;   // first of this lane's 8 dims

  const int n = p.context_lens[b];
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int64_t begin64 = static_cast<int64_t>(lo) + static_cast<int64_t>(j) * p.partition_size;
  const int64_t rowbase = (static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(g) * G) *
                          p.max_parts + j;   // index of (b, h = g*G, j)

  if (begin64 >= n) {
    if (p.write_empty) {
      for (int i = threadIdx.x; i < G * D; i += kBlock) {
        const int h = i / D;
        p.part_out[(rowbase + static_cast<int64_t>(h) * p.max_parts) * D + (i % D)] = 0.0f;
      }
      if (threadIdx.x < G) {
        p.part_max[rowbase + static_cast<int64_t>(threadIdx.x) * p.max_parts] = -INFINITY;
        p.part_sum[rowbase + static_cast<int64_t>(threadIdx.x) * p.max_parts] = 0.0f;
      }
    }
    return;
  }
  const int begin = static_cast<int>(begin64);
  const int end = static_cast<int>(min(begin64 + p.partition_size, static_cast<int64_t>(n)));

  // q rows of the group: 8 bf16 per lane per head.
  uint4 qv[G];
  {
    const uint16_t* qb = p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * G) * D + e0;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = load16(qb + h * D);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  const uint16_t* kbase = p.k + static_cast<int64_t>(g) * p.head_stride;
  const uint16_t* vbase = p.v + static_cast<int64_t>(g) * p.head_stride;
  const int c_first = begin / CH;
  const int c_last = (end - 1) / CH;

  for (int c = c_first + wave; c <= c_last; c += kWaves) {
    const int tchunk = c * CH;
    uint4 kr[NI], vr[NI];
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t0 = tchunk + i * TPI;               // first key of this load (wave-uniform)
      const int t = t0 + r;
      valid[i] = (t >= begin) && (t < end);
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (t0 + TPI > begin && t0 < end) {            // some key of this load is live
        const int page = bt[t0 >> p.page_shift];     // page_size % TPI == 0: one page per load
        const int64_t pbase = static_cast<int64_t>(page) * p.page_stride;
        const int off = (t & (p.page_size - 1)) * p.token_stride + e0;
        if (valid[i]) {
          kr[i] = load16(kbase + pbase + off);
          vr[i] = load16(vbase + pbase + off);
        }
      }
    }

    // scores s[i][h] (log2 domain), replicated over the LPT lanes of a key
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = dot2_bf16(kr[i].x, qv[h].x, 0.0f);
        a = dot2_bf16(kr[i].y, qv[h].y, a);
        a = dot2_bf16(kr[i].z, qv[h].z, a);
        a = dot2_bf16(kr[i].w, qv[h].w, a);
        a = row_sum16(a);
        if constexpr (LPT == 32) a += xor16(a);
        s[i][h] = valid[i] ? a * p.scale_log2 : -INFINITY;
      }
    }

    // online softmax update, then P.V
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) cm = fmaxf(cm, s[i][h]);
      const float mn = fmaxf(m[h], cm);
      const float base = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = fast_exp2(m[h] - base);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        s[i][h] = fast_exp2(s[i][h] - base);
        l[h] += s[i][h];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[8];
      vf[0] = bf16_lo(vr[i].x); vf[1] = bf16_hi(vr[i].x);
      vf[2] = bf16_lo(vr[i].y); vf[3] = bf16_hi(vr[i].y);
      vf[4] = bf16_lo(vr[i].z); vf[5] = bf16_hi(vr[i].z);
      vf[6] = bf16_lo(vr[i].w); vf[7] = bf16_hi(vr[i].w);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(s[i][h], vf[e], acc[h][e]);
      }
    }
  }

  // Merge the TPI key-slot groups of this wave (lanes r*LPT + e), fixed order.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
    if constexpr (TPI == 4) M = fmaxf(M, xor16(M));
    M = fmaxf(M, xor32(M));
    const float sc = (M == -INFINITY) ? 0.0f : fast_exp2(m[h] - M);
    float lw = l[h] * sc;
    if constexpr (TPI == 4) lw += xor16(lw);
    lw += xor32(lw);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc[h][e] * sc;
      if constexpr (TPI == 4) a += xor16(a);
      a += xor32(a);
      acc[h][e] = a;
    }
    m[h] = M;
    l[h] = lw;
  }
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_acc[wave][h][e0 + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[wave][h] = m[h];
      red_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // Merge the four waves and write the normalised partial, fp32.
  for (int i = threadIdx.x; i < G * D; i += kBlock) {
    const int h = i / D;
    const int d = i % D;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
    float W = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = (red_m[w][h] == -INFINITY) ? 0.0f : fast_exp2(red_m[w][h] - M);
      W += red_l[w][h] * sc;
      o += red_acc[w][h][d] * sc;
    }
    const int64_t row = rowbase + static_cast<int64_t>(h) * p.max_parts;
    p.part_out[row * D + d] = o / W;
    if (d == 0) {
      p.part_max[row] = M * kLn2;
      p.part_sum[row] = W;
    }
  }
}

// One block per (q head, sequence): M = max m_j, W = sum l_j e^(m_j - M),
// out = sum_j (l_j e^(m_j - M) / W) o_j over live partitions, ascending j
// within each of the block's partition groups, groups added in fixed order.
template <int D>
__global__ __launch_bounds__(kBlock) void merge_kernel(const MergeParams p) {
  constexpr int TPR = D / 4;                  // threads per row (float4 each)
  constexpr int NGRP = kBlock / TPR;          // partition groups per block
  __shared__ float red[kBlock];
  __shared__ float4 part[NGRP][TPR];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int n = p.context_lens[b];
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int live = (n > lo) ? static_cast<int>((static_cast<int64_t>(n - lo) + p.partition_size - 1) /
                                               p.partition_size)
                            : 0;
  const int64_t row = static_cast<int64_t>(b) * p.num_q_heads + h;
  const float* pm = p.part_max + row * p.max_parts;
  const float* pl = p.part_sum + row * p.max_parts;
  const float* po = p.part_out + row * p.max_parts * D;

  // M over live partitions
  float M = -INFINITY;
  for (int jj = threadIdx.x; jj < live; jj += kBlock) M = fmaxf(M, pm[jj]);
  M = wave_max(M);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  uint16_t* out = p.out + row * D;
  if (live == 0 || M == -INFINITY) {
    for (int d = threadIdx.x; d < D; d += kBlock) out[d] = 0;
    if (p.lse && threadIdx.x == 0) p.lse[row] = -INFINITY;
    return;
  }
  float W = 0.0f;
  for (int jj = threadIdx.x; jj < live; jj += kBlock) {
    const float mj = pm[jj];
    const float lj = pl[jj];
    if (mj != -INFINITY && lj != 0.0f) W += lj * __expf(mj - M);
  }
  W = wave_sum(W);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = W;
  __syncthreads();
  W = (red[0] + red[1]) + (red[2] + red[3]);

  const int grp = threadIdx.x / TPR;
  const int d4 = threadIdx.x % TPR;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int jj = grp; jj < live; jj += NGRP) {
    const float mj = pm[jj];
    const float lj = pl[jj];
    if (mj == -INFINITY || lj == 0.0f) continue;
    const float w = lj * __expf(mj - M) / W;
    const float4 o = reinterpret_cast<const float4*>(po + static_cast<int64_t>(jj) * D)[d4];
    a.x = fmaf(w, o.x, a.x);
    a.y = fmaf(w, o.y, a.y);
    a.z = fmaf(w, o.z, a.z);
    a.w = fmaf(w, o.w, a.w);
  }
  part[grp][d4] = a;
  __syncthreads();
  if (grp == 0) {
    float4 t = part[0][d4];
#pragma unroll
    for (int q = 1; q < NGRP; ++q) {
      const float4 u = part[q][d4];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    uint2 packed;
    packed.x = static_cast<uint32_t>(f32_to_bf16_rne(t.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(t.y)) << 16);
    packed.y = static_cast<uint32_t>(f32_to_bf16_rne(t.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(t.w)) << 16);
    reinterpret_cast<uint2*>(out)[d4] = packed;
  }
  if (p.lse && threadIdx.x == 0) p.lse[row] = M + __logf(W);
}

// ---- launchers -----------------------------------------------------------------

template <int D, int G>
static hipError_t launch_split_dg(const SplitParams& p, int batch, int num_kv_heads,
                                  hipStream_t stream) {
  dim3 grid(p.max_parts, num_kv_heads, batch);
  hipLaunchKernelGGL((split_kernel<D, G>), grid, dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_split_d(const SplitParams& p, int group, int batch, int num_kv_heads,
                                 hipStream_t stream) {
  switch (group) {
    case 1: return launch_split_dg<D, 1>(p, batch, num_kv_heads, stream);
    case 2: return launch_split_dg<D, 2>(p, batch, num_kv_heads, stream);
    case 4: return launch_split_dg<D, 4>(p, batch, num_kv_heads, stream);
    case 8: return launch_split_dg<D, 8>(p, batch, num_kv_heads, stream);
    case 16:
      if constexpr (D == 128) return launch_split_dg<D, 16>(p, batch, num_kv_heads, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split(const SplitParams& p, int head_dim, int group, int batch,
                        int num_kv_heads, hipStream_t stream) {
  if (head_dim == 128) return launch_split_d<128>(p, group, batch, num_kv_heads, stream);
  if (head_dim == 256) return launch_split_d<256>(p, group, batch, num_kv_heads, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, int batch, hipStream_t stream) {
  dim3 grid(p.num_q_heads, batch);
  if (head_dim == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kBlock), 0, stream, p);
  } else if (head_dim == 256) {
    hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(kBlock), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
