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

// ---- lane-level exchange helpers (partner = lane ^ W) ---------------------------

template <int W>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (W == 1) return dpp<0xB1>(x);       // quad_perm [1,0,3,2]
  else if constexpr (W == 2) return dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  else if constexpr (W == 4)
    return u2f(static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(f2u(x)), 0x101f)));
  else if constexpr (W == 8) return dpp<kRowRor8>(x);   // i -> i+8 mod 16 == i ^ 8
  else if constexpr (W == 16) return xor16(x);
  else return xor32(x);
}

// Sum (kMax = false) or max over the lanes that differ in bits [lo, hi) of
// the lane id; every such lane gets the result.
template <int LO, int HI, bool kMax>
__device__ __forceinline__ float reduce_bits(float x) {
  if constexpr (LO < HI) {
    const float y = xor_lane<(1 << LO)>(x);
    x = kMax ? fmaxf(x, y) : x + y;
    return reduce_bits<LO + 1, HI, kMax>(x);
  } else {
    return x;
  }
}

constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }

// Compile-time geometry of the split kernel for head_dim D and group G.
//
// Score layout: LQ lanes share one key row, each holding D/LQ of its dims
// (NQL 16-byte pieces); a pass covers TQ = 64/LQ keys.  The LQ partial dot
// products of every head are combined by a reduce-scatter: at step s lanes
// j and j ^ (LQ >> (s+1)) trade halves of their remaining head slots, and the
// q rows are pre-permuted per lane (slot h of lane j holds head h ^ pi(j)) so
// each step is one uniform "own[k] + partner[k + half]".  After NSCAT steps a
// lane owns VH heads (slot k = head k ^ pi(j)); leftover steps, when G < LQ,
// are plain sums.
//
// Value layout: LV = D/8 lanes per key row, 8 dims each, TV = 64/LV keys per
// load; the accumulator of a lane holds its 8 dims for all G heads.
template <int D, int G>
struct Geo {
  static constexpr int LQ = (G * D / 128) > 4 ? G * D / 128 : 4;
  static constexpr int LOG_LQ = ilog2c(LQ);
  static constexpr int NQL = D / (8 * LQ);
  static constexpr int TQ = 64 / LQ;
  static constexpr int LV = D / 8;
  static constexpr int TV = 64 / LV;
  static constexpr int CH = (G >= 16) ? 16 : (D == 128 ? 32 : 16);   // keys per chunk
  static constexpr int NTQ = CH / TQ;
  static constexpr int NV = CH / TV;
  static constexpr int LOG_G = ilog2c(G);
  static constexpr int NSCAT = LOG_G < LOG_LQ ? LOG_G : LOG_LQ;
  static constexpr int VH = G >> NSCAT;
  static_assert(NTQ >= 1 && NV >= 1 && NQL >= 1, "geometry");
};

// pi(j): which head sits in slot 0 of lane j (within its LQ-lane key group).
template <int D, int G>
__device__ __forceinline__ int head_perm(int j) {
  using g = Geo<D, G>;
  int pi = 0;
#pragma unroll
  for (int s = 0; s < g::NSCAT; ++s) pi |= ((j >> (g::LOG_LQ - 1 - s)) & 1) * (G >> (s + 1));
  return pi;
}

// Reduce-scatter of v[0..G) over the LQ lanes of a key group; returns with
// v[0..VH) holding complete sums for heads k ^ pi(j).
template <int D, int G, int S>
__device__ __forceinline__ void scatter_step(float (&v)[G]) {
  using g = Geo<D, G>;
  if constexpr (S < g::NSCAT) {
    constexpr int W = g::LQ >> (S + 1);
    constexpr int HALF = G >> (S + 1);
#pragma unroll
    for (int k = 0; k < HALF; ++k) v[k] += xor_lane<W>(v[k + HALF]);
    scatter_step<D, G, S + 1>(v);
  } else if constexpr (S < g::LOG_LQ) {
    constexpr int W = g::LQ >> (S + 1);
    v[0] += xor_lane<W>(v[0]);
    scatter_step<D, G, S + 1>(v);
  }
}

// Page table of one wave: the partition [begin, end) is cut into aligned
// chunks of CH keys and wave w takes chunks c0 = first + w, c0 + 4, ...  The
// physical page of every page those chunks touch sits in one lane of `ptab`
// (lane = chunk-in-group << ppc_shift | page-in-chunk), loaded from the block
// table once per group of 64 >> ppc_shift chunks and read back with
// v_readlane, so no K/V load waits on a block-table read.
struct WaveKeys {
  const int32_t* bt;
  int begin, end;
  int c0, nk;
  int ppc_shift;
  int ptab;
  int group;
};

template <int CH>
__device__ __forceinline__ void load_page_table(WaveKeys& wk, int grp, int lane, int page_shift) {
  const int per_group = 64 >> wk.ppc_shift;
  const int k = grp * per_group + (lane >> wk.ppc_shift);
  const int sub = lane & ((1 << wk.ppc_shift) - 1);
  const int c = wk.c0 + k * kWaves;
  const int pi = ((c * CH) >> page_shift) + sub;
  const bool live = k < wk.nk && pi >= (wk.begin >> page_shift) && pi <= ((wk.end - 1) >> page_shift);
  wk.ptab = live ? wk.bt[pi] : 0;
  wk.group = grp;
}

// Make sure `ptab` covers chunk k of the wave (reloads once per group).
template <int CH>
__device__ __forceinline__ void ensure_pages(WaveKeys& wk, int k, int lane, int page_shift) {
  const int grp = k >> (6 - wk.ppc_shift);
  if (grp != wk.group) load_page_table<CH>(wk, grp, lane, page_shift);
}

// Physical page of key t of the wave's k-th chunk (table already loaded).
template <int CH>
__device__ __forceinline__ int page_of(const WaveKeys& wk, int k, int t, int page_shift) {
  const int kk = k & ((64 >> wk.ppc_shift) - 1);
  const int tchunk = (wk.c0 + k * kWaves) * CH;
  const int slot = (kk << wk.ppc_shift) + ((t >> page_shift) - (tchunk >> page_shift));
  return __builtin_amdgcn_readlane(wk.ptab, slot);
}

// Buffer descriptor over one (page, KV head) tile; reads at offsets past
// `tile_bytes` return zeros, which is how dead keys are masked without
// branching or touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int page,
                                                            uint32_t page_bytes, int tile_bytes) {
  const char* tile = reinterpret_cast<const char*>(base) +
                     static_cast<uint64_t>(static_cast<uint32_t>(page)) * page_bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), static_cast<short>(0),
                                           tile_bytes, 0x00020000);
}

constexpr int kDeadBit = 0x40000000;   // OR-ed into a dead key's offset: past any tile

__device__ __forceinline__ uint4 tile_load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 1 when key t lies outside [begin, end), as the dead-offset bit.
__device__ __forceinline__ int dead_bit(int t, int begin, int end) {
  return (static_cast<uint32_t>(t - begin) >= static_cast<uint32_t>(end - begin)) ? kDeadBit : 0;
}

template <int D, int G>
struct KRegs {
  uint4 v[Geo<D, G>::NTQ][Geo<D, G>::NQL];
};
template <int D, int G>
struct VRegs {
  uint4 v[Geo<D, G>::NV];
};

// K pieces of chunk k in the score layout; dead keys hold 0.  `koff` is this
// lane's byte offset inside a tile for slot 0 (slot row r plus its dims); the
// slot of the first key of a pass is added through the scalar offset.
template <int D, int G>
__device__ __forceinline__ void load_k(KRegs<D, G>& kr, const WaveKeys& wk, int k, int lane,
                                       const uint16_t* kbase, const SplitParams& p, int koff) {
  using g = Geo<D, G>;
  const int tchunk = (wk.c0 + k * kWaves) * g::CH;
  const int r = lane / g::LQ;
#pragma unroll
  for (int u = 0; u < g::NTQ; ++u) {
    const int t0 = tchunk + u * g::TQ;                 // keys t0 .. t0+TQ-1 share one page
    const int page = page_of<g::CH>(wk, k, t0, p.page_shift);
    const auto rs = tile_rsrc(kbase, page, p.page_bytes, p.tile_bytes);
    const int soff = (t0 & (p.page_size - 1)) * p.token_bytes;
    const int voff = koff | dead_bit(t0 + r, wk.begin, wk.end);
#pragma unroll
    for (int s = 0; s < g::NQL; ++s) kr.v[u][s] = tile_load(rs, voff + s * 16 * g::LQ, soff);
  }
}

// V rows of chunk k in the value layout; dead keys hold 0.
template <int D, int G>
__device__ __forceinline__ void load_v(VRegs<D, G>& vr, const WaveKeys& wk, int k, int lane,
                                       const uint16_t* vbase, const SplitParams& p, int voff0) {
  using g = Geo<D, G>;
  const int tchunk = (wk.c0 + k * kWaves) * g::CH;
  const int r = lane / g::LV;
#pragma unroll
  for (int i = 0; i < g::NV; ++i) {
    const int t0 = tchunk + i * g::TV;
    const int page = page_of<g::CH>(wk, k, t0, p.page_shift);
    const auto rs = tile_rsrc(vbase, page, p.page_bytes, p.tile_bytes);
    const int soff = (t0 & (p.page_size - 1)) * p.token_bytes;
    vr.v[i] = tile_load(rs, voff0 | dead_bit(t0 + r, wk.begin, wk.end), soff);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kBlock) void split_kernel(const SplitParams p) {
  using g = Geo<D, G>;
  constexpr int CH = g::CH;

  __shared__ float red_acc[kWaves][G][D];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ float p_lds[kWaves][CH][G];     // probabilities, key-major
  __shared__ float a_lds[kWaves][G];         // per-head rescale factor of the chunk

  const int j = blockIdx.x;
  const int gk = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int n = p.context_lens[b];
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int64_t begin64 = static_cast<int64_t>(lo) + static_cast<int64_t>(j) * p.partition_size;
  const int64_t rowbase = (static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * G) *
                          p.max_parts + j;   // index of (b, h = gk*G, j)

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

  WaveKeys wk;
  wk.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  wk.begin = static_cast<int>(begin64);
  wk.end = static_cast<int>(min(begin64 + p.partition_size, static_cast<int64_t>(n)));
  const int c_first = wk.begin / CH;
  const int c_last = (wk.end - 1) / CH;
  wk.c0 = c_first + wave;
  wk.nk = (wk.c0 <= c_last) ? (c_last - wk.c0) / kWaves + 1 : 0;
  wk.ppc_shift = (CH > p.page_size) ? (ilog2c(CH) - p.page_shift) : 0;
  wk.ptab = 0;
  wk.group = -1;

  const uint16_t* kbase = p.k + static_cast<int64_t>(gk) * p.head_stride;
  const uint16_t* vbase = p.v + static_cast<int64_t>(gk) * p.head_stride;

  const int jq = lane % g::LQ;               // lane within its key group (score layout)
  const int pi = head_perm<D, G>(jq);
  // this lane writes p for its heads if it is the first copy among the
  // lanes that a trailing plain-sum step left holding the same values
  const bool p_writer = (jq & ((g::LQ >> g::NSCAT) - 1)) == 0;

  // per-lane byte offsets inside a tile (slot row + dims); keys of one
  // pass are consecutive slots of one page, so the pass adds a scalar
  const int koff = (lane / g::LQ) * p.token_bytes + 16 * (lane % g::LQ);
  const int voff0 = (lane / g::LV) * p.token_bytes + 16 * (lane % g::LV);

  KRegs<D, G> kr;
  VRegs<D, G> vr;
  if (wk.nk > 0) {
    ensure_pages<CH>(wk, 0, lane, p.page_shift);
    load_k<D, G>(kr, wk, 0, lane, kbase, p, koff);
    load_v<D, G>(vr, wk, 0, lane, vbase, p, voff0);
  }

  // q pieces, pre-permuted per lane: slot h holds head h ^ pi.
  uint4 qv[G][g::NQL];
  {
    const uint16_t* qb = p.q + (static_cast<int64_t>(b) * p.num_q_heads + gk * G) * D + 8 * jq;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int s = 0; s < g::NQL; ++s) qv[h][s] = load16(qb + (h ^ pi) * D + s * 8 * g::LQ);
  }

  float m_own[g::VH], l_own[g::VH];
#pragma unroll
  for (int v = 0; v < g::VH; ++v) {
    m_own[v] = -INFINITY;
    l_own[v] = 0.0f;
  }
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

  const int rq = lane / g::LQ;
  for (int k = 0; k < wk.nk; ++k) {
    const int tchunk = (wk.c0 + k * kWaves) * CH;

    // scores of this lane's keys, then reduce-scatter over the key group
    float s_own[g::NTQ][g::VH];
#pragma unroll
    for (int u = 0; u < g::NTQ; ++u) {
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int s = 0; s < g::NQL; ++s) {
          a = dot2_bf16(kr.v[u][s].x, qv[h][s].x, a);
          a = dot2_bf16(kr.v[u][s].y, qv[h][s].y, a);
          a = dot2_bf16(kr.v[u][s].z, qv[h][s].z, a);
          a = dot2_bf16(kr.v[u][s].w, qv[h][s].w, a);
        }
        v[h] = a;
      }
      scatter_step<D, G, 0>(v);
      const int t = tchunk + u * g::TQ + rq;
      const bool live = t >= wk.begin && t < wk.end;
#pragma unroll
      for (int vh = 0; vh < g::VH; ++vh) s_own[u][vh] = live ? v[vh] * p.scale_log2 : -INFINITY;
    }

    // K registers are free: start streaming the next chunk's K now (the
    // scheduling barriers keep the compiler from hoisting these loads above
    // the last reads of the registers they overwrite)
    __builtin_amdgcn_sched_barrier(0);
    if (k + 1 < wk.nk) {
      ensure_pages<CH>(wk, k + 1, lane, p.page_shift);
      load_k<D, G>(kr, wk, k + 1, lane, kbase, p, koff);
    }

    // online softmax for the heads this lane owns; the running max of a head
    // is the same on every lane that owns it (max over all keys of the chunk)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int vh = 0; vh < g::VH; ++vh) {
      float cm = s_own[0][vh];
#pragma unroll
      for (int u = 1; u < g::NTQ; ++u) cm = fmaxf(cm, s_own[u][vh]);
      cm = reduce_bits<g::LOG_LQ, 6, true>(cm);
      const float mn = fmaxf(m_own[vh], cm);
      const float base = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = fast_exp2(m_own[vh] - base);
      m_own[vh] = mn;
      float ls = 0.0f;
      const int h = vh ^ pi;
#pragma unroll
      for (int u = 0; u < g::NTQ; ++u) {
        const float pr = fast_exp2(s_own[u][vh] - base);
        ls += pr;
        if (p_writer) p_lds[wave][u * g::TQ + rq][h] = pr;
      }
      l_own[vh] = l_own[vh] * alpha + ls;
      if (p_writer && rq == 0) a_lds[wave][h] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // rescale the accumulators, then P.V in the value layout
    {
      float al[G];
#pragma unroll
      for (int h = 0; h < G; ++h) al[h] = a_lds[wave][h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
    }
    const int rv = lane / g::LV;
#pragma unroll
    for (int i = 0; i < g::NV; ++i) {
      float pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = p_lds[wave][i * g::TV + rv][h];
      float vf[8];
      vf[0] = bf16_lo(vr.v[i].x); vf[1] = bf16_hi(vr.v[i].x);
      vf[2] = bf16_lo(vr.v[i].y); vf[3] = bf16_hi(vr.v[i].y);
      vf[4] = bf16_lo(vr.v[i].z); vf[5] = bf16_hi(vr.v[i].z);
      vf[6] = bf16_lo(vr.v[i].w); vf[7] = bf16_hi(vr.v[i].w);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    __builtin_amdgcn_sched_barrier(0);
    if (k + 1 < wk.nk) load_v<D, G>(vr, wk, k + 1, lane, vbase, p, voff0);
  }

  // Wave totals: l over the key groups that own the same head, the
  // accumulators over the key slots of the value layout.  All lanes of a
  // head share one running max, so no rescaling is needed here.
#pragma unroll
  for (int vh = 0; vh < g::VH; ++vh) l_own[vh] = reduce_bits<g::LOG_LQ, 6, false>(l_own[vh]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = reduce_bits<ilog2c(g::LV), 6, false>(acc[h][e]);
  if (lane < g::LV) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_acc[wave][h][lane * 8 + e] = acc[h][e];
  }
  if (lane < g::LQ && p_writer) {
#pragma unroll
    for (int vh = 0; vh < g::VH; ++vh) {
      red_m[wave][vh ^ pi] = m_own[vh];
      red_l[wave][vh ^ pi] = l_own[vh];
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
