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
// Two attention routines over a key range, both reading every K/V row with
// 16-byte lane loads of contiguous (page, head) tiles:
//
// attend_range_mfma (groups of 4-16 heads, head_dim 64 and 512, FP8 and f32
// pools): per 16-key chunk, S^T[16 keys x 16 heads] = K.Q^T and O += P.V on
// the matrix cores.  bf16 products are exact and sums fp32; P (and f32 pool
// elements) enter as three exact bf16 terms.  The softmax keeps a lazy
// per-head reference max in the log2 domain.  Waves take every fourth chunk
// and are merged once at the end; at head_dim 512 they split the dims of
// each chunk instead.
//
// attend_range_valu (groups of 1 and 2 heads): a K or V row of D bf16 is
// read as D/8 lanes x 16 bytes, one wave load covering 1 KB of consecutive
// keys; q.k partial dots with v_dot2_f32_bf16, summed over the D/8 lanes of
// a row with DPP; P stays fp32 and multiplies V widened to fp32.  Each group
// of D/8 lanes that shares a key slot keeps its own running (max, sum,
// accumulator); the groups and the waves are merged once at the end, in a
// fixed order.
#include <hip/hip_runtime.h>

#include <atomic>

#include "pa_device.h"
#include "pa_mfma.h"
#include "pa_params.h"
#include "pa_profile.h"
#include "pa_validate.h"

namespace pa {

constexpr int kWaves = 4;               // waves of a fixed-partition block
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
  // keys per chunk: 8 for D = 256 with G >= 8, which keeps the K/V buffers
  // small enough for two waves per SIMD
  static constexpr int CH = (D == 256 && G >= 8) ? 8 : (G >= 16) ? 16 : (D == 128 ? 32 : 16);
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
  int step;        // waves sharing the range: chunk k of this wave is c0 + k*step
  int ppc_shift;
  int ptab;
  int group;
};

template <int CH>
__device__ __forceinline__ void load_page_table(WaveKeys& wk, int grp, int lane, int page_shift) {
  const int per_group = 64 >> wk.ppc_shift;
  const int k = grp * per_group + (lane >> wk.ppc_shift);
  const int sub = lane & ((1 << wk.ppc_shift) - 1);
  const int c = wk.c0 + k * wk.step;
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
  const int tchunk = (wk.c0 + k * wk.step) * CH;
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

// K/V rows are read exactly once per call: non-temporal loads (cache policy
// nt) stream them past the caches, which raises the sustained read rate of
// gfx950 from about 6.0 to 6.7 TB/s in a 2 GiB read of random 8 KB tiles.
constexpr int kStreamPolicy = 2;   // nt

__device__ __forceinline__ uint4 tile_load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy));
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
  const int tchunk = (wk.c0 + k * wk.step) * g::CH;
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
  const int tchunk = (wk.c0 + k * wk.step) * g::CH;
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

// Virtual head h of a KV group is query h / gq, q head h % gq; its q and out
// rows sit head_offset(h) rows after the group's first row.  With one query,
// head_offset(h) = h.  Padding heads (h >= vheads) alias head 0 for their q
// loads and write no output.
__device__ __forceinline__ int64_t head_offset(const SplitParams& p, int h) {
  const int hh = h < p.vheads ? h : 0;
  const int s = hh / p.gq;
  return static_cast<int64_t>(s) * p.q_heads + (hh - s * p.gq);
}

// Keys [lo, hi) that head h of sequence b may see, within [begin, end): query
// s of a multi-query row sees up to n - S + s when causal, and a window
// counts back from its last key.  With one query this is [begin, end) itself.
__device__ __forceinline__ void head_bounds(const SplitParams& p, int n, int h, int begin, int end,
                                            int& lo_h, int& hi_h) {
  const int sq = (h < p.vheads ? h : 0) / p.gq;
  const int hi = p.causal ? min(n, n - p.num_queries + 1 + sq) : n;
  const int lo = p.window > 0 ? max(0, hi - p.window) : 0;
  lo_h = max(lo, begin);
  hi_h = min(hi, end);
}

// Merge of the NW waves' states of one range and the write of its result.
// Wave w left, per head h < G, the reference max red_m[w][h] (log2 domain, -inf
// if it saw no key) its sum red_l[w][h] and unnormalised accumulator
// red_acc[(w*G + h)*D + d] are relative to, and the largest score it saw,
// red_mt[w][h] (>= red_m[w][h]; the same array when the reference is the
// running max).  Results are expressed relative to the largest score of the
// range, so the partial's max is that score.  Writes the fp32 partial
// of head h to out + h*hstride*D, mx[h*hstride] (natural-log max) and
// sm[h*hstride] (sum) -- or, when `final_out` is set (the range is the row's
// only one), the bf16 output of head h to final_out + head_offset(h)*D and
// its log-sum-exp to final_lse[head_offset(h)].  A head that saw no key
// (possible only for the early queries of a multi-query row) gets o = 0, max
// -inf, sum 0.
//
// With NSL > 1 the waves split the dims instead of the keys (wave w holds dims
// w*D/NSL .. +D/NSL of every head): they share one state, red_*[0][h], and
// red_acc is slice-major, [w][h][D/NSL].
template <int D, int G, int NW, int NSL = 1>
__device__ __forceinline__ void write_range(const SplitParams& p, const float* red_acc,
                                            const float (*red_m)[G], const float (*red_mt)[G],
                                            const float (*red_l)[G], float* out, float* mx,
                                            float* sm, int64_t hstride, uint16_t* final_out,
                                            float* final_lse) {
  constexpr int D4 = D / 4;        // a thread takes 4 consecutive dims of one head
  constexpr int NS = NSL > 1 ? 1 : NW;   // wave states to merge
  constexpr int DW = D / NSL;            // dims of one slice
  for (int i = threadIdx.x; i < G * D4; i += 64 * NW) {
    const int h = i / D4;
    const int d = (i % D4) * 4;
    if (h >= p.vheads) continue;     // padding head
    float M = red_mt[0][h];
#pragma unroll
    for (int w = 1; w < NS; ++w) M = fmaxf(M, red_mt[w][h]);
    float W = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NS; ++w) {
      const float sc = (red_m[w][h] == -INFINITY) ? 0.0f : fast_exp2(red_m[w][h] - M);
      W += red_l[w][h] * sc;
      const float4 a =
          *reinterpret_cast<const float4*>(&red_acc[((w + d / DW) * G + h) * DW + d % DW]);
      o.x += a.x * sc;
      o.y += a.y * sc;
      o.z += a.z * sc;
      o.w += a.w * sc;
    }
    const bool any = W > 0.0f;
    const float inv = any ? p.out_scale / W : 0.0f;   // out_scale: V pool scale (1 for bf16)
    if (final_out) {
      const int64_t ho = head_offset(p, h);
      uint2 packed;
      packed.x = pack_bf16(f32_to_bf16_rne(o.x * inv), f32_to_bf16_rne(o.y * inv));
      packed.y = pack_bf16(f32_to_bf16_rne(o.z * inv), f32_to_bf16_rne(o.w * inv));
      *reinterpret_cast<uint2*>(final_out + ho * D + d) = packed;
      if (d == 0 && final_lse) final_lse[ho] = any ? M * kLn2 + __logf(W) : -INFINITY;
    } else {
      *reinterpret_cast<float4*>(out + h * hstride * D + d) =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      if (d == 0) {
        mx[h * hstride] = any ? M * kLn2 : -INFINITY;
        sm[h * hstride] = W;
      }
    }
  }
}

// Attention of the G q heads of KV head gk of sequence b over keys
// [begin, end) (begin < end), by the NW waves of the block, on the vector
// ALUs: wave w takes chunks w, w + NW, ..., keeps its own running state, and
// the waves are merged at the end (write_range).
template <int D, int G, int NW>
__device__ __forceinline__ void attend_range_valu(const SplitParams& p, int b, int gk, int begin,
                                                  int end, float* out, float* mx, float* sm,
                                                  int64_t hstride, uint16_t* final_out,
                                                  float* final_lse) {
  using g = Geo<D, G>;
  constexpr int CH = g::CH;

  __shared__ float red_acc[NW][G][D];
  __shared__ float red_m[NW][G];
  __shared__ float red_l[NW][G];
  __shared__ float p_lds[NW][CH][G];         // probabilities, key-major
  __shared__ float a_lds[NW][G];             // per-head rescale factor of the chunk

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  WaveKeys wk;
  wk.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  wk.begin = begin;
  wk.end = end;
  const int c_first = begin / CH;
  const int c_last = (end - 1) / CH;
  wk.c0 = c_first + wave;
  wk.step = NW;
  wk.nk = (wk.c0 <= c_last) ? (c_last - wk.c0) / NW + 1 : 0;
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

  const int64_t row0 = static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * p.gq;

  // q pieces, pre-permuted per lane: slot h holds head h ^ pi.
  uint4 qv[G][g::NQL];
  {
    const uint16_t* qb = p.q + row0 * D + 8 * jq;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int s = 0; s < g::NQL; ++s) qv[h][s] = load16(qb + head_offset(p, h ^ pi) * D + s * 8 * g::LQ);
  }

  // keys each owned head may see
  int lo_h[g::VH], hi_h[g::VH];
  {
    const int n = p.context_lens[b];
#pragma unroll
    for (int vh = 0; vh < g::VH; ++vh) head_bounds(p, n, vh ^ pi, begin, end, lo_h[vh], hi_h[vh]);
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
    const int tchunk = (wk.c0 + k * NW) * CH;
    KRegs<D, G> kr;
    VRegs<D, G> vr;
    ensure_pages<CH>(wk, k, lane, p.page_shift);
    load_k<D, G>(kr, wk, k, lane, kbase, p, koff);
    load_v<D, G>(vr, wk, k, lane, vbase, p, voff0);

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
#pragma unroll
      for (int vh = 0; vh < g::VH; ++vh)
        s_own[u][vh] = (t >= lo_h[vh] && t < hi_h[vh]) ? v[vh] * p.scale_log2 : -INFINITY;
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

  write_range<D, G, NW>(p, &red_acc[0][0][0], red_m, red_m, red_l, out, mx, sm, hstride,
                        final_out, final_lse);
  __syncthreads();   // the shared buffers are reused by the block's next range
}

// ---- matrix-core range routine (wide groups) ------------------------------------
//
// For groups of 8 or more (virtual) heads the vector-ALU layout needs G*8
// accumulators and G q pieces per lane; on MFMA the 16 heads of a tile share
// one operand column each and a lane holds D/4 accumulators.  Per wave and
// chunk of 16 keys (always inside one page):
//   scores  S^T[16 keys x 16 heads] = K[16 x D] . Q^T[D x 16]    (16x16x32, D/32 steps)
//           A = K rows loaded straight from the page (lane: key c, dims
//           32ks + 8g .. +8), B = q (lane: head c, same dims), exact bf16
//           products, fp32 sums; D lane holds keys 4g .. 4g+3 of head c.
//   softmax per head c over the chunk (max across the 4 lane groups), with a
//           reference max that moves only when a score passes it by more than
//           8 (log2 domain): P <= 2^8 and the accumulators are rescaled rarely.
//   P.V     O[16 heads x D] += P[16 x 16 keys] . V[16 keys x D] (16x16x16)
//           A = P exactly as the score D layout left it (head c, keys 4g+i),
//           split into three bf16 terms hi + mid + lo, which represent the fp32
//           value exactly; B = V columns from the wave's LDS tile (row-major,
//           rows padded to D + 16 elements) by transposed reads.
// Padding heads (c >= vheads) get q = 0 and write nothing.  The loads of chunk k+1
// are issued as soon as chunk k's registers are free: K after the scores, V
// after its LDS write.
//
// f32 pools (F32): every K or V element splits exactly into three bf16 terms
// hi + mid + lo (as P does), so the scores take three MFMAs per step and P.V
// nine (P's three terms times V's three), all with exact products and fp32
// sums; V goes through three bf16 LDS tiles, one per term.  A step's 8 dims
// are two 16-byte loads (dims 32ks + 8g .. +4 and +4 .. +8).
//
// FP8 pools (F8): K and V hold one OCP E4M3 byte per element.  They are
// converted to bf16 in registers (exact: every E4M3 value is a bf16 value);
// the per-pool scales are folded into the softmax scale (K) and the output
// (V) by the host.  A 16-byte K load then covers two score steps: lane g
// holds dims 64j + 16g .. +16 of its key, the first 8 for step 2j and the
// last 8 for step 2j+1, and q is loaded with the same dims order (the
// contraction over dims does not depend on it).  V rows are converted on
// their way into the LDS tile, which stays bf16.
// Element type of the K/V pools.
enum : int { kKvBf16 = 0, kKvFp8 = 1, kKvF32 = 2 };

template <int D, int G, int KV = kKvBf16>
struct MfmaGeo {
  static constexpr bool F8 = KV == kKvFp8;
  static constexpr bool F32 = KV == kKvF32;
  // A wave's chunk is SUB tiles of 16 keys (a tile never spans two pages);
  // their loads are issued together and one softmax update covers them.
  // Measured on the bs64 decode: two tiles per chunk made the FP8 call slower
  // (125 against 119.5 us) and the bf16 one spill, so a chunk is one tile.
  static constexpr int SUB = 1;
  static constexpr int KC = 16 * SUB;    // keys per chunk
  static constexpr int KS = D / 32;      // score k-steps
  static constexpr int NT = D / 16;      // P.V output tiles
  static constexpr int EB = F8 ? 1 : F32 ? 4 : 2;   // bytes per pool element
  static constexpr int NK = KS * EB / 2; // 16-byte K loads per lane and 16-key tile
  static constexpr int LV = D * EB / 16; // lanes per V row in the load layout (16 B each)
  static constexpr int TV = 64 / LV;     // V rows per load
  static constexpr int NV = 16 / TV;     // V loads per 16-key tile
  static constexpr int VD = 16 / EB;     // dims per V lane load
  static constexpr int VPAD = D + 16;    // LDS row stride of the V tile (bf16 elements)
  static_assert(G >= 1 && G <= 16, "one 16-column MFMA tile holds the group");
};

// 16 E4M3 bytes -> 16 bf16 (exact), bytes 0..7 into lo, 8..15 into hi.
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w, bool high_word) {
  return __builtin_bit_cast(uint32_t, high_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ void fp8x16_bf16(uint4 x, uint4& lo, uint4& hi) {
  lo = make_uint4(fp8x2_bf16(x.x, false), fp8x2_bf16(x.x, true), fp8x2_bf16(x.y, false),
                  fp8x2_bf16(x.y, true));
  hi = make_uint4(fp8x2_bf16(x.z, false), fp8x2_bf16(x.z, true), fp8x2_bf16(x.w, false),
                  fp8x2_bf16(x.w, true));
}

//
// head_dim 512 (the global-layer head size of a model that mixes 256 and 512
// per layer [vllm.cpp kernel matrix, row KERNEL-ATTN-PAGED]) splits the dims
// instead of the keys: the NW waves walk the same
// chunks, wave w holding dims 128w .. 128w+127 of K, q, V and the output (the
// D = 128 geometry per wave).  Their partial scores are summed through LDS in
// wave order, so every wave has the same scores and the same softmax state,
// and each writes its own output columns.
//
// Issue priority from progress: a SIMD's instruction arbiter prefers its
// oldest wave, so of the blocks resident on one CU (each owning the same
// number of keys in the balanced split) the first dispatched pulls ahead,
// finishes early and leaves its slot idle while the last one is still
// streaming.  A wave of the balanced split therefore lowers its priority as
// its block advances: 3 until the block has passed one half of its keys, 2
// until three quarters, 1 until nine tenths, then 0.  The leaders yield to
// the laggards at each step and the blocks of a CU end close together.
// Priority changes only the order of issue, never a result.  The steps are
// given as key indices of the range's row, so the loop only compares
// wave-uniform integers.
struct PrioKeys {
  bool on;
  int t50, t75, t90;   // first key at which the block has passed 1/2, 3/4, 9/10 of its keys
};

__device__ __forceinline__ void progress_priority(const PrioKeys& pk, int t, int& cur) {
  const int lvl = 3 - (t >= pk.t50 ? 1 : 0) - (t >= pk.t75 ? 1 : 0) - (t >= pk.t90 ? 1 : 0);
  if (lvl == cur) return;
  cur = lvl;
  if (lvl == 3) __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// pk: where the block's progress steps fall (pk.on false, as for the fixed
// partitions, leaves the priority alone).
template <int D, int G, int NW, int KV>
__device__ __forceinline__ void attend_range_mfma(const SplitParams& p, int b, int gk, int begin,
                                                  int end, float* out, float* mx, float* sm,
                                                  int64_t hstride, uint16_t* final_out,
                                                  float* final_lse,
                                                  const PrioKeys& pk = PrioKeys{false, 0, 0, 0}) {
  constexpr int NSL = D > 256 ? NW : 1;   // dim slices
  constexpr int DW = D / NSL;             // dims of one wave
  using mg = MfmaGeo<DW, G, KV>;
  constexpr bool F8 = mg::F8;
  constexpr bool F32 = mg::F32;
  constexpr int KC = mg::KC;
  constexpr int SUB = mg::SUB;
  constexpr int kVTerms = F32 ? 3 : 1;    // bf16 V tiles per wave (hi, mid, lo for f32)
  constexpr int kVTileBytes = KC * mg::VPAD * 2;
  constexpr int kTileBytes = NW * kVTerms * kVTileBytes;
  constexpr int kRedBytes = NW * G * DW * 4;
  // the V tiles of the loop and the wave states of the epilogue share one buffer
  __shared__ __align__(16) char lds[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
  // partial scores of the dim slices, double-buffered (one barrier per chunk)
  __shared__ f32x4_t sx[NSL > 1 ? 2 : 1][NSL][64];
  __shared__ float red_m[NW][G];
  __shared__ float red_mt[NW][G];
  __shared__ float red_l[NW][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int slice = NSL > 1 ? wave : 0;
  uint16_t (*vt)[mg::VPAD] =
      reinterpret_cast<uint16_t (*)[mg::VPAD]>(lds + wave * kVTerms * kVTileBytes);

  WaveKeys wk;
  wk.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  wk.begin = begin;
  wk.end = end;
  const int c_first = begin / KC;
  const int c_last = (end - 1) / KC;
  wk.c0 = c_first + (NSL > 1 ? 0 : wave);
  wk.step = NSL > 1 ? 1 : NW;
  wk.nk = (wk.c0 <= c_last) ? (c_last - wk.c0) / wk.step + 1 : 0;
  // pages per chunk: 1, or 2 when a 32-key chunk meets 16-key pages
  wk.ppc_shift = (KC > p.page_size) ? (ilog2c(KC) - p.page_shift) : 0;
  wk.ptab = 0;
  wk.group = -1;

  // pool bases of KV head gk (head_stride counts pool elements), at the
  // wave's dim slice
  const int64_t slice_bytes = static_cast<int64_t>(slice) * DW * mg::EB;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const char*>(p.k) + static_cast<int64_t>(gk) * p.head_stride * mg::EB + slice_bytes);
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const char*>(p.v) + static_cast<int64_t>(gk) * p.head_stride * mg::EB + slice_bytes);

  const int64_t row0 = static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * p.gq;
  const bool head_live = c16 < p.vheads;

  // B operand of the scores: q of head c16, dims 32ks + 8g .. +8 (bf16 pools)
  // or 64j + 16g + 8(ks & 1) .. +8 with j = ks / 2 (FP8 pools)
  uint4 qb[mg::KS];
  {
    const uint16_t* qrow = p.q + (row0 + head_offset(p, head_live ? c16 : 0)) * D + slice * DW;
#pragma unroll
    for (int ks = 0; ks < mg::KS; ++ks) {
      const int d0 = F8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g;
      qb[ks] = head_live ? load16(qrow + d0) : make_uint4(0, 0, 0, 0);
    }
  }
  int lo_h = 0, hi_h = 0;          // no key for a padding head
  if (head_live) head_bounds(p, p.context_lens[b], c16, begin, end, lo_h, hi_h);

  f32x4_t acc[mg::NT];
#pragma unroll
  for (int nt = 0; nt < mg::NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;         // per head c16, equal on its 4 lanes
  float m_top = -INFINITY;         // largest score of head c16 so far (>= m_ref, < m_ref + 8)
  float l_sum = 0.0f;              // this lane's share of head c16's sum

  // K: lane (g, c16) reads key c16 of each tile, 16 bytes at 64 * i + 16 * g,
  // straight into the A-operand layout.  (Loading whole rows to LDS instead,
  // with direct global->LDS loads, and reading the operand back measured
  // slower on the bs64 decode: 198 against 193 us.)
  const int koff = c16 * p.token_bytes + (F32 ? 32 : 16) * g;
  // byte offset of K load i within the lane's row share
  auto kload_off = [](int i) { return F32 ? 128 * (i >> 1) + 16 * (i & 1) : 64 * i; };
  const int voff0 = (lane / mg::LV) * p.token_bytes + 16 * (lane % mg::LV);
  uint4 kr[SUB][mg::NK], vr[SUB][mg::NV];
  auto issue_k = [&](int k) {
    const int t0 = (wk.c0 + k * wk.step) * KC;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int tu = t0 + 16 * u;
      const auto rs = tile_rsrc(kbase, page_of<KC>(wk, k, tu, p.page_shift), p.page_bytes, p.tile_bytes);
      const int soff = (tu & (p.page_size - 1)) * p.token_bytes;
      const int voff = koff | dead_bit(tu + c16, wk.begin, wk.end);
#pragma unroll
      for (int i = 0; i < mg::NK; ++i) kr[u][i] = tile_load(rs, voff + kload_off(i), soff);
    }
  };
  auto issue_v = [&](int k) {
    const int t0 = (wk.c0 + k * wk.step) * KC;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int tu = t0 + 16 * u;
      const auto rs = tile_rsrc(vbase, page_of<KC>(wk, k, tu, p.page_shift), p.page_bytes, p.tile_bytes);
      const int soff = (tu & (p.page_size - 1)) * p.token_bytes;
#pragma unroll
      for (int j = 0; j < mg::NV; ++j)
        vr[u][j] = tile_load(rs, voff0 | dead_bit(tu + mg::TV * j + lane / mg::LV, wk.begin, wk.end),
                             soff + mg::TV * j * p.token_bytes);
    }
  };

  if (wk.nk > 0) {
    ensure_pages<KC>(wk, 0, lane, p.page_shift);
    issue_k(0);
    issue_v(0);
  }
  const uint16_t* brow = &vt[4 * g + (c16 >> 2)][4 * (c16 & 3)];
  int prio = -1;
  for (int k = 0; k < wk.nk; ++k) {
    const int t0 = (wk.c0 + k * wk.step) * KC;
    if (pk.on) progress_priority(pk, t0, prio);
    const bool more = k + 1 < wk.nk;
    f32x4_t sc[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      sc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint4* kv = kr[u];
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < mg::NK; ++i) {
          uint4 a0, a1;
          fp8x16_bf16(kv[i], a0, a1);
          sc[u] = mfma(a0, qb[2 * i], sc[u]);
          sc[u] = mfma(a1, qb[2 * i + 1], sc[u]);
        }
      } else if constexpr (F32) {
#pragma unroll
        for (int ks = 0; ks < mg::KS; ++ks) {
          const uint4 x0 = kv[2 * ks], x1 = kv[2 * ks + 1];
          uint4 h, m, l;
          split3_bf16x2(u2f(x0.x), u2f(x0.y), h.x, m.x, l.x);
          split3_bf16x2(u2f(x0.z), u2f(x0.w), h.y, m.y, l.y);
          split3_bf16x2(u2f(x1.x), u2f(x1.y), h.z, m.z, l.z);
          split3_bf16x2(u2f(x1.z), u2f(x1.w), h.w, m.w, l.w);
          sc[u] = mfma(l, qb[ks], sc[u]);
          sc[u] = mfma(m, qb[ks], sc[u]);
          sc[u] = mfma(h, qb[ks], sc[u]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < mg::KS; ++ks) sc[u] = mfma(kv[ks], qb[ks], sc[u]);
      }
    }
    if (more) {
      ensure_pages<KC>(wk, k + 1, lane, p.page_shift);
      issue_k(k + 1);
    }
    if constexpr (NSL > 1) {
      static_assert(SUB == 1, "one score tile per chunk");
      sx[k & 1][slice][lane] = sc[0];
      __syncthreads();
      f32x4_t t = sx[k & 1][0][lane];
#pragma unroll
      for (int w = 1; w < NSL; ++w) t += sx[k & 1][w][lane];
      sc[0] = t;
    }

    // lane holds keys t0 + 16u + 4g + i of head c16; a chunk inside every
    // live head's key range needs no mask (padding heads' values are unused)
    float s[SUB][4];
    float cm = -INFINITY;
    const bool inside = !head_live || (t0 >= lo_h && t0 + KC <= hi_h);
    if (__builtin_amdgcn_read_exec() == __ballot(inside)) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[u][i] = sc[u][i] * p.scale_log2;
          cm = fmaxf(cm, s[u][i]);
        }
    } else {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * u + 4 * g + i;
          s[u][i] = (t >= lo_h && t < hi_h) ? sc[u][i] * p.scale_log2 : -INFINITY;
          cm = fmaxf(cm, s[u][i]);
        }
    }
    cm = fmaxf(cm, xor16(cm));
    cm = fmaxf(cm, xor32(cm));
    m_top = fmaxf(m_top, cm);
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
      for (int nt = 0; nt < mg::NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= ar[i];
    }
    const float base = (m_ref == -INFINITY) ? 0.0f : m_ref;
    uint2 pa_hi[SUB], pa_mid[SUB], pa_lo[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = fast_exp2(s[u][i] - base);
        l_sum += e[i];
      }
      split3_bf16x2(e[0], e[1], pa_hi[u].x, pa_mid[u].x, pa_lo[u].x);
      split3_bf16x2(e[2], e[3], pa_hi[u].y, pa_mid[u].y, pa_lo[u].y);
    }

    // V rows to the wave's tile (as bf16), then the next chunk's V loads
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int j = 0; j < mg::NV; ++j) {
        // 16-byte units of the row: a lane's VD dims are units m * VD / 8 ..
        uint4* row = reinterpret_cast<uint4*>(&vt[16 * u + mg::TV * j + lane / mg::LV][0]);
        const int m = lane % mg::LV;
        if constexpr (F32) {
          // 4 dims of one key, as three bf16 terms into the three tiles
          const uint4 x = vr[u][j];
          uint2 h, mm, l;
          split3_bf16x2(u2f(x.x), u2f(x.y), h.x, mm.x, l.x);
          split3_bf16x2(u2f(x.z), u2f(x.w), h.y, mm.y, l.y);
          const int r = 16 * u + mg::TV * j + lane / mg::LV;
          char* base = lds + wave * kVTerms * kVTileBytes + r * mg::VPAD * 2 + 8 * m;
          *reinterpret_cast<uint2*>(base) = h;
          *reinterpret_cast<uint2*>(base + kVTileBytes) = mm;
          *reinterpret_cast<uint2*>(base + 2 * kVTileBytes) = l;
        } else if constexpr (F8) {
          // the two 16-byte halves are written in an order that puts the 16
          // lanes of one write pass on 16 different 4-bank groups
          uint4 lo, hi;
          fp8x16_bf16(vr[u][j], lo, hi);
          const int swap = (mg::LV == 8 ? m : m >> 3) & 1;
          const uint4 first = make_uint4(swap ? hi.x : lo.x, swap ? hi.y : lo.y,
                                         swap ? hi.z : lo.z, swap ? hi.w : lo.w);
          const uint4 second = make_uint4(swap ? lo.x : hi.x, swap ? lo.y : hi.y,
                                          swap ? lo.z : hi.z, swap ? lo.w : hi.w);
          row[2 * m + swap] = first;
          row[2 * m + 1 - swap] = second;
        } else {
          row[m] = vr[u][j];
        }
      }
    if (more) issue_v(k + 1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P.V in groups of 8 output tiles: the group's transposed reads first, then
    // its MFMAs term-major, so no MFMA waits on the one before it and the
    // reads' latency is paid once per group
    constexpr int kGroupTiles = F32 ? (mg::NT < 4 ? mg::NT : 4) : (mg::NT < 8 ? mg::NT : 8);
    if constexpr (F32) {
      // P's three terms times V's three: nine exact-product MFMAs per tile
#pragma unroll
      for (int n0 = 0; n0 < mg::NT; n0 += kGroupTiles) {
        uint2 bv[3][kGroupTiles];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
          for (int n = 0; n < kGroupTiles; ++n)
            bv[t][n] = lds_read_tr(brow + t * (kVTileBytes / 2) + 16 * (n0 + n));
#pragma unroll
        for (int t = 2; t >= 0; --t) {
#pragma unroll
          for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_lo[0], bv[t][n], acc[n0 + n]);
#pragma unroll
          for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_mid[0], bv[t][n], acc[n0 + n]);
#pragma unroll
          for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_hi[0], bv[t][n], acc[n0 + n]);
        }
      }
    } else
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int n0 = 0; n0 < mg::NT; n0 += kGroupTiles) {
        uint2 bv[kGroupTiles];
#pragma unroll
        for (int n = 0; n < kGroupTiles; ++n)
          bv[n] = lds_read_tr(brow + 16 * u * mg::VPAD + 16 * (n0 + n));
#pragma unroll
        for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_lo[u], bv[n], acc[n0 + n]);
#pragma unroll
        for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_mid[u], bv[n], acc[n0 + n]);
#pragma unroll
        for (int n = 0; n < kGroupTiles; ++n) acc[n0 + n] = mfma16(pa_hi[u], bv[n], acc[n0 + n]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }

  // head c16's sum over the 4 lane groups
  l_sum += xor16(l_sum);
  l_sum += xor32(l_sum);

  __syncthreads();                 // every wave is done with its V tile
  float* red_acc = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    if (h < G) {
#pragma unroll
      for (int nt = 0; nt < mg::NT; ++nt) red_acc[(wave * G + h) * DW + 16 * nt + c16] = acc[nt][i];
    }
  }
  if (g == 0 && head_live && (NSL == 1 || wave == 0)) {
    red_m[wave][c16] = m_ref;
    red_mt[wave][c16] = m_top;
    red_l[wave][c16] = l_sum;
  }
  __syncthreads();
  write_range<D, G, NW, NSL>(p, red_acc, red_m, red_mt, red_l, out, mx, sm, hstride, final_out,
                             final_lse);
  __syncthreads();   // the shared buffers are reused by the block's next range
}

// Groups of 4 to 16 heads run on the matrix cores, 1 and 2 on the vector
// ALUs (measured on the bs64 GQA-4 decode: 199 us on MFMA against 206 us);
// head_dim 64 and 512 always take the matrix cores.
template <int D, int G>
constexpr bool kUseMfma = G >= 4 || D == 64 || D == 512;

// Waves per SIMD the compiler must fit the range kernels' registers into.
// (head_dim 512 holds the D = 128 registers per wave)
template <int D, int G, int KV = kKvBf16>
constexpr int kMinWaves = KV == kKvF32 ? (D == 64 ? 3 : D == 256 ? 1 : 2)
                          : (KV != kKvBf16 || kUseMfma<D, G>)
                              ? (D == 64 ? 4 : (D == 128 || D == 512) ? 3 : 2)
                              : 1;

// FP8 and f32 pools always take the matrix-core routine.
template <int D, int G, int NW, int KV = kKvBf16>
__device__ __forceinline__ void attend_range(const SplitParams& p, int b, int gk, int begin,
                                             int end, float* out, float* mx, float* sm,
                                             int64_t hstride, uint16_t* final_out = nullptr,
                                             float* final_lse = nullptr,
                                             const PrioKeys& pk = PrioKeys{false, 0, 0, 0}) {
  if constexpr (KV != kKvBf16 || kUseMfma<D, G>)
    attend_range_mfma<D, G, NW, KV>(p, b, gk, begin, end, out, mx, sm, hstride, final_out,
                                    final_lse, pk);
  else
    attend_range_valu<D, G, NW>(p, b, gk, begin, end, out, mx, sm, hstride, final_out, final_lse);
}

// Called by a whole wave, with count(b) items in each of the hkv rows of
// sequence b: the sum of count(b) over the sequences, and the sequence
// holding item x of the rows laid end to end (with the items of one row
// before that sequence).
template <typename F>
__device__ __forceinline__ int64_t wave_items(int batch, F count) {
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) s += (b0 + lane < batch) ? count(b0 + lane) : 0;
  return wave_sum64(s);
}

template <typename F>
__device__ __forceinline__ void wave_find_item(int batch, int hkv, int64_t x, F count, int& b_out,
                                               int64_t& pre_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int64_t len = (b0 + lane < batch) ? count(b0 + lane) : 0;
    const int64_t incl = wave_scan64(len);
    const uint64_t hit = __ballot(hkv * (base + incl) > x);
    if (hit) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      b_out = b0 + l;
      pre_out = base + __shfl(incl, l) - __shfl(len, l);
      return;
    }
    base += __shfl(incl, 63);
  }
  b_out = batch;
  pre_out = base;
}

// Fixed partitions: one block per (partition j, KV head gk, sequence b),
// handling keys [lo + j*P, lo + (j+1)*P).  Blocks are dispatched in the order
// of their linear index i = blockIdx.y * gridDim.x + blockIdx.x (a 2-D grid
// only past 65,536 blocks; indices past the last block exit at once): block i
// takes the i-th partition with a key, in row-major
// order over (b, gk) and ascending j, or, past the last of those, the empty
// partitions in the same order.  So every partition with keys starts before
// any empty one, and the empty ones fill the slots that the last partitions
// with keys leave idle.
template <int D, int G>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kMinWaves<D, G>)))
void split_kernel(const SplitParams p, int batch) {
  __shared__ int sh_item[3];
  const int64_t i = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  if (i >= static_cast<int64_t>(p.max_parts) * p.kv_heads * batch) return;   // whole block
  if (threadIdx.x < 64) {
    const int hkv = p.kv_heads;
    const int P = p.partition_size;
    auto live_of = [&](int bb) -> int64_t {   // partitions j < max_parts with a key
      const int nn = p.context_lens[bb];
      const int64_t len = nn - (p.window > 0 ? max(0, nn - p.window) : 0);
      return len > 0 ? min(static_cast<int64_t>(p.max_parts), (len + P - 1) / P) : 0;
    };
    auto dead_of = [&](int bb) -> int64_t { return p.max_parts - live_of(bb); };
    const int64_t W = wave_items(batch, live_of) * hkv;
    int bb;
    int64_t pre, off, cnt, first;
    if (i < W) {
      wave_find_item(batch, hkv, i, live_of, bb, pre);
      cnt = live_of(bb);
      off = i - pre * hkv;
      first = 0;
    } else {
      wave_find_item(batch, hkv, i - W, dead_of, bb, pre);
      cnt = dead_of(bb);
      off = i - W - pre * hkv;
      first = live_of(bb);
    }
    if (threadIdx.x == 0) {
      sh_item[0] = static_cast<int>(first + off % cnt);
      sh_item[1] = static_cast<int>(off / cnt);
      sh_item[2] = bb;
    }
  }
  __syncthreads();
  const int j = sh_item[0];
  const int gk = sh_item[1];
  const int b = sh_item[2];
  const int n = p.context_lens[b];
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int64_t begin64 = static_cast<int64_t>(lo) + static_cast<int64_t>(j) * p.partition_size;
  const int64_t rowbase = (static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * p.gq) *
                          p.max_parts + j;   // index of (b, h = gk*Gq, j)
  if (begin64 >= n) {
    if (p.write_empty) {
      for (int e = threadIdx.x; e < p.vheads * D; e += kBlock) {
        const int h = e / D;
        p.part_out[(rowbase + static_cast<int64_t>(h) * p.max_parts) * D + (e % D)] = 0.0f;
      }
      if (threadIdx.x < p.vheads) {
        p.part_max[rowbase + static_cast<int64_t>(threadIdx.x) * p.max_parts] = -INFINITY;
        p.part_sum[rowbase + static_cast<int64_t>(threadIdx.x) * p.max_parts] = 0.0f;
      }
    }
    return;
  }
  const int end = static_cast<int>(min(begin64 + p.partition_size, static_cast<int64_t>(n)));
  attend_range<D, G, kWaves>(p, b, gk, static_cast<int>(begin64), end, p.part_out + rowbase * D,
                     p.part_max + rowbase, p.part_sum + rowbase, p.max_parts);
}

// ---- balanced split -----------------------------------------------------------
//
// Rows are (sequence b, KV head g), r = b*Hkv + g, with len_b = ctx_b - lo_b
// attended keys; laid end to end they form T = Hkv * sum_b len_b units of work
// (one key of one KV head).  Block i of the nb used blocks owns the units
// [s_i, s_i+1) with s_i = floor(i*T/nb), so every block streams the same number
// of K/V bytes whatever the mix of context lengths.  A block's share is cut at
// row ends into segments; segment (r, i) writes its fp32 partial to slot
// r + i, which is unique (each segment starts at the (r + i)-th boundary of
// the merged row/block boundary sequence) and makes the slots of one row
// contiguous, in ascending key order.  A row that lies inside one block's share
// is written out directly by that block.  Every call rewrites every row's
// record, (first block << 12) | pieces, from the block holding the row's first
// piece (0 pieces for a sequence with no key), and the merge kernel combines
// the pieces of the rows with two or more, in ascending order.  Every block
// derives the split from the context lengths itself (a scan by one wave), so
// no plan has to be built and read back.  The split points depend on the
// context lengths of the whole batch and on nothing else (not on where pages
// live).

__device__ __forceinline__ int64_t seq_len(const int32_t* ctx, int b, int window) {
  const int n = ctx[b];
  const int lo = window > 0 ? max(0, n - window) : 0;
  return static_cast<int64_t>(n - lo);
}


// Keys (per KV head) of all sequences: sum_b len_b.  Called by a whole wave.
// Units of one row of sequence b on the key line: its keys, after `cost`
// units that stand for the row's prologue (none for a row with no key).
__device__ __forceinline__ int64_t row_span(const int32_t* ctx, int b, int window, int cost) {
  const int64_t len = seq_len(ctx, b, window);
  return len > 0 ? len + cost : 0;
}

__device__ __forceinline__ int64_t total_units(const int32_t* ctx, int batch, int window, int cost) {
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
  for (int b0 = 0; b0 < batch; b0 += 64)
    s += (b0 + lane < batch) ? row_span(ctx, b0 + lane, window, cost) : 0;
  return wave_sum64(s);
}

// Sequence b that holds unit x (0 <= x < T) and the units of one row before
// it, pre_b = sum_{b' < b} span_b'.  Called by a whole wave; all lanes get
// the result.
__device__ __forceinline__ void locate_unit(const int32_t* ctx, int batch, int window, int cost,
                                            int hkv, int64_t x, int& b_out, int64_t& pre_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int64_t len = (b0 + lane < batch) ? row_span(ctx, b0 + lane, window, cost) : 0;
    const int64_t incl = wave_scan64(len);
    const uint64_t hit = __ballot(hkv * (base + incl) > x);
    if (hit) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      b_out = b0 + l;
      pre_out = base + __shfl(incl, l) - __shfl(len, l);
      return;
    }
    base += __shfl(incl, 63);
  }
  b_out = batch;
  pre_out = base;
}


// Waves per block of the balanced split.  Where a wave's state is large (G*D
// of 2048 floats or more, bf16 pools on the matrix cores: head_dim 256 groups
// of 8 and 16, head_dim 128 groups of 16), one block holds all the waves a CU
// keeps (4 x the waves per SIMD): half or a third as many ranges, so fewer
// prologues, epilogue merges of the waves' states and cut rows (d256w window
// decode 57.2 -> 53.7 us, bs64 4-query verify 211.7 -> 200.4 us).  Elsewhere
// 4-wave blocks measured faster (bs64 decode 188 against 192 us, FP8 107
// against 123 us).
template <int D, int G, int KV>
constexpr int kBalWaves = (KV == kKvBf16 && kUseMfma<D, G> && D <= 256 && G * D >= 2048)
                              ? 4 * kMinWaves<D, G, KV>
                              : kWaves;

template <int D, int G, int KV>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 64 * kBalWaves<D, G, KV>)))
__attribute__((amdgpu_waves_per_eu(kMinWaves<D, G, KV>)))
void balanced_split_kernel(const SplitParams p, const BalancedLayout bl) {
  constexpr int NWB = kBalWaves<D, G, KV>;
  __shared__ int64_t sh_total;
  __shared__ int64_t sh_pre;
  __shared__ int sh_b;
  const int i = blockIdx.x;
  const int hkv = p.kv_heads;
  // sequences with no key: output 0, log-sum-exp -inf (block i takes b = i,
  // i + grid, ...; the out rows of a sequence are contiguous)
  for (int b = i; b < bl.batch; b += gridDim.x) {
    if (p.context_lens[b] > 0) continue;
    const int64_t r0 = static_cast<int64_t>(b) * p.num_q_heads;
    for (int j = threadIdx.x; j < p.num_q_heads * D; j += 64 * NWB) bl.out[r0 * D + j] = 0;
    if (bl.lse)
      for (int j = threadIdx.x; j < p.num_q_heads; j += 64 * NWB) bl.lse[r0 + j] = -INFINITY;
    if (bl.row_info)
      for (int g = threadIdx.x; g < hkv; g += 64 * NWB) bl.row_info[static_cast<int64_t>(b) * hkv + g] = 0;
  }
  if (!bl.seg_out) {
    // No workspace: block i takes whole rows (b, g) = i, i + grid, ... and
    // writes their bf16 outputs directly; no partials, no merge.
    for (int64_t r = i; r < bl.rows; r += gridDim.x) {
      const int b = static_cast<int>(r / hkv);
      const int gk = static_cast<int>(r - static_cast<int64_t>(b) * hkv);
      const int n = p.context_lens[b];
      if (n <= 0) continue;                                  // written above
      const int lo = p.reach > 0 ? max(0, n - p.reach) : 0;
      const int64_t h0 = static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * p.gq;
      attend_range<D, G, NWB, KV>(p, b, gk, lo, n, nullptr, nullptr, nullptr, 1, bl.out + h0 * D,
                                     bl.lse ? bl.lse + h0 : nullptr);
    }
    return;
  }
  if (threadIdx.x < 64) {
    const int64_t T = total_units(p.context_lens, bl.batch, p.reach, bl.row_cost) * hkv;
    int b = 0;
    int64_t pre = 0;
    if (T > 0) {
      const int nb = used_blocks(T, gridDim.x, bl.min_units);
      if (i < nb)
        locate_unit(p.context_lens, bl.batch, p.reach, bl.row_cost, hkv,
                    static_cast<int64_t>(i) * T / nb, b, pre);
    }
    if (threadIdx.x == 0) {
      sh_total = T;
      sh_b = b;
      sh_pre = pre;
    }
  }
  __syncthreads();
  const int64_t T = sh_total;
  if (T == 0) return;
  const int nb = used_blocks(T, gridDim.x, bl.min_units);
  if (i >= nb) return;
  const int64_t s0 = static_cast<int64_t>(i) * T / nb;
  const int64_t s1 = static_cast<int64_t>(i + 1) * T / nb;
  int b = sh_b;
  int64_t pre = sh_pre;                                  // units of one row before sequence b
  const int gq = p.gq;
  const int cost = bl.row_cost;
  while (b < bl.batch) {
    const int n = p.context_lens[b];
    const int lo = p.reach > 0 ? max(0, n - p.reach) : 0;
    const int64_t len = n - lo;
    const int64_t span = len > 0 ? len + cost : 0;
    const int64_t seq0 = pre * hkv;                      // first unit of sequence b
    if (seq0 >= s1) break;
    for (int gk = 0; gk < hkv && len > 0; ++gk) {
      // row (b, gk): units off .. off + cost stand for its prologue, its keys
      // lo .. n are units k0 = off + cost .. k0 + len; a block whose share
      // holds none of its keys leaves it alone
      const int64_t off = seq0 + static_cast<int64_t>(gk) * span;
      const int64_t k0 = off + cost;
      if (k0 >= s1) break;
      const int64_t x0 = s0 > k0 ? s0 : k0;
      const int64_t x1 = (s1 < k0 + len) ? s1 : k0 + len;
      if (x1 <= x0) continue;
      const int begin = lo + static_cast<int>(x0 - k0);
      const int end = lo + static_cast<int>(x1 - k0);
      // a row whose keys lie inside this block's share gets its final output here
      const bool whole = k0 >= s0 && k0 + len <= s1;
      const int64_t r = static_cast<int64_t>(b) * hkv + gk;
      const int64_t slot = r + i;
      const int64_t h0 = static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(gk) * gq;
      // key of this row at which the block has passed num/den of its units
      auto key_at = [&](int num, int den) {
        const int64_t t = lo + (s0 + (s1 - s0) * num / den - k0);
        return static_cast<int>(t < -(1 << 30) ? -(1 << 30) : t > (1 << 30) ? (1 << 30) : t);
      };
      const PrioKeys pk{true, key_at(1, 2), key_at(3, 4), key_at(9, 10)};
      attend_range<D, G, NWB, KV>(p, b, gk, begin, end, bl.seg_out + slot * G * D,
                                 bl.seg_max + slot * G, bl.seg_sum + slot * G, 1,
                                 whole ? bl.out + h0 * D : nullptr,
                                 (whole && bl.lse) ? bl.lse + h0 : nullptr, pk);
      // the block holding a row's first piece records where its pieces are:
      // slots r + i .. r + i + count - 1 (count 1: written here already)
      if (x0 == k0 && threadIdx.x == 0)
        bl.row_info[r] = (i << 12) | (block_of(k0 + len - 1, T, nb) - i + 1);
    }
    pre += span;
    ++b;
  }
}

// Merge of the cut rows: block (r, y) combines the pieces of row r = (b, g),
// float4 units y*256 .. +256 of its G*D (virtual) head dims.  All pieces are
// read in one go (up to kBatch at a time, with a running max across
// batches), in ascending slot order; rows not cut (whole, or with no key) were
// written by the split kernel (which rewrites every row's record each call).
template <int D, int G>
__global__ __launch_bounds__(kBlock) void balanced_merge_kernel(const BalancedLayout bl,
                                                               int num_q_heads) {
  constexpr int kBatch = 8;
  constexpr int D4 = D / 4;
  const int r = blockIdx.x;
  const int info = bl.row_info[r];
  const int count = info & 0xfff;
  const int first = info >> 12;
  // rows with one piece (or none) are done; the slot range stays inside the
  // workspace whatever the record holds
  if (count < 2 || first < 0 || first + count > kMaxBalancedBlocks) return;
  const int64_t slot0 = r + static_cast<int64_t>(first);
  const int u = blockIdx.y * kBlock + threadIdx.x;
  if (u >= G * D4) return;
  const int h = u / D4;
  const int d = (u % D4) * 4;
  // output row of virtual head h (query h / gq, q head h % gq); padding heads
  // write nothing
  if (h >= bl.vheads) return;
  const int gq = bl.gq;
  const int hkv = bl.rows / bl.batch;
  const int b = r / hkv;
  const int64_t h0 = static_cast<int64_t>(b) * num_q_heads + static_cast<int64_t>(r - b * hkv) * gq;
  const int64_t ho = h0 + static_cast<int64_t>(h / gq) * bl.q_heads + (h % gq);
  const float* pm = bl.seg_max + slot0 * G + h;
  const float* pl = bl.seg_sum + slot0 * G + h;
  const float* po = bl.seg_out + (slot0 * G + h) * D + d;
  float M = -INFINITY, W = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < count; k0 += kBatch) {
    float mk[kBatch], lk[kBatch];
    float4 ok[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool in = k0 + k < count;
      mk[k] = in ? pm[(k0 + k) * G] : -INFINITY;
      lk[k] = in ? pl[(k0 + k) * G] : 0.0f;
      ok[k] = in ? *reinterpret_cast<const float4*>(po + static_cast<int64_t>(k0 + k) * G * D)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mn = fmaxf(Mn, mk[k]);
    if (Mn == -INFINITY) continue;            // no piece so far saw a key for this head
    const float a = __expf(M - Mn);           // 0 while M is -inf
    W *= a;
    o.x *= a; o.y *= a; o.z *= a; o.w *= a;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = lk[k] * __expf(mk[k] - Mn);   // 0 for an empty piece (l = 0, m = -inf)
      W += w;
      o.x = fmaf(w, ok[k].x, o.x);
      o.y = fmaf(w, ok[k].y, o.y);
      o.z = fmaf(w, ok[k].z, o.z);
      o.w = fmaf(w, ok[k].w, o.w);
    }
    M = Mn;
  }
  uint16_t* dst = bl.out + ho * D + d;
  if (M == -INFINITY) {                       // no piece saw a key for this head
    *reinterpret_cast<uint2*>(dst) = make_uint2(0, 0);
    if (d == 0 && bl.lse) bl.lse[ho] = -INFINITY;
    return;
  }
  const float inv = 1.0f / W;
  *reinterpret_cast<uint2*>(dst) =
      make_uint2(pack_bf16(f32_to_bf16_rne(o.x * inv), f32_to_bf16_rne(o.y * inv)),
                 pack_bf16(f32_to_bf16_rne(o.z * inv), f32_to_bf16_rne(o.w * inv)));
  if (d == 0 && bl.lse) bl.lse[ho] = M + __logf(W);
}

// ---- merge -----------------------------------------------------------------------

// Where the partials of one (sequence, q head) live.
struct FixedSlots {      // partition j at row*max_parts + j
  const float* po; const float* pm; const float* pl;
  int count;
  __device__ int64_t idx(int k) const { return k; }
};

// One block per (q head, sequence): M = max m_k, W = sum l_k e^(m_k - M),
// out = sum_k (l_k e^(m_k - M) / W) o_k over the partials k of the row, in
// ascending k within each of the block's partition groups, the groups added
// in fixed order.  `stride` is the distance between consecutive partials in
// elements of m/l (times D for o).
// One block merges dims [slice*D/DS, (slice+1)*D/DS) of a row, DS = D/32
// blocks per row: TPR = 8 threads cover the slice (4 dims each), and the 32
// groups of them take partitions grp, grp + 32, ... in ascending order, the
// groups' sums then added in ascending group order.
template <int D>
constexpr int kMergeSlices = D / 32;

template <int D>
__device__ __forceinline__ void merge_row(const float* pm, const float* pl, const float* po,
                                          int64_t stride, int count, uint16_t* out, float* lse,
                                          int slice) {
  constexpr int TPR = D / 4 / kMergeSlices<D>;   // threads per row slice (float4 each)
  constexpr int NGRP = kBlock / TPR;             // partition groups per block
  __shared__ float red[kWaves];
  __shared__ float4 part[NGRP][TPR];

  float M = -INFINITY;
  for (int jj = threadIdx.x; jj < count; jj += kBlock) M = fmaxf(M, pm[jj * stride]);
  M = wave_max(M);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  if (count == 0 || M == -INFINITY) {
    for (int d = threadIdx.x; d < D / kMergeSlices<D>; d += kBlock) out[slice * (D / kMergeSlices<D>) + d] = 0;
    if (lse && slice == 0 && threadIdx.x == 0) *lse = -INFINITY;
    return;
  }
  float W = 0.0f;
  for (int jj = threadIdx.x; jj < count; jj += kBlock) {
    const float mj = pm[jj * stride];
    const float lj = pl[jj * stride];
    if (mj != -INFINITY && lj != 0.0f) W += lj * __expf(mj - M);
  }
  W = wave_sum(W);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = W;
  __syncthreads();
  W = (red[0] + red[1]) + (red[2] + red[3]);

  const int grp = threadIdx.x / TPR;
  const int d4 = slice * TPR + threadIdx.x % TPR;   // float4 of the row
  // partitions grp, grp + NGRP, ... in ascending order, U of them loaded
  // together (a partition without a key has weight 0 and o = 0)
  constexpr int U = 8;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = grp; j0 < count; j0 += U * NGRP) {
    float w[U];
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * NGRP;
      const bool in = jj < count;
      const float mj = in ? pm[jj * stride] : -INFINITY;
      const float lj = in ? pl[jj * stride] : 0.0f;
      o[u] = in ? reinterpret_cast<const float4*>(po + jj * stride * D)[d4] : make_float4(0.f, 0.f, 0.f, 0.f);
      w[u] = (mj == -INFINITY || lj == 0.0f) ? 0.0f : lj * __expf(mj - M) / W;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a.x = fmaf(w[u], o[u].x, a.x);
      a.y = fmaf(w[u], o[u].y, a.y);
      a.z = fmaf(w[u], o[u].z, a.z);
      a.w = fmaf(w[u], o[u].w, a.w);
    }
  }
  part[grp][threadIdx.x % TPR] = a;
  __syncthreads();
  if (grp == 0) {
    float4 t = part[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < NGRP; ++q) {
      const float4 u = part[q][threadIdx.x];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    uint2 packed;
    packed.x = static_cast<uint32_t>(f32_to_bf16_rne(t.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(t.y)) << 16);
    packed.y = static_cast<uint32_t>(f32_to_bf16_rne(t.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(t.w)) << 16);
    reinterpret_cast<uint2*>(out)[d4] = packed;
  }
  if (lse && slice == 0 && threadIdx.x == 0) *lse = M + __logf(W);
}

// Fixed partitions: live partitions j < ceil((ctx - lo) / P).
template <int D>
__global__ __launch_bounds__(kBlock) void merge_kernel(const MergeParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int n = p.context_lens[b];
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  // live partitions, at most max_parts: a context past the partitions'
  // reach (outside the contract) merges the ones written and reads nothing
  // beyond its own row
  const int64_t nlive = (n > lo) ? (static_cast<int64_t>(n - lo) + p.partition_size - 1) /
                                       p.partition_size
                                 : 0;
  const int live = static_cast<int>(nlive < p.max_parts ? nlive : p.max_parts);
  const int64_t row = static_cast<int64_t>(b) * p.num_q_heads + h;
  merge_row<D>(p.part_max + row * p.max_parts, p.part_sum + row * p.max_parts,
               p.part_out + row * p.max_parts * D, 1, live, p.out + row * D,
               p.lse ? p.lse + row : nullptr, blockIdx.z);
}

// ---- launchers -----------------------------------------------------------------

template <int D, int G>
static hipError_t launch_split_dg(const SplitParams& p, int batch, int num_kv_heads,
                                  hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(p.max_parts) * num_kv_heads * batch;
  const int64_t gx = blocks < 65536 ? blocks : 65536;
  const int64_t gy = (blocks + gx - 1) / gx;
  if (gy > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy));
  launch_profiled(split_kernel<D, G>, grid, dim3(kBlock), 0, stream, p, batch);
  return hipGetLastError();
}

template <int D, int G, int KV>
static hipError_t launch_balanced_dg(const SplitParams& p, const BalancedLayout& bl, int grid,
                                     hipStream_t stream) {
  launch_profiled(balanced_split_kernel<D, G, KV>, dim3(grid), dim3(64 * kBalWaves<D, G, KV>), 0, stream, p,
                  bl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !bl.seg_out) return e;   // no workspace: rows were written whole
  hipLaunchKernelGGL((balanced_merge_kernel<D, G>), dim3(bl.rows, (G * D / 4 + kBlock - 1) / kBlock),
                     dim3(kBlock), 0, stream, bl, p.num_q_heads);
  return hipGetLastError();
}

// Resident blocks per CU of the balanced split kernel (a property of the
// code object, the same on every gfx950 device; threads that race on the
// first call store the same value).
template <int D, int G, int KV>
static int blocks_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, balanced_split_kernel<D, G, KV>,
                                                     64 * kBalWaves<D, G, KV>, 0) !=
            hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
static hipError_t launch_split_d(const SplitParams& p, int group, int batch, int num_kv_heads,
                                 hipStream_t stream) {
  switch (group) {
    case 1: return launch_split_dg<D, 1>(p, batch, num_kv_heads, stream);
    case 2: return launch_split_dg<D, 2>(p, batch, num_kv_heads, stream);
    case 4: return launch_split_dg<D, 4>(p, batch, num_kv_heads, stream);
    case 8: return launch_split_dg<D, 8>(p, batch, num_kv_heads, stream);
    case 16: return launch_split_dg<D, 16>(p, batch, num_kv_heads, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split(const SplitParams& p, int head_dim, int group, int batch,
                        int num_kv_heads, hipStream_t stream) {
  if (head_dim == 64) return launch_split_d<64>(p, group, batch, num_kv_heads, stream);
  if (head_dim == 128) return launch_split_d<128>(p, group, batch, num_kv_heads, stream);
  if (head_dim == 256) return launch_split_d<256>(p, group, batch, num_kv_heads, stream);
  if (head_dim == 512) return launch_split_d<512>(p, group, batch, num_kv_heads, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, int batch, hipStream_t stream) {
  dim3 grid(p.num_q_heads, batch, head_dim / 32);   // kMergeSlices<head_dim>
  if (head_dim == 64) {
    launch_profiled(merge_kernel<64>, grid, dim3(kBlock), 0, stream, p);
  } else if (head_dim == 128) {
    launch_profiled(merge_kernel<128>, grid, dim3(kBlock), 0, stream, p);
  } else if (head_dim == 256) {
    launch_profiled(merge_kernel<256>, grid, dim3(kBlock), 0, stream, p);
  } else if (head_dim == 512) {
    launch_profiled(merge_kernel<512>, grid, dim3(kBlock), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int G, int KV>
static int balanced_blocks(int num_cus, int max_blocks) {
  const int n = blocks_per_cu<D, G, KV>() * num_cus;
  return n < max_blocks ? n : max_blocks;
}

// Calls f.template operator()<D, G, KV>() for a supported (head_dim, padded
// group, pool element type) triple; returns `none` otherwise.  (f32 pools at
// head_dim 256 run one wave per SIMD: their K and V registers do not fit two.)
template <typename R, typename F>
static R dispatch_dg(int head_dim, int group, int kv, R none, F&& f) {
#define PA_CASE(DD, GG)                                                                \
  if (head_dim == DD && group == GG) {                                                 \
    if (kv == kKvBf16) return f.template operator()<DD, GG, kKvBf16>();                \
    if (kv == kKvFp8) return f.template operator()<DD, GG, kKvFp8>();                  \
    if (kv == kKvF32) return f.template operator()<DD, GG, kKvF32>();                  \
    return none;                                                                       \
  }
  PA_CASE(64, 1) PA_CASE(64, 2) PA_CASE(64, 4) PA_CASE(64, 8) PA_CASE(64, 16)
  PA_CASE(128, 1) PA_CASE(128, 2) PA_CASE(128, 4) PA_CASE(128, 8) PA_CASE(128, 16)
  PA_CASE(256, 1) PA_CASE(256, 2) PA_CASE(256, 4) PA_CASE(256, 8) PA_CASE(256, 16)
  PA_CASE(512, 1) PA_CASE(512, 2) PA_CASE(512, 4) PA_CASE(512, 8) PA_CASE(512, 16)
#undef PA_CASE
  return none;
}

// Blocks the balanced split uses for num_cus compute units (occupancy x CUs, capped).
int balanced_grid(int head_dim, int group, int num_cus, int max_blocks, int kv) {
  return dispatch_dg<int>(head_dim, group, kv, 0, [&]<int D, int G, int KV>() {
    return balanced_blocks<D, G, KV>(num_cus, max_blocks);
  });
}

// Units charged for starting a row: kRowCostUnits for 4-wave blocks (half
// that over bf16 pools), twice that for the blocks that hold all the waves of
// a CU.  bs64 4-query verify, 12-wave blocks: 194.5 us at 256 against 202.1 at
// 128 and 195.4 at 384; d256w, 8-wave blocks: 53.5 us at 128 and 256; bs64
// decode, bf16: 187.5-187.8 us at 64 against 188.6-188.7 at 128 (long
// contexts 0.3 us and the tiny call 0.4 us slower at 64); FP8 pools keep 128
// (106.5 against 108.5 us at 64).
int balanced_row_cost(int head_dim, int group, int kv) {
  return dispatch_dg<int>(head_dim, group, kv, kRowCostUnits, [&]<int D, int G, int KV>() {
    if (kBalWaves<D, G, KV> > kWaves) return 2 * kRowCostUnits;
    return KV == kKvBf16 ? kRowCostUnits / 2 : kRowCostUnits;
  });
}

// Balanced split, then the merge of the rows several blocks shared: the whole
// of pa_decode (bf16, FP8 or f32 pools).
hipError_t launch_balanced(const SplitParams& sp, const BalancedLayout& bl, int head_dim, int group,
                           int grid, hipStream_t stream, int kv) {
  return dispatch_dg<hipError_t>(head_dim, group, kv, hipErrorInvalidValue,
                                 [&]<int D, int G, int KV>() {
                                   return launch_balanced_dg<D, G, KV>(sp, bl, grid, stream);
                                 });
}

}  // namespace pa
