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
//
// Work split: heads form groups of 64 (one block = 4 waves x 16 heads); a
// row is (head group, sequence), ordered group-major.  The keys of all rows,
// laid end to end (T = groups * sum of context lengths), are cut into nb
// equal contiguous ranges, one per block; a block writes one partial per row
// piece it covers.  Group-major order puts the two head groups of the same
// keys T/2 units apart, i.e. in blocks i and i + nb/2, which the dispatcher
// places on the same XCD (nb a multiple of 16), so the second read of a
// cache tile is served by that XCD's L2.
//
// S queries per sequence (mla_absorbed_decode_multiquery): query s, head h is
// query head s*H + h of its sequence, so a sequence has S*H heads in
// ceil(S*H / 64) groups that share its key range; the absorption treats
// q_nope [B][S][H][128] as B*S rows of H heads, W_UK[h] / W_UV[h] serve every
// query, and under the causal in-block mask head s*H + h drops the keys
// t >= n - S + 1 + s of its sequence.
//
// FP8 latent cache (mla_absorbed_decode_fp8): rows of 656 bytes hold the
// latent as E4M3 in blocks of 64 with one power-of-two scale byte per block
// and the rope part in bf16 [vllm.cpp kernel matrix, row KERNEL-KV-CACHE-DSA:
// the fp8_ds_mla dequant read, e4m3 * 2^(scale byte - 127), rope bf16].  The
// staging lanes widen each 16-byte latent chunk to bf16 with the block's
// scale (v_cvt_scalef32_pk_bf16_fp8, exact for any result in bf16's normal
// range), so the LDS tile, and everything after it, is the bf16 path's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_mfma.h"
#include "pa_validate.h"

namespace pa {

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
constexpr int kGroup = kHeadsPerWave * kMlaWaves;   // heads per block
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kRowPad = kRow + 16; // LDS row stride (elements) of a cache tile row: 296 dwords,
                                   // conflict-free for the score and transposed reads
static_assert(kGroup == kMlaBlockHeads, "head group size");

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
  float* seg_out;          // [slots][64][512] normalised partial o_lat
  float* seg_max;          // [slots][64] natural-log-domain reference max
  float* seg_sum;          // [slots][64] sum of exp(s - max)
  uint16_t* out;           // [B][S][H][128]
  int64_t page_stride;
  int32_t token_stride;
  int32_t bt_stride;
  int32_t batch;
  int32_t num_heads;       // query heads per sequence: S * H (query s, head h -> s*H + h)
  int32_t w_heads;         // H, the heads of W_UK / W_UV
  int32_t num_queries;     // S
  int32_t abs_rows;        // B * S, the rows of the absorption
  int32_t groups;          // ceil(num_heads / 64)
  int32_t page_size;
  int32_t page_shift;
  int32_t split_grid;      // blocks launched for the split kernel
  int32_t min_keys;        // keys per block below which fewer blocks are used
  float scale_log2;
};

// ---- 1. absorption: q_abs = q_nope . W_UK[h] on MFMA, split in three; rope copied ---
//
// Block (h, jq, bt): q_abs[r][h][jq*128 .. +128) for the query rows
// r = 64*bt .. +64, in tiles of 16 that share one staged W_UK tile (r = b*S + s:
// q_nope [B][S][H][128] is [B*S][H][128], and row r*H + h of the result is
// head s*H + h of sequence b, the numbering of the later kernels).  Each tile
// is the product [16 r x 128 d] . [128 d x 128 j] of exact bf16 operands
// (MFMA, fp32 accumulation).  A = q_nope rows straight from memory (8
// consecutive d per lane); B = the W_UK[h] tile staged in LDS row-major
// ([d][j]) and read with transposed reads, which give each lane 4
// consecutive d of one column j.  Wave w computes j tiles 2w and 2w+1.  The
// three bf16 terms of a tile go through LDS so that each row's 128 columns
// leave as 16-byte stores.
constexpr int kWukPad = 128 + 16;  // LDS row stride of the W_UK tile: 72 dwords, conflict-free
constexpr int kAbsTiles = 4;       // 16-row tiles per absorb block
constexpr int kAbsOutPad = 128 + 8;

__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p) {
  __shared__ __align__(16) uint16_t ws[kNope][kWukPad];
  __shared__ __align__(16) uint16_t os[3][16][kAbsOutPad];   // hi, mid, lo of one tile
  const int h = blockIdx.x;
  const int jq = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const uint16_t* wsrc = p.w_uk + static_cast<int64_t>(h) * kNope * kLat + jq * 128;
  uint4 wst[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {          // 128 rows x 16 chunks of 16 B
    const int c = t + 256 * k;
    wst[k] = load16(wsrc + static_cast<int64_t>(c >> 4) * kLat + (c & 15) * 8);
  }
  // A operand of a tile: row b0 + c16, d = 32ks + 8g .. +8
  auto load_a = [&](int b0, int nb, uint4 (&qa)[kNope / 32]) {
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ++ks)
      qa[ks] = c16 < nb ? load16(p.q_nope + (static_cast<int64_t>(b0 + c16) * p.w_heads + h) * kNope +
                                 32 * ks + 8 * g)
                        : make_uint4(0, 0, 0, 0);
  };
  const int r0 = blockIdx.z * 16 * kAbsTiles;
  uint4 qa[kNope / 32];
  load_a(r0, min(16, p.abs_rows - r0), qa);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = t + 256 * k;
    *reinterpret_cast<uint4*>(&ws[c >> 4][(c & 15) * 8]) = wst[k];
  }
  __syncthreads();
  for (int tt = 0; tt < kAbsTiles; ++tt) {
    const int b0 = r0 + 16 * tt;
    if (b0 >= p.abs_rows) break;
    const int nb = min(16, p.abs_rows - b0);
    uint4 qn[kNope / 32];                // the next tile's A operand, in flight
    const int b1 = b0 + 16;
    const bool more = tt + 1 < kAbsTiles && b1 < p.abs_rows;
    if (more) load_a(b1, min(16, p.abs_rows - b1), qn);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int nt = 2 * wave + u;
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kNope / 32; ++ks) {
        // lane (g, a) points at rows 32ks + 8g + a/4 (+4), columns 16nt + 4(a%4)
        const uint16_t* bp = &ws[32 * ks + 8 * g + (c16 >> 2)][16 * nt + 4 * (c16 & 3)];
        const uint2 k03 = lds_read_tr(bp);
        const uint2 k47 = lds_read_tr(bp + 4 * kWukPad);
        c = mfma(qa[ks], make_uint4(k03.x, k03.y, k47.x, k47.y), c);
      }
      // D: lane holds q_abs[b0 + 4g + i][jq*128 + 16nt + c16]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t hi, mid, lo;
        split3_bf16(c[i], hi, mid, lo);
        os[0][4 * g + i][16 * nt + c16] = hi;
        os[1][4 * g + i][16 * nt + c16] = mid;
        os[2][4 * g + i][16 * nt + c16] = lo;
      }
    }
    __syncthreads();
    // 3 terms x 16 rows x 16 chunks of 8 columns, three 16-byte stores per thread
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int e = t + 256 * k;
      const int term = e >> 8, bb = (e >> 4) & 15, ch = e & 15;
      if (bb < nb) {
        const int64_t row = static_cast<int64_t>(b0 + bb) * p.w_heads + h;
        uint16_t* dst = term == 0 ? p.q_hi + row * kRow : (term == 1 ? p.q_mid : p.q_lo) + row * kLat;
        *reinterpret_cast<uint4*>(dst + jq * 128 + 8 * ch) =
            *reinterpret_cast<const uint4*>(&os[term][bb][8 * ch]);
      }
    }
    __syncthreads();   // os is rewritten by the next tile
    if (jq == 0 && t < nb * (kRope / 8)) {   // rope part: exact bf16, one term
      const int rb = t / (kRope / 8), rc = t % (kRope / 8);
      const int64_t row = static_cast<int64_t>(b0 + rb) * p.w_heads + h;
      *reinterpret_cast<uint4*>(p.q_hi + row * kRow + kLat + 8 * rc) =
          load16(p.q_rope + row * kRope + 8 * rc);
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < kNope / 32; ++ks) qa[ks] = qn[ks];
    }
  }
}

// ---- 2. split attention over the latent cache ----------------------------------------

// Tile row of the key that MFMA row m (0..15) of a 16-key half handles.  The
// transposed P.V reads of one 16-lane group touch the rows of m = 4g .. 4g+3;
// mapping them to rows 2i + (g&1) + 8(g>>1) (four rows two apart) puts the
// four 32-byte pieces in disjoint LDS banks (rows are 292 dwords apart),
// and keeps the score operand reads of rows m = 0..7 conflict-free.
__device__ __forceinline__ int key_row(int m) { return 2 * (m & 3) + ((m >> 2) & 1) + 8 * (m >> 3); }

// Sum of the context lengths.  Called by a whole wave.
__device__ __forceinline__ int64_t mla_total(const int32_t* ctx, int batch) {
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) s += (b0 + lane < batch) ? ctx[b0 + lane] : 0;
  return wave_sum64(s);
}

// Sequence b holding key y (0 <= y < S) of a group's key line, and the keys
// before it.  Called by a whole wave.
__device__ __forceinline__ void mla_locate(const int32_t* ctx, int batch, int64_t y, int& b_out,
                                           int64_t& pre_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int64_t len = (b0 + lane < batch) ? ctx[b0 + lane] : 0;
    const int64_t incl = wave_scan64(len);
    const uint64_t hit = __ballot(base + incl > y);
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

// 16 E4M3 bytes times the power-of-two scale s -> 16 bf16, bytes 0..7 into lo.
__device__ __forceinline__ uint32_t fp8x2_bf16_scaled(uint32_t w, float s, bool high_word) {
  return __builtin_bit_cast(uint32_t, high_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, true)
                                                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, false));
}
__device__ __forceinline__ void fp8x16_bf16_scaled(uint4 x, float s, uint4& lo, uint4& hi) {
  lo = make_uint4(fp8x2_bf16_scaled(x.x, s, false), fp8x2_bf16_scaled(x.x, s, true),
                  fp8x2_bf16_scaled(x.y, s, false), fp8x2_bf16_scaled(x.y, s, true));
  hi = make_uint4(fp8x2_bf16_scaled(x.z, s, false), fp8x2_bf16_scaled(x.z, s, true),
                  fp8x2_bf16_scaled(x.w, s, false), fp8x2_bf16_scaled(x.w, s, true));
}

// Attention of the heads of group hg of sequence b over keys [begin, end);
// writes the normalised partial, its max and its sum to slot.
// Score D layout: lane l holds S^T[MFMA row 4*(l/16)+i (+16)][head l%16]; MFMA
// row m of each 16-key half is tile row key_row(m).  Those 8 values are
// exactly the A operand of P.V for head l%16 when the P.V k-slots 8g..8g+7
// are taken as the keys of rows {4g..4g+3, 16+4g..16+4g+3}; the B operand
// (those keys, 16 latent columns) comes from two transposed LDS reads of the
// key-major tile.  The softmax keeps a per-head reference max and rescales
// the accumulators only when a score exceeds it by more than 8 (log2
// domain), so P stays below 2^8 and rescaling is rare.
// CAUSAL: head s*H + h (query s of S) sees only keys t < n - S + 1 + s; a
// head with no such key in [begin, end) writes a zero partial with max -inf
// and sum 0.
template <bool F8, bool CAUSAL>
__device__ __forceinline__ void mla_segment(const MlaParams& p, int b, int n, int hg, int begin,
                                            int end, int64_t slot,
                                            uint16_t (*crow2)[kTileKeys][kRowPad],
                                            uint16_t (*qlo_s)[kLat + 8]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int hb = hg * kGroup;
  const int nh = min(kGroup, p.num_heads - hb);
  const int h0 = hb + wave * kHeadsPerWave;
  const bool active = wave * kHeadsPerWave < nh;   // waves past the last head only stage tiles
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;

  __syncthreads();   // the previous segment is done with qlo_s and crow

  // Staging of one tile: 32 keys x 72 chunks of 16 B.  Wave w stages keys
  // 8w .. 8w+7, lane l key 8w + l/8 and its chunks l%8 + 8k (k < 9), so each
  // lane resolves one page per tile and the chunk offsets are constants.
  // FP8 rows: lane l loads E4M3 latent chunks l%8 + 8k (k < 4, 16 dims each,
  // block (l%8)/4 + 2k), rope chunk l%8 and the 8 scale bytes.
  // The page of the next tile's key is fetched one tile ahead.
  constexpr int kChunks = F8 ? 5 : kRow / 8 / 8;   // 16-byte loads per lane and tile
  const int skey = wave * 8 + (lane >> 3);
  const int schunk = lane & 7;
  uint4 stage[kChunks];
  uint2 sbytes = make_uint2(0, 0);   // FP8: the row's block-scale bytes
  auto page_of = [&](int t0) -> int {
    const int t = t0 + skey;
    return (t >= begin && t < end) ? bt[t >> p.page_shift] : -1;
  };
  auto load_tile = [&](int t0, int page) {
    if constexpr (F8) {
      const char* src = reinterpret_cast<const char*>(p.cache) +
                        static_cast<int64_t>(max(page, 0)) * p.page_stride +
                        static_cast<int64_t>((t0 + skey) & (p.page_size - 1)) * p.token_stride;
      const uint16_t* lat = reinterpret_cast<const uint16_t*>(src + 16 * schunk);
#pragma unroll
      for (int k = 0; k < 4; ++k) stage[k] = page >= 0 ? load16(lat + 64 * k) : make_uint4(0, 0, 0, 0);
      stage[4] = page >= 0 ? load16(reinterpret_cast<const uint16_t*>(src + kMlaFp8Rope + 16 * schunk))
                           : make_uint4(0, 0, 0, 0);
      sbytes = page >= 0 ? *reinterpret_cast<const uint2*>(src + kMlaFp8Scales) : make_uint2(0, 0);
    } else {
      const uint16_t* src = p.cache + static_cast<int64_t>(max(page, 0)) * p.page_stride +
                            static_cast<int64_t>((t0 + skey) & (p.page_size - 1)) * p.token_stride +
                            schunk * 8;
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
        stage[k] = page >= 0 ? load16(src + 64 * k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](uint16_t (*dst)[kRowPad]) {
    if constexpr (F8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // block (schunk >> 2) + 2k: byte of sbytes.x (k < 2) or sbytes.y
        const uint32_t word = k < 2 ? sbytes.x : sbytes.y;
        const uint32_t sb = (word >> (8 * ((schunk >> 2) + 2 * (k & 1)))) & 0xffu;
        uint4 lo, hi;
        fp8x16_bf16_scaled(stage[k], u2f(sb << 23), lo, hi);
        *reinterpret_cast<uint4*>(&dst[skey][16 * (schunk + 8 * k)]) = lo;
        *reinterpret_cast<uint4*>(&dst[skey][16 * (schunk + 8 * k) + 8]) = hi;
      }
      *reinterpret_cast<uint4*>(&dst[skey][kLat + 8 * schunk]) = stage[4];
    } else {
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
        *reinterpret_cast<uint4*>(&dst[skey][(schunk + 8 * k) * 8]) = stage[k];
    }
  };
  const int first_tile = begin / kTileKeys;
  const int last_tile = (end - 1) / kTileKeys;
  load_tile(first_tile * kTileKeys, page_of(first_tile * kTileKeys));
  int page_next = first_tile < last_tile ? page_of((first_tile + 1) * kTileKeys) : -1;

  // Q^T operand for all 18 k-steps: head h0 + c16, dims 32*ks + 8g .. +8;
  // hi (18 steps) and mid (16 latent steps) in registers, lo in LDS, where
  // each 1 KB row is one direct global->LDS load of the wave (64 lanes x 16 B).
  uint4 qh[kKS], qm[kKSL];
  if (active) {
    const int64_t hrow = static_cast<int64_t>(b) * p.num_heads + h0 + c16;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qh[ks] = load16(p.q_hi + hrow * kRow + 32 * ks + 8 * g);
#pragma unroll
    for (int ks = 0; ks < kKSL; ++ks) qm[ks] = load16(p.q_mid + hrow * kLat + 32 * ks + 8 * g);
  }
  for (int r = wave; r < nh; r += kMlaWaves)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(p.q_lo + (static_cast<int64_t>(b) * p.num_heads + hb + r) * kLat + 8 * lane),
        (__attribute__((address_space(3))) void*)(&qlo_s[r][0]), 16, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  f32x4_t acc[kLat / 16];
#pragma unroll
  for (int jt = 0; jt < kLat / 16; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;     // per head c16 (same on the 4 lanes of the head)
  float l_sum = 0.0f;          // this lane's share of the head's denominator

  // Tiles alternate between two LDS buffers: tile k+1 is stored into the
  // other buffer right after tile k's P.V, so one barrier per tile (at the
  // top: tile k is complete and the other buffer's readers are done) orders
  // everything.
  store_tile(crow2[0]);
  for (int tile = first_tile; tile <= last_tile; ++tile) {
    const int t0 = tile * kTileKeys;
    uint16_t (*crow)[kRowPad] = crow2[(tile - first_tile) & 1];
    uint16_t (*cnext)[kRowPad] = crow2[(tile - first_tile + 1) & 1];
    __syncthreads();
    // The next tile's loads are issued inside the score loop, between MFMAs
    // (waves without heads issue and store them here).
    const bool more = tile < last_tile;
    const int page_now = page_next;
    if (more) page_next = tile + 1 < last_tile ? page_of(t0 + 2 * kTileKeys) : -1;
    if (!active) {
      if (more) {
        load_tile(t0 + kTileKeys, page_now);
        store_tile(cnext);
      }
      continue;
    }

    // scores S^T for keys t0 .. t0+31 (two 16-key M tiles), heads h0 .. h0+15.
    // The LDS operands of step ks+1 are read while the MFMAs of step ks run;
    // the scheduling barriers keep the compiler from hoisting all 18 steps'
    // reads (which would need ~200 more registers).
    f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const uint16_t* arow0 = &crow[key_row(c16)][8 * g];
    const uint16_t* arow1 = &crow[16 + key_row(c16)][8 * g];
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
        sc[0] = mfma(a0, qlv, sc[0]);
        sc[1] = mfma(a1, qlv, sc[1]);
        sc[0] = mfma(a0, qm[ks], sc[0]);
        sc[1] = mfma(a1, qm[ks], sc[1]);
      }
      sc[0] = mfma(a0, qh[ks], sc[0]);
      sc[1] = mfma(a1, qh[ks], sc[1]);
      if (ks == 2 && more) load_tile(t0 + kTileKeys, page_now);
      a0 = n0;
      a1 = n1;
      qlv = nl;
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds keys t0 + 16*mt + key_row(4g + i) for head c16
    float pv[8];
    float cm = -INFINITY;
    const int end_h = CAUSAL ? min(end, n - p.num_queries + 1 + (h0 + c16) / p.w_heads) : end;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * mt + key_row(4 * g + i);
        const float v = (t >= begin && t < end_h) ? sc[mt][i] * p.scale_log2 : -INFINITY;
        pv[4 * mt + i] = v;
        cm = fmaxf(cm, v);
      }
    cm = fmaxf(cm, xor16(cm));
    cm = fmaxf(cm, xor32(cm));
    // move the reference max when a score passes it by more than 8
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
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      e[k] = fast_exp2(pv[k] - base);
      l_sum += e[k];
    }
    uint4 pa_hi, pa_mid, pa_lo;
    split3_bf16x2(e[0], e[1], pa_hi.x, pa_mid.x, pa_lo.x);
    split3_bf16x2(e[2], e[3], pa_hi.y, pa_mid.y, pa_lo.y);
    split3_bf16x2(e[4], e[5], pa_hi.z, pa_mid.z, pa_lo.z);
    split3_bf16x2(e[6], e[7], pa_hi.w, pa_mid.w, pa_lo.w);
    // O[heads][latent] += P . C over the 32 keys of the tile; lane (g, a)
    // points the transposed reads at the rows of keys key_row(4g + a/4) and
    // 16 + key_row(4g + a/4), columns 16*jt + 4*(a%4).
    const int krow = key_row(4 * g + (c16 >> 2));
    const uint16_t* brow0 = &crow[krow][4 * (c16 & 3)];
    const uint16_t* brow1 = &crow[16 + krow][4 * (c16 & 3)];
    // Two N-tiles per step, the next pair's transposed reads in flight, the
    // MFMAs of the pair interleaved so no MFMA waits on the one before it.
    uint2 ka0 = lds_read_tr(brow0), ka1 = lds_read_tr(brow1);
    uint2 kb0 = lds_read_tr(brow0 + 16), kb1 = lds_read_tr(brow1 + 16);
#pragma unroll
    for (int jt = 0; jt < kLat / 16; jt += 2) {
      const uint4 bopa = make_uint4(ka0.x, ka0.y, ka1.x, ka1.y);
      const uint4 bopb = make_uint4(kb0.x, kb0.y, kb1.x, kb1.y);
      if (jt + 2 < kLat / 16) {
        ka0 = lds_read_tr(brow0 + 16 * (jt + 2));
        ka1 = lds_read_tr(brow1 + 16 * (jt + 2));
        kb0 = lds_read_tr(brow0 + 16 * (jt + 3));
        kb1 = lds_read_tr(brow1 + 16 * (jt + 3));
      }
      acc[jt] = mfma(pa_lo, bopa, acc[jt]);
      acc[jt + 1] = mfma(pa_lo, bopb, acc[jt + 1]);
      acc[jt] = mfma(pa_mid, bopa, acc[jt]);
      acc[jt + 1] = mfma(pa_mid, bopb, acc[jt + 1]);
      acc[jt] = mfma(pa_hi, bopa, acc[jt]);
      acc[jt + 1] = mfma(pa_hi, bopb, acc[jt + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store_tile(cnext);
  }
  if (!active) return;

  // denominators: lanes of one head (c16) across the 4 key groups
  l_sum += xor16(l_sum);
  l_sum += xor32(l_sum);
  float lr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lr[i] = __shfl(l_sum, 4 * g + i);
  const int64_t srow = slot * kGroup + wave * kHeadsPerWave;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = p.seg_out + (srow + 4 * g + i) * kLat;
    const float inv = (!CAUSAL || lr[i] > 0.0f) ? 1.0f / lr[i] : 0.0f;
#pragma unroll
    for (int jt = 0; jt < kLat / 16; ++jt) dst[16 * jt + c16] = acc[jt][i] * inv;
  }
  if (g == 0) {
    p.seg_max[srow + c16] = m_ref * kLn2;
    p.seg_sum[srow + c16] = l_sum;
  }
}

template <bool F8, bool CAUSAL>
__global__ __launch_bounds__(kMlaThreads) void mla_split_kernel(const MlaParams p) {
  __shared__ __align__(16) uint16_t crow[2][kTileKeys][kRowPad];
  __shared__ __align__(16) uint16_t qlo_s[kGroup][kLat + 8];
  __shared__ int64_t sh[4];
  __shared__ int sh_b;

  if (threadIdx.x < 64) {
    const int64_t S = mla_total(p.context_lens, p.batch);
    const int64_t T = S * p.groups;
    const int nb = used_blocks(T, p.split_grid, p.min_keys);
    const int i = blockIdx.x;
    const int64_t u0 = T * i / nb;
    int b = p.batch;
    int64_t pre = 0;
    if (i < nb && S > 0) mla_locate(p.context_lens, p.batch, u0 % S, b, pre);
    if (threadIdx.x == 0) {
      sh[0] = S;
      sh[1] = (i < nb) ? u0 : 0;
      sh[2] = (i < nb) ? T * (i + 1) / nb : 0;
      sh[3] = pre;
      sh_b = b;
    }
  }
  __syncthreads();
  const int i = blockIdx.x;
  const int64_t S = sh[0];
  const int64_t u1 = sh[2];
  int64_t u = sh[1];
  if (u >= u1) return;
  int hg = static_cast<int>(u / S);
  int b = sh_b;
  int64_t pre = sh[3];
  while (u < u1) {
    const int64_t row_start = hg * S + pre;
    const int n = p.context_lens[b];
    const int begin = static_cast<int>(u - row_start);
    const int end = static_cast<int>(min(u1 - row_start, static_cast<int64_t>(n)));
    if (end > begin)
      mla_segment<F8, CAUSAL>(p, b, n, hg, begin, end, static_cast<int64_t>(hg) * p.batch + b + i,
                              crow, qlo_s);
    u = row_start + n;
    pre += n;
    if (++b == p.batch) {
      b = 0;
      pre = 0;
      ++hg;
    }
  }
}

// ---- 3. merge of the partials, then out = W_UV[h] . o_lat on MFMA ---------------------
//
// Block (h, bt, s) handles sequences ROWS*bt .. +ROWS (ROWS = 8 or 16) of
// head s*H + h (query s, W_UV[h]; hg below is that head's group): row
// (group hg, b) was cut into pieces by blocks i0 .. i1 of the split
// (recomputed here from the context lengths), whose partials sit in slots
// r + i0 .. r + i1 with r = hg*batch + b.  The max M and the total
// W = sum l_i e^(m_i - M) of a row are wave reductions over its pieces; o_lat
// is the (l_i e^(m_i - M) / W)-weighted sum of the pieces in ascending i
// (eight pieces' loads in flight), written to LDS as three bf16 terms; then
// out[b][dv] = sum_j o_lat[b][j] W_UV[h][dv][j] on MFMA with A = o_lat (rows
// past ROWS zero) and B = W_UV rows, whose 8 consecutive latent dims per lane
// are contiguous in memory; wave w computes dv tile w.  The W_UV loads are
// issued first, so they overlap the merge.  An empty context, or a query that
// sees no key, gives 0.
constexpr int kMergeThreads = 512;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeWts = 64;      // piece weights kept in LDS per row

template <int ROWS>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_uv_kernel(const MlaParams p) {
  static_assert(ROWS == 8 || ROWS == 16, "rows per block");
  __shared__ __align__(16) uint16_t ohi[16][kLat + 8];
  __shared__ __align__(16) uint16_t omid[16][kLat + 8];
  __shared__ __align__(16) uint16_t olo[16][kLat + 8];
  __shared__ float wts[ROWS][kMergeWts];
  __shared__ int64_t sh_slot[ROWS];
  __shared__ int sh_cnt[ROWS];
  __shared__ float sh_m[ROWS], sh_iw[ROWS];
  const int hw = blockIdx.x;                       // head of W_UV
  const int h = blockIdx.z * p.w_heads + hw;       // query head
  const int b0 = blockIdx.y * ROWS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int hg = h / kGroup;
  const int hl = h % kGroup;
  const int nrow = min(ROWS, p.batch - b0);

  // W_UV[h] rows of dv tile `wave`, all 16 k-steps, in flight from the start
  const uint16_t* wuv = p.w_uv + static_cast<int64_t>(hw) * kDv * kLat +
                        static_cast<int64_t>(16 * wave + c16) * kLat + 8 * g;
  uint4 bw[kLat / 32];
#pragma unroll
  for (int ks = 0; ks < kLat / 32; ++ks) bw[ks] = load16(wuv + 32 * ks);

  if (tid < 64) {
    const int64_t S = mla_total(p.context_lens, p.batch);
    const int64_t T = S * p.groups;
    const int nb = used_blocks(T, p.split_grid, p.min_keys);
    // keys of the sequences before b0, then the prefix within the tile
    int64_t before = 0;
    for (int c0 = 0; c0 < b0; c0 += 64) before += (c0 + lane < b0) ? p.context_lens[c0 + lane] : 0;
    before = wave_sum64(before);
    const int64_t len = (lane < nrow) ? p.context_lens[b0 + lane] : 0;
    const int64_t pre = before + wave_scan64(len) - len;
    if (lane < ROWS) {
      int64_t slot = 0;
      int cnt = 0;
      if (lane < nrow && len > 0) {
        const int64_t start = hg * S + pre;
        const int i0 = block_of(start, T, nb);
        const int i1 = block_of(start + len - 1, T, nb);
        slot = static_cast<int64_t>(hg) * p.batch + b0 + lane + i0;
        cnt = i1 - i0 + 1;
      }
      sh_slot[lane] = slot;
      sh_cnt[lane] = cnt;
    }
  }
  if constexpr (ROWS < 16) {   // rows ROWS..15 of the MFMA A operand stay zero
    for (int i = tid; i < (16 - ROWS) * (kLat / 8); i += kMergeThreads) {
      const int r = ROWS + i / (kLat / 8), c8 = (i % (kLat / 8)) * 8;
      *reinterpret_cast<uint4*>(&ohi[r][c8]) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&omid[r][c8]) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&olo[r][c8]) = make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();
  // per row: M and W over its pieces, lanes striding over the pieces (max and
  // sum read together, the first 64 pieces' terms kept); wave w takes rows
  // w, w + 8
#pragma unroll
  for (int bb = wave; bb < ROWS; bb += kMergeWaves) {
    const int cnt = sh_cnt[bb];
    const int64_t slot = sh_slot[bb];
    const bool mine = lane < cnt;
    const float m0 = mine ? p.seg_max[(slot + lane) * kGroup + hl] : -INFINITY;
    const float l0 = mine ? p.seg_sum[(slot + lane) * kGroup + hl] : 0.0f;
    float M = m0;
    for (int k = lane + 64; k < cnt; k += 64) M = fmaxf(M, p.seg_max[(slot + k) * kGroup + hl]);
    M = wave_max(M);
    if (M == -INFINITY) M = 0.0f;   // no piece saw a key: every weight is 0
    float wk = mine ? l0 * __expf(m0 - M) : 0.0f;
    if (mine) wts[bb][lane] = wk;
    for (int k = lane + 64; k < cnt; k += 64)
      wk += p.seg_sum[(slot + k) * kGroup + hl] * __expf(p.seg_max[(slot + k) * kGroup + hl] - M);
    const float W = wave_sum(wk);
    if (lane == 0) {
      sh_m[bb] = M;
      sh_iw[bb] = W > 0.0f ? 1.0f / W : 0.0f;
    }
  }
  __syncthreads();
  // o_lat for ROWS sequences x 512 dims: wave w takes rows w, w + 8; lane l
  // dims 8l .. 8l+8
#pragma unroll
  for (int bb = wave; bb < ROWS; bb += kMergeWaves) {
    const int d0 = lane * 8;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    const int cnt = sh_cnt[bb];
    const int64_t slot = sh_slot[bb];
    const float M = sh_m[bb], iw = sh_iw[bb];
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float4 v[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t srow = (slot + min(k0 + u, cnt - 1)) * kGroup + hl;
        v[u][0] = *reinterpret_cast<const float4*>(p.seg_out + srow * kLat + d0);
        v[u][1] = *reinterpret_cast<const float4*>(p.seg_out + srow * kLat + d0 + 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        const int64_t srow = (slot + min(k, cnt - 1)) * kGroup + hl;
        const float w = k < cnt ? (k < kMergeWts ? wts[bb][k]
                                                 : p.seg_sum[srow] * __expf(p.seg_max[srow] - M)) * iw
                                : 0.0f;
        o[0] = fmaf(w, v[u][0].x, o[0]);
        o[1] = fmaf(w, v[u][0].y, o[1]);
        o[2] = fmaf(w, v[u][0].z, o[2]);
        o[3] = fmaf(w, v[u][0].w, o[3]);
        o[4] = fmaf(w, v[u][1].x, o[4]);
        o[5] = fmaf(w, v[u][1].y, o[5]);
        o[6] = fmaf(w, v[u][1].z, o[6]);
        o[7] = fmaf(w, v[u][1].w, o[7]);
      }
    }
    uint16_t h8[8], m8[8], l8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split3_bf16(o[e], h8[e], m8[e], l8[e]);
    *reinterpret_cast<uint4*>(&ohi[bb][d0]) = make_uint4(pack_bf16(h8[0], h8[1]), pack_bf16(h8[2], h8[3]),
                                                         pack_bf16(h8[4], h8[5]), pack_bf16(h8[6], h8[7]));
    *reinterpret_cast<uint4*>(&omid[bb][d0]) = make_uint4(pack_bf16(m8[0], m8[1]), pack_bf16(m8[2], m8[3]),
                                                          pack_bf16(m8[4], m8[5]), pack_bf16(m8[6], m8[7]));
    *reinterpret_cast<uint4*>(&olo[bb][d0]) = make_uint4(pack_bf16(l8[0], l8[1]), pack_bf16(l8[2], l8[3]),
                                                         pack_bf16(l8[4], l8[5]), pack_bf16(l8[6], l8[7]));
  }
  __syncthreads();
  // out[b][dv]: wave w takes dv tile w
  f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kLat / 32; ++ks) {
    const uint4 a_hi = *reinterpret_cast<const uint4*>(&ohi[c16][32 * ks + 8 * g]);
    const uint4 a_mid = *reinterpret_cast<const uint4*>(&omid[c16][32 * ks + 8 * g]);
    const uint4 a_lo = *reinterpret_cast<const uint4*>(&olo[c16][32 * ks + 8 * g]);
    c = mfma(a_lo, bw[ks], c);
    c = mfma(a_mid, bw[ks], c);
    c = mfma(a_hi, bw[ks], c);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bb = 4 * g + i;
    if (bb < nrow)
      p.out[(static_cast<int64_t>(b0 + bb) * p.num_heads + h) * kDv + 16 * wave + c16] =
          f32_to_bf16_rne(c[i]);
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

}  // extern "C"

namespace {

int mla_decode_impl(const void* q_nope, const void* q_rope, const void* kv_cache,
                    const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                    const int32_t* block_table, int32_t block_table_stride,
                    const int32_t* context_lens, int32_t batch, int32_t num_heads,
                    int32_t max_pages_per_seq, float scale, int32_t partition_size, void* out,
                    void* workspace, size_t workspace_bytes, void* stream, bool fp8,
                    int32_t num_queries, bool causal) {
  int rc = pa::check_mla(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out, fp8, num_queries);
  if (rc) return rc;
  const int32_t qheads = num_queries * num_heads;   // query heads per sequence
  pa::MlaPlan plan;
  if (!pa::plan_mla(batch, qheads, max_pages_per_seq, cache->page_size, partition_size, &plan))
    return pa::fail(PA_ERR_SHAPE, "no launch plan for these shapes");
  if (!workspace || workspace_bytes < plan.bytes)
    return pa::fail(PA_ERR_WORKSPACE, "workspace must hold mla_absorbed_decode_workspace_size() = " +
                                          std::to_string(plan.bytes) + " bytes (num_heads " +
                                          std::to_string(qheads) + ")");
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
  p.seg_out = reinterpret_cast<float*>(ws + plan.off_seg_out);
  p.seg_max = reinterpret_cast<float*>(ws + plan.off_seg_max);
  p.seg_sum = reinterpret_cast<float*>(ws + plan.off_seg_sum);
  p.out = static_cast<uint16_t*>(out);
  p.page_stride = cache->page_stride;
  p.token_stride = static_cast<int32_t>(cache->token_stride);
  p.bt_stride = block_table_stride;
  p.batch = batch;
  p.num_heads = qheads;
  p.w_heads = num_heads;
  p.num_queries = num_queries;
  p.abs_rows = batch * num_queries;
  p.groups = plan.groups;
  p.page_size = cache->page_size;
  int shift = 0;
  while ((1 << shift) < cache->page_size) ++shift;
  p.page_shift = shift;
  // The split's block count is fixed by the build, not the device (so are the
  // results): kSplitCUs blocks for 256 compute units.
  const int cus = pa::kSplitCUs;
  // Explicit partition size: about that many keys per block.  Library choice:
  // one block per CU (a multiple of 16, so the head groups of a key range
  // share an XCD), each block at least kMlaMinKeys keys.
  if (partition_size > 0) {
    p.split_grid = plan.max_blocks;
    p.min_keys = partition_size;
  } else {
    p.split_grid = std::max(16, std::min(plan.max_blocks, cus / 16 * 16));
    p.min_keys = pa::kMlaMinKeys;
  }
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::clear_error();
  const int btiles = (p.abs_rows + 16 * pa::kAbsTiles - 1) / (16 * pa::kAbsTiles);
  hipLaunchKernelGGL(pa::mla_absorb_kernel, dim3(num_heads, pa::kMlaLat / 128, btiles), dim3(256),
                     0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("absorb: ") + hipGetErrorString(e));
  // one query, or no mask: every head sees the whole context
  const bool masked = causal && num_queries > 1;
  const dim3 sg(p.split_grid), st(pa::kMlaThreads);
  if (fp8 && masked)
    hipLaunchKernelGGL((pa::mla_split_kernel<true, true>), sg, st, 0, s, p);
  else if (fp8)
    hipLaunchKernelGGL((pa::mla_split_kernel<true, false>), sg, st, 0, s, p);
  else if (masked)
    hipLaunchKernelGGL((pa::mla_split_kernel<false, true>), sg, st, 0, s, p);
  else
    hipLaunchKernelGGL((pa::mla_split_kernel<false, false>), sg, st, 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("split: ") + hipGetErrorString(e));
  // 16 sequences per merge block (a full MFMA tile, W_UV read half as often)
  // when that still gives a block per CU, else 8
  if (static_cast<int64_t>(num_heads) * num_queries * ((batch + 15) / 16) >= cus)
    hipLaunchKernelGGL(pa::mla_merge_uv_kernel<16>,
                       dim3(num_heads, (batch + 15) / 16, num_queries), dim3(pa::kMergeThreads),
                       0, s, p);
  else
    hipLaunchKernelGGL(pa::mla_merge_uv_kernel<8>,
                       dim3(num_heads, (batch + 7) / 8, num_queries), dim3(pa::kMergeThreads),
                       0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("merge: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

int mla_absorbed_decode(const void* q_nope, const void* q_rope, const void* kv_cache,
                        const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                        const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* context_lens, int32_t batch, int32_t num_heads,
                        int32_t max_pages_per_seq, float scale, int32_t partition_size, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_impl(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out, workspace, workspace_bytes, stream, false, 1,
                         false);
}

int mla_absorbed_decode_fp8(const void* q_nope, const void* q_rope, const void* kv_cache,
                            const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                            const int32_t* block_table, int32_t block_table_stride,
                            const int32_t* context_lens, int32_t batch, int32_t num_heads,
                            int32_t max_pages_per_seq, float scale, int32_t partition_size,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_impl(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out, workspace, workspace_bytes, stream, true, 1,
                         false);
}

int mla_absorbed_decode_multiquery(const void* q_nope, const void* q_rope, const void* kv_cache,
                                   const pa_kv_layout* cache, const void* w_uk, const void* w_uv,
                                   const int32_t* block_table, int32_t block_table_stride,
                                   const int32_t* context_lens, int32_t batch, int32_t num_heads,
                                   int32_t num_queries, int32_t causal, int32_t max_pages_per_seq,
                                   float scale, int32_t partition_size, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return mla_decode_impl(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out, workspace, workspace_bytes, stream, false,
                         num_queries, causal != 0);
}

int mla_absorbed_decode_multiquery_fp8(const void* q_nope, const void* q_rope,
                                       const void* kv_cache, const pa_kv_layout* cache,
                                       const void* w_uk, const void* w_uv,
                                       const int32_t* block_table, int32_t block_table_stride,
                                       const int32_t* context_lens, int32_t batch,
                                       int32_t num_heads, int32_t num_queries, int32_t causal,
                                       int32_t max_pages_per_seq, float scale,
                                       int32_t partition_size, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return mla_decode_impl(q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                         block_table_stride, context_lens, batch, num_heads, max_pages_per_seq,
                         scale, partition_size, out, workspace, workspace_bytes, stream, true,
                         num_queries, causal != 0);
}

}  // extern "C"
