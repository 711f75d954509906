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
// (v_mfma_f32_32x32x16_bf16): per 32-key tile and 32-head column block,
// S^T[32 keys x 32 heads] = C[32 x 576] . Q^T, and O[32 heads x 512] += P[32 x
// 32 keys] . C[32 x 512].  The cache and W_UV are exact bf16; each fp32 operand
// (q_abs, P, o_lat) enters as three bf16 terms hi + mid + lo, which represent
// an fp32 value exactly (3 x 8 significant bits), so the MFMAs multiply the
// fp32 operands exactly and only the fp32 accumulation rounds, at three MFMAs
// instead of one.
//
// Work split: heads form groups of 64 (one block = 4 waves: two wave pairs of
// 32 heads, the two waves of a pair splitting the latent dims); a row is
// (head group, sequence), ordered group-major.  The keys of all rows, laid end
// to end (T = groups * sum of context lengths), are cut into nb equal
// contiguous ranges, one per block; a block writes one partial per row piece
// it covers.
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
#include <type_traits>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_mfma.h"
#include "pa_profile.h"
#include "pa_validate.h"

namespace pa {

constexpr int kLat = kMlaLat;      // 512
constexpr int kRow = kMlaRow;      // 576
constexpr int kNope = kMlaNope;    // 128
constexpr int kRope = kMlaRope;    // 64
constexpr int kDv = kMlaDv;        // 128
constexpr int kTileKeys = kMlaTileKeys;   // keys per LDS tile
constexpr int kMlaWaves = 4;       // two wave pairs of 32 heads
constexpr int kGroup = 64;         // heads per block
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaDeadBit = 0x40000000;   // OR-ed into a dead key's offset: past any page
static_assert(kGroup == kMlaBlockHeads, "head group size");

struct MlaSplit;

// The partial slots of one (head group, sequence) row: slot .. slot + cnt - 1,
// in ascending key order.
struct MlaRowSlots {
  int64_t slot;
  int32_t cnt;
  int32_t pad;
};

struct MlaParams {
  const uint16_t* q_nope;
  const uint16_t* q_rope;
  const uint16_t* cache;
  const uint16_t* w_uk;
  const uint16_t* w_uv;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* q_hi;          // q_abs | q_rope, first terms (the split kernel's operand order)
  uint16_t* q_mid;         // second and third terms of q_abs
  uint16_t* q_lo;
  float* seg_out;          // [slots][64][512] partial o_lat, unnormalised: sum of P V
  float* seg_max;          // [slots][64] natural-log-domain reference max
  float* seg_sum;          // [slots][64] sum of exp(s - max)
  MlaSplit* split_plan;    // the split plan, written by the absorb kernel
  MlaRowSlots* row_slots;  // [groups][batch], written with it
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
  int32_t split_grid;      // blocks launched for the split kernel (and partial slots)
  int32_t min_tiles;       // fewest 32-key tiles a piece of a row is given
  int32_t explicit_size;   // the caller fixed the piece size (min_tiles tiles)
  float scale_log2;
};

// q_abs (three bf16 terms) and q_rope in the workspace, in the split kernel's
// operand order: for sequence b, 32-head tile ht (heads 32ht .. +32 of the
// S*H heads), half d of the dims and k-step ks, the 16-byte pieces of the 64
// lanes in one 1 KB run.  Lane c + 32hh holds head 32ht + c, dims 256d + 16ks
// + 8hh .. +8 of the latent part (ks < 16) or, in the hi term only, rope dims
// 32d + 16(ks - 16) + 8hh .. +8 (ks = 16, 17), and sits at position 2c + hh
// of the run.  Each q load of the split kernel then reads one 1 KB run, and
// the absorption writes each head's two pieces of a run as 32 contiguous
// bytes.  Offset of a piece in 16-byte chunks (pos = 2c + hh):
constexpr int kQHiSteps = kMlaLat / 32 + kMlaRope / 32;   // 18: latent and rope k-steps
constexpr int kQLoSteps = kMlaLat / 32;                   // 16
__device__ __forceinline__ int64_t q_piece(int64_t tile, int half, int ks, int pos, int steps) {
  return ((tile * 2 + half) * steps + ks) * 64 + pos;
}

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

__device__ void mla_write_plan(const MlaParams& p);

// One more slice of blocks (x = H) holds the block that plans the split
// kernel's work once per call (the split and merge kernels read the plan).
__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p) {
  if (blockIdx.x == p.w_heads) {
    if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 64) mla_write_plan(p);
    return;
  }
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
    // (q row r = b S + s, head h: head s H + h of sequence b)
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int e = t + 256 * k;
      const int term = e >> 8, bb = (e >> 4) & 15, ch = e & 15;
      if (bb < nb) {
        const int r = b0 + bb, sb = r / p.num_queries;
        const int vh = (r - sb * p.num_queries) * p.w_heads + h;
        const int j = jq * 128 + 8 * ch;            // latent dims j .. j+7
        const int64_t tile = static_cast<int64_t>(sb) * ((p.num_heads + 31) >> 5) + (vh >> 5);
        const int64_t at = q_piece(tile, j >> 8, (j & 255) >> 4, 2 * (vh & 31) + ((j >> 3) & 1),
                                   term == 0 ? kQHiSteps : kQLoSteps);
        uint16_t* dst = term == 0 ? p.q_hi : (term == 1 ? p.q_mid : p.q_lo);
        *reinterpret_cast<uint4*>(dst + 8 * at) = *reinterpret_cast<const uint4*>(&os[term][bb][8 * ch]);
      }
    }
    __syncthreads();   // os is rewritten by the next tile
    if (jq == 0 && t < nb * (kRope / 8)) {   // rope part: exact bf16, one term
      const int rb = t / (kRope / 8), rc = t % (kRope / 8);
      const int r = b0 + rb, sb = r / p.num_queries;
      const int vh = (r - sb * p.num_queries) * p.w_heads + h;
      const int64_t row = static_cast<int64_t>(r) * p.w_heads + h;
      const int jr = 8 * rc;                       // rope dims jr .. jr+7
      const int64_t tile = static_cast<int64_t>(sb) * ((p.num_heads + 31) >> 5) + (vh >> 5);
      const int64_t at = q_piece(tile, jr >> 5, kQLoSteps + ((jr & 31) >> 4),
                                 2 * (vh & 31) + ((jr >> 3) & 1), kQHiSteps);
      *reinterpret_cast<uint4*>(p.q_hi + 8 * at) = load16(p.q_rope + row * kRope + 8 * rc);
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < kNope / 32; ++ks) qa[ks] = qn[ks];
    }
  }
}

// ---- 2. split attention over the latent cache ----------------------------------------

// Two ways to cut the work of the split kernel, chosen per call from the
// context lengths alone (deterministic, the same on every device), both
// merged by log-sum-exp in ascending key order:
//
// Pieces of rows: row (group hg, sequence b) of T_b = ceil(ctx_b / 32) tiles
// is cut into n_b = ceil(T_b / L) pieces, piece j taking tiles
// [j T_b / n_b, (j+1) T_b / n_b), the same for every group.  Group hg's
// pieces are blocks (and partial slots) hg*N .. hg*N + N - 1, sequence b's
// from the prefix sum of n_{b' < b}, with N = sum_b n_b rounded up to a
// multiple of 8 (the groups' pieces of one key range then sit on one XCD).
// L is the least tile count >= lmin whose pieces fit in nb blocks.  Every
// block owns one range of one row: no block pays for a second row's start
// (q loads, a drained and refilled tile pipeline, a second partial), which
// costs about as much as three or four tiles.
//
// The key line: the keys of all rows laid end to end (group-major), cut into
// equal ranges, one per block, so a block may cover the end of one row and
// the start of the next; segment (row r, block i) writes slot r + i.  Taken
// at the library's choice when rows are too few for even pieces (the largest
// piece more than kMlaRowSlack tiles above the mean), as in a multi-query
// verify whose many head groups leave two or three blocks per row.
constexpr int kMlaRowSlack = 3;
// Key line: units before each row's keys that stand for its prologue (q
// terms, the tile pipeline's refill, one more partial), so a block whose
// range starts several rows gets fewer keys.
constexpr int kMlaRowCost = 64;

struct MlaSplit {
  bool rows;   // pieces of rows, else the key line
  int L;       // pieces of rows: tiles per piece, at most
  int N;       // pieces of rows: blocks per head group (0: no key anywhere)
  int64_t S;   // key line: units per group (each row's keys after kMlaRowCost units)
  int nb;      // key line: blocks used
};

__device__ __forceinline__ int mla_tiles(const int32_t* ctx, int b) { return (ctx[b] + 31) >> 5; }

// explicit: the caller fixed the piece size (lmin tiles): pieces of rows.
__device__ __forceinline__ MlaSplit mla_plan(const int32_t* ctx, int batch, int groups, int lmin,
                                             int nb, bool explicit_size) {
  const int lane = threadIdx.x & 63;
  int64_t tiles = 0, keys = 0;
  int tmax = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int t = (b0 + lane < batch) ? mla_tiles(ctx, b0 + lane) : 0;
    const int n = (b0 + lane < batch) ? ctx[b0 + lane] : 0;
    keys += n > 0 ? n + kMlaRowCost : 0;   // units of the key line
    tiles += t;
    tmax = max(tmax, t);
  }
  tiles = wave_sum64(tiles);
  keys = wave_sum64(keys);
  tmax = static_cast<int>(wave_max(static_cast<float>(tmax)));   // exact below 2^24
  // the first 64 rows' tile counts stay in a register: the search below
  // evaluates pieces() a dozen times, and a pass over the lengths in memory
  // would put a dependent global load in each
  const int t_first = lane < batch ? mla_tiles(ctx, lane) : 0;
  auto pieces = [&](int L) {          // blocks per head group for L tiles per piece
    float n = static_cast<float>((t_first + L - 1) / L);   // counts below 2^24: the float sum is exact
    for (int b0 = 64; b0 < batch; b0 += 64)
      n += (b0 + lane < batch) ? static_cast<float>((mla_tiles(ctx, b0 + lane) + L - 1) / L) : 0.0f;
    return (static_cast<int64_t>(wave_sum(n)) + 7) / 8 * 8;
  };
  auto fits = [&](int L) { return groups * pieces(L) <= nb; };
  int lo = static_cast<int>(max<int64_t>(lmin, (groups * tiles + nb - 1) / nb));
  int L = lo;
  if (tmax > 0 && !fits(lo)) {        // gallop, then bisect: fits(lo) false, fits(hi) true
    int step = max(1, lo / 8);
    int hi = lo + step;
    while (hi < tmax && !fits(hi)) {
      lo = hi;
      step *= 2;
      hi = lo + step;
    }
    if (hi >= tmax) hi = tmax;        // one piece per row fits (the host sizes the grid so)
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      if (fits(mid)) hi = mid;
      else lo = mid;
    }
    L = hi;
  }
  MlaSplit sp{true, L, tmax > 0 ? static_cast<int>(pieces(L)) : 0, keys, 0};
  const int64_t mean = (groups * tiles + nb - 1) / nb;
  if (!explicit_size && L > mean + kMlaRowSlack) {
    sp.rows = false;
    sp.nb = used_blocks(groups * keys, nb, int64_t{kMlaMinKeys});
  }
  return sp;
}

// The split plan of this call, written once to the workspace.  Called by a
// whole wave.
__device__ void mla_write_plan(const MlaParams& p) {
  const MlaSplit sp = mla_plan(p.context_lens, p.batch, p.groups, p.min_tiles, p.split_grid,
                               p.explicit_size);
  const int lane = threadIdx.x & 63;
  if (lane == 0) *p.split_plan = sp;
  // each row's partial slots: pieces of rows, slots hg N + (pieces before b)
  // .. + n_b - 1; the key line, slots hg B + b + i for the blocks i0 .. i1
  // whose ranges cut the row
  int64_t before = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < p.batch ? p.context_lens[b] : 0;
    // pieces of the row, or its units on the key line
    const int64_t a = sp.rows ? ((n + 31) / 32 + sp.L - 1) / sp.L : (n > 0 ? n + kMlaRowCost : 0);
    const int64_t pre = before + wave_scan64(a) - a;
    before += wave_sum64(a);
    if (b < p.batch) {
      for (int hg = 0; hg < p.groups; ++hg) {
        MlaRowSlots r{0, 0, 0};
        if (sp.rows) {
          r.slot = static_cast<int64_t>(hg) * sp.N + pre;
          r.cnt = static_cast<int32_t>(a);
        } else if (n > 0) {
          const int64_t T = sp.S * p.groups;
          const int64_t start = hg * sp.S + pre + kMlaRowCost;   // the row's first key
          const int i0 = block_of(start, T, sp.nb);
          const int i1 = block_of(start + n - 1, T, sp.nb);
          r.slot = static_cast<int64_t>(hg) * p.batch + b + i0;
          r.cnt = i1 - i0 + 1;
        }
        p.row_slots[static_cast<int64_t>(hg) * p.batch + b] = r;
      }
    }
  }
}

// Sequence b holding key y (0 <= y < S) of a group's key line, and the keys
// before it.  Called by a whole wave.
// c_first: this lane's context length among the first 64 (0 past the batch).
__device__ __forceinline__ void mla_locate(const int32_t* ctx, int batch, int64_t y, int c_first,
                                           int& b_out, int64_t& pre_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int64_t n = b0 == 0 ? c_first : ((b0 + lane < batch) ? ctx[b0 + lane] : 0);
    const int64_t len = n > 0 ? n + kMlaRowCost : 0;   // the row's units
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


// Sequence b whose pieces hold piece k (0 <= k < sum_b n_b) of a head group,
// and the pieces before b.  Called by a whole wave; b = batch past the last.
// c_first: this lane's context length among the first 64 (0 past the batch).
__device__ __forceinline__ void mla_piece_row(const int32_t* ctx, int batch, int L, int k,
                                              int c_first, int& b_out, int& pre_out) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int t = b0 == 0 ? (c_first + 31) >> 5 : ((b0 + lane < batch) ? mla_tiles(ctx, b0 + lane) : 0);
    const int n = (t + L - 1) / L;
    const int incl = static_cast<int>(wave_scan64(n));
    const uint64_t hit = __ballot(base + incl > k);
    if (hit) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      b_out = b0 + l;
      pre_out = base + __shfl(incl, l) - __shfl(n, l);
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

// Split-kernel geometry.  A block's 64-head group is two wave pairs; pair w/2
// takes heads 32 (w/2) .. +32 (one 32x32 MFMA column block), and within a pair
// wave half d = w % 2 holds latent dims 256d .. 256d+255 and rope dims
// 512 + 32d .. +32 of q and of the output accumulators.
constexpr int kPairHeads = 32;
constexpr int kHalfLat = kLat / 2;                       // 256
constexpr int kHalfRope = kRope / 2;                     // 32
constexpr int kLatSteps = kHalfLat / 16;                 // 16 score k-steps (32x32x16)
constexpr int kRopeSteps = kHalfRope / 16;               // 2
constexpr int kDimTiles = kHalfLat / 32;                 // 8 P.V output tiles of 32 dims
constexpr int kRowChunks = kRow / 8;                     // 72 16-byte chunks per 576-wide row
constexpr int kTileElems = kTileKeys * kRow;             // one LDS tile, bf16 elements
constexpr int kWaveLoads = kTileElems * 2 / 1024 / kMlaWaves;   // 9 one-KB wave loads per tile
constexpr int kTileBufs = 3;

// LDS position (in 16-byte chunks) of chunk c of tile row r: rows of 72
// chunks back to back, c's low three bits XOR-ed with swz(r).  The 8 rows a
// score read serves per LDS cycle get 8 distinct swz values, and the 4 rows
// x 2 chunks of a 16-lane transposed read get 8 distinct bank groups (even
// swz for rows 0-3 of an 8-row block, odd for rows 4-7), so both read forms
// run without bank conflicts (32 banks of 4 bytes; measured).
__device__ __forceinline__ int swz(int r) { return 2 * (r & 3) + ((r >> 2) & 1); }

// Value of lane l ^ 32 combined with this lane's: v_permlane32_swap exchanges
// the two 32-lane halves of a register pair (a VALU operation, no LDS).
__device__ __forceinline__ float xhalf(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  // lanes 0-31 receive lane l + 32 in r[1], lanes 32-63 lane l - 32 in r[0]
  return u2f((threadIdx.x & 32) ? r[0] : r[1]);
}

// Keeps x computed at this point: an empty asm that reads it.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// x *= f for an accumulator element held in an AGPR, through one temporary
// VGPR: the rare rescale of the 128 accumulators then needs no VGPR copy of
// them (VALU instructions cannot read AGPRs).
__device__ __forceinline__ void scale_in_agpr(float& x, float f) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(x), "=&v"(t)
      : "v"(f));
}

struct MlaSplitLds {
  uint16_t tile[kTileBufs][kTileElems];
  f32x4_t xs[2][kMlaWaves][4][64];   // partial scores of each wave, double-buffered
};

// Attention of the heads of group hg of sequence b over keys [begin, end);
// writes the unnormalised partial (sum over the keys of P V, P = e^(s - max)),
// its max and its sum to slot.
//
// Per 32-key tile t0 .. t0+31, wave (pair, half):
//   scores   S^T[32 keys x 32 heads] over the wave's dims on
//            v_mfma_f32_32x32x16_bf16: A = cache rows from LDS (lane c: key c,
//            8 dims), B = q (lane: head c, 8 dims), 16 latent k-steps x 3 q
//            terms + 2 rope k-steps.  The two halves of a pair trade partials
//            through LDS and add them: a + b = b + a exactly, so both hold the
//            same scores bit for bit, and the same softmax state.
//   softmax  D element i of lane l is key t0 + 8(i/4) + 4(l/32) + i%4 of head
//            l%32; lazy reference max (moves when passed by more than 8 in the
//            log2 domain, P <= 2^8), P split in three bf16 terms.
//   P.V      O[32 heads x 256 dims] += P[32 x 32 keys] . C[32 keys x 256]: 8 dim
//            tiles x 2 k-steps x 3 P terms.  The P registers are the A operand
//            as they stand when k-slot 8h + j of k-step kk is taken as key
//            16kk + 4h + j (j < 4) or 16kk + 8 + 4h + (j - 4); the B operand is
//            two transposed LDS reads (ds_read_b64_tr_b16) of those key rows.
// Pipeline: iteration it computes the scores of tile it and the softmax and
// P.V of tile it-1; tile it+1 is loaded during iteration it straight from
// global memory into its LDS buffer (buffer_load ... lds, whose buffer range
// turns dead keys into zeros), three tiles resident; one barrier per
// iteration orders the tile loads, the partial-score exchange and the reuse
// of buffers.  FP8 rows are widened in registers and stored at the end of
// the iteration instead.
// CAUSAL: head s*H + h (query s of S) sees only keys t < n - S + 1 + s; a
// head with no such key in [begin, end) writes a zero partial with max -inf
// and sum 0.
template <bool F8, bool CAUSAL>
__device__ __forceinline__ void mla_segment(const MlaParams& p, int b, int n, int hg, int begin,
                                            int end, int64_t slot, MlaSplitLds& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int c = lane & 31;
  const int hh = lane >> 5;
  const int hb = hg * kGroup;
  const int nh = min(kGroup, p.num_heads - hb);
  const bool active = pair * kPairHeads < nh;      // pairs past the last head only load tiles
  const int h0 = hb + pair * kPairHeads;
  const bool head_ok = pair * kPairHeads + c < nh;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;

  __syncthreads();   // the previous segment is done with the tiles and partials

  const int first_tile = begin / kTileKeys;
  const int ntiles = (end - 1) / kTileKeys - first_tile + 1;
  const int token_bytes = p.token_stride * (F8 ? 1 : 2);

  // ---- page table: lane l holds the physical page of logical page pbase + l ----
  // (entries past the segment's last page read as 0; reloaded when a tile
  // reaches beyond the 64 pages held, so no tile load waits on the table)
  const int plast = (end - 1) >> p.page_shift;
  int pbase = (first_tile * kTileKeys) >> p.page_shift;
  auto load_ptab = [&](int base) {
    const int pi = base + lane;
    return pi <= plast ? bt[pi] : 0;
  };
  int ptab = load_ptab(pbase);
  auto ensure_ptab = [&](int t0) {     // wave-uniform
    if ((((t0 + kTileKeys - 1) >> p.page_shift) - pbase) >= 64) {
      pbase = t0 >> p.page_shift;
      ptab = load_ptab(pbase);
    }
  };

  // ---- tile loads ----
  // bf16 rows: wave load u = 9w + j (j < 9) fills LDS chunks 64u .. 64u+63 of
  // the tile; lane i brings the chunk that belongs at position 64u + i.  Waves
  // 0 and 1 fill rows 0..15, waves 2 and 3 rows 16..31, so each wave reads one
  // page (16-key pages included) through that page's buffer range.
  // chunk offsets of this lane's loads within its half-tile (tile-independent)
  const int hf = wave >> 1;
  int lvoff[kWaveLoads];
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int pos = 64 * (kWaveLoads * wave + j) + lane;
    const int r = pos / kRowChunks;
    lvoff[j] = (r - 16 * hf) * token_bytes + 16 * ((pos - r * kRowChunks) ^ swz(r));
  }
  // One tile's loads: set up (page, buffer range, dead-key offsets) once,
  // then load j of 9, issued between the MFMAs of the score k-steps.
  struct TileLoad {
    __amdgpu_buffer_rsrc_t rs;
    int soff, buf;
  } tl_next;
  auto setup_tile = [&](int it) {
    const int t0 = (first_tile + it) * kTileKeys;
    ensure_ptab(t0);
    const int k0 = t0 + 16 * hf;
    const int page = __builtin_amdgcn_readlane(ptab, (k0 >> p.page_shift) - pbase);
    const char* pg = reinterpret_cast<const char*>(p.cache) +
                     static_cast<int64_t>(page) * p.page_stride * 2;
    tl_next.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(pg), static_cast<short>(0),
                                                   (p.page_size - 1) * token_bytes + kRow * 2,
                                                   0x00020000);
    tl_next.soff = (k0 & (p.page_size - 1)) * token_bytes;
    tl_next.buf = it % kTileBufs;
    if (!(k0 >= begin && k0 + 16 <= end)) {   // wave-uniform: an edge tile
#pragma unroll
      for (int j = 0; j < kWaveLoads; ++j) {
        const int key = t0 + (64 * (kWaveLoads * wave + j) + lane) / kRowChunks;
        lvoff[j] = (lvoff[j] & ~kMlaDeadBit) | ((key >= begin && key < end) ? 0 : kMlaDeadBit);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kWaveLoads; ++j) lvoff[j] &= ~kMlaDeadBit;
    }
  };
  auto load_part = [&](int j) {
    const int u = kWaveLoads * wave + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        tl_next.rs, (__attribute__((address_space(3))) void*)(&sm.tile[tl_next.buf][512 * u]), 16,
        lvoff[j], tl_next.soff, 0, 0);
  };
  auto issue_tile = [&](int it) {
    setup_tile(it);
#pragma unroll
    for (int j = 0; j < kWaveLoads; ++j) load_part(j);
  };
  // FP8 rows, staged in registers: lane l takes key 8w + l/8 and its latent
  // E4M3 chunks l%8 + 8k (k < 4, 16 dims each), rope chunk l%8 and the
  // row's 8 scale bytes; dead keys stage zeros.
  const int skey = wave * 8 + (lane >> 3);
  const int schunk = lane & 7;
  uint4 stage[F8 ? 5 : 1];
  uint2 sbytes = make_uint2(0, 0);
  auto stage_tile = [&](int it) {
    if constexpr (F8) {
      const int t0 = (first_tile + it) * kTileKeys;
      ensure_ptab(t0);
      const int t = t0 + skey;
      const bool live = t >= begin && t < end;
      const int page = __shfl(ptab, (t >> p.page_shift) - pbase);
      const char* src = reinterpret_cast<const char*>(p.cache) +
                        static_cast<int64_t>(page) * p.page_stride +
                        static_cast<int64_t>(t & (p.page_size - 1)) * p.token_stride;
      const uint16_t* lat = reinterpret_cast<const uint16_t*>(src + 16 * schunk);
#pragma unroll
      for (int k = 0; k < 4; ++k) stage[k] = live ? load16(lat + 64 * k) : make_uint4(0, 0, 0, 0);
      stage[4] = live ? load16(reinterpret_cast<const uint16_t*>(src + kMlaFp8Rope + 16 * schunk))
                      : make_uint4(0, 0, 0, 0);
      sbytes = live ? *reinterpret_cast<const uint2*>(src + kMlaFp8Scales) : make_uint2(0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (F8) {
      uint4* row = reinterpret_cast<uint4*>(&sm.tile[buf][skey * kRow]);
      const int sw = swz(skey);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // block (schunk >> 2) + 2k: byte of sbytes.x (k < 2) or sbytes.y
        const uint32_t word = k < 2 ? sbytes.x : sbytes.y;
        const uint32_t sb = (word >> (8 * ((schunk >> 2) + 2 * (k & 1)))) & 0xffu;
        uint4 lo, hi;
        fp8x16_bf16_scaled(stage[k], u2f(sb << 23), lo, hi);
        const int c0 = 2 * (schunk + 8 * k);
        row[c0 ^ sw] = lo;
        row[(c0 + 1) ^ sw] = hi;
      }
      row[(kLat / 8 + schunk) ^ sw] = stage[4];
    }
  };

  // ---- q: B operand of the scores, head h0 + c, dims of this wave's half ----
  // (the workspace holds them in this order: each load is 1 KB in one piece)
  uint4 qh[kLatSteps + kRopeSteps], qm[kLatSteps], ql[kLatSteps];
  {
    static_assert(kQHiSteps == kLatSteps + kRopeSteps && kQLoSteps == kLatSteps, "q layout");
    const int64_t tile = static_cast<int64_t>(b) * ((p.num_heads + 31) >> 5) + (h0 >> 5);
    const int pos = 2 * c + hh;
    const uint16_t* qhi = p.q_hi + 8 * q_piece(tile, half, 0, pos, kQHiSteps);
    const uint16_t* qmid = p.q_mid + 8 * q_piece(tile, half, 0, pos, kQLoSteps);
    const uint16_t* qlo = p.q_lo + 8 * q_piece(tile, half, 0, pos, kQLoSteps);
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kLatSteps; ++ks) {
      qh[ks] = head_ok ? load16(qhi + 512 * ks) : z;
      qm[ks] = head_ok ? load16(qmid + 512 * ks) : z;
      ql[ks] = head_ok ? load16(qlo + 512 * ks) : z;
    }
#pragma unroll
    for (int ks = kLatSteps; ks < kLatSteps + kRopeSteps; ++ks) qh[ks] = head_ok ? load16(qhi + 512 * ks) : z;
  }

  // ---- per-lane LDS addresses (bytes within a tile) ----
  // score A operand: row c, chunk 32*half + 2ks + hh (latent), 64 + 4*half + 2ks + hh (rope)
  int sa[4], sr[kRopeSteps];
  {
    const int sw = swz(c);
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[r] = 16 * (c * kRowChunks + ((32 * half + 2 * r + hh) ^ sw));
#pragma unroll
    for (int ks = 0; ks < kRopeSteps; ++ks)
      sr[ks] = 16 * (c * kRowChunks + ((kLat / 8 + 4 * half + 2 * ks + hh) ^ sw));
  }
  // P.V B operand: 16-lane group g = lane/16 reads rows 16kk + 4hh + a/4 (and
  // + 8), dims 256*half + 32dt + 16(g & 1) + 4(a & 3), a = lane % 16
  int tb[2];
  {
    const int a = lane & 15;
    const int r = 4 * hh + (a >> 2);
    const int sw = swz(r);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      tb[q] = 16 * (r * kRowChunks + ((32 * half + 4 * q + 2 * ((lane >> 4) & 1) + ((a & 3) >> 1)) ^ sw)) +
              8 * (a & 1);
  }

  f32x16_t acc[kDimTiles];
#pragma unroll
  for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  float m_ref = -INFINITY;     // head c, the same on lanes c and c + 32 and on both halves
  float l_sum = 0.0f;          // this lane's share of head c's denominator
  const int end_h = CAUSAL ? min(end, n - p.num_queries + 1 + (h0 + c) / p.w_heads) : end;
  f32x16_t s_mine;             // this wave's partial scores of the previous tile
#pragma unroll
  for (int i = 0; i < 16; ++i) s_mine[i] = 0.0f;

  auto next_tile = [&](int it) {   // load tile it (if any) into its buffer in one go
    if (it < ntiles) {
      if constexpr (F8) stage_tile(it);
      else issue_tile(it);
    }
  };
  auto tile_ready = [&](int it) {  // tile it is in LDS for every wave
    if constexpr (F8) {
      if (it < ntiles) store_tile(it % kTileBufs);
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  };

  // Iteration it: the score MFMAs of tile it run with the softmax of tile
  // it-1 (VALU) placed between them in slices, one slice per k-step; then
  // the P.V MFMAs of tile it-1, with the exchange write of tile it's partial
  // scores.  SC / SM: whether there is a tile it / a tile it-1.
  auto iteration = [&](int it, auto sc_on, auto sm_on) {
    constexpr bool SC = decltype(sc_on)::value;
    constexpr bool SM = decltype(sm_on)::value;
    tile_ready(it);
    // tile it+1: FP8 rows are staged now (their loads first); bf16 rows go
    // straight to LDS, one load per score k-step
    const bool more = it + 1 < ntiles;
    if constexpr (F8)
      if (more) stage_tile(it + 1);
    // LDS reads next: the first two score operands of tile it and the
    // partner's partial scores of tile it-1, so that the bf16 tile's set-up
    // (branches, each closing the compiler's scheduling region) runs while
    // they are in flight
    const char* tl = reinterpret_cast<const char*>(&sm.tile[it % kTileBufs][0]);
    auto aread = [&](int ks) {
      return ks < kLatSteps ? *reinterpret_cast<const uint4*>(tl + sa[ks & 3] + 128 * (ks >> 2))
                            : *reinterpret_cast<const uint4*>(tl + sr[ks - kLatSteps]);
    };
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0;
    if constexpr (SC) {
      a0 = aread(0);
      a1 = aread(1);
    }
    f32x4_t px[4];   // softmax state of tile it-1
    if constexpr (SM) {
      const f32x4_t* src = &sm.xs[(it - 1) & 1][wave ^ 1][0][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) px[q] = src[64 * q];
    }
    if constexpr (!F8 && !SC) {
      if (more) issue_tile(it + 1);
    } else if constexpr (!F8) {
      if (more) setup_tile(it + 1);
    }
    float v[16];
    float cm = -INFINITY, nref = m_ref, alpha = 1.0f, base = 0.0f, lpart = 0.0f;
    bool bump = false;
    uint4 ph[2], pm[2], pl[2];
    const int t0p = (first_tile + it - 1) * kTileKeys;
    const bool inner = __builtin_amdgcn_read_exec() ==
                       __ballot(t0p >= begin && t0p + kTileKeys <= end_h);
    auto softmax_slice = [&](int k) {
      // each slice ends with its results pinned (an empty asm that reads
      // them), so the optimiser cannot sink the work towards its later uses
      if (k == 0) {           // full scores: this half plus the partner's
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[4 * q + e] = s_mine[4 * q + e] + px[q][e];
            pin(v[4 * q + e]);
          }
      } else if (k == 1 || k == 2) {   // scale and mask (keys outside [begin, end_h))
        if (inner) {                     // wave-uniform: no key of the tile is masked
#pragma unroll
          for (int i = 8 * (k - 1); i < 8 * k; ++i) {
            v[i] *= p.scale_log2;
            pin(v[i]);
          }
        } else {
          const int lo = begin - t0p, hi = end_h - t0p;
#pragma unroll
          for (int i = 8 * (k - 1); i < 8 * k; ++i) {
            const int r = 8 * (i >> 2) + 4 * hh + (i & 3);
            v[i] = (r >= lo && r < hi) ? v[i] * p.scale_log2 : -INFINITY;
            pin(v[i]);
          }
        }
      } else if (k == 3) {    // per-head max over the 32 keys
#pragma unroll
        for (int i = 0; i < 16; ++i) cm = fmaxf(cm, v[i]);
        cm = fmaxf(cm, xhalf(cm));
        pin(cm);
      } else if (k == 4) {    // reference max (moves when passed by more than 8)
        bump = cm > m_ref + 8.0f;
        nref = bump ? cm : m_ref;
        alpha = (m_ref == -INFINITY) ? 0.0f : fast_exp2(m_ref - nref);
        base = (nref == -INFINITY) ? 0.0f : nref;
        pin(nref);
        pin(alpha);
        pin(base);
      } else if (k >= 5 && k <= 8) {
#pragma unroll
        for (int i = 4 * (k - 5); i < 4 * (k - 4); ++i) {
          v[i] = fast_exp2(v[i] - base);
          lpart += v[i];
          pin(v[i]);
        }
        pin(lpart);
      } else if (k >= 9 && k <= 12) {   // P in three bf16 terms, two pairs per slice
        const int kk = (k - 9) >> 1, q0 = ((k - 9) & 1) * 2;
#pragma unroll
        for (int q = q0; q < q0 + 2; ++q) {
          uint32_t hi2, mi2, lo2;
          split3_bf16x2(v[8 * kk + 2 * q], v[8 * kk + 2 * q + 1], hi2, mi2, lo2);
          pin(hi2);
          pin(mi2);
          pin(lo2);
          if (q == 0) { ph[kk].x = hi2; pm[kk].x = mi2; pl[kk].x = lo2; }
          if (q == 1) { ph[kk].y = hi2; pm[kk].y = mi2; pl[kk].y = lo2; }
          if (q == 2) { ph[kk].z = hi2; pm[kk].z = mi2; pl[kk].z = lo2; }
          if (q == 3) { ph[kk].w = hi2; pm[kk].w = mi2; pl[kk].w = lo2; }
        }
      }
    };
    // scores of tile it, softmax slices of tile it-1 between the k-steps
    f32x16_t sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
    if constexpr (SC) {
      // the operand of k-step ks is read two steps ahead; the softmax slices
      // start two steps in, once the partner's partial scores have arrived
#pragma unroll
      for (int ks = 0; ks < kLatSteps + kRopeSteps; ++ks) {
        uint4 a2 = a1;
        if (ks + 2 < kLatSteps + kRopeSteps) a2 = aread(ks + 2);
        if (ks < kLatSteps) {
          sc = mfma32(a0, ql[ks], sc);
          sc = mfma32(a0, qm[ks], sc);
        }
        sc = mfma32(a0, qh[ks], sc);
        if constexpr (SM)
          if (ks >= 2) softmax_slice(ks - 2);
        if constexpr (!F8)
          if (ks < kWaveLoads && more) load_part(ks);
        a0 = a1;
        a1 = a2;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 13; ++k) softmax_slice(k);
    }
    if constexpr (SM) {
      // the rare rescale of the accumulators (heads whose reference moved).
      // A head whose reference moves from -inf has seen no key, so its
      // accumulators are still exactly 0 and need none: the first tile of a
      // range, where every head's reference moves, skips it.
      const bool rescale = bump && m_ref != -INFINITY;
      l_sum = l_sum * alpha + lpart;
      m_ref = nref;
      if (__builtin_amdgcn_read_exec() & __ballot(rescale)) {
        // accumulator element i of a lane is head 8(i/4) + 4hh + i%4
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ar = __shfl(alpha, 8 * (i >> 2) + 4 * hh + (i & 3));
#pragma unroll
          for (int dt = 0; dt < kDimTiles; ++dt) {
            float x = acc[dt][i];
            scale_in_agpr(x, ar);
            acc[dt][i] = x;
          }
        }
      }
      // P.V of tile it-1: the B operands of dim tile dt+1 are read while dt's
      // MFMAs run; the exchange write of tile it's scores goes in after dt 0
      const uint32_t tvb = lds_addr(&sm.tile[(it - 1) % kTileBufs][0]);
      uint32_t tv0 = tvb + tb[0], tv1 = tvb + tb[1];
      // the two bases are fixed here, so each read is base + constant and the
      // constant goes into the instruction's offset field
      pin(tv0);
      pin(tv1);
      auto bread = [&](int dt, int kk) {
        const uint32_t a0 = ((dt & 1) ? tv1 : tv0) + 128 * (dt >> 1) + 16 * kk * kRowChunks * 16;
        const uint2 b0 = lds_read_tr_at(a0);
        const uint2 b1 = lds_read_tr_at(a0 + 8 * kRowChunks * 16);
        return make_uint4(b0.x, b0.y, b1.x, b1.y);
      };
      uint4 b0 = bread(0, 0), b1 = bread(0, 1);
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) {
        uint4 n0 = b0, n1 = b1;
        if (dt + 1 < kDimTiles) {
          n0 = bread(dt + 1, 0);
          n1 = bread(dt + 1, 1);
        }
        // the reads stay ahead of this tile's six MFMAs, which hide their latency
        __builtin_amdgcn_sched_barrier(0);
        acc[dt] = mfma32(pl[0], b0, acc[dt]);
        acc[dt] = mfma32(pl[1], b1, acc[dt]);
        acc[dt] = mfma32(pm[0], b0, acc[dt]);
        acc[dt] = mfma32(pm[1], b1, acc[dt]);
        acc[dt] = mfma32(ph[0], b0, acc[dt]);
        acc[dt] = mfma32(ph[1], b1, acc[dt]);
        if (SC && dt == 0) {
          f32x4_t* dst = &sm.xs[it & 1][wave][0][lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[64 * q] = f32x4_t{sc[4 * q], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]};
        }
        b0 = n0;
        b1 = n1;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (SC) {
      f32x4_t* dst = &sm.xs[it & 1][wave][0][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[64 * q] = f32x4_t{sc[4 * q], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]};
    }
    if constexpr (SC) s_mine = sc;
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  next_tile(0);
  iteration(0, T_{}, F_{});
  for (int it = 1; it < ntiles; ++it) iteration(it, T_{}, T_{});
  iteration(ntiles, F_{}, T_{});
  if (!active) return;

  // denominators: head c's sum over lanes c and c + 32; accumulator element
  // i is head 8(i/4) + 4hh + i%4
  const float l_tot = l_sum + xhalf(l_sum);
  const int64_t srow = slot * kGroup + pair * kPairHeads;
  // the accumulators leave as they are (the stores take them from the
  // AGPRs); the merge weighs each piece by e^(m - M) / W
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hr = 8 * (i >> 2) + 4 * hh + (i & 3);
    float* dst = p.seg_out + (srow + hr) * kLat + kHalfLat * half + c;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) dst[32 * dt] = acc[dt][i];
  }
  if (half == 0 && hh == 0) {
    p.seg_max[srow + c] = m_ref * kLn2;
    p.seg_sum[srow + c] = l_tot;
  }
}

template <bool F8, bool CAUSAL>
__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(1)))
void mla_split_kernel(const MlaParams p) {
  __shared__ MlaSplitLds sm;
  __shared__ int64_t sh[4];
  __shared__ int sh_b, sh_rows, sh_n;
  const int i = blockIdx.x;
  if (threadIdx.x < 64) {
    // the first 64 context lengths, loaded beside the plan, so the searches
    // below and the row's length wait for no further load
    const int c_first = static_cast<int>(threadIdx.x) < p.batch ? p.context_lens[threadIdx.x] : 0;
    const MlaSplit sp = *p.split_plan;
    int b = p.batch;
    if (sp.rows) {                            // piece j of row (hg, b): tiles [j T / n, (j+1) T / n)
      // Work unit k = (piece k / groups, head group k % groups), taken in an
      // XCD-aware order: the hardware deals consecutive blocks to the 8 XCDs
      // in turn, so block i takes unit (i % 8) (grid / 8) + i / 8 and each
      // XCD runs a run of consecutive units.  The head groups of a piece (one
      // set of latent tiles) and the pieces of a row (one set of q rows) then
      // meet in one L2.  The partial slot stays hg N + piece.
      const int nbk = p.split_grid;
      const int k = (nbk & 7) == 0 ? (i & 7) * (nbk >> 3) + (i >> 3) : i;
      const int piece = k / p.groups;
      const int hg = piece < sp.N ? k - piece * p.groups : p.groups;
      int pre = 0;
      if (hg < p.groups) mla_piece_row(p.context_lens, p.batch, sp.L, piece, c_first, b, pre);
      const int nlen = b < 64 ? __shfl(c_first, b) : (b < p.batch ? p.context_lens[b] : 0);
      if (threadIdx.x == 0) {
        sh[0] = b < p.batch ? hg : p.groups;  // past the last piece: nothing to do
        sh_n = nlen;
        if (b < p.batch) {
          const int T = (nlen + 31) >> 5, nj = (T + sp.L - 1) / sp.L;
          const int j = piece - pre;
          sh[1] = static_cast<int64_t>(j) * T / nj;
          sh[2] = static_cast<int64_t>(j + 1) * T / nj;
          sh[3] = static_cast<int64_t>(hg) * sp.N + piece;
        }
      }
    } else {                                  // units [i T / nb, (i+1) T / nb) of the key line
      const int64_t T = sp.S * p.groups;
      const int64_t u0 = T * i / sp.nb;
      int64_t pre = 0;
      if (i < sp.nb && sp.S > 0) mla_locate(p.context_lens, p.batch, u0 % sp.S, c_first, b, pre);
      if (threadIdx.x == 0) {
        sh[0] = sp.S;
        sh[1] = (i < sp.nb) ? u0 : 0;
        sh[2] = (i < sp.nb) ? T * (i + 1) / sp.nb : 0;
        sh[3] = pre;
      }
    }
    if (threadIdx.x == 0) {
      sh_b = b;
      sh_rows = sp.rows;
    }
  }
  __syncthreads();
  // the block's segments (one for a piece of a row), one mla_segment call site
  const bool rows = sh_rows;
  int b = sh_b;
  int hg = rows ? static_cast<int>(sh[0]) : 0;
  const int64_t S = rows ? 0 : sh[0];
  int64_t u = rows ? 0 : sh[1], u1 = rows ? 1 : sh[2], pre = rows ? 0 : sh[3];
  if (rows ? hg >= p.groups : u >= u1) return;
  if (!rows) hg = static_cast<int>(u / S);
  const int n_row = sh_n;
  while (u < u1) {
    const int n = rows ? n_row : p.context_lens[b];
    int begin, end;
    int64_t slot;
    if (rows) {
      begin = kTileKeys * static_cast<int>(sh[1]);
      end = min(n, kTileKeys * static_cast<int>(sh[2]));
      slot = sh[3];
      u = u1;
    } else {                                  // the key line, row by row
      const int64_t row_start = hg * S + pre;
      const int64_t k0 = row_start + (n > 0 ? kMlaRowCost : 0);   // the row's first key
      begin = static_cast<int>(max(u, k0) - k0);
      end = static_cast<int>(min(u1 - k0, static_cast<int64_t>(n)));
      slot = static_cast<int64_t>(hg) * p.batch + b + i;
      u = k0 + n;
    }
    if (end > begin) mla_segment<F8, CAUSAL>(p, b, n, hg, begin, end, slot, sm);
    if (!rows) {
      pre += n > 0 ? n + kMlaRowCost : 0;
      if (++b == p.batch) {
        b = 0;
        pre = 0;
        ++hg;
      }
    }
  }
}

// ---- 3. merge of the partials, then out = W_UV[h] . o_lat on MFMA ---------------------
//
// Block (h, bt, s) handles sequences ROWS*bt .. +ROWS (ROWS = 8 or 16) of
// head s*H + h (query s, W_UV[h]; hg below is that head's group): row
// (group hg, b) was cut into pieces whose partials sit in the slots the
// absorb kernel's plan block listed for it, in ascending key order.  The max
// M and the total W = sum l_i e^(m_i - M) of a row are wave reductions over
// its pieces, loaded together with the first eight pieces' partials; o_lat
// is the (e^(m_i - M) / W)-weighted sum of the pieces' unnormalised partials
// in ascending i (eight pieces' loads in flight), written to LDS as three
// bf16 terms; then
// out[b][dv] = sum_j o_lat[b][j] W_UV[h][dv][j] on MFMA with A = o_lat (rows
// past ROWS zero) and B = W_UV rows, whose 8 consecutive latent dims per lane
// are contiguous in memory; wave w computes dv tile w.  With 8 rows the W_UV
// loads are issued first, so they overlap the merge; with 16 (the verify
// step's grids, two blocks or more per CU) they follow it, which keeps the
// kernel within the registers of two resident blocks per CU.  An empty
// context, or a query that sees no key, gives 0.
constexpr int kMergeThreads = 512;
constexpr int kMergeWaves = kMergeThreads / 64;

template <int ROWS>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_uv_kernel(const MlaParams p) {
  static_assert(ROWS == 8 || ROWS == 16, "rows per block");
  __shared__ __align__(16) uint16_t ohi[16][kLat + 8];
  __shared__ __align__(16) uint16_t omid[16][kLat + 8];
  __shared__ __align__(16) uint16_t olo[16][kLat + 8];
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
  auto load_wuv = [&]() {
#pragma unroll
    for (int ks = 0; ks < kLat / 32; ++ks) bw[ks] = load16(wuv + 32 * ks);
  };
  if constexpr (ROWS < 16) load_wuv();   // 16 rows: after the merge (registers for 2 blocks per CU)

  if constexpr (ROWS < 16) {   // rows ROWS..15 of the MFMA A operand stay zero
    for (int i = tid; i < (16 - ROWS) * (kLat / 8); i += kMergeThreads) {
      const int r = ROWS + i / (kLat / 8), c8 = (i % (kLat / 8)) * 8;
      *reinterpret_cast<uint4*>(&ohi[r][c8]) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&omid[r][c8]) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&olo[r][c8]) = make_uint4(0, 0, 0, 0);
    }
  }
  // per row (wave w takes rows w, w + 8): its pieces' maxima and sums and the
  // first eight pieces' partials are loaded together; then M, W and the
  // weighted sum of the partials in ascending piece order (the weights of
  // the first 64 pieces from the lanes that computed them)
#pragma unroll
  for (int bb = wave; bb < ROWS; bb += kMergeWaves) {
    const MlaRowSlots ri = bb < nrow ? p.row_slots[static_cast<int64_t>(hg) * p.batch + b0 + bb]
                                     : MlaRowSlots{0, 0, 0};
    const int cnt = ri.cnt;
    const int64_t slot = ri.slot;
    const int d0 = lane * 8;
    float4 v[8][2];
    auto load_group = [&](int k0) {   // pieces k0 .. k0+7 (the last repeated past cnt)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t srow = (slot + min(k0 + u, cnt - 1)) * kGroup + hl;
        v[u][0] = *reinterpret_cast<const float4*>(p.seg_out + srow * kLat + d0);
        v[u][1] = *reinterpret_cast<const float4*>(p.seg_out + srow * kLat + d0 + 4);
      }
    };
    if (cnt > 0) load_group(0);
    const bool mine = lane < cnt;
    const float m0 = mine ? p.seg_max[(slot + lane) * kGroup + hl] : -INFINITY;
    const float l0 = mine ? p.seg_sum[(slot + lane) * kGroup + hl] : 0.0f;
    float M = m0;
    for (int k = lane + 64; k < cnt; k += 64) M = fmaxf(M, p.seg_max[(slot + k) * kGroup + hl]);
    M = wave_max(M);
    if (M == -INFINITY) M = 0.0f;   // no piece saw a key: every weight is 0
    const float e_mine = mine ? __expf(m0 - M) : 0.0f;   // a piece's weight before 1/W
    float wk = l0 * e_mine;
    for (int k = lane + 64; k < cnt; k += 64)
      wk += p.seg_sum[(slot + k) * kGroup + hl] * __expf(p.seg_max[(slot + k) * kGroup + hl] - M);
    const float W = wave_sum(wk);
    const float iw = W > 0.0f ? 1.0f / W : 0.0f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      if (k0 > 0) load_group(k0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        const int64_t srow = (slot + min(k, cnt - 1)) * kGroup + hl;
        const float w = k < cnt ? (k < 64 ? __shfl(e_mine, k) : __expf(p.seg_max[srow] - M)) * iw
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
  if constexpr (ROWS == 16) load_wuv();
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
  p.split_plan = reinterpret_cast<pa::MlaSplit*>(ws + plan.off_split_plan);
  p.row_slots = reinterpret_cast<pa::MlaRowSlots*>(ws + plan.off_row_slots);
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
  // The split's grid is fixed by the shapes and the build, not the device (so
  // are the results): plan.max_blocks blocks, kSplitCUs (one per compute unit
  // of MI355X) for the library's choice; each piece gets at least
  // partition_size keys, or kMlaMinKeys for the library's choice.
  const int cus = pa::kSplitCUs;
  p.split_grid = plan.max_blocks;
  p.min_tiles = (partition_size > 0 ? partition_size : pa::kMlaMinKeys) / pa::kMlaTileKeys;
  p.explicit_size = partition_size > 0;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::clear_error();
  const int btiles = (p.abs_rows + 16 * pa::kAbsTiles - 1) / (16 * pa::kAbsTiles);
  hipLaunchKernelGGL(pa::mla_absorb_kernel, dim3(num_heads + 1, pa::kMlaLat / 128, btiles), dim3(256),
                     0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_LAUNCH, std::string("absorb: ") + hipGetErrorString(e));
  // one query, or no mask: every head sees the whole context
  const bool masked = causal && num_queries > 1;
  const dim3 sg(p.split_grid), st(pa::kMlaThreads);
  if (fp8 && masked)
    pa::launch_profiled(pa::mla_split_kernel<true, true>, sg, st, 0, s, p);
  else if (fp8)
    pa::launch_profiled(pa::mla_split_kernel<true, false>, sg, st, 0, s, p);
  else if (masked)
    pa::launch_profiled(pa::mla_split_kernel<false, true>, sg, st, 0, s, p);
  else
    pa::launch_profiled(pa::mla_split_kernel<false, false>, sg, st, 0, s, p);
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
