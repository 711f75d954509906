// pa_device.h -- small device helpers for the gfx950 kernels: bf16 packing,
// wave64 cross-lane reductions built on DPP and ds_swizzle, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// The two bf16 values packed in one dword, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// a.x*b.x + a.y*b.y + c on packed bf16 pairs (v_dot2_f32_bf16): the bf16
// products are exact in fp32, accumulation is fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP row rotations (rows are 16 lanes on wave64).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return u2f(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(f2u(x)), kCtrl, 0xf, 0xf, false)));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kRowRor8>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor2>(x);
  x += dpp<kRowRor1>(x);
  return x;
}

// Value of lane (lane ^ 16) within each 32-lane half (ds_swizzle bitmask mode).
__device__ __forceinline__ float xor16(float x) {
  return u2f(static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(f2u(x)), 0x401f)));
}
// Value of lane (lane ^ 32).
__device__ __forceinline__ float xor32(float x) {
  const int src = (static_cast<int>(threadIdx.x & 63) ^ 32) << 2;
  return u2f(static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(f2u(x)))));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kRowRor8>(x));
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor2>(x));
  x = fmaxf(x, dpp<kRowRor1>(x));
  x = fmaxf(x, xor16(x));
  x = fmaxf(x, xor32(x));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x += xor16(x);
  x += xor32(x);
  return x;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---- balanced splits: T units cut into nb equal contiguous ranges ----------
// Block i owns units [floor(i*T/nb), floor((i+1)*T/nb)).

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) v += __shfl_xor(v, w);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int64_t wave_scan64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) {
    const int64_t u = __shfl_up(v, w);
    if (lane >= w) v += u;
  }
  return v;
}

// Block holding unit x: the largest i with floor(i*T/nb) <= x.
__device__ __forceinline__ int block_of(int64_t x, int64_t T, int nb) {
  return static_cast<int>(((x + 1) * nb - 1) / T);
}

// Blocks used for T units: ceil(T / min_units), at least 1 and at most grid.
__device__ __forceinline__ int used_blocks(int64_t T, int grid, int64_t min_units) {
  const int64_t want = (T + min_units - 1) / min_units;
  return static_cast<int>(want < 1 ? 1 : (want < grid ? want : grid));
}

}  // namespace pa
