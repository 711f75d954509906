// pa_mfma.h -- gfx950 matrix-core helpers shared by the GQA and MLA kernels:
// bf16 MFMA wrappers, the transposed LDS read that feeds them a key-major tile,
// and the exact three-term bf16 split of an fp32 operand.
//
// Lane layouts (wave64, 16x16 output tiles; g = lane / 16, c = lane % 16):
//   16x16x32:  A lane holds A[c][8g .. 8g+7],  B lane holds B[8g .. 8g+7][c]
//   16x16x16:  A lane holds A[c][4g .. 4g+3],  B lane holds B[4g .. 4g+3][c]
//   both:      D lane holds D[4g .. 4g+3][c]
// 32x32x16 (h = lane / 32, c = lane % 32; confirmed by an in-bounds probe):
//   A lane holds A[c][8h .. 8h+7],  B lane holds B[8h .. 8h+7][c],
//   D element i (0..15) of a lane is D[8(i / 4) + 4h + i % 4][c]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;

// Two fp32 -> two bf16 packed in one dword (low half from a), round to
// nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// split3_bf16 for a pair, on the hardware conversion: a = hi + mid + lo in the
// low halves, b in the high halves, exactly (the same argument: each residual
// is exact in fp32 and the last has at most 8 significant bits).
__device__ __forceinline__ void split3_bf16x2(float a, float b, uint32_t& hi, uint32_t& mid,
                                              uint32_t& lo) {
  hi = cvt_bf16x2(a, b);
  const float ra = a - u2f(hi << 16), rb = b - u2f(hi & 0xffff0000u);
  mid = cvt_bf16x2(ra, rb);
  lo = cvt_bf16x2(ra - u2f(mid << 16), rb - u2f(mid & 0xffff0000u));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// D = A.B + C, 16x16x32, bf16 operands (8 per lane), fp32 accumulation.
__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// D = A.B + C, 32x32x16, bf16 operands (8 per lane), fp32 accumulation.
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D = A.B + C, 16x16x16, bf16 operands (4 per lane), fp32 accumulation.
__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                    __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Transposed 64-bit LDS read (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane j receives element k (k < 4) of the 4 bf16 that lane 4k + j/4
// addresses, at position j % 4: with lane a pointing at row a/4, columns
// 4(a%4) .. +4 of a row-major tile, lane j gets column j of rows 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Byte address of p (which points into LDS) in the LDS aperture.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// lds_read_tr at an LDS byte address: written as base + constant, the
// constant goes into the instruction's offset field instead of costing an
// address add per read.
__device__ __forceinline__ uint2 lds_read_tr_at(uint32_t addr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)(addr));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace pa
