// MFMA operand helpers shared by the decode, prefill and MLA kernels.
//
// 16x16 tiles, lane l, j = l / 16 (gfx950 layouts, measured):
//   A [16 x K]: lane l holds row l % 16, K-slots (j, 0..e-1)
//   B [K x 16]: lane l holds column l % 16, K-slots (j, 0..e-1)
//   C [16 x 16] f32: lane l holds rows 4j + 0..3 of column l % 16
// Only the C layout fixes meaning; the K-slot order just has to agree
// between A and B.
//
// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// with in[L] = the four 16-bit values at lane L's address,
//   out[i][e] = in[4e + (i >> 2)][i & 3].
// So for V^T as the A operand of O^T += V^T . P^T (rows = value dims, K =
// tokens 4j + e), lane i of group j points at row 4j + (i >> 2) and columns
// 16b + 4(i & 3) .. +3 of a row-major [token][d] tile and receives
// V[4j + e][16b + i] for e = 0..3.
#pragma once

#include "device_common.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <class DT>
struct Mfma;

template <>
struct Mfma<BF16> {
  // C += A(16 x 32) . B(32 x 16), 8 elements per lane
  static __device__ __forceinline__ f32x4_t qk(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // C += A(16 x 16) . B(16 x 16), 4 elements per lane
  static __device__ __forceinline__ f32x4_t pv(const uint2 &a, const uint2 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return BF16::pack2(lo, hi); }
  static __device__ __forceinline__ float to_f(uint16_t x) { return BF16::to_f(x); }
  static __device__ __forceinline__ uint16_t from_f(float x) { return BF16::from_f(x); }
};

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ f32x4_t qk(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(const uint2 &a, const uint2 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const _Float16 a = _Float16(lo), b = _Float16(hi);
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
  }
  static __device__ __forceinline__ float to_f(uint16_t x) { return float(__builtin_bit_cast(_Float16, x)); }
  static __device__ __forceinline__ uint16_t from_f(float x) {
    return __builtin_bit_cast(uint16_t, _Float16(x));
  }
};

// Transposed 64-bit LDS read (four 16-bit values), see the layout above.
__device__ __forceinline__ uint2 lds_read_tr16(const void *p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s *)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace pkv
