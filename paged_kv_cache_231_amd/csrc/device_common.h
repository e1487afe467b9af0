// Device helpers: element types, conversions, wave reductions, split ranges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace pkv {

// Element types.  bf16 is kept as its bit pattern (uint16_t).
struct F32 {
  using T = float;
  static __device__ __forceinline__ float to_f(T x) { return x; }
  static __device__ __forceinline__ T from_f(float x) { return x; }
};
struct F16 {
  using T = _Float16;
  static __device__ __forceinline__ float to_f(T x) { return float(x); }
  static __device__ __forceinline__ T from_f(float x) { return T(x); }
};
struct BF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float to_f(T x) { return __uint_as_float(uint32_t(x) << 16); }
  // Hardware conversion (v_cvt_pk_bf16_f32): round to nearest even, NaN
  // stays NaN.
  static __device__ __forceinline__ T from_f(float f) { return __builtin_bit_cast(T, (__bf16)f); }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Sentinel for "no key seen yet": finite, so exp2(m - m_new) stays defined
// when a part of the history is empty; masked scores are -inf.
constexpr float kNoMax = -1e30f;

// 16-byte load marked nontemporal: K/V cache rows are streamed once per
// (query, KV head), and the streaming hint lifts HBM read throughput.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), with
// the gfx950 row-swap instructions instead of an LDS round trip.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// a group gets the group's sum.  Within a 16-lane row DPP does it: two quad
// swaps, then the half-row and row mirrors (each pairs a lane with one of the
// other, already reduced, half).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Visible keys of query i: positions [0, n).  Clamped to the table's reach
// so a plan changed behind the library's back cannot index past the table.
__device__ __forceinline__ uint32_t visible_keys(const PlanView &p, uint32_t i, int causal,
                                                 uint32_t *seq_out) {
  const uint32_t seq = p.words[p.qseq + i];
  uint64_t n;  // the causal count needs no length
  if (causal) n = uint64_t(p.words[p.qpos + i]) + 1;
  else n = p.words[p.lens + seq];
  const uint64_t reach = uint64_t(p.W) * p.ps;
  if (n > reach) n = reach;
  *seq_out = seq;
  return uint32_t(n);
}

__device__ __forceinline__ uint32_t ceil_div_u(uint32_t a, uint32_t b) { return a / b + (a % b != 0); }

// First visible key under a sliding window: the last `window` of the visible
// keys [0, n) stay, [n - window, n); window 0 keeps them all.
__device__ __forceinline__ uint32_t window_lo(uint32_t n, uint32_t window) {
  return window != 0u && n > window ? n - window : 0u;
}

}  // namespace pkv
