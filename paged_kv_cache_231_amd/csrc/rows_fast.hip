// Bandwidth-bound decode kernel (VALU + DPP), specialised on element type,
// head dimension and q heads per block.
//
// Computes the same attention as the generic kernel (ruDNN 0.1.7
// `paged_attention` page, `DevicePlan::attention` doc) for head_dim ==
// value_dim in {64, 128, 256}.  Each K/V row of the cache is read once per
// (query, KV head) and serves all GT q heads of its group: no per-head KV
// repeat (module doc).
//
// Layout on the chip.  A block of four waves owns one (query, group of GT q
// heads, split part); its waves take the part's pages in turn.  Within a
// wave, a token's row of D elements is read by LPT lanes with one 16-byte
// load each (LPT = D * sizeof(T) / 16), so the wave reads TPW = 64 / LPT
// tokens per load instruction and each lane row (LPT lanes) keeps its own
// online softmax.  The q.k partial sums are combined across the LPT lanes with
// DPP (quad swaps and row mirrors), never through LDS.  At the end the lane
// rows are merged with shuffles and the four waves through LDS.

#include "device_common.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;

template <class DT>
struct Vec;  // 16-byte chunk of a K/V/Q row and its dot/convert helpers

template <>
struct Vec<F32> {
  static constexpr int E = 4;
  static __device__ __forceinline__ float dot(const uint4 &q, const uint4 &k) {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  }
  static __device__ __forceinline__ void to_f(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <>
struct Vec<BF16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
  static __device__ __forceinline__ float dot(const uint4 &q, const uint4 &k) {
    float s = d2(q.x, k.x, 0.f);
    s = d2(q.y, k.y, s);
    s = d2(q.z, k.z, s);
    return d2(q.w, k.w, s);
  }
  static __device__ __forceinline__ void to_f(const uint4 &v, float *f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(w[j] << 16);
      f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
};

template <>
struct Vec<F16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  }
  static __device__ __forceinline__ float dot(const uint4 &q, const uint4 &k) {
    float s = d2(q.x, k.x, 0.f);
    s = d2(q.y, k.y, s);
    s = d2(q.z, k.z, s);
    return d2(q.w, k.w, s);
  }
  static __device__ __forceinline__ void to_f(const uint4 &v, float *f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2_t h = __builtin_bit_cast(f16x2_t, w[j]);
      f[2 * j] = float(h.x);
      f[2 * j + 1] = float(h.y);
    }
  }
};

template <class DT, int D, int GT>
__global__ __launch_bounds__(256) void rows_fast_kernel(RowArgs a) {
  using T = typename DT::T;
  using V = Vec<DT>;
  constexpr int E = V::E;            // elements per lane per 16-byte load
  constexpr int LPT = D / E;         // lanes per token row
  constexpr int TPW = 64 / LPT;      // tokens per wave load
  constexpr int CH = GT >= 8 ? 2 : 4;  // tokens per lane row per step
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0, "bad lane split");

  __shared__ float s_acc[kWaves][GT][D];
  __shared__ float s_m[kWaves][GT], s_l[kWaves][GT];

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
  const uint32_t row = lane / LPT, col = lane % LPT;
  const uint32_t groups = a.hq / GT;
  const uint32_t part = blockIdx.x % a.splits;
  const uint32_t hg = (blockIdx.x / a.splits) % groups;
  const uint32_t qi = blockIdx.x / a.splits / groups;
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  uint32_t seq;
  const uint32_t n = visible_keys(a.plan, i, a.causal, &seq);
  const uint32_t ps = a.plan.ps;
  const uint32_t used_pages = ceil_div_u(n, ps);
  const uint32_t p_begin = part * a.pages_per_split;
  uint32_t p_end = p_begin + a.pages_per_split;
  if (p_end > used_pages) p_end = used_pages;
  if (a.splits > 1 && p_begin >= p_end) return;  // empty part: the merge skips it

  const uint32_t h0 = hg * GT;
  const uint32_t kvh = h0 / (a.hq / a.hkv);
  uint4 qv[GT];
  const T *qbase = static_cast<const T *>(a.q) + (uint64_t(i) * a.hq + h0) * D + col * E;
#pragma unroll
  for (int g = 0; g < GT; ++g) qv[g] = *reinterpret_cast<const uint4 *>(qbase + uint64_t(g) * D);

  float m[GT], l[GT], acc[GT][E];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNoMax;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const T *kb = static_cast<const T *>(a.k) + uint64_t(kvh) * D + col * E;
  const T *vb = static_cast<const T *>(a.v) + uint64_t(kvh) * D + col * E;
  const uint32_t *table = a.plan.words + a.plan.table + uint64_t(seq) * a.plan.W;
  const float sl2 = a.scale_log2;

  for (uint32_t p = p_begin + wv; p < p_end; p += kWaves) {
    const uint32_t page = table[p];
    if (page >= a.plan.N) continue;  // never read outside the pool
    const uint32_t tok0 = p * ps;
    const uint32_t cnt = n - tok0 < ps ? n - tok0 : ps;
    const T *kp = kb + uint64_t(page) * a.k_page;
    const T *vp = vb + uint64_t(page) * a.v_page;
    for (uint32_t sb = 0; sb < cnt; sb += TPW * CH) {
      uint4 kk[CH], vv[CH];
      bool ok[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t slot = sb + c * TPW + row;
        ok[c] = slot < cnt;
        kk[c] = make_uint4(0, 0, 0, 0);
        vv[c] = make_uint4(0, 0, 0, 0);
        if (ok[c]) {
          kk[c] = load_stream16(kp + uint64_t(slot) * a.k_tok);
          vv[c] = load_stream16(vp + uint64_t(slot) * a.v_tok);
        }
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float x[CH];
        float mb = kNoMax;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          x[c] = group_sum<LPT>(V::dot(qv[g], kk[c])) * sl2;
          x[c] = ok[c] ? x[c] : -INFINITY;
          mb = fmaxf(mb, x[c]);
        }
        const float m_new = fmaxf(m[g], mb);
        const float alpha = fast_exp2(m[g] - m_new);
        m[g] = m_new;
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float pr = fast_exp2(x[c] - m_new);
          l[g] += pr;
          float vf[E];
          V::to_f(vv[c], vf);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pr, vf[e], acc[g][e]);
        }
      }
    }
  }

  // merge the lane rows of this wave
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off, 64);
      const float lo = __shfl_xor(l[g], off, 64);
      const float mn = fmaxf(m[g], mo);
      const float a1 = fast_exp2(m[g] - mn), a2 = fast_exp2(mo - mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ao = __shfl_xor(acc[g][e], off, 64);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wv][g][col * E + e] = acc[g][e];
    }
    if (col == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        s_m[wv][g] = m[g];
        s_l[wv][g] = l[g];
      }
    }
  }
  __syncthreads();

  // merge the four waves and write this block's result
  for (uint32_t idx = tid; idx < uint32_t(GT * D); idx += 256) {
    const uint32_t g = idx / D, d = idx % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(s_m[w][g] - M);
      num = fmaf(s_acc[w][g][d], sc, num);
      den = fmaf(s_l[w][g], sc, den);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    if (a.splits == 1) {
      T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h0) * D;
      out[idx] = DT::from_f(num * inv);
    } else {
      const uint64_t r = (uint64_t(i) * a.splits + part) * a.hq + h0;
      a.ws_o[r * D + idx] = num * inv;
      if (d == 0) a.ws_lse[r + g] = M + fast_log2(den);
    }
  }
}

template <class DT, int D>
hipError_t launch_gt(const RowArgs &a, int gt, dim3 grid, hipStream_t st) {
  switch (gt) {
    case 1: launch_k((rows_fast_kernel<DT, D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: launch_k((rows_fast_kernel<DT, D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: launch_k((rows_fast_kernel<DT, D, 4>), grid, dim3(256), 0, st, a); break;
    case 8: launch_k((rows_fast_kernel<DT, D, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <class DT>
hipError_t launch_d(const RowArgs &a, int gt, dim3 grid, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_gt<DT, 64>(a, gt, grid, st);
    case 128: return launch_gt<DT, 128>(a, gt, grid, st);
    case 256: return launch_gt<DT, 256>(a, gt, grid, st);
    default: return hipErrorNotSupported;
  }
}

int group_tile(const RowArgs &a) {
  const uint32_t g = a.hq / a.hkv;
  for (int gt = 8; gt >= 1; gt >>= 1)
    if (g % uint32_t(gt) == 0) return gt;
  return 1;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool rows_fast_supported(const RowArgs &a, pkv_dtype dt) {
  if (a.pdim != 0 || a.d != a.dv || a.window != 0 || a.kv_fp8) return false;  // neither here
  if (a.d != 64 && a.d != 128 && a.d != 256) return false;
  if (dt != PKV_F32 && dt != PKV_F16 && dt != PKV_BF16) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v)) return false;
  if (a.out && !aligned16(a.out)) return false;
  return true;
}

hipError_t launch_rows_fast(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const int gt = group_tile(a);
  const uint64_t blocks = uint64_t(a.n_queries) * (a.hq / uint32_t(gt)) * a.splits;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));
  switch (dt) {
    case PKV_F32: return launch_d<F32>(a, gt, grid, st);
    case PKV_F16: return launch_d<F16>(a, gt, grid, st);
    case PKV_BF16: return launch_d<BF16>(a, gt, grid, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
