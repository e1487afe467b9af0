// Generic per-query attention kernel and the split merge kernel.
//
// The generic kernel serves every shape the specialised kernels do not:
// any head/value dimension up to 1024, any page size, F32/F16/BF16, and the
// MLA position term.  One wave handles one (query, q head, split part): it
// walks the visible keys of its part one token at a time through the block
// table, keeping an online softmax in base 2.  It is the correctness
// backstop, not a fast path.
//
// The split/merge arithmetic follows the ruDNN 0.1.7 `paged_attention` page
// (`attention_into_split` doc: parts of the visible history, merged through
// FP32 statistics).  Part j covers logical pages [j*pp, (j+1)*pp) of the
// query's block-table row; each part writes its normalised f32 output and
// its log2-sum-exp2, and the merge kernel combines the non-empty parts.

#include "device_common.h"

namespace pkv {

namespace {

constexpr int kMaxPerLane = 16;  // 1024 / 64
constexpr int kMaxPosPerLane = 4;  // 256 / 64

template <class DT>
__global__ __launch_bounds__(64) void rows_generic_kernel(RowArgs a) {
  using T = typename DT::T;
  const uint32_t lane = threadIdx.x;
  const uint32_t unit = blockIdx.x;
  const uint32_t part = unit % a.splits;
  const uint32_t h = (unit / a.splits) % a.hq;
  const uint32_t qi = unit / a.splits / a.hq;
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  uint32_t seq;
  const uint32_t n = visible_keys(a.plan, i, a.causal, &seq);
  const uint64_t span = uint64_t(a.pages_per_split) * a.plan.ps;
  const uint64_t lo = window_lo(n, a.window);
  const uint64_t p0 = uint64_t(part) * span;
  const uint64_t t0 = p0 > lo ? p0 : lo;
  const uint64_t t1 = p0 + span < n ? p0 + span : uint64_t(n);
  if (a.splits > 1 && t0 >= t1) return;  // empty part: the merge skips it

  const uint32_t g = h / (a.hq / a.hkv);
  const T *q = static_cast<const T *>(a.q) + (uint64_t(i) * a.hq + h) * a.d;
  const T *k = static_cast<const T *>(a.k) + uint64_t(g) * a.d;
  const T *v = static_cast<const T *>(a.v) + uint64_t(g) * a.dv;
  float qr[kMaxPerLane], acc[kMaxPerLane], qpr[kMaxPosPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const uint32_t d = lane + 64u * j;
    qr[j] = d < a.d ? DT::to_f(q[d]) : 0.f;
    acc[j] = 0.f;
  }
  const T *qp = nullptr, *kp = nullptr;
  if (a.pdim) {
    qp = static_cast<const T *>(a.qp) + (uint64_t(i) * a.hq + h) * a.pdim;
    kp = static_cast<const T *>(a.kp);
  }
#pragma unroll
  for (int j = 0; j < kMaxPosPerLane; ++j) {
    const uint32_t d = lane + 64u * j;
    qpr[j] = (a.pdim && d < a.pdim) ? DT::to_f(qp[d]) : 0.f;
  }

  float m = kNoMax, l = 0.f;
  const uint32_t *table = a.plan.words + a.plan.table + uint64_t(seq) * a.plan.W;
  for (uint64_t t = t0; t < t1; ++t) {
    const uint32_t page = table[t / a.plan.ps];
    if (page >= a.plan.N) continue;  // never read outside the pool
    const uint32_t slot = uint32_t(t % a.plan.ps);
    const T *kr = k + uint64_t(page) * a.k_page + uint64_t(slot) * a.k_tok;
    const T *vr = v + uint64_t(page) * a.v_page + uint64_t(slot) * a.v_tok;
    float part_dot = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const uint32_t d = lane + 64u * j;
      if (d < a.d) part_dot += qr[j] * DT::to_f(kr[d]);
    }
    if (a.pdim) {
      const T *kpr = kp + uint64_t(page) * a.kp_page + uint64_t(slot) * a.kp_tok;
#pragma unroll
      for (int j = 0; j < kMaxPosPerLane; ++j) {
        const uint32_t d = lane + 64u * j;
        if (d < a.pdim) part_dot += qpr[j] * DT::to_f(kpr[d]);
      }
    }
    const float x = wave_sum(part_dot) * a.scale_log2;
    const float m_new = fmaxf(m, x);
    const float alpha = fast_exp2(m - m_new);
    const float p = fast_exp2(x - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const uint32_t d = lane + 64u * j;
      if (d < a.dv) acc[j] = acc[j] * alpha + p * DT::to_f(vr[d]);
    }
    m = m_new;
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.splits == 1) {
    T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * a.dv;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const uint32_t d = lane + 64u * j;
      if (d < a.dv) out[d] = DT::from_f(acc[j] * inv);
    }
  } else {
    const uint64_t row = (uint64_t(i) * a.splits + part) * a.hq + h;
    float *o = a.ws_o + row * a.dv;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const uint32_t d = lane + 64u * j;
      if (d < a.dv) o[d] = acc[j] * inv;
    }
    if (lane == 0) a.ws_lse[row] = m + fast_log2(l);
  }
}

// Merge of the non-empty parts of one (query, head):
//   M = max_j lse_j,  w_j = 2^(lse_j - M),  out = sum_j w_j o_j / sum_j w_j.
// One block per (query, head).  The part statistics are read in parallel
// (one part per thread) and reduced through LDS; each thread then owns value
// elements d = tid, tid + 256, ... and sums over the parts with independent,
// unrolled loads so that many are in flight at once.
template <class DT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  using T = typename DT::T;
  __shared__ float s_w[256];  // splits <= 256
  __shared__ float s_red[8];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
  const uint32_t h = blockIdx.x % a.hq;
  const uint32_t qi = blockIdx.x / a.hq;
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  uint32_t seq;
  const uint32_t n = visible_keys(a.plan, i, a.causal, &seq);
  const uint32_t used_pages = ceil_div_u(n, a.plan.ps);
  uint32_t parts = ceil_div_u(used_pages, a.pages_per_split);
  if (parts > a.splits) parts = a.splits;
  // parts wholly before the window are empty: skip them
  const uint32_t first = window_lo(n, a.window) / a.plan.ps / a.pages_per_split;
  parts = parts > first ? parts - first : 0u;
  const uint64_t base = uint64_t(i) * a.splits + first;

  const float lse = tid < parts ? a.ws_lse[(base + tid) * a.hq + h] : -INFINITY;
  float mx = wave_max(fmaxf(lse, kNoMax));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float w = tid < parts ? fast_exp2(lse - mx) : 0.f;
  s_w[tid] = w;
  const float ws = wave_sum(w);
  if (lane == 0) s_red[4 + wv] = ws;
  __syncthreads();
  const float total = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);
  const float inv = total > 0.f ? 1.f / total : 0.f;

  T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * a.dv;
  const uint64_t stride = uint64_t(a.hq) * a.dv;  // between parts
  const float *o = a.ws_o + (base * a.hq + h) * a.dv;
  for (uint32_t d = tid; d < a.dv; d += 256) {
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    uint32_t p = 0;
    for (; p + 4 <= parts; p += 4) {
      const float o0 = o[(p + 0) * stride + d], o1 = o[(p + 1) * stride + d];
      const float o2 = o[(p + 2) * stride + d], o3 = o[(p + 3) * stride + d];
      acc0 = fmaf(s_w[p + 0], o0, acc0);
      acc1 = fmaf(s_w[p + 1], o1, acc1);
      acc2 = fmaf(s_w[p + 2], o2, acc2);
      acc3 = fmaf(s_w[p + 3], o3, acc3);
    }
    for (; p < parts; ++p) acc0 = fmaf(s_w[p], o[p * stride + d], acc0);
    out[d] = DT::from_f(((acc0 + acc1) + (acc2 + acc3)) * inv);
  }
}

}  // namespace

hipError_t launch_rows_generic(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint64_t blocks = uint64_t(a.n_queries) * a.hq * a.splits;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));
  switch (dt) {
    case PKV_F32: launch_k(rows_generic_kernel<F32>, grid, dim3(64), 0, st, a); break;
    case PKV_F16: launch_k(rows_generic_kernel<F16>, grid, dim3(64), 0, st, a); break;
    case PKV_BF16: launch_k(rows_generic_kernel<BF16>, grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint64_t blocks = uint64_t(a.n_queries) * a.hq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));
  switch (dt) {
    case PKV_F32: launch_k(merge_kernel<F32>, grid, dim3(256), 0, st, a); break;
    case PKV_F16: launch_k(merge_kernel<F16>, grid, dim3(256), 0, st, a); break;
    case PKV_BF16: launch_k(merge_kernel<BF16>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
