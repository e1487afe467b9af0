// Cache append (ruDNN 0.1.7 `paged_attention` page, `DevicePlan::append`
// and `append_with_report` docs): every query of the plan stores its new
// key and value rows, all KV heads, at the cache slot of its own absolute
// position: slot qpos % ps of page table[qseq][qpos / ps].  In the cache
// layout [pages, ps, Hkv, D] the Hkv * D elements of one slot are
// contiguous, as are the query's Hkv * D new elements, so each query is two
// contiguous block copies (K, then V).  The host has checked the write plan
// (no two queries share a slot), so blocks never overlap and the copies
// may run in any order.  Pure data movement: HBM-bound, one read and one
// write of every new byte.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace pkv {

namespace {

// Copies in units of U (16, 4 or 2 bytes): k_units / v_units per query's K
// / V block, the K block's units first.  One wave per query and chunk:
// wave w of block (x, y) copies units [y * kWaveChunk, (y + 1) * kWaveChunk)
// of query 4x + w, kPer units per lane, every source load issued before the
// slot lookup is waited for and before any store, so a wave keeps kPer
// loads in flight and the whole grid fits the chip in one round.  (One
// block of 256 threads per query with one unit per thread took two rounds
// of load latency: 7.6 us for 4216 queries of 4 KB; eight queries per
// block with every thread issuing all their loads first measured slower
// still.)
constexpr uint32_t kQPB = 4;                  // queries (waves) per block
constexpr uint32_t kPer = 4;                  // units per lane per chunk
constexpr uint32_t kWaveChunk = 64u * kPer;   // units per (query, chunk)
template <class U>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const PlanView &p = a.plan;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t i = blockIdx.x * kQPB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (i >= a.n_queries) return;
  const uint32_t per_q = a.k_units + a.v_units;
  const uint32_t u0 = blockIdx.y * kWaveChunk;
  const U *src_k = static_cast<const U *>(a.new_k) + uint64_t(i) * a.k_units;
  const U *src_v = static_cast<const U *>(a.new_v) + uint64_t(i) * a.v_units;
  // unconditional loads from a per-lane address (units past the query's
  // end read its unit 0 and are not stored): no branch for the compiler to
  // wait at
  U x[kPer];
#pragma unroll
  for (uint32_t e = 0; e < kPer; ++e) {
    const uint32_t u = u0 + 64u * e + lane;
    const uint32_t uc = u < per_q ? u : 0u;
    const U *src = uc < a.k_units ? src_k + uc : src_v + (uc - a.k_units);
    x[e] = __builtin_nontemporal_load(src);
  }
  // keep the loads here, ahead of the slot lookup (the compiler would sink
  // a load into the branch of its store, behind the lookup's scalar loads)
  asm volatile("" ::: "memory");
  // plan words through the constant address space (they do not change
  // while the kernel runs): scalar loads, counted apart from the data loads
  const __attribute__((address_space(4))) uint32_t *w =
      (const __attribute__((address_space(4))) uint32_t *)p.words;
  const uint32_t seq = w[p.qseq + i];
  const uint32_t pos = w[p.qpos + i];
  const uint32_t page = w[p.table + uint64_t(seq) * p.W + pos / p.ps];
  const bool ok = page < p.N;  // never write outside the pool
  const uint64_t slot = uint64_t(page) * p.ps + pos % p.ps;
  U *dst_k = static_cast<U *>(a.k) + slot * a.k_units;
  U *dst_v = static_cast<U *>(a.v) + slot * a.v_units;
#pragma unroll
  for (uint32_t e = 0; e < kPer; ++e) {
    const uint32_t u = u0 + 64u * e + lane;
    U *dst = u < a.k_units ? dst_k + u : dst_v + (u - a.k_units);
    if (ok && u < per_q) *dst = x[e];
  }
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

bool aligned(const void *ptr, uintptr_t b) { return (reinterpret_cast<uintptr_t>(ptr) & (b - 1)) == 0; }

}  // namespace

hipError_t launch_append(AppendArgs a, uint64_t k_block_bytes, uint64_t v_block_bytes,
                         hipStream_t st) {
  if (a.n_queries == 0) return hipSuccess;
  const void *ptrs[] = {a.new_k, a.new_v, a.k, a.v};
  auto fits = [&](uint64_t b) {
    if (k_block_bytes % b || v_block_bytes % b) return false;
    for (const void *q : ptrs)
      if (!aligned(q, b)) return false;
    return true;
  };
  const uint64_t unit = fits(16) ? 16 : fits(4) ? 4 : 2;
  a.k_units = uint32_t(k_block_bytes / unit);
  a.v_units = uint32_t(v_block_bytes / unit);
  const uint64_t per_q = uint64_t(a.k_units) + a.v_units;  // <= 2 * 2^32 / 2: checked below
  const uint64_t chunks = per_q / kWaveChunk + (per_q % kWaveChunk != 0);
  if (per_q > 0xFFFFFFFFull || chunks > 65535) return hipErrorInvalidValue;
  const dim3 grid((a.n_queries + kQPB - 1) / kQPB, uint32_t(chunks));
  if (unit == 16)
    launch_k(append_kernel<u32x4_t>, grid, dim3(256), 0, st, a);
  else if (unit == 4)
    launch_k(append_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  else
    launch_k(append_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
