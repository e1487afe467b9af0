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
// / V block.  Block (x, y) copies units [y * kChunk, (y + 1) * kChunk) of
// query x: the slot address is one chain of scalar loads per block, and the
// source loads do not wait for it.  (Eight queries per block, each thread
// issuing all their loads before the stores, measured slower: 14.8 against
// 10.7 us for 4216 queries.)
constexpr uint32_t kChunk = 2048;  // units per block: 8 per thread

template <class U>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const PlanView &p = a.plan;
  const uint32_t i = blockIdx.x;
  const uint32_t per_q = a.k_units + a.v_units;
  const uint32_t u0 = blockIdx.y * kChunk;
  const uint32_t u1 = per_q - u0 < kChunk ? per_q : u0 + kChunk;
  const uint32_t seq = p.words[p.qseq + i];
  const uint32_t pos = p.words[p.qpos + i];
  const uint32_t page = p.words[p.table + uint64_t(seq) * p.W + pos / p.ps];
  const uint64_t slot = uint64_t(page) * p.ps + pos % p.ps;
  const bool ok = page < p.N;  // never write outside the pool
  for (uint32_t u = u0 + threadIdx.x; u < u1; u += 256) {
    if (u < a.k_units) {
      const U x = __builtin_nontemporal_load(static_cast<const U *>(a.new_k) + uint64_t(i) * a.k_units + u);
      if (ok) static_cast<U *>(a.k)[slot * a.k_units + u] = x;
    } else {
      const uint32_t w = u - a.k_units;
      const U x = __builtin_nontemporal_load(static_cast<const U *>(a.new_v) + uint64_t(i) * a.v_units + w);
      if (ok) static_cast<U *>(a.v)[slot * a.v_units + w] = x;
    }
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
  const uint64_t chunks = per_q / kChunk + (per_q % kChunk != 0);
  if (per_q > 0xFFFFFFFFull || chunks > 65535) return hipErrorInvalidValue;
  const dim3 grid(a.n_queries, uint32_t(chunks));
  if (unit == 16)
    launch_k(append_kernel<u32x4_t>, grid, dim3(256), 0, st, a);
  else if (unit == 4)
    launch_k(append_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  else
    launch_k(append_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
