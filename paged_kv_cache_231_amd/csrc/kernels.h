// Kernel argument blocks and launchers shared by the host dispatcher
// (api.cpp) and the HIP sources.  All strides are in elements.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkv {

// Per-kernel timing.  While the host dispatcher times a launch it sets this
// thread's LaunchEvents; the next launch_k records the kernel's own start
// and end in them (part of its dispatch, so no separate event packets sit
// between kernels), marks them used and clears them.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchEvents &launch_events();  // this thread's (defined in api.cpp)

// Every kernel of the library is launched through here.
template <typename... Args, typename F = void (*)(Args...)>
inline void launch_k(F kernel, const dim3 &grid, const dim3 &block, uint32_t shmem, hipStream_t st,
                     Args... args) {
  LaunchEvents &ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev.start, ev.stop, 0u, args...);
  if (ev.start) {
    ev.start = ev.stop = nullptr;
    ev.used = true;
  }
}

// Where a kernel finds the schedule inside the device plan words.
struct PlanView {
  const uint32_t *words;  // device copy of the spec-v1 plan
  uint32_t lens, qseq, qpos, table;  // word offsets of the sections
  uint32_t W, ps, N;                 // table width, page size, pool pages
};

// One launch of a per-query ("row") kernel over a list of queries.
struct RowArgs {
  PlanView plan;
  const uint32_t *qlist;  // device list of query indices, or null = 0..n-1
  uint32_t n_queries;     // queries in the list (grid)
  uint32_t hq, hkv, d, dv, pdim;  // pdim: MLA position dim, 0 for attention
  uint32_t splits, pages_per_split;
  int causal;
  uint32_t window;   // > 0: only the last `window` visible keys (0 = all)
  float scale_log2;  // scale * log2(e) (* k_scale for an FP8 key cache): base-2 scores
  uint32_t kv_fp8;   // K and V hold FP8 E4M3 bytes (decode MFMA kernels only)
  float v_scale;     // output factor: the FP8 value cache's scale, else 1
  const void *q, *k, *v;     // MLA: k = v = latent
  const void *qp, *kp;       // MLA position parts (null for attention)
  uint64_t k_page, k_tok;    // k: page stride, token stride
  uint64_t v_page, v_tok;
  uint64_t kp_page, kp_tok;
  void *out;                 // [Q, hq, dv] in the input dtype
  float *ws_o, *ws_lse;      // [Q, splits, hq, dv], [Q, splits, hq] (splits > 1)
  // Balanced schedule (bal_waves > 0 units): the row queries' tile
  // positions are cut into equal ranges, one per group of segq units (decode:
  // waves, segq = KV heads x 16-head groups; MLA: blocks, segq = 64-head
  // groups); pieces cut by a range boundary go to ws_o/ws_lse slots (2 per
  // unit, one row per head of the unit).  bal_rec[2r], bal_rec[2r + 1]:
  // first tile and tile count of row query r; bal_rec[2 n_queries]: total.
  uint32_t *bal_rec;
  uint32_t bal_waves;
};

struct MergeArgs {
  PlanView plan;
  const uint32_t *qlist;
  uint32_t n_queries;
  uint32_t hq, hkv, dv, splits, pages_per_split;
  int causal;
  uint32_t window;
  const float *ws_o, *ws_lse;
  void *out;
  const uint32_t *bal_rec;  // balanced schedule (bal_waves > 0), as in RowArgs
  uint32_t bal_waves;
};

// Query tiles of the chunked-prefill kernel.
struct TileArgs {
  PlanView plan;
  const uint32_t *tiles;  // device {first, count} pairs
  uint32_t n_tiles;
  uint32_t hq, hkv, d, dv;
  int causal;
  uint32_t window;   // > 0: only the last `window` visible keys (0 = all)
  float scale_log2;  // includes the key scale of an FP8 cache
  uint32_t kv_fp8;   // 1: k and v hold E4M3 codes
  float v_scale;     // value scale of an FP8 cache (1 otherwise)
  const void *q, *k, *v;
  uint64_t k_page, k_tok, v_page, v_tok;
  void *out;
};

// Cache append: query i's new K/V blocks (Hkv * D, Hkv * Dv elements) to
// the slot of its position; k_units / v_units are set by the launcher.
struct AppendArgs {
  PlanView plan;
  uint32_t n_queries;
  uint32_t k_units, v_units;  // copy units per query's K and V block
  const void *new_k, *new_v;
  void *k, *v;                // the caches written (in place or copies)
};

hipError_t launch_append(AppendArgs a, uint64_t k_block_bytes, uint64_t v_block_bytes,
                         hipStream_t st);
hipError_t launch_rows_generic(const RowArgs &a, pkv_dtype dt, hipStream_t st);
// Fast VALU decode; returns hipErrorNotSupported when the shape is not one
// of its specialisations (the caller then uses the generic kernel).
bool rows_fast_supported(const RowArgs &a, pkv_dtype dt);
hipError_t launch_rows_fast(const RowArgs &a, pkv_dtype dt, hipStream_t st);
// MFMA decode (F16/BF16, head_dim == value_dim in {64, 128, 256}).
bool rows_mfma_supported(const RowArgs &a, pkv_dtype dt);
uint64_t rows_mfma_blocks(const RowArgs &a);
int rows_mfma_blocks_per_cu(const RowArgs &a, pkv_dtype dt);
hipError_t launch_rows_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st);
// Balanced MFMA decode: the wave-range kernel, then the merge of the pieces
// cut by range boundaries.  balanced_waves_per_cu: resident waves per CU of
// the wave-range kernel.  The merge takes the heads per unit: 16 for the
// decode waves, kMlaBlockHeads for the MLA blocks.
int balanced_waves_per_cu(uint32_t d, uint32_t ps, pkv_dtype dt);
hipError_t launch_rows_balanced(const RowArgs &a, pkv_dtype dt, hipStream_t st);
hipError_t launch_merge_balanced(const MergeArgs &a, pkv_dtype dt, uint32_t unit_heads,
                                 hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, pkv_dtype dt, hipStream_t st);
// MLA on MFMA (F16/BF16, rank 512, position dim 64): one block per
// (query, 64-head group, split part); balanced: one block per CU, each
// (range, 64-head group), bal_waves = the block count.
constexpr uint32_t kMlaBlockHeads = 64;
bool mla_mfma_supported(const RowArgs &a, pkv_dtype dt);
uint64_t mla_mfma_blocks(const RowArgs &a);
hipError_t launch_mla_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st);
// Blocks of a balanced MLA launch on `cus` compute units with slot rows
// for `slot_rows` (two kMlaBlockHeads-row slots per block): whole groups of
// 8 x head-group blocks, 0 when none fits.
uint32_t mla_balanced_blocks(const RowArgs &a, uint32_t cus, uint64_t slot_rows);
hipError_t launch_mla_balanced(const RowArgs &a, pkv_dtype dt, hipStream_t st);
bool tiles_supported(const TileArgs &a, pkv_dtype dt);
hipError_t launch_tiles(const TileArgs &a, pkv_dtype dt, hipStream_t st);

}  // namespace pkv
