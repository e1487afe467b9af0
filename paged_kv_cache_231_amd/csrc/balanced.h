// Balanced schedule, shared by the decode and MLA kernels.  The key tiles of
// the row queries are numbered query after query (TT keys per tile, one
// number per tile position, shared by the segq units that attend the same
// keys for different heads) and the numbers are cut into equal contiguous
// ranges, one per group of segq units; unit g of group k attends its heads
// over range k.  A unit is a wave (decode) or a block (MLA).  Every unit
// finds its range from a prefix of the tile counts that it computes itself,
// so no launch or synchronisation precedes it; one unit also stores, per row
// query, its first tile and tile count for the merge.  A range is a list of
// pieces, one per query it touches.  A piece that is a whole query writes
// the output directly; a piece cut by a range boundary writes f32 partials
// (normalised o and base-2 lse) to a slot of its unit: slot 2u when it is
// the unit's first piece and its query began in an earlier range, else slot
// 2u + 1 (its query goes on into the next range).  The merge kernel combines
// the cut pieces.

#pragma once

#include "device_common.h"

namespace pkv {
namespace bal {

// Visible keys of query i (the causal count needs no length load), capped
// at the table's reach.
__device__ __forceinline__ uint32_t row_keys(const RowArgs &a, uint32_t seq, uint32_t pos) {
  const uint64_t reach = uint64_t(a.plan.W) * a.plan.ps;
  uint64_t n = a.causal ? uint64_t(pos) + 1u : uint64_t(a.plan.words[a.plan.lens + seq]);
  return uint32_t(n < reach ? n : reach);
}

// Tiles of TT keys of a query with n visible keys, on the TT-key grid from
// the tile that holds its first visible key (the window's start).
template <uint32_t TT>
__device__ __forceinline__ uint32_t key_tiles(const RowArgs &a, uint32_t n) {
  return ceil_div_u(n, TT) - window_lo(n, a.window) / TT;
}

// Inclusive prefix sum over the 64 lanes of a full wave, on DPP: shifts by
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside
// the row add 0), then the last lane of row 0 added to row 1 and of row 2
// to row 3, then lane 31 added to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, uint32_t) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Tile prefix over 64 consecutive row queries base .. base + 63: lane l
// holds v = tiles of query base + l (0 past the end) and excl = first tile
// of that query, with the query's index i, sequence and visible keys n (so
// a piece needs no second look-up); end = first tile after the chunk.
struct Chunk {
  uint32_t base, end;
  uint32_t v, excl;
  uint32_t i, seq, n;
};

template <uint32_t TT>
__device__ __forceinline__ void scan_chunk(Chunk &c, const RowArgs &a, uint32_t base,
                                           uint32_t carry, uint32_t lane) {
  const uint32_t r = base + lane;
  const uint32_t rc = r < a.n_queries ? r : a.n_queries - 1u;
  const uint32_t i = a.qlist ? a.qlist[rc] : rc;
  const uint32_t seq = a.plan.words[a.plan.qseq + i];
  const uint32_t n = row_keys(a, seq, a.plan.words[a.plan.qpos + i]);
  const uint32_t v = r < a.n_queries ? key_tiles<TT>(a, n) : 0u;
  const uint32_t x = wave_incl_scan(v, lane);
  c.base = base;
  c.v = v;
  c.excl = carry + x - v;
  c.end = carry + __builtin_amdgcn_readlane(x, 63);
  c.i = i;
  c.seq = seq;
  c.n = n;
}

// One unit's walk over its range [t0, t_end): the chunk holding the current
// query qi and the next tile t.
struct Range {
  uint32_t t0, t, t_end, qi;
  Chunk ch;
};

// A piece: row query qi (query i of sequence seq, n visible keys), its
// tiles [tt0, tt1) of ntq; first = the unit's first piece.
struct Piece {
  uint32_t qi, tt0, tt1, ntq;
  uint32_t i, seq, n;
  bool first;
};

// Range of group grp_k of `groups`.  Returns false when the range is empty
// (more groups than tiles).  With `record`, stores bal_rec: {first tile,
// tiles} of every row query and the total at [2 n_queries].  The host
// keeps n_queries * (most tiles of a query) below 2^31, so tile numbers and
// groups * tiles-per-group do not overflow.
template <uint32_t TT>
__device__ __forceinline__ bool find_range(Range &rg, const RowArgs &a, uint32_t groups,
                                           uint32_t grp_k, bool record, uint32_t lane) {
  const uint32_t R = a.n_queries;
  // Total tiles T and the super-chunk of row queries holding this group's
  // first tile: chunks of 64 queries (coalesced loads, one wave sum each);
  // lane l adds up chunks l*m .. l*m + m - 1.
  // The tile counts of kBatch chunks are loaded together, each level of
  // the plan-word indirection (row list, query words, sequence length) for
  // all of them at once with no branch between the loads; rows past the end
  // read the last row and count 0.
  // (The causal count needs no length: that level is skipped.)  When all
  // chunks fit one batch (R <= 64 kBatch), the batch's chunks stay in
  // registers, so the range's chunk is taken from them instead of loaded
  // again.
  constexpr uint32_t kBatch = 8;
  const uint32_t nch = (R + 63u) / 64u;
  const uint32_t m = (nch + 63u) / 64u;
  const uint64_t reach = uint64_t(a.plan.W) * a.plan.ps;
  const uint32_t *words = a.plan.words;
  uint32_t s = 0, carry = 0;
  Chunk kc[kBatch];
  for (uint32_t c0 = 0; c0 < nch; c0 += kBatch) {
    uint32_t vb[kBatch], nb[kBatch], qi[kBatch], sq[kBatch], pq[kBatch];
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      const uint32_t r = (c0 + b) * 64u + lane;
      qi[b] = r < R ? r : R - 1u;
    }
    if (a.qlist) {
#pragma unroll
      for (uint32_t b = 0; b < kBatch; ++b) qi[b] = a.qlist[qi[b]];
    }
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      sq[b] = words[a.plan.qseq + qi[b]];
      pq[b] = words[a.plan.qpos + qi[b]];
    }
    if (a.causal) {
#pragma unroll
      for (uint32_t b = 0; b < kBatch; ++b) nb[b] = pq[b] + 1u;
    } else {
#pragma unroll
      for (uint32_t b = 0; b < kBatch; ++b) nb[b] = words[a.plan.lens + sq[b]];
    }
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      if (uint64_t(nb[b]) > reach) nb[b] = uint32_t(reach);
      vb[b] = (c0 + b) * 64u + lane < R ? ceil_div_u(nb[b], TT) - window_lo(nb[b], a.window) / TT : 0u;
    }
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      const uint32_t c = c0 + b;
      if (c >= nch) break;
      const uint32_t r = c * 64u + lane;
      const uint32_t v = vb[b];
      const uint32_t x = wave_incl_scan(v, lane);
      const uint32_t tot = __builtin_amdgcn_readlane(x, 63);
      if (c / m == lane) s += tot;
      if (record && r < R) {
        a.bal_rec[2u * r] = carry + x - v;
        a.bal_rec[2u * r + 1u] = v;
      }
      if (c0 == 0u) {
        kc[b].base = c * 64u;
        kc[b].v = v;
        kc[b].excl = carry + x - v;
        kc[b].end = carry + tot;
        kc[b].i = qi[b];
        kc[b].seq = sq[b];
        kc[b].n = nb[b];
      }
      carry += tot;
    }
  }
  const uint32_t sx = wave_incl_scan(s, lane);
  const uint32_t T = __builtin_amdgcn_readlane(sx, 63);
  if (record && lane == 0u) a.bal_rec[2u * R] = T;
  const uint32_t tpg = T / groups + (T % groups != 0u);
  rg.t0 = rg.t = grp_k * tpg;
  if (rg.t >= T) return false;
  rg.t_end = T - rg.t < tpg ? T : rg.t + tpg;
  if (nch <= kBatch) {
    // the first kept chunk that ends after t (t < T, so one does)
    bool found = false;
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b)
      if (!found && b < nch && kc[b].end > rg.t) {
        rg.ch = kc[b];
        found = true;
      }
  } else {
    // super-chunk lane: the last one starting at or before t (its sum is > 0)
    const uint64_t sel = __ballot(sx - s <= rg.t);
    const uint32_t lb = 63u - uint32_t(__builtin_clzll(sel));
    scan_chunk<TT>(rg.ch, a, lb * m * 64u, __builtin_amdgcn_readlane(sx - s, lb), lane);
    while (rg.ch.end <= rg.t) scan_chunk<TT>(rg.ch, a, rg.ch.base + 64u, rg.ch.end, lane);
  }
  rg.qi = rg.ch.base + 63u - uint32_t(__builtin_clzll(__ballot(rg.ch.excl <= rg.t)));
  return true;
}

// Next piece of the range, or false when the range is done.
template <uint32_t TT>
__device__ __forceinline__ bool next_piece(Range &rg, const RowArgs &a, uint32_t lane, Piece &p) {
  while (rg.t < rg.t_end) {
    if (rg.qi - rg.ch.base >= 64u) scan_chunk<TT>(rg.ch, a, rg.ch.base + 64u, rg.ch.end, lane);
    const uint32_t li = rg.qi - rg.ch.base;
    const uint32_t c0 = __builtin_amdgcn_readlane(rg.ch.excl, li);
    const uint32_t ntq = __builtin_amdgcn_readlane(rg.ch.v, li);  // tiles of this query
    if (c0 + ntq <= rg.t) {  // a query with no tiles
      ++rg.qi;
      continue;
    }
    p.qi = rg.qi;
    p.i = __builtin_amdgcn_readlane(rg.ch.i, li);
    p.seq = __builtin_amdgcn_readlane(rg.ch.seq, li);
    p.n = __builtin_amdgcn_readlane(rg.ch.n, li);
    p.ntq = ntq;
    p.tt0 = rg.t - c0;
    p.tt1 = ntq - p.tt0 < rg.t_end - rg.t ? ntq : p.tt0 + (rg.t_end - rg.t);
    p.first = rg.t == rg.t0;
    rg.t += p.tt1 - p.tt0;
    if (p.tt1 == ntq) ++rg.qi;
    return true;
  }
  return false;
}

// Slot of a cut piece of unit u (see the schedule above).
__device__ __forceinline__ uint32_t piece_slot(const Piece &p, uint32_t u) {
  return (p.first && p.tt0 > 0u) ? 2u * u : 2u * u + 1u;
}

}  // namespace bal
}  // namespace pkv
