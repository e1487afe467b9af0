// MLA decode kernel on MFMA: absorbed queries against one shared latent head
// plus a position part (ruDNN 0.1.7 `paged_attention` page, `DevicePlan::mla`
// doc), for latent rank 512 and position dim 64.
//
// For one query every q head attends the same cache rows, so scores and the
// output are dense contractions over the latent:
//   S^T[tokens x heads] = latent . q_abs^T + k_pos . q_pos^T   (576-deep)
//   O^T[rank x heads]  += latent^T . P^T                        (token-deep)
// A block owns one (query, split part, 64-head group) in the split grid, or
// one equal range of the queries' 32-token tiles and a 64-head group in the
// balanced grid (pieces of several queries in turn).  Its eight waves (two
// per SIMD) take two roles: four score waves (16 heads each: scores, online
// softmax, probabilities into LDS) work on tile kt while four value waves
// (128 output dims of all 64 heads each, the 128 x 64 f32 tile in VGPRs)
// accumulate tile kt - 1, so on every SIMD one wave's softmax arithmetic
// runs under the other's matrix instructions.  Latent and k_pos rows travel
// HBM -> LDS directly into a four-stage ring; the latent is read from LDS as
// the A operand of q.k and, transposed, as the A operand of the value
// product (16x16x32 with 32 tokens per step).  The online softmax is kept in
// base 2 with lazy rescaling.  Split parts, and balanced pieces cut by a
// range boundary, write f32 partials that a merge kernel combines.

#include "balanced.h"
#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kWaves = 8;          // two per SIMD: four score waves, four value waves
constexpr int kThreads = 64 * kWaves;
constexpr int kRoleWaves = 4;      // waves per role
constexpr int kHeadsPerBlock = kRoleWaves * 16;
static_assert(kHeadsPerBlock == int(kMlaBlockHeads), "slot rows per block of the balanced merge");
constexpr int kTT = 32;            // tokens per tile (two 16-row M-tiles)
constexpr int kStages = 4;         // LDS ring stages
constexpr int kTableCache = 1024;  // block-table entries cached in LDS
constexpr float kSlack = 8.0f;     // lazy-rescale threshold (log2 units)
// Waves that issue the ring's DMA: 0 all eight, 1 the value waves, 2 the
// score waves.
constexpr int kDmaRole = 2;
// The refill of interval k (tile k + 2) is issued at its start (false) or
// at its end, just before the barrier (true).
constexpr bool kDmaAtTail = false;

// LDS layout of one ring stage: 32 latent rows of R bf16/f16 (row stride 2R
// bytes), then 32 position rows of P.  Within each 256-byte segment of a
// latent row, 16-byte chunk c of row r sits in slot c ^ (r & 15).  A
// 16-byte LDS read is served eight lanes at a time, and is free of bank
// conflicts when each eight lanes take eight distinct 16-byte units of one
// 128-byte half (measured): the q.k operand reads (one row per lane, lanes
// c16 = 0..7 rows 0..7) are.  The transposed value reads (32 lanes per
// cycle, four lanes per row) take their rows in an order that puts the
// eight rows of a cycle into distinct 32-byte slot pairs (see pv_row
// below).  Position rows (128 bytes) keep chunk c of row r in slot
// c ^ ((r >> 1) & 7).

template <int R, int P>
struct MLds {
  static constexpr int kLatRow = R * 2;            // 1024 bytes
  static constexpr int kPosRow = P * 2;            // 128 bytes
  static constexpr int kLat = kTT * kLatRow;
  static constexpr int kPos = kTT * kPosRow;
  static constexpr int kStage = kLat + kPos;
  static constexpr int kBytes = kStages * kStage;
  static constexpr int kLatCPR = R / 8;            // 16-byte chunks per latent row
  static constexpr int kPosCPR = P / 8;            // per position row
  static __device__ __forceinline__ uint32_t lat_slot(uint32_t c, uint32_t r) { return c ^ (r & 15u); }
  static __device__ __forceinline__ uint32_t pos_slot(uint32_t c, uint32_t r) { return c ^ ((r >> 1) & 7u); }
};

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (inline assembly: the compiler's wait insertion would otherwise drain the
// ring before every LDS read; the ring's explicit waits order it).  The first
// form takes a per-lane address, the second a uniform base plus a per-lane
// 32-bit byte offset.  The LDS base goes in through an M0 operand, so the
// compiler itself sets M0 and knows what it holds.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void dma16_s(const void *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char *)(p)));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One piece of work for the whole block: query i (sequence seq), tokens
// [t_lo, t_hi), the block's 64 heads from hb.  The result goes to the output
// rows of the query (direct) or, normalised with its base-2 lse, to f32 rows
// row_base + (head - hb) of ws_o / ws_lse.  Every wave of the block calls it
// with the same arguments; it starts by rewriting the table cache and the
// ring, so a caller running pieces back to back passes a block barrier
// first.
//
// Schedule.  Barrier B_k (k = 0 .. n) opens interval k, in which score
// waves process tile k (k < n) into probability buffer k % 2 and value
// waves accumulate tile k - 1 (k >= 1) from buffer (k - 1) % 2; every wave
// issues its share of tile k + 2's DMA into the stage tile k - 2 used, and
// before B_{k+1} waits for its share of tile k + 1.  One more interval
// hands the denominators to the value waves.
template <class DT, int R, int P>
__device__ __forceinline__ void mla_piece(const RowArgs &a, uint32_t i, uint32_t seq, uint32_t t_lo,
                                          uint32_t t_hi, uint32_t hb, bool direct, uint64_t row_base) {
  using M = Mfma<DT>;
  using L = MLds<R, P>;
  using T = typename DT::T;
  constexpr int KS = R / 32;                  // q.k steps over the latent (16)
  constexpr int KP = P / 32;                  // q.k steps over the position part (2)
  constexpr int MBW = R / 16 / kRoleWaves;    // 16-dim output blocks per value wave (8)
  constexpr int NBW = kHeadsPerBlock / 16;    // 16-head column blocks (4)
  constexpr int kPBytes = kHeadsPerBlock * kTT * 2;  // one tile's probabilities, bf16/f16
  constexpr int kLoads = kTT / (kDmaRole == 0 ? kWaves : kRoleWaves) + 1;  // DMA instructions per issuing wave per tile
  __shared__ __align__(1024) unsigned char lds[L::kBytes];
  __shared__ uint32_t tcache[kTableCache];
  // P of a tile: the 16-byte chunk j (K slots 8j .. 8j+7 of the value
  // product) of head 16 nb + c16 at 1024 nb + 256 j + 16 c16, so every eight
  // lanes of a store or load touch eight consecutive chunks
  __shared__ __align__(16) unsigned char pl[2][kPBytes];
  __shared__ float pal[2][kHeadsPerBlock];    // per head: rescale factor of the tile
  __shared__ float fin[2][kHeadsPerBlock];    // per head: final reference and denominator

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  const bool scorer = wv < uint32_t(kRoleWaves);
  const uint32_t rw = scorer ? wv : wv - uint32_t(kRoleWaves);  // index within the role
  const uint32_t ps = a.plan.ps;
  const bool pow2 = (ps & (ps - 1)) == 0;
  const uint32_t ps_shift = pow2 ? uint32_t(__builtin_ctz(ps)) : 0u;
  auto page_of = [&](uint32_t tok) { return pow2 ? tok >> ps_shift : tok / ps; };

  // Block-table entries of the part, cached in LDS as a window of
  // kTableCache logical pages starting at page `wb` (moved forward when a
  // tile reaches past it, which only parts longer than the window need).
  const uint32_t *table = a.plan.words + a.plan.table + uint64_t(seq) * a.plan.W;
  const uint32_t lp_end = t_hi > t_lo ? page_of(t_hi - 1) + 1 : 0u;
  uint32_t wb = page_of(t_lo);
  auto fill_window = [&]() {
    for (uint32_t e = tid; e < uint32_t(kTableCache) && wb + e < lp_end; e += kThreads) {
      const uint32_t pg = table[wb + e];
      tcache[e] = pg < a.plan.N ? pg : 0u;  // never read outside the pool
    }
  };
  fill_window();

  const float sl2 = a.scale_log2;
  const T *lat = static_cast<const T *>(a.k);
  const T *kpos = static_cast<const T *>(a.kp);
  __syncthreads();  // table cache ready

  // DMA of tile kt, issued by the waves of kDmaRole (all eight, or the four
  // of one role): issuing wave d of nd loads latent rows (32 / nd) d ..
  // (one whole row per instruction: uniform row base, per-lane chunk
  // offset) and the position rows beside them (one instruction; with eight
  // issuers lanes 0..31 only).  Lane l locates row (32 / nd) d + l/8 (mod
  // the rows it owns); the latent loads take the page and slot of lanes 0,
  // 8, 16, ...  Rows past the end read row 0 of page 0; their latent is
  // zeroed before the value product.
  constexpr int nd = kDmaRole == 0 ? kWaves : kRoleWaves;
  constexpr int kRowsPer = kTT / nd;  // latent rows per issuing wave
  const bool issuer = kDmaRole == 0 || (kDmaRole == 1) == !scorer;
  const uint32_t dw = kDmaRole == 0 ? wv : rw;  // index among the issuers
  uint32_t lat_voff[kRowsPer];  // byte offset of the chunk lane l fetches
#pragma unroll
  for (int n2 = 0; n2 < kRowsPer; ++n2) lat_voff[n2] = 16u * L::lat_slot(lane, dw * uint32_t(kRowsPer) + n2);
  const uint32_t pos_r = dw * uint32_t(kRowsPer) + ((lane >> 3) % uint32_t(kRowsPer));
  const uint32_t pos_voff = 16u * L::pos_slot(lane % L::kPosCPR, pos_r);
  auto issue = [&](uint32_t kt) {
    if (!issuer) return;
    unsigned char *stage = lds + (kt % kStages) * L::kStage;
    const uint32_t t0 = t_lo + kt * kTT;
    const uint32_t tok = t0 + pos_r;
    const bool ok = tok < t_hi;
    const uint32_t lp = ok ? page_of(tok) : wb;
    const uint32_t slot = ok ? tok - lp * ps : 0u;
    const uint32_t page = ok ? tcache[lp - wb] : 0u;
    // every lane forms the 64-bit address of the row it locates (vector
    // arithmetic, once per tile: a cache may hold more than 2^32 elements);
    // each row's instruction then reads the two halves of its row's address
    const uint64_t ra = reinterpret_cast<uint64_t>(lat + (uint64_t(page) * a.k_page + uint64_t(slot) * a.k_tok));
    const uint32_t ra_lo = uint32_t(ra), ra_hi = uint32_t(ra >> 32);
#pragma unroll
    for (int n2 = 0; n2 < kRowsPer; ++n2) {
      const uint32_t rr = dw * uint32_t(kRowsPer) + n2;
      // (the builtin returns int: widen through uint32_t, never sign-extend)
      const uint64_t rs = uint64_t(uint32_t(__builtin_amdgcn_readlane(ra_lo, 8 * n2))) |
                          (uint64_t(uint32_t(__builtin_amdgcn_readlane(ra_hi, 8 * n2))) << 32);
      dma16_s(reinterpret_cast<const T *>(rs), lat_voff[n2],
              __builtin_amdgcn_readfirstlane(lds_addr(stage + rr * L::kLatRow)));
    }
    const uint64_t off = uint64_t(page) * a.kp_page + uint64_t(slot) * a.kp_tok;
    if (lane < 8u * uint32_t(kRowsPer))
      dma16(reinterpret_cast<const unsigned char *>(kpos + off) + pos_voff,
            __builtin_amdgcn_readfirstlane(lds_addr(stage + L::kLat + uint32_t(kRowsPer) * dw * L::kPosRow)));
  };
  // before issuing tile kt: move the table window if the tile reaches past
  // it (every wave calls this at the same point of an interval)
  auto window_for = [&](uint32_t kt) {
    const uint32_t t0 = t_lo + kt * kTT;
    const uint32_t last = (t0 + kTT < t_hi ? t0 + kTT : t_hi) - 1u;
    if (page_of(last) >= wb + uint32_t(kTableCache)) {
      block_sync_lds();  // every wave is done with the old entries
      wb = page_of(t0);
      fill_window();
      __syncthreads();
    }
  };

  // Token order.  The value product's K slots of lane group j are the rows
  // pv_row(j, 0..3) of the tile, then the same rows + 16 (the order that
  // keeps its transposed reads free of bank conflicts, see below).
  //   pv_row(j, e) = 4 (j & 1) + (j >> 1) + 2 (e & 1) + 8 (e >> 1): the rows
  //   of lanes 0..31 are 0,2,4,..,14, those of lanes 32..63 the odd rows,
  //   one row of each slot pair per LDS cycle.
  // A score lane (j, c16) holds rows 4j .. 4j+3 of each M-tile; one lane
  // swap (below) gives it rows pv_row(j, 0..3) instead, its value K slots.
  auto pv_row_of = [](uint32_t jj, uint32_t e) {
    return 4u * (jj & 1u) + (jj >> 1) + 2u * (e & 1u) + 8u * (e >> 1);
  };
  // q.k: lane (j, c16) reads chunk 4ks + j of row c16 + 16 mt (the swizzle
  // permutes chunks inside 256-byte segments: a per-lane base plus an
  // immediate segment offset); position rows likewise.
  uint32_t qk_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qk_off[u] = c16 * L::kLatRow + 16u * L::lat_slot(4u * u + j, c16);
  uint32_t pos_off[KP];
#pragma unroll
  for (int ks = 0; ks < KP; ++ks) pos_off[ks] = c16 * L::kPosRow + 16u * L::pos_slot(4u * ks + j, c16);
  // V^T: a transposed read gives lane (j, i) dim 16b + i of four rows,
  // supplied by the group's lanes: lane (j, c16) supplies row pv_row(j,
  // c16 >> 2) (+16 for the second read), dims 16b + 4 (c16 & 3) .. +3, i.e.
  // chunk 2b + ((c16 & 3) >> 1), half c16 & 1; a value wave's blocks are
  // b = 8 rw + mb.
  const uint32_t e4 = c16 >> 2, q4 = c16 & 3u;
  const uint32_t pv_row = pv_row_of(j, e4);
  uint32_t pv_off[MBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
    pv_off[mb] = pv_row * L::kLatRow + 8u * (q4 & 1u) + 16u * L::lat_slot(2u * mb + (q4 >> 1), pv_row) + 256u * rw;

  const uint32_t n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTT - 1) / kTT : 0u;
  // the interval skeleton shared by both roles (same barriers in every wave)
  auto prologue = [&]() {
    if (n_tiles > 0u) issue(0);
    if (n_tiles > 1u) {
      window_for(1);
      issue(1);
    }
    if (n_tiles > 1u) wait_vm<kLoads>();
    else wait_vm<0>();
    block_sync_lds();  // B_0: tile 0 ready
  };
  auto interval_head = [&](uint32_t k) {
    if (k + 2 < n_tiles) {
      window_for(k + 2);
      if (!kDmaAtTail) issue(k + 2);
    }
  };
  auto interval_tail = [&](uint32_t k) {
    if (kDmaAtTail && k + 2 < n_tiles) issue(k + 2);
    // this wave's share of tile k + 1 has landed (tile k + 2's may not)
    if (k + 2 < n_tiles) wait_vm<kLoads>();
    else wait_vm<0>();
    block_sync_lds();  // B_{k+1}
  };

  if (scorer) {
    // Score waves: column c16 is head hb + 16 rw + c16 (heads past hq
    // compute on head 0's query and are never stored).
    uint4 qa[KS], qp[KP];
    {
      const uint32_t h = hb + 16u * rw + c16;
      const uint64_t row = uint64_t(i) * a.hq + (h < a.hq ? h : 0u);
      const T *qrow = static_cast<const T *>(a.q) + row * R;
      const T *prow = static_cast<const T *>(a.qp) + row * P;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const uint4 *>(qrow + 8 * (4 * ks + j));
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) qp[ks] = *reinterpret_cast<const uint4 *>(prow + 8 * (4 * ks + j));
      // finish these loads here: a wait the compiler placed at their first
      // use would also drain the ring's DMA loads
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qa[ks].x), "v"(qa[ks].y), "v"(qa[ks].z), "v"(qa[ks].w));
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) asm volatile("" ::"v"(qp[ks].x), "v"(qp[ks].y), "v"(qp[ks].z), "v"(qp[ks].w));
    }
    float m = kNoMax, lsum = 0.f;  // the head's reference (base 2), this lane's share of l
    prologue();
    for (uint32_t k = 0; k <= n_tiles; ++k) {
      interval_head(k);
      if (k < n_tiles) {
        const uint32_t t0 = t_lo + k * kTT;
        const unsigned char *st_lat = lds + (k % kStages) * L::kStage;
        const unsigned char *st_pos = st_lat + L::kLat;
        // S^T: both M-tiles of this wave's 16 heads, two accumulators each;
        // read r (k-step r / 2, M-tile r % 2) is issued kAhead reads ahead
        // and the order is fenced.
        f32x4_t acc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int c = 0; c < 2; ++c) acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        {
          constexpr int kReads = 2 * (KS + KP), kAhead = 6;
          auto load_a = [&](int r) -> uint4 {
            const int ks = r >> 1, mt = r & 1;
            if (ks < KS)
              return *reinterpret_cast<const uint4 *>(st_lat + mt * (16 * L::kLatRow) + qk_off[ks & 3] +
                                                      256 * (ks >> 2));
            return *reinterpret_cast<const uint4 *>(st_pos + mt * (16 * L::kPosRow) + pos_off[ks - KS]);
          };
          uint4 ka[kAhead + 1];
#pragma unroll
          for (int r = 0; r < kAhead; ++r) ka[r] = load_a(r);
#pragma unroll
          for (int r = 0; r < kReads; ++r) {
            if (r + kAhead < kReads) ka[(r + kAhead) % (kAhead + 1)] = load_a(r + kAhead);
            const int ks = r >> 1, mt = r & 1;
            acc[mt][ks & 1] = M::qk(ka[r % (kAhead + 1)], ks < KS ? qa[ks] : qp[ks - KS], acc[mt][ks & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // lane (j, c16) holds tokens 16 mt + 4 j + e of head 16 rw + c16:
        // masked past the end, scaled to base 2
        float x[2][4];
        float lmx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool vis = t0 + 16u * mt + 4u * j + uint32_t(e) < t_hi;
            x[mt][e] = vis ? (acc[mt][0][e] + acc[mt][1][e]) * sl2 : -INFINITY;
            lmx = fmaxf(lmx, x[mt][e]);
          }
        // Lazy rescaling: the reference moves only when the head's tile max
        // passes it by more than kSlack, so probabilities stay below
        // 2^kSlack; the factor goes to the value waves with the
        // probabilities.
        const float tm = rows4_max(lmx);
        float alpha = 1.f;
        if (tm > m + kSlack) {
          alpha = fast_exp2(m - tm);
          m = tm;
          lsum *= alpha;
        }
        float pr[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) pr[mt][e] = fast_exp2(x[mt][e] - m);
        lsum += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
        // into value-product order: pack the even and odd rows separately;
        // one swap of lanes 32..63 of the even pairs with lanes 0..31 of the
        // odd pairs delivers them (lanes of j = 0 get rows (0, 2) and
        // (8, 10), j = 1 (4, 6) (12, 14), j = 2 (1, 3) (9, 11), j = 3 (5, 7)
        // (13, 15)), rows + 16 from the second M-tile
        const auto lo = __builtin_amdgcn_permlane32_swap(M::pack2(pr[0][0], pr[0][2]), M::pack2(pr[0][1], pr[0][3]),
                                                         false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(M::pack2(pr[1][0], pr[1][2]), M::pack2(pr[1][1], pr[1][3]),
                                                         false, false);
        *reinterpret_cast<uint4 *>(&pl[k & 1u][1024u * rw + 256u * j + 16u * c16]) =
            make_uint4(lo[0], lo[1], hi[0], hi[1]);
        if (j == 0u) pal[k & 1u][16u * rw + c16] = alpha;
      } else {
        // denominators and references for the value waves
        const float l_tot = rows4_sum(lsum);
        if (j == 0u) {
          fin[0][16u * rw + c16] = m;
          fin[1][16u * rw + c16] = l_tot;
        }
      }
      interval_tail(k);
    }
    return;
  }

  // Value waves: o[mb][nb] holds O^T[dim 128 rw + 16 mb + 4 j + e][head hb +
  // 16 nb + c16].
  f32x4_t o[MBW][NBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) o[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  prologue();
  for (uint32_t k = 0; k <= n_tiles; ++k) {
    interval_head(k);
    if (k >= 1u) {
      // value product of tile k - 1
      const uint32_t kv = k - 1u;
      const unsigned char *st_lat = lds + (kv % kStages) * L::kStage;
      float al[NBW];
      bool moved = false;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        al[nb] = pal[kv & 1u][16u * nb + c16];
        moved |= al[nb] != 1.f;
      }
      if (__any(moved)) {
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) o[mb][nb] *= al[nb];
      }
      uint4 pb[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        pb[nb] = *reinterpret_cast<const uint4 *>(&pl[kv & 1u][1024u * nb + 256u * j + 16u * c16]);
      constexpr int kPvAhead = 3;
      auto load_v = [&](int mb) -> uint4 {
        const unsigned char *p0 = st_lat + pv_off[mb];
        const uint2 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * L::kLatRow);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 va[kPvAhead + 1];
#pragma unroll
      for (int mb = 0; mb < kPvAhead; ++mb) va[mb] = load_v(mb);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        if (mb + kPvAhead < MBW) va[(mb + kPvAhead) % (kPvAhead + 1)] = load_v(mb + kPvAhead);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) o[mb][nb] = M::qk(va[mb % (kPvAhead + 1)], pb[nb], o[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k + 1 == n_tiles) {
      // tile k is the last: zero its latent rows past the end (they are
      // also V; no value wave reads the stage before the next barrier, and
      // the score waves mask those rows)
      const uint32_t t0 = t_lo + k * kTT;
      unsigned char *st_lat = lds + (k % kStages) * L::kStage;
      if (t0 + kTT > t_hi)
        for (uint32_t e = tid - 64u * kRoleWaves; e < uint32_t(kTT * L::kLatCPR); e += 64u * kRoleWaves) {
          const uint32_t r = e / L::kLatCPR;
          if (t0 + r >= t_hi)
            *reinterpret_cast<uint4 *>(st_lat + r * L::kLatRow + 16u * (e % L::kLatCPR)) =
                make_uint4(0, 0, 0, 0);
        }
    }
    interval_tail(k);
  }

  // normalise and write: lane holds O^T[dim 128 rw + 16 mb + 4j + e][head hb + 16 nb + c16]
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const uint32_t hl = 16u * nb + c16, h = hb + hl;
    if (h >= a.hq) continue;
    const float mh = fin[0][hl], l_tot = fin[1][hl];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (direct) {
      T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * R + 128u * rw + 4u * j;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        uint2 w;
        w.x = M::pack2(o[mb][nb][0] * inv, o[mb][nb][1] * inv);
        w.y = M::pack2(o[mb][nb][2] * inv, o[mb][nb][3] * inv);
        *reinterpret_cast<uint2 *>(out + 16 * mb) = w;
      }
    } else {
      const uint64_t r = row_base + hl;
      float *wo = a.ws_o + r * R + 128u * rw + 4u * j;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) *reinterpret_cast<f32x4_t *>(wo + 16 * mb) = o[mb][nb] * inv;
      if (rw == 0u && j == 0u) a.ws_lse[r] = mh + fast_log2(l_tot);
    }
  }
}

// Split grid: one block per (query, split part, 64-head group).
template <class DT, int R, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_kernel(RowArgs a, uint32_t head_groups) {
  // Blocks are dispatched round-robin over the eight XCDs.  The head groups
  // of one (query, part) read the same cache rows, so they get consecutive
  // logical numbers on one XCD (the second read then hits that XCD's L2);
  // logical order is part-major (the first parts of every query start first).
  const uint32_t bid = blockIdx.x, span8 = 8u * head_groups;
  const uint32_t logical = (bid / span8) * span8 + (bid % 8u) * head_groups + (bid % span8) / 8u;
  const uint32_t per_part = a.n_queries * head_groups;
  if (logical >= per_part * a.splits) return;
  const uint32_t part = logical / per_part;
  const uint32_t rest = logical % per_part;
  const uint32_t hgi = rest % head_groups;
  const uint32_t qi = rest / head_groups;
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  uint32_t seq;
  const uint32_t n = visible_keys(a.plan, i, a.causal, &seq);
  const uint64_t span = uint64_t(a.pages_per_split) * a.plan.ps;
  const uint64_t lo64 = uint64_t(part) * span;
  if (a.splits > 1 && lo64 >= n) return;  // empty part: the merge skips it
  const uint32_t t_lo = uint32_t(lo64 < n ? lo64 : n);
  const uint32_t t_hi = uint32_t(lo64 + span < n ? lo64 + span : n);
  const uint32_t hb = hgi * kHeadsPerBlock;
  mla_piece<DT, R, P>(a, i, seq, t_lo, t_hi, hb, a.splits == 1,
                      (uint64_t(i) * a.splits + part) * a.hq + hb);
}

// Balanced grid (balanced.h) with blocks as units: block u of the launch
// attends 64-head group g = u % head_groups over range u / head_groups, so
// every block streams the same number of 32-token tiles whatever the length
// mix.  The head groups of one range are numbered onto one XCD and run side
// by side, so the second read of each latent tile hits that XCD's L2.
template <class DT, int R, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_balanced_kernel(RowArgs a, uint32_t head_groups) {
  const uint32_t bid = blockIdx.x, span8 = 8u * head_groups;
  const uint32_t u = (bid / span8) * span8 + (bid % 8u) * head_groups + (bid % span8) / 8u;
  const uint32_t groups = a.bal_waves / head_groups;
  const uint32_t grp_k = u / head_groups, g = u % head_groups;
  if (grp_k >= groups) return;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bal::Range rg;
  if (!bal::find_range<kTT>(rg, a, groups, grp_k, u == 0u && wv == 0u, lane)) return;
  const uint32_t hb = g * kHeadsPerBlock;
  bal::Piece pc;
  while (bal::next_piece<kTT>(rg, a, lane, pc)) {
    const uint32_t i = pc.i, seq = pc.seq, n = pc.n;  // found with the range
    const uint32_t t_lo = pc.tt0 * kTT;
    const uint32_t t_hi = pc.tt1 * kTT < n ? pc.tt1 * kTT : n;
    const bool whole = pc.tt0 == 0u && pc.tt1 == pc.ntq;
    const uint32_t slot = bal::piece_slot(pc, u);
    __syncthreads();  // the previous piece's ring and table cache are free
    mla_piece<DT, R, P>(a, i, seq, t_lo, t_hi, hb, whole, uint64_t(slot) * kHeadsPerBlock);
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool mla_mfma_supported(const RowArgs &a, pkv_dtype dt) {
  if (dt != PKV_F16 && dt != PKV_BF16) return false;
  if (a.d != 512 || a.dv != 512 || a.pdim != 64 || a.hkv != 1) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.qp) || !aligned16(a.kp)) return false;
  if (a.splits == 1 && !aligned16(a.out)) return false;
  return true;
}

uint64_t mla_mfma_blocks(const RowArgs &a) {
  // rounded up to whole groups of 8 * hg (see the XCD mapping)
  const uint64_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const uint64_t n = uint64_t(a.n_queries) * hg * a.splits;
  return (n + 8 * hg - 1) / (8 * hg) * (8 * hg);
}

uint32_t mla_balanced_blocks(const RowArgs &a, uint32_t cus, uint64_t slot_rows) {
  const uint64_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  uint64_t b = slot_rows / (2 * kHeadsPerBlock);
  if (cus < b) b = cus;
  b -= b % (8 * hg);
  return uint32_t(b);
}

hipError_t launch_mla_balanced(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint32_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  if (a.bal_waves == 0 || a.bal_waves % (8 * hg) != 0) return hipErrorInvalidValue;
  const dim3 grid(a.bal_waves);
  if (dt == PKV_BF16)
    launch_k((mla_balanced_kernel<BF16, 512, 64>), grid, dim3(kThreads), 0, st, a, hg);
  else
    launch_k((mla_balanced_kernel<F16, 512, 64>), grid, dim3(kThreads), 0, st, a, hg);
  return hipGetLastError();
}

hipError_t launch_mla_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint32_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const uint64_t blocks = mla_mfma_blocks(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));  // a multiple of 8 * hg
  if (dt == PKV_BF16)
    launch_k((mla_kernel<BF16, 512, 64>), grid, dim3(kThreads), 0, st, a, hg);
  else
    launch_k((mla_kernel<F16, 512, 64>), grid, dim3(kThreads), 0, st, a, hg);
  return hipGetLastError();
}

}  // namespace pkv
