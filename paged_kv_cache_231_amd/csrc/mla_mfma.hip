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
// balanced grid (pieces of several queries in turn); its four waves (one
// per SIMD) own 16 heads each, with the 512 x 16 f32 output tile in VGPRs
// and the loop-invariant query operands in AGPRs (MFMA reads them there).
// Latent and k_pos rows travel HBM -> LDS directly into a four-stage ring
// (three 32-token tiles ahead); the latent is read from LDS as the A operand
// of q.k and, transposed, as the A operand of the value product (16x16x32
// with 32 tokens per step).  The online softmax is kept in base 2 with lazy
// rescaling.  Split parts, and balanced pieces cut by a range boundary,
// write f32 partials that a merge kernel combines.

#include "balanced.h"
#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;          // one wave per SIMD
constexpr int kHeadsPerBlock = kWaves * 16;
static_assert(kHeadsPerBlock == int(kMlaBlockHeads), "slot rows per block of the balanced merge");
constexpr int kTT = 32;            // tokens per tile (two 16-row M-tiles)
constexpr int kStages = 4;         // LDS ring stages
constexpr int kTableCache = 1024;  // block-table entries cached in LDS
constexpr float kSlack = 8.0f;     // lazy-rescale threshold (log2 units)

// LDS layout of one ring stage: 32 latent rows of R bf16/f16 (row stride 2R
// bytes), then 32 position rows of P.  Within each 256-byte segment of a
// latent row, 16-byte chunk c of row r sits in slot c ^ (r & 15): the q.k
// operand reads (one row per lane, eight lanes per LDS cycle) then fall into
// distinct banks.  The transposed value reads (32 lanes per cycle, four
// lanes per row) take their rows in an order that puts the eight rows of a
// cycle into distinct 32-byte slot pairs (see pv_row below).  Position rows
// (128 bytes) keep chunk c of row r in slot c ^ ((r >> 1) & 7).

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
  static constexpr int kLatPerWave = kTT / kWaves;  // latent rows each wave loads
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

// Keep a loop-invariant MFMA operand in AGPRs (the MFMA reads it there).
__device__ __forceinline__ void to_agpr(uint4 &x) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+a"(v));
  x = __builtin_bit_cast(uint4, v);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One piece of work for the whole block: query i (sequence seq), tokens
// [t_lo, t_hi), this wave's 16 heads from h0.  The result goes to the output
// rows of the query (direct) or, normalised with its base-2 lse, to f32
// rows row0 + c16 of ws_o / ws_lse.  Every wave of the block calls it with
// the same query and tokens; it starts by rewriting the table cache and the
// ring, so a caller running pieces back to back passes a block barrier
// first.
template <class DT, int R, int P>
__device__ __forceinline__ void mla_piece(const RowArgs &a, uint32_t i, uint32_t seq, uint32_t t_lo,
                                          uint32_t t_hi, uint32_t h0, bool direct, uint64_t row0) {
  using M = Mfma<DT>;
  using L = MLds<R, P>;
  using T = typename DT::T;
  constexpr int KS = R / 32;   // q.k steps over the latent (16)
  constexpr int KP = P / 32;   // q.k steps over the position part (2)
  constexpr int DB = R / 16;   // 16-wide output blocks (32)
  constexpr int kLoads = L::kLatPerWave + 1;  // DMA instructions per wave per tile
  __shared__ __align__(1024) unsigned char lds[L::kBytes];
  __shared__ uint32_t tcache[kTableCache];

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t c16 = lane & 15u, j = lane >> 4;
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
    for (uint32_t e = tid; e < uint32_t(kTableCache) && wb + e < lp_end; e += 256) {
      const uint32_t pg = table[wb + e];
      tcache[e] = pg < a.plan.N ? pg : 0u;  // never read outside the pool
    }
  };
  fill_window();

  // this wave's heads: column c16 -> head h0 + c16; columns of heads past hq
  // compute on head 0's query and are not stored
  uint4 qa[KS], qp[KP];
  {
    const uint32_t h = h0 + c16;
    const uint64_t row = uint64_t(i) * a.hq + (h < a.hq ? h : 0u);
    const T *qrow = static_cast<const T *>(a.q) + row * R;
    const T *prow = static_cast<const T *>(a.qp) + row * P;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const uint4 *>(qrow + 8 * (4 * ks + j));
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) qp[ks] = *reinterpret_cast<const uint4 *>(prow + 8 * (4 * ks + j));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) to_agpr(qa[ks]);
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) to_agpr(qp[ks]);
  }
  f32x4_t o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNoMax, lsum = 0.f;
  const float sl2 = a.scale_log2;
  const T *lat = static_cast<const T *>(a.k);
  const T *kpos = static_cast<const T *>(a.kp);
  __syncthreads();  // table cache ready

  // DMA of tile kt: wave wv loads latent rows 8wv .. 8wv+7 (one whole row
  // per instruction: uniform row base, per-lane chunk offset) and position
  // rows 8wv .. 8wv+7 (one instruction, lane l row 8wv + l/8).  Lane l
  // locates row 8wv + l/8; the latent loads take the page and slot of lanes
  // 0, 8, .., 56.  Rows past the end read row 0 of page 0; their latent is
  // zeroed before use.
  uint32_t lat_voff[L::kLatPerWave];  // byte offset of the chunk lane l fetches
#pragma unroll
  for (int n2 = 0; n2 < L::kLatPerWave; ++n2)
    lat_voff[n2] = 16u * L::lat_slot(lane, wv * uint32_t(L::kLatPerWave) + n2);
  const uint32_t pos_r = wv * uint32_t(L::kLatPerWave) + (lane >> 3);
  const uint32_t pos_voff = 16u * L::pos_slot(lane % L::kPosCPR, pos_r);
  auto issue = [&](uint32_t kt) {
    unsigned char *stage = lds + (kt % kStages) * L::kStage;
    const uint32_t t0 = t_lo + kt * kTT;
    const uint32_t tok = t0 + pos_r;
    const bool ok = tok < t_hi;
    const uint32_t lp = ok ? page_of(tok) : wb;
    const uint32_t slot = ok ? tok - lp * ps : 0u;
    const uint32_t page = ok ? tcache[lp - wb] : 0u;
#pragma unroll
    for (int n2 = 0; n2 < L::kLatPerWave; ++n2) {
      const uint32_t rr = wv * uint32_t(L::kLatPerWave) + n2;
      const uint32_t pg = __builtin_amdgcn_readlane(page, 8 * n2);
      const uint32_t sl = __builtin_amdgcn_readlane(slot, 8 * n2);
      const T *row = lat + (pg * uint32_t(a.k_page) + sl * uint32_t(a.k_tok));
      dma16_s(row, lat_voff[n2], __builtin_amdgcn_readfirstlane(lds_addr(stage + rr * L::kLatRow)));
    }
    const uint32_t off = page * uint32_t(a.kp_page) + slot * uint32_t(a.kp_tok);
    dma16(reinterpret_cast<const unsigned char *>(kpos + off) + pos_voff,
          __builtin_amdgcn_readfirstlane(lds_addr(stage + L::kLat + 8u * wv * L::kPosRow)));
  };
  // before issuing tile kt: move the table window if the tile reaches past it
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

  // Per-lane LDS read offsets.  The swizzle only permutes 16-byte chunks
  // inside a 256-byte segment of a row, so each read is a per-lane base plus
  // an immediate segment offset.
  //   q.k:  lane (j, c16) reads chunk 4ks + j of row c16 (+16 for M-tile 1):
  //         segment ks >> 2, in-segment slot (4 (ks & 3) + j) ^ c16
  //   pos:  chunk 4ks + j of position row c16 (+16)
  //   V^T:  a transposed read gives lane (j, i) dim 16b + i of four rows,
  //         supplied by the group's lanes: lane (j, c16) supplies row
  //         pv_row(j, c16 >> 2) (+16 for the second read), dims 16b +
  //         4 (c16 & 3) .. +3, i.e. chunk 2b + ((c16 & 3) >> 1), half c16 & 1.
  //         pv_row(j, e) = 4 (j & 1) + (j >> 1) + 2 (e & 1) + 8 (e >> 1): the
  //         rows of lanes 0..31 are 0,2,4,..,14, those of lanes 32..63 the
  //         odd rows, one row of each slot pair per LDS cycle.
  uint32_t qk_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qk_off[u] = c16 * L::kLatRow + 16u * ((4u * u + j) ^ c16);
  uint32_t pos_off[KP];
#pragma unroll
  for (int ks = 0; ks < KP; ++ks) pos_off[ks] = c16 * L::kPosRow + 16u * L::pos_slot(4u * ks + j, c16);
  const uint32_t e4 = c16 >> 2, q4 = c16 & 3u;
  const uint32_t pv_row = 4u * (j & 1u) + (j >> 1) + 2u * (e4 & 1u) + 8u * (e4 >> 1);
  uint32_t pv_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    pv_off[u] = pv_row * L::kLatRow + 8u * (q4 & 1u) + 16u * ((2u * u + (q4 >> 1)) ^ pv_row);

  const uint32_t n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTT - 1) / kTT : 0u;
  for (uint32_t kt = 0; kt < n_tiles && kt < uint32_t(kStages - 1); ++kt) {
    window_for(kt);
    issue(kt);
  }

  for (uint32_t kt = 0; kt < n_tiles; ++kt) {
    const uint32_t t0 = t_lo + kt * kTT;
    const uint32_t ahead = n_tiles - 1 - kt;
    if (ahead >= 2) wait_vm<2 * kLoads>();
    else if (ahead == 1) wait_vm<kLoads>();
    else wait_vm<0>();
    unsigned char *st_lat = lds + (kt % kStages) * L::kStage;
    unsigned char *st_pos = st_lat + L::kLat;
    if (t0 + kTT > t_hi) {
      // last tile: zero the latent of rows past the end (it is also V)
      block_sync_lds();
      for (uint32_t e = tid; e < uint32_t(kTT * L::kLatCPR); e += 256) {
        const uint32_t r = e / L::kLatCPR;
        if (t0 + r >= t_hi)
          *reinterpret_cast<uint4 *>(st_lat + r * L::kLatRow + 16u * (e % L::kLatCPR)) =
              make_uint4(0, 0, 0, 0);
      }
    }
    block_sync_lds();

    // S^T = latent . q_abs^T + k_pos . q_pos^T; M-tile mt holds tokens
    // 16 mt + c16 (A rows).  Both M-tiles advance together with four
    // accumulators each (k-step mod 4): eight independent MFMA chains.
    // Reads r = 0 .. 2 (KS + KP) - 1 go in order (k-step r / 2, M-tile
    // r % 2); read r + kAhead is issued before the MFMA of read r, and the
    // order is fenced so the LDS latency hides behind the MFMAs in flight.
    constexpr int kCh = 4;
    f32x4_t acc[2][kCh];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c = 0; c < kCh; ++c) acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
        acc[mt][ks % kCh] = M::qk(ka[r % (kAhead + 1)], ks < KS ? qa[ks] : qp[ks - KS], acc[mt][ks % kCh]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    f32x4_t s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) s[mt] = (acc[mt][0] + acc[mt][1]) + (acc[mt][2] + acc[mt][3]);

    // online softmax per head; lane (j, c16) holds tokens 16 mt + 4 j + e.
    // Probabilities are exp2 of the scaled score minus the head's current
    // reference m.  Lazy rescaling: the reference only moves when a head's
    // max exceeds it by more than kSlack (base 2), so probabilities stay
    // below 2^kSlack and most tiles skip what follows the threshold test.
    // A lane above m + kSlack means its head's max is too, so the head
    // maxima are formed only then.
    float x[2][4];
    float lmx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool vis = t0 + 16u * mt + 4u * j + e < t_hi;
        x[mt][e] = vis ? s[mt][e] * sl2 : -INFINITY;
        lmx = fmaxf(lmx, x[mt][e]);
      }
    float p[2][4];
    uint4 pb;
    // P^T operand in the value reads' row order: lane (j, c16) holds rows
    // 4j .. 4j+3 of each M-tile and needs rows pv_row(j, 0..3).  Pack the
    // even and odd rows separately; one swap of lanes 32..63 of the even
    // pairs with lanes 0..31 of the odd pairs delivers them: lanes of j = 0
    // get rows (0, 2) and (8, 10), j = 1 (4, 6) (12, 14), j = 2 (1, 3)
    // (9, 11), j = 3 (5, 7) (13, 15).
    auto probs = [&]() {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[mt][e] = fast_exp2(x[mt][e] - m);
      const auto lo = __builtin_amdgcn_permlane32_swap(M::pack2(p[0][0], p[0][2]), M::pack2(p[0][1], p[0][3]),
                                                       false, false);
      const auto hi = __builtin_amdgcn_permlane32_swap(M::pack2(p[1][0], p[1][2]), M::pack2(p[1][1], p[1][3]),
                                                       false, false);
      pb = make_uint4(lo[0], lo[1], hi[0], hi[1]);
    };
    probs();
    if (__any(lmx > m + kSlack)) {
      const float mx = rows4_max(lmx);
      const float m_new = mx > m + kSlack ? mx : m;
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      probs();
    }
    lsum += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));

    // O^T += latent^T . P^T over 32 tokens: K slots 8j .. 8j+3 are rows
    // pv_row(j, 0..3), slots 8j+4 .. 8j+7 the same rows + 16.  The two
    // transposed reads of block b + kPvAhead are issued before the MFMA of
    // block b and the order is fenced, so every MFMA finds its operand
    // loaded (left to itself the compiler reads one block at a time and
    // waits for each pair).
    {
      constexpr int kPvAhead = 4;
      auto load_v = [&](int b) -> uint4 {
        const unsigned char *p0 = st_lat + pv_off[b & 7] + 256 * (b >> 3);
        const uint2 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * L::kLatRow);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 va[kPvAhead + 1];
#pragma unroll
      for (int b = 0; b < kPvAhead; ++b) va[b] = load_v(b);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        if (b + kPvAhead < DB) va[(b + kPvAhead) % (kPvAhead + 1)] = load_v(b + kPvAhead);
        o[b] = M::qk(va[b % (kPvAhead + 1)], pb, o[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (kt + kStages - 1 < n_tiles) {
      window_for(kt + kStages - 1);
      issue(kt + kStages - 1);
    }
  }

  // normalise and write: lane holds O^T[d = 16b + 4j + e][head c16]
  const float l_tot = rows4_sum(lsum);
  const uint32_t h = h0 + c16;
  if (h >= a.hq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (direct) {
    T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * R;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      uint2 w;
      w.x = M::pack2(o[b][0] * inv, o[b][1] * inv);
      w.y = M::pack2(o[b][2] * inv, o[b][3] * inv);
      *reinterpret_cast<uint2 *>(out + 16 * b + 4 * j) = w;
    }
  } else {
    const uint64_t r = row0 + c16;
    float *wo = a.ws_o + r * R;
#pragma unroll
    for (int b = 0; b < DB; ++b) *reinterpret_cast<f32x4_t *>(wo + 16 * b + 4 * j) = o[b] * inv;
    if (j == 0) a.ws_lse[r] = m + fast_log2(l_tot);
  }
}

// Split grid: one block per (query, split part, 64-head group).
template <class DT, int R, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
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
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t h0 = hgi * kHeadsPerBlock + wv * 16u;
  mla_piece<DT, R, P>(a, i, seq, t_lo, t_hi, h0, a.splits == 1,
                      (uint64_t(i) * a.splits + part) * a.hq + h0);
}

// Balanced grid (balanced.h) with blocks as units: block u of the launch
// attends 64-head group g = u % head_groups over range u / head_groups, so
// every block streams the same number of 32-token tiles whatever the length
// mix.  The head groups of one range are numbered onto one XCD and run side
// by side, so the second read of each latent tile hits that XCD's L2.
template <class DT, int R, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
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
  const uint32_t h0 = g * kHeadsPerBlock + wv * 16u;
  bal::Piece pc;
  while (bal::next_piece<kTT>(rg, a, lane, pc)) {
    const uint32_t i = __builtin_amdgcn_readfirstlane(a.qlist ? a.qlist[pc.qi] : pc.qi);
    uint32_t seq;
    const uint32_t n = __builtin_amdgcn_readfirstlane(visible_keys(a.plan, i, a.causal, &seq));
    seq = __builtin_amdgcn_readfirstlane(seq);
    const uint32_t t_lo = pc.tt0 * kTT;
    const uint32_t t_hi = pc.tt1 * kTT < n ? pc.tt1 * kTT : n;
    const bool whole = pc.tt0 == 0u && pc.tt1 == pc.ntq;
    const uint32_t slot = bal::piece_slot(pc, u);
    __syncthreads();  // the previous piece's ring and table cache are free
    mla_piece<DT, R, P>(a, i, seq, t_lo, t_hi, h0, whole,
                        uint64_t(slot) * kHeadsPerBlock + wv * 16u);
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
    launch_k((mla_balanced_kernel<BF16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  else
    launch_k((mla_balanced_kernel<F16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  return hipGetLastError();
}

hipError_t launch_mla_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint32_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const uint64_t blocks = mla_mfma_blocks(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));  // a multiple of 8 * hg
  if (dt == PKV_BF16)
    launch_k((mla_kernel<BF16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  else
    launch_k((mla_kernel<F16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  return hipGetLastError();
}

}  // namespace pkv
