// Chunked-prefill kernel on MFMA: causal attention at absolute positions for
// runs of consecutive queries of one sequence ("tiles" of the plan).
//
// Computes the attention of the ruDNN 0.1.7 `paged_attention` page
// (`DevicePlan::attention` doc: packed queries, paged K/V, `causal` by the
// absolute positions of the plan, prefill chunks included).  A tile's queries
// are consecutive positions p0, p0+1, ... of one sequence, so they share the
// key rows 0..p_last, and every (query, q head) of one KV head forms a dense
// contraction with those rows.
//
// A block owns 128 q-rows (a q-row is one (query, q head) pair; with G q
// heads per KV head that is 128/G queries x G heads) of one tile and one KV
// head; each of its four waves owns 32 q-rows as two MFMA N-tiles.  Keys are
// walked in tiles of 32 rows.  K and V rows travel HBM -> LDS directly
// (gfx950 global_load_lds, no registers on the way) into a ring of four
// stages, three tiles ahead of the tile being computed, so the load latency
// hides behind the MFMA work.  Each wave computes S^T = K . Q^T (tokens on
// the M side), applies the absolute-position mask and an online softmax in
// base 2, and accumulates O^T += V^T . P^T, with V^T read by transposed LDS
// loads.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled by
// row, which keeps both read patterns at most two-way banked.  The block
// table of the sequence is cached in LDS.  Blocks that share a (tile, KV
// head) are numbered so they land on one XCD and share its L2.

#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kPW = 4;             // waves per block
constexpr int kRowsPerBlock = 128; // q-rows per block (32 per wave)
constexpr int kTT = 32;            // key rows per tile
constexpr int kStages = 4;         // LDS ring stages (3 tiles in flight)
constexpr int kTableCache = 1024;  // block-table entries cached in LDS
constexpr float kSlack = 8.0f;     // lazy-rescale threshold (log2 units)

template <int D>
struct PLds {
  static constexpr int kRowB = D * 2;              // bytes per row (unpadded)
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int kTile = kTT * kRowB;        // one K or V tile
  static constexpr int kStage = 2 * kTile;         // K then V
  static constexpr int kBytes = kStages * kStage;
  static constexpr int RPW = 1024 / kRowB;         // rows per wave load (64 lanes x 16 B)
  static constexpr int NI = kTT / (RPW * kPW);     // loads per wave per tensor per tile
  // chunk c of row r sits in slot c ^ swz(r): rows sharing a 256-byte bank
  // line get different XOR keys
  static __device__ __forceinline__ uint32_t swz(uint32_t r) {
    return D == 64 ? (r >> 1) & 7u : r & 15u;
  }
};

// Float max without IEEE canonicalisation of the inputs (fmaxf quiets both
// operands first): the running max is only a reference point, and a NaN
// score still reaches the output through its exponent.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max over the four 16-lane rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows4_vmax(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Compiler-level memory barriers around the raw hardware barrier: LDS loads
// and stores may not move across, and no wait for outstanding global loads
// is implied (the ring waits for those explicitly).
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// 16 bytes land at LDS byte address lds_base + 16 * l.  Written as inline
// assembly so the compiler's wait insertion does not treat every later LDS
// read as dependent on it: the ring's explicit vmcnt waits and barriers order
// these loads against the reads.  The LDS base is an M0 operand, so the
// compiler sets M0 itself and knows what it holds.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char *)(p)));
}

// Makes the compiler finish the loads of x here (it cannot see the DMA
// loads, so a wait it placed later for x would drain them too).
__device__ __forceinline__ void settle(const uint4 &x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <class DT, int D>
__global__ __launch_bounds__(256) void prefill_kernel(TileArgs a, uint32_t n_sub,
                                                      uint32_t n_groups) {
  using M = Mfma<DT>;
  using L = PLds<D>;
  using T = typename DT::T;
  constexpr int KS = D / 32, DB = D / 16;
  constexpr int kLoadsPerTile = 2 * L::NI;  // per thread: K and V
  __shared__ __align__(1024) unsigned char lds[L::kBytes];
  __shared__ uint32_t tcache[kTableCache];

  // Blocks are dispatched round-robin over the eight XCDs (blockIdx.x % 8).
  // The (tile, KV head) groups are dealt to the XCDs in turn, group g to XCD
  // g % 8, and the n_sub blocks of a group run back to back on its XCD, so
  // they share the group's K/V rows in that XCD's L2.  Dealing groups (not
  // contiguous ranges) spreads every tile's work over all XCDs: tiles of
  // one chunk have similar key counts while chunks differ widely.
  const uint32_t k = blockIdx.x / 8u;
  const uint32_t group = (k / n_sub) * 8u + blockIdx.x % 8u;
  if (group >= n_groups) return;
  const uint32_t sub = k % n_sub;
  const uint32_t kvh = group % a.hkv;
  const uint32_t tile = group / a.hkv;

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  const PlanView &pv = a.plan;
  const uint32_t first = a.tiles[2 * tile], count = a.tiles[2 * tile + 1];
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t qb_n = kRowsPerBlock / grp;  // queries per block
  const uint32_t q_lo = sub * qb_n;
  if (q_lo >= count) return;
  const uint32_t q_hi = q_lo + qb_n < count ? q_lo + qb_n : count;
  const uint32_t seq = pv.words[pv.qseq + first];
  const uint32_t p0 = pv.words[pv.qpos + first];
  const uint32_t len = pv.words[pv.lens + seq];
  uint64_t k_end64 = a.causal ? uint64_t(p0) + q_hi : uint64_t(len);
  const uint64_t reach = uint64_t(pv.W) * pv.ps;
  if (k_end64 > reach) k_end64 = reach;
  const uint32_t k_end = uint32_t(k_end64);
  const uint32_t ps = pv.ps;
  const bool pow2 = (ps & (ps - 1)) == 0;
  const uint32_t ps_shift = pow2 ? uint32_t(__builtin_ctz(ps)) : 0u;

  // block table of the sequence, first kTableCache entries, into LDS
  const uint32_t *table = pv.words + pv.table + uint64_t(seq) * pv.W;
  // (each entry holds the element offset of the page's first row: K and V
  // share their strides since head_dim == value_dim)
  const uint32_t page_elems = uint32_t(a.k_page);
  const uint32_t n_lp = (k_end + ps - 1) / ps;
  for (uint32_t e = tid; e < n_lp && e < uint32_t(kTableCache); e += 256) {
    const uint32_t pg = table[e];
    tcache[e] = (pg < pv.N ? pg : 0u) * page_elems;  // never read outside the pool
  }

  // this wave's q-rows: N-tile nt, column c16 -> q-row 32*wv + 16*nt + c16
  uint4 qb[2][KS];
  uint32_t pos[2];
  bool row_ok[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint32_t r = 32u * wv + 16u * nt + c16;
    const uint32_t qq = r / grp, h = r % grp;
    row_ok[nt] = r < qb_n * grp && q_lo + qq < q_hi;
    pos[nt] = p0 + q_lo + qq;
    const T *qrow = static_cast<const T *>(a.q) +
                    (uint64_t(first + q_lo + qq) * a.hq + kvh * grp + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[nt][ks] = row_ok[nt] ? *reinterpret_cast<const uint4 *>(qrow + 8 * (4 * ks + j))
                              : make_uint4(0, 0, 0, 0);
  }
  // smallest position among the block's queries: key tiles wholly at or
  // below it need no causal mask
  const uint32_t pos_min = p0 + q_lo;
  // last visible key of each q-row: position (causal) or the last key
  uint32_t lim[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) lim[nt] = a.causal && pos[nt] < k_end - 1u ? pos[nt] : k_end - 1u;

  f32x4_t o[2][DB];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int b = 0; b < DB; ++b) o[nt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {kNoMax, kNoMax};
  // a row's reference moves only when a raw score passes (m + kSlack) /
  // scale_log2; kNoMax makes the first visible score do so
  float thr[2] = {kNoMax, kNoMax};
  // Softmax denominators on the matrix core: one more 16-row output block
  // per N-tile whose A operand is all ones, so each of its rows accumulates
  // the sum of P over the keys for the lane's q-row (rescaled with O).
  f32x4_t lacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  uint4 ones;
  ones.x = ones.y = ones.z = ones.w = M::pack2(1.f, 1.f);
  const float sl2 = a.scale_log2;
  const float inv_sl2 = 1.f / sl2;
  const T *kbase = static_cast<const T *>(a.k) + uint64_t(kvh) * D;
  const T *vbase = static_cast<const T *>(a.v) + uint64_t(kvh) * D;
  __syncthreads();  // table cache ready (Q loads may still be in flight: fine)

  // DMA of key tile kt into its ring stage: wave wv, load n covers rows
  // RPW*(NI*wv + n) .. +RPW-1; lane -> row r0 + lane / CPR, slot lane % CPR,
  // which holds chunk slot ^ swz(row) of the cache row.  Rows past the end
  // read row 0 of page 0 (inside the pool) and are zeroed before use.
  // Per-lane parts of the DMA addresses: load n of a wave covers rows
  // r0(n) .. r0(n)+RPW-1, lane -> row r0(n) + lane / CPR and slot lane % CPR,
  // which holds chunk slot ^ swz(row) of the cache row.  For a power-of-two
  // page size the token's slot in its page is (kt*kTT mod ps) + (row mod ps),
  // so its element offset splits into a per-tile uniform part and the
  // per-lane part kept here.
  const uint32_t tok_elems = uint32_t(a.k_tok);
  uint32_t lane_off[L::NI];
#pragma unroll
  for (int n = 0; n < L::NI; ++n) {
    const uint32_t r = L::RPW * (L::NI * wv + n) + lane / L::CPR;
    const uint32_t chunk = (lane % L::CPR) ^ L::swz(r);
    lane_off[n] = (pow2 ? (r & (ps - 1u)) * tok_elems : 0u) + 8u * chunk;
  }
  // DMA of key tile kt into its ring stage.  Rows past the end read row 0 of
  // page 0 (inside the pool) and are zeroed before use.
  auto issue = [&](uint32_t kt) {
    unsigned char *stage = lds + (kt % kStages) * L::kStage;
    const uint32_t tok0 = kt * kTT;
    const uint32_t tile_off = pow2 ? (tok0 & (ps - 1u)) * tok_elems : 0u;
#pragma unroll
    for (int n = 0; n < L::NI; ++n) {
      const uint32_t r0 = L::RPW * (L::NI * wv + n);
      const uint32_t r = r0 + lane / L::CPR;
      const uint32_t tok = tok0 + r;
      const bool ok = tok < k_end;
      uint32_t off;
      if (pow2) {
        const uint32_t lp = ok ? tok >> ps_shift : 0u;  // entry 0 exists whenever a tile does
        const uint32_t pbase = lp < uint32_t(kTableCache)
                                   ? tcache[lp]
                                   : (table[lp] < pv.N ? table[lp] : 0u) * page_elems;
        off = ok ? pbase + tile_off + lane_off[n] : lane_off[n] - (r & (ps - 1u)) * tok_elems;
      } else {
        const uint32_t lp = ok ? tok / ps : 0u;
        const uint32_t slot = ok ? tok - lp * ps : 0u;
        const uint32_t pbase = !ok ? 0u
                               : lp < uint32_t(kTableCache)
                                   ? tcache[lp]
                                   : (table[lp] < pv.N ? table[lp] : 0u) * page_elems;
        off = pbase + slot * tok_elems + lane_off[n];
      }
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage + r0 * L::kRowB));
      dma16(kbase + off, dst);
      dma16(vbase + off, dst + uint32_t(L::kTile));
    }
  };

  // Transposed value reads: lane (j, c16) supplies key row pv_row(j,
  // c16 >> 2) (+16 for the second read), value dims 16b + 4 (c16 & 3) .. +3.
  // pv_row(j, e) = 4 (j & 1) + (j >> 1) + 2 (e & 1) + 8 (e >> 1) puts rows
  // 0,2,..,14 on lanes 0..31 and the odd rows on lanes 32..63, so the eight
  // rows one LDS cycle serves land in distinct 32-byte slot pairs.
  uint32_t pv_off[DB];
  {
    const uint32_t e4 = c16 >> 2, q4 = c16 & 3u;
    const uint32_t pr = 4u * (j & 1u) + (j >> 1) + 2u * (e4 & 1u) + 8u * (e4 >> 1);
#pragma unroll
    for (int b = 0; b < DB; ++b)
      pv_off[b] = pr * L::kRowB + 8u * (q4 & 1u) + 16u * ((2u * b + (q4 >> 1)) ^ L::swz(pr));
  }

  const uint32_t n_tiles = (k_end + kTT - 1) / kTT;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qb[nt][ks]);
  for (uint32_t kt = 0; kt < n_tiles && kt < uint32_t(kStages - 1); ++kt) issue(kt);

  // Tile kt's ring stage is complete and visible to every wave once each
  // thread has seen its own loads of kt land and the block has passed a
  // barrier (which also means every wave finished reading the stage the next
  // refill overwrites).  `later` = tiles issued after kt that may still be
  // in flight.
  auto ready = [&](uint32_t kt, uint32_t later) {
    if (later >= 2) wait_vm<2 * kLoadsPerTile>();
    else if (later == 1) wait_vm<kLoadsPerTile>();
    else wait_vm<0>();
    const uint32_t t0 = kt * kTT;
    if (t0 + kTT > k_end) {
      // last tile: rows past the end hold whatever row 0 of page 0 holds;
      // zero their V (a NaN there must not reach the product)
      unsigned char *vt_lds = lds + (kt % kStages) * L::kStage + L::kTile;
      block_sync_lds();
      for (uint32_t e = tid; e < uint32_t(kTT * L::CPR); e += 256) {
        const uint32_t r = e / L::CPR;
        if (t0 + r >= k_end)
          *reinterpret_cast<uint4 *>(vt_lds + r * L::kRowB + 16u * (e % L::CPR)) = make_uint4(0, 0, 0, 0);
      }
    }
    block_sync_lds();
  };
  // S^T of key tile kt for both 16-row halves and both N-tiles: eight
  // independent MFMA chains (even and odd k-steps apart), sixteen per SIMD
  // with two waves, which keeps the 16x16x32 pipe full
  auto scores = [&](uint32_t kt, f32x4_t (&sc)[2][2]) {
    const unsigned char *kt_lds = lds + (kt % kStages) * L::kStage;
    uint4 ka[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint32_t r = 16u * mb + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[mb][ks] = *reinterpret_cast<const uint4 *>(kt_lds + r * L::kRowB +
                                                      16u * ((4u * ks + j) ^ L::swz(r)));
    }
    f32x4_t acc[2][2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[mb][nt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mb][nt][ks & 1] = M::qk(ka[mb][ks], qb[nt][ks], acc[mb][nt][ks & 1]);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sc[mb][nt] = acc[mb][nt][0] + acc[mb][nt][1];
  };

  // Software pipeline: the scores of tile kt+1 are issued before the
  // softmax and value product of tile kt, so the matrix core works on the
  // next tile while the VALU computes this tile's exponentials.
  f32x4_t s[2][2];
  if (n_tiles) {
    ready(0, n_tiles - 1 < 2u ? n_tiles - 1 : 2u);
    scores(0, s);
  }
  for (uint32_t kt = 0; kt < n_tiles; ++kt) {
    const uint32_t t0 = kt * kTT;
    unsigned char *vt_lds = lds + (kt % kStages) * L::kStage + L::kTile;
    // issued so far: tiles 0 .. kt+2
    if (kt + 1 < n_tiles) ready(kt + 1, kt + 2 < n_tiles ? 1u : 0u);

    // scores of tile kt, masked where a key is not visible
    float x[2][2][4];  // [N-tile][half][row]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[nt][mb][e] = s[mb][nt][e];
    const bool full = a.causal ? (t0 + kTT - 1 <= pos_min && t0 + kTT <= k_end)
                               : (t0 + kTT <= k_end);
    if (!full) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // key row 16mb + 4j + e of the tile is visible iff its index is at
        // most lim[nt] - t0 - 4j (one signed compare per score)
        const int d = int(lim[nt]) - int(t0) - int(4u * j);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[nt][mb][e] = 16 * mb + e <= d ? x[nt][mb][e] : -INFINITY;
      }
    }

    // One straight-line block: the MFMAs of tile kt+1's scores interleaved
    // with tile kt's softmax arithmetic.  After the last tile the scores
    // read a ring stage whose contents are not used (in bounds).
    f32x4_t s_next[2][2];
    scores(kt + 1, s_next);
    // online softmax (base 2): each probability is exp2(score * scale_log2
    // - m) with one FMA, against the row's current reference m
    uint4 pb[2];
    auto probs = [&](int nt) {
      float p[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[mb][e] = fast_exp2(__builtin_fmaf(x[nt][mb][e], sl2, -m[nt]));
      // P^T operand in the value reads' row order (see pv_off): pack even
      // and odd rows of each half, then one swap of lanes 32..63 of the even
      // pairs with lanes 0..31 of the odd pairs
      const auto lo = __builtin_amdgcn_permlane32_swap(M::pack2(p[0][0], p[0][2]),
                                                       M::pack2(p[0][1], p[0][3]), false, false);
      const auto hi = __builtin_amdgcn_permlane32_swap(M::pack2(p[1][0], p[1][2]),
                                                       M::pack2(p[1][1], p[1][3]), false, false);
      pb[nt] = make_uint4(lo[0], lo[1], hi[0], hi[1]);
    };
    // this lane's largest raw score of each N-tile (8 of the row's 32 keys)
    float lmax[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      lmax[nt] = vmax3(vmax3(x[nt][0][0], x[nt][0][1], x[nt][0][2]),
                       vmax3(x[nt][0][3], x[nt][1][0], x[nt][1][1]),
                       vmax(x[nt][1][2], x[nt][1][3]));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) probs(nt);
    // schedule of the block: the key-tile reads first, then one MFMA per
    // five VALU instructions
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
#pragma unroll
    for (int i = 0; i < 4 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    // Lazy rescaling: the reference only moves when a row's max exceeds it
    // by more than kSlack (base 2), so probabilities stay below 2^kSlack and
    // most tiles take none of this.  The result is the same softmax:
    // numerator and denominator share the reference.  A lane above its
    // threshold means its row's max is too, so the row maxima are formed
    // only here.
    if (__any(lmax[0] > thr[0] || lmax[1] > thr[1])) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mt = rows4_vmax(lmax[nt]) * sl2;
        const float m_new = mt > m[nt] + kSlack ? mt : m[nt];
        const float alpha = fast_exp2(m[nt] - m_new);
        m[nt] = m_new;
        thr[nt] = (m_new + kSlack) * inv_sl2;
#pragma unroll
        for (int b = 0; b < DB; ++b) o[nt][b] *= alpha;
        lacc[nt] *= alpha;
        probs(nt);
      }
    }

    // The value product runs at a raised wave priority: the other wave of
    // the SIMD (from another block) issues in its gaps, not the reverse.
    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T . P^T over the 32 keys: K slots 8j .. 8j+3 are key rows
    // pv_row(j, 0..3), slots 8j+4 .. 8j+7 the same rows + 16.  The reads of
    // block b + kPvAhead are issued before the MFMAs of block b and the
    // order is fenced, so the transposed-read latency hides behind the
    // MFMAs in flight.
    {
      constexpr int kPvAhead = 3;
      auto load_v = [&](int b) -> uint4 {
        const unsigned char *p0 = vt_lds + pv_off[b];
        const uint2 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * L::kRowB);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 va[kPvAhead + 1];
#pragma unroll
      for (int b = 0; b < kPvAhead && b < DB; ++b) va[b] = load_v(b);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        if (b + kPvAhead < DB) va[(b + kPvAhead) % (kPvAhead + 1)] = load_v(b + kPvAhead);
        o[0][b] = M::qk(va[b % (kPvAhead + 1)], pb[0], o[0][b]);
        o[1][b] = M::qk(va[b % (kPvAhead + 1)], pb[1], o[1][b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lacc[0] = M::qk(ones, pb[0], lacc[0]);
    lacc[1] = M::qk(ones, pb[1], lacc[1]);
    __builtin_amdgcn_s_setprio(0);
    // refill the stage of tile kt-1 (every wave passed this iteration's
    // barrier, so none still reads it)
    if (kt + kStages - 1 < n_tiles) issue(kt + kStages - 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) s[mb][nt] = s_next[mb][nt];
  }

  // normalise and write: lane holds O^T[d = 16b + 4j + e][q-row c16]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l_tot = lacc[nt][0];  // every row of the ones block holds the sum
    if (!row_ok[nt]) continue;
    const uint32_t r = 32u * wv + 16u * nt + c16;
    const uint32_t qq = r / grp, h = r % grp;
    T *out = static_cast<T *>(a.out) + (uint64_t(first + q_lo + qq) * a.hq + kvh * grp + h) * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      uint2 w;
      w.x = M::pack2(o[nt][b][0] * inv, o[nt][b][1] * inv);
      w.y = M::pack2(o[nt][b][2] * inv, o[nt][b][3] * inv);
      *reinterpret_cast<uint2 *>(out + 16 * b + 4 * j) = w;
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool tiles_supported(const TileArgs &a, pkv_dtype dt) {
  if (dt != PKV_F16 && dt != PKV_BF16) return false;
  if (a.d != a.dv || (a.d != 64 && a.d != 128)) return false;
  if (a.hq / a.hkv > uint32_t(kRowsPerBlock)) return false;
  return aligned16(a.q) && aligned16(a.k) && aligned16(a.v) && aligned16(a.out);
}

hipError_t launch_tiles(const TileArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t qb_n = kRowsPerBlock / grp;
  const uint32_t n_sub = (PKV_TILE_MAX + qb_n - 1) / qb_n;
  const uint64_t n_groups = uint64_t(a.n_tiles) * a.hkv;
  if (n_groups == 0) return hipSuccess;
  // eight XCD lanes of ceil(groups / 8) groups, n_sub blocks each
  const uint64_t blocks = (n_groups + 7) / 8 * 8 * n_sub;
  if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>(blocks));
  const uint32_t ng = uint32_t(n_groups);
  if (dt == PKV_BF16) {
    if (a.d == 64) launch_k((prefill_kernel<BF16, 64>), grid, dim3(256), 0, st, a, n_sub, ng);
    else launch_k((prefill_kernel<BF16, 128>), grid, dim3(256), 0, st, a, n_sub, ng);
  } else {
    if (a.d == 64) launch_k((prefill_kernel<F16, 64>), grid, dim3(256), 0, st, a, n_sub, ng);
    else launch_k((prefill_kernel<F16, 128>), grid, dim3(256), 0, st, a, n_sub, ng);
  }
  return hipGetLastError();
}

}  // namespace pkv
