// Decode kernel on MFMA for F16/BF16, head_dim == value_dim in {64, 128, 256}.
//
// Computes the attention of the ruDNN 0.1.7 `paged_attention` page
// (`DevicePlan::attention` doc) for queries attended one at a time.  For one
// query and one KV head, the G q heads of its group (no per-head KV repeat,
// module doc) form a dense contraction: S^T[tokens x heads] = K . Q^T over
// the head dimension, then O^T[d x heads] += V^T . P^T over the tokens.  Both
// run on 16x16 MFMA tiles with the tokens on the M side, so the softmax
// probabilities come out of the first product already in the B-operand
// layout of the second.  K and V rows are read whole from HBM (16 bytes per
// lane, streaming hint, one instruction per few rows), written to a per-wave
// LDS tile, and read back in the MFMA layouts: K rows as the A operand, V^T
// with transposed LDS reads.
//
// A block of four waves owns one (query, KV head, group of up to 16 q heads,
// split part); its waves take 16-token tiles of the part in turn, each with
// its own online softmax (base 2), merged through LDS at the end.  Max and
// sum reductions across lanes use shuffles; no cross-wave traffic happens
// inside the token loop.
//
// MFMA lane layouts used (16x16 tiles, lane l, j = l / 16):
//   A [16 x K]: lane l holds row l % 16, K-slots (j, 0..e-1)
//   B [K x 16]: lane l holds column l % 16, K-slots (j, 0..e-1)
//   C [16 x 16] f32: lane l holds rows 4j + 0..3 of column l % 16
// Only the C layout fixes meaning; the K-slot order just has to agree
// between A and B, and it does because both are filled with one mapping.

#include "balanced.h"
#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16;   // tokens per wave iteration
constexpr int kHeads = 16;  // q heads per block (MFMA N)

template <int D>
struct Lds {
  static constexpr int kRow = D * 2 + 16;  // bytes per staged row (padding spreads banks)
  static constexpr int kTileBytes = 2 * kTile * kRow;  // K tile, then V tile
  static constexpr int kOStride = D + 4;   // floats per head row in the merge area
  static constexpr int kVBytes = kWaves * kTileBytes;
  static constexpr int kOBytes = kWaves * kHeads * kOStride * 4;
  static constexpr int kBytes = kVBytes > kOBytes ? kVBytes : kOBytes;
};

// K/V rows of one 16-token tile as loaded from the cache: each load
// instruction covers RPI whole rows (CPR 16-byte chunks each, lane l taking
// row RPI*n + l/CPR, chunk l%CPR), read with the streaming hint.  Whole-row
// instructions keep HBM busy; the MFMA layouts are produced from LDS.  F8:
// the cache holds one FP8 E4M3 byte per element (half the chunks per row,
// twice the rows per instruction); rows are widened to the query type when
// staged.
template <int D, bool F8>
struct TileRegs {
  static constexpr int EB = F8 ? 1 : 2;     // bytes per cache element
  static constexpr int CPR = D * EB / 16;   // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per load instruction
  static constexpr int NL = 16 / RPI;       // loads per lane per tensor
  uint4 k[NL], v[NL];
  uint32_t valid16;  // bit r: token r of the tile exists
};

// Two FP8 E4M3 codes (bytes 0, 1 or 2, 3 of x) widened exactly to the query
// type (every E4M3 value is a bf16 and an f16 value); the hardware scale
// operand is 1.
template <class DT>
__device__ __forceinline__ uint32_t widen_f8(uint32_t x, bool hi);
template <>
__device__ __forceinline__ uint32_t widen_f8<BF16>(uint32_t x, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen_f8<F16>(uint32_t x, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
}

// Where the tokens of the wave's tiles live.  With PAGE_UNIFORM (page size a
// power of two >= 16) every tile lies inside one page; the page numbers of
// up to 64 consecutive tiles of the wave are held one per lane and read with
// readlane, so the token loop issues no table loads.
// The wave's k-th tile starts at token t_lo + 16 (first + step k): step 4
// when the four waves of a block interleave over one range, 1 when a wave
// owns a contiguous range.
template <bool PAGE_UNIFORM>
struct TileMap {
  const uint32_t *table;
  uint32_t t_lo, t_hi, first, step, ps, ps_shift, n_pages_pool;
  uint32_t lo;         // first visible key (sliding window); rows before it are masked
  uint32_t lane_page;  // page of tile (base + lane)
  uint32_t base;       // first tile held in lane_page

  __device__ __forceinline__ uint32_t tile_start(uint32_t k) const {
    return t_lo + (first + step * k) * 16u;
  }
  __device__ __forceinline__ void fill(uint32_t k0, uint32_t lane) {
    base = k0;
    const uint32_t t0 = tile_start(k0 + lane);
    lane_page = (PAGE_UNIFORM && t0 < t_hi) ? table[t0 >> ps_shift] : 0u;
  }
};

template <class DT, int D, bool PU, bool F8>
__device__ __forceinline__ void load_tile(TileRegs<D, F8> &t, const RowArgs &a, TileMap<PU> &map,
                                          const unsigned char *kbase,
                                          const unsigned char *vbase, uint32_t k,
                                          uint32_t lane) {
  using TR = TileRegs<D, F8>;
  const uint32_t t0 = map.tile_start(k);
  const uint32_t chunk = lane % TR::CPR;
  // A row past the end reads row 0 of page 0 (inside the pool whenever any
  // token exists).  Its K feeds only scores masked to -inf and its V is
  // replaced by zeros when staged (a select, so NaN never leaks).  The loads
  // are unconditional, which keeps them in flight across the attention of
  // the previous tile.  Element offsets are 64-bit: a cache tensor may hold
  // more than 2^32 elements.
  if constexpr (PU) {
    const uint32_t page = __builtin_amdgcn_readlane(map.lane_page, k - map.base);
    const uint32_t rows = map.t_hi - t0 < 16u ? map.t_hi - t0 : 16u;
    const bool page_ok = page < map.n_pages_pool;  // never read outside the pool
    const uint32_t before = map.lo > t0 ? map.lo - t0 : 0u;  // rows before the window
    t.valid16 = page_ok && before < 16u ? ((1u << rows) - 1u) & ~((1u << before) - 1u) : 0u;
    const uint32_t slot0 = t0 & (map.ps - 1);
    // the page's first element (uniform: scalar arithmetic)
    const uint64_t kpb = uint64_t(page) * a.k_page, vpb = uint64_t(page) * a.v_page;
#pragma unroll
    for (int n = 0; n < TR::NL; ++n) {
      const uint32_t r = TR::RPI * n + lane / TR::CPR;
      const bool ok = page_ok && r < rows;
      const uint64_t ko = ok ? kpb + uint64_t(slot0 + r) * a.k_tok : 0u;
      const uint64_t vo = ok ? vpb + uint64_t(slot0 + r) * a.v_tok : 0u;
      t.k[n] = load_stream16(kbase + ko * TR::EB + 16u * chunk);
      t.v[n] = load_stream16(vbase + vo * TR::EB + 16u * chunk);
    }
  } else {
    uint32_t valid = 0;
#pragma unroll
    for (int n = 0; n < TR::NL; ++n) {
      const uint32_t r = TR::RPI * n + lane / TR::CPR;
      const uint32_t tok = t0 + r;
      bool ok = tok >= map.lo && tok < map.t_hi;
      const uint32_t lp = map.ps_shift != 32u ? tok >> map.ps_shift : tok / map.ps;
      const uint32_t slot = tok - lp * map.ps;
      const uint32_t page = ok ? map.table[lp] : 0u;
      ok = ok && page < map.n_pages_pool;  // never read outside the pool
      valid |= ok ? 1u << r : 0u;
      const uint64_t ko = ok ? uint64_t(page) * a.k_page + uint64_t(slot) * a.k_tok : 0u;
      const uint64_t vo = ok ? uint64_t(page) * a.v_page + uint64_t(slot) * a.v_tok : 0u;
      t.k[n] = load_stream16(kbase + ko * TR::EB + 16u * chunk);
      t.v[n] = load_stream16(vbase + vo * TR::EB + 16u * chunk);
    }
    // every lane knows the rows it loaded; OR them across the wave
    uint32_t all = valid;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) all |= __shfl_xor(all, o, 64);
    t.valid16 = all & 0xffffu;
  }
}

constexpr float kSlack = 8.0f;  // lazy-rescale threshold (log2 units)

// Online-softmax state of one wave: the reference m (base 2, uniform across
// the four lane groups of a head; within kSlack below the running max or
// above it), this lane's partial sum and O^T tiles, both relative to m.
template <int D>
struct WaveState {
  f32x4_t o[D / 16];
  float m, lsum;
};

template <class DT, int D, bool F8>
__device__ __forceinline__ void attend_tile(WaveState<D> &st, const TileRegs<D, F8> &t,
                                            const uint4 *qb, unsigned char *vt, float sl2,
                                            uint32_t lane) {
  using M = Mfma<DT>;
  using L = Lds<D>;
  constexpr int KS = D / 32, DB = D / 16;
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  // stage the K and V rows in the query type (the cache rows' byte layout;
  // FP8 rows widened, each 16-byte chunk of codes to two chunks); rows past
  // the end get zero V
  using TR = TileRegs<D, F8>;
  unsigned char *kt = vt;
  unsigned char *vtile = vt + kTile * L::kRow;
#pragma unroll
  for (int n = 0; n < TR::NL; ++n) {
    const uint32_t r = TR::RPI * n + lane / TR::CPR;
    const bool keep = (t.valid16 >> r) & 1u;
    if constexpr (F8) {
      const uint32_t off = r * L::kRow + 32u * (lane % TR::CPR);
      const uint4 kw = t.k[n], vw = t.v[n];
      *reinterpret_cast<uint4 *>(kt + off) =
          make_uint4(widen_f8<DT>(kw.x, false), widen_f8<DT>(kw.x, true),
                     widen_f8<DT>(kw.y, false), widen_f8<DT>(kw.y, true));
      *reinterpret_cast<uint4 *>(kt + off + 16) =
          make_uint4(widen_f8<DT>(kw.z, false), widen_f8<DT>(kw.z, true),
                     widen_f8<DT>(kw.w, false), widen_f8<DT>(kw.w, true));
      const uint4 v0 = make_uint4(widen_f8<DT>(vw.x, false), widen_f8<DT>(vw.x, true),
                                  widen_f8<DT>(vw.y, false), widen_f8<DT>(vw.y, true));
      const uint4 v1 = make_uint4(widen_f8<DT>(vw.z, false), widen_f8<DT>(vw.z, true),
                                  widen_f8<DT>(vw.w, false), widen_f8<DT>(vw.w, true));
      *reinterpret_cast<uint4 *>(vtile + off) = keep ? v0 : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(vtile + off + 16) = keep ? v1 : make_uint4(0, 0, 0, 0);
    } else {
      const uint32_t off = r * L::kRow + 16u * (lane % TR::CPR);
      *reinterpret_cast<uint4 *>(kt + off) = t.k[n];
      *reinterpret_cast<uint4 *>(vtile + off) = keep ? t.v[n] : make_uint4(0, 0, 0, 0);
    }
  }

  // S^T = K . Q^T : A = K[token c16][chunk 4ks + j]; rows = tokens 4j+0..3,
  // column = head c16
  f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 ka = *reinterpret_cast<const uint4 *>(kt + c16 * L::kRow + 16 * (4 * ks + j));
    s = M::qk(ka, qb[ks], s);
  }

  // Online softmax against the head's reference st.m (base 2).  Lazy
  // rescaling: the reference only moves when the head's max exceeds it by
  // more than kSlack, so probabilities stay below 2^kSlack and most tiles
  // skip the cross-lane max and the rescale.  A lane above st.m + kSlack
  // means its head's max is too.  o, lsum and st.m share the reference, so
  // the partial results (and lse = st.m + log2 lsum) are the same softmax.
  float x[4];
  float lmx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool v = (t.valid16 >> (4 * j + e)) & 1u;
    x[e] = v ? s[e] * sl2 : -INFINITY;
    lmx = fmaxf(lmx, x[e]);
  }
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = fast_exp2(x[e] - st.m);
  if (__any(lmx > st.m + kSlack)) {
    const float mt = rows4_max(lmx);
    const float m_new = mt > st.m + kSlack ? mt : st.m;
    const float alpha = fast_exp2(st.m - m_new);
    st.m = m_new;
    st.lsum *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b) st.o[b] *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(x[e] - m_new);
  }
  st.lsum += (p[0] + p[1]) + (p[2] + p[3]);
  uint2 pb;
  pb.x = M::pack2(p[0], p[1]);
  pb.y = M::pack2(p[2], p[3]);

  // O^T += V^T . P^T : A = V^T[d = 16b + c16][tokens 4j+0..3], one
  // transposed LDS read per block of 16 value dims
  const unsigned char *vrow = vtile + (4 * j + (c16 >> 2)) * L::kRow + 8 * (c16 & 3);
#pragma unroll
  for (int b = 0; b < DB; ++b) st.o[b] = M::pv(lds_read_tr16(vrow + 32 * b), pb, st.o[b]);
}

// Q^T of heads h0 .. h0 + nh - 1 of query i as the B operand of q.k:
// column = head c16, K-slot chunk 4 ks + j; absent heads are zero.
template <class DT, int D>
__device__ __forceinline__ void load_q(uint4 (&qb)[D / 32], const RowArgs &a, uint32_t i,
                                       uint32_t h0, uint32_t nh, uint32_t lane) {
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  const typename DT::T *qrow =
      static_cast<const typename DT::T *>(a.q) + (uint64_t(i) * a.hq + h0 + c16) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qb[ks] = c16 < nh ? *reinterpret_cast<const uint4 *>(qrow + 8 * (4 * ks + j))
                      : make_uint4(0, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void reset_state(WaveState<D> &st) {
#pragma unroll
  for (int b = 0; b < D / 16; ++b) st.o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = kNoMax;
  st.lsum = 0.f;
}

// Attends the wave's n_tiles tiles of `map` with a software pipeline, two
// tiles in flight: while one tile is attended the next one's loads run.  The
// steady-state loop issues its loads unconditionally, so the wait before
// each tile covers only that tile's loads; page numbers are refilled once
// per 64 tiles, outside the loop.
template <class DT, int D, bool PU, bool F8>
__device__ __forceinline__ void stream_tiles(WaveState<D> &st, TileMap<PU> &map,
                                             uint32_t n_tiles, const RowArgs &a,
                                             const unsigned char *kbase,
                                             const unsigned char *vbase, const uint4 *qb,
                                             unsigned char *vt, float sl2, uint32_t lane) {
  TileRegs<D, F8> ta, tb;
  for (uint32_t c0 = 0; c0 < n_tiles; c0 += 64) {
    const uint32_t cn = n_tiles - c0 < 64u ? n_tiles - c0 : 64u;
    map.fill(c0, lane);
    uint32_t k = 0;
    if (cn >= 4) {
      load_tile<DT, D, PU, F8>(ta, a, map, kbase, vbase, c0, lane);
      load_tile<DT, D, PU, F8>(tb, a, map, kbase, vbase, c0 + 1, lane);
      for (; k + 3 < cn; k += 2) {
        attend_tile<DT, D, F8>(st, ta, qb, vt, sl2, lane);
        load_tile<DT, D, PU, F8>(ta, a, map, kbase, vbase, c0 + k + 2, lane);
        attend_tile<DT, D, F8>(st, tb, qb, vt, sl2, lane);
        load_tile<DT, D, PU, F8>(tb, a, map, kbase, vbase, c0 + k + 3, lane);
      }
    } else {
      load_tile<DT, D, PU, F8>(ta, a, map, kbase, vbase, c0, lane);
      if (cn > 1) load_tile<DT, D, PU, F8>(tb, a, map, kbase, vbase, c0 + 1, lane);
    }
    // at most three tiles left: k in ta, k + 1 in tb
    if (k < cn) {
      attend_tile<DT, D, F8>(st, ta, qb, vt, sl2, lane);
      if (k + 2 < cn) load_tile<DT, D, PU, F8>(ta, a, map, kbase, vbase, c0 + k + 2, lane);
    }
    if (k + 1 < cn) attend_tile<DT, D, F8>(st, tb, qb, vt, sl2, lane);
    if (k + 2 < cn) attend_tile<DT, D, F8>(st, ta, qb, vt, sl2, lane);
  }
}

template <bool PU>
__device__ __forceinline__ void init_map(TileMap<PU> &map, const RowArgs &a, uint32_t seq,
                                         uint32_t t_lo, uint32_t t_hi, uint32_t first,
                                         uint32_t step) {
  const uint32_t ps = a.plan.ps;
  map.table = a.plan.words + a.plan.table + uint64_t(seq) * a.plan.W;
  map.t_lo = t_lo;
  map.t_hi = t_hi;
  map.first = first;
  map.step = step;
  map.ps = ps;
  const bool pow2 = (ps & (ps - 1)) == 0;
  map.ps_shift = pow2 ? uint32_t(__builtin_ctz(ps)) : 32u;
  map.n_pages_pool = a.plan.N;
  map.lo = 0;
}

template <class DT, int D, bool PU, bool F8>
__global__ __launch_bounds__(256) void decode_mfma_kernel(RowArgs a) {
  using M = Mfma<DT>;
  constexpr int KS = D / 32;  // 32-wide K steps of q.k (also 16-byte chunks per lane per row)
  constexpr int DB = D / 16;  // 16-wide value blocks
  using L = Lds<D>;
  __shared__ __align__(16) unsigned char lds[L::kBytes];
  __shared__ float s_m[kWaves][kHeads], s_l[kWaves][kHeads];

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t hgk = (grp + kHeads - 1) / kHeads;
  // Part-major block order: the first parts of every query (full length)
  // are dispatched before the later, partly filled ones.
  const uint32_t per_part = a.n_queries * a.hkv * hgk;
  const uint32_t part = blockIdx.x / per_part;
  const uint32_t rest = blockIdx.x % per_part;
  const uint32_t hsel = rest % (a.hkv * hgk);
  const uint32_t qi = rest / (a.hkv * hgk);
  const uint32_t kvh = hsel / hgk, sub = hsel % hgk;
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  uint32_t seq;
  const uint32_t n = visible_keys(a.plan, i, a.causal, &seq);
  const uint32_t lo = window_lo(n, a.window);
  const uint32_t ps = a.plan.ps;
  const uint64_t span = uint64_t(a.pages_per_split) * ps;
  const uint64_t lo64 = uint64_t(part) * span;
  // empty part (past the keys, or wholly before the window): the merge skips it
  if (a.splits > 1 && (lo64 >= n || lo64 + span <= lo)) return;
  // tiles stay on the 16-key grid (one page each when PU); rows before the
  // window are masked
  const uint32_t lo_grid = PU ? lo & ~15u : lo;
  uint32_t t_lo = uint32_t(lo64 < n ? lo64 : n);
  if (t_lo < lo_grid) t_lo = lo_grid;
  const uint32_t t_hi = uint32_t(lo64 + span < n ? lo64 + span : n);
  const uint32_t h0 = kvh * grp + sub * kHeads;               // first q head of the block
  const uint32_t nh = grp - sub * kHeads < kHeads ? grp - sub * kHeads : kHeads;

  uint4 qb[KS];
  load_q<DT, D>(qb, a, i, h0, nh, lane);
  WaveState<D> st;
  reset_state<D>(st);

  constexpr uint32_t EB = F8 ? 1u : 2u;  // bytes per cache element
  const unsigned char *kbase = static_cast<const unsigned char *>(a.k) + uint64_t(kvh) * D * EB;
  const unsigned char *vbase = static_cast<const unsigned char *>(a.v) + uint64_t(kvh) * D * EB;
  unsigned char *vt = lds + wv * L::kTileBytes;  // this wave's V tile
  TileMap<PU> map;
  init_map<PU>(map, a, seq, t_lo, t_hi, wv, 4u);
  map.lo = lo;
  const uint32_t first = t_lo + wv * 16u;
  const uint32_t n_tiles = first < t_hi ? (t_hi - first + 63u) / 64u : 0u;
  stream_tiles<DT, D, PU, F8>(st, map, n_tiles, a, kbase, vbase, qb, vt, a.scale_log2, lane);

  // per-head sum over the four lane groups (m is already uniform across them)
  const float lsum = rows4_sum(st.lsum);
  __syncthreads();  // every wave is done with its V tile: reuse LDS for the merge
  float *so = reinterpret_cast<float *>(lds);
  {
    float *mine = so + wv * kHeads * L::kOStride + c16 * L::kOStride;
#pragma unroll
    for (int b = 0; b < DB; ++b)
      *reinterpret_cast<f32x4_t *>(mine + 16 * b + 4 * j) = st.o[b];
    if (j == 0) {
      s_m[wv][c16] = st.m;
      s_l[wv][c16] = lsum;
    }
  }
  __syncthreads();

  for (uint32_t idx = tid; idx < nh * uint32_t(D); idx += 256) {
    const uint32_t h = idx / D, d = idx % D;
    float mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(s_m[w][h] - mx);
      num = fmaf(so[(w * kHeads + h) * L::kOStride + d], sc, num);
      den = fmaf(s_l[w][h], sc, den);
    }
    const float inv = den > 0.f ? a.v_scale / den : 0.f;  // v_scale: FP8 value cache
    if (a.splits == 1) {
      auto *out = static_cast<uint16_t *>(a.out) + (uint64_t(i) * a.hq + h0 + h) * D;
      out[d] = M::from_f(num * inv);
    } else {
      const uint64_t r = (uint64_t(i) * a.splits + part) * a.hq + h0 + h;
      a.ws_o[r * D + d] = num * inv;
      if (d == 0) a.ws_lse[r] = mx + fast_log2(den);
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced schedule (balanced.h) with waves as units.  With the block-per-part
// grid above, the work of a CU is whatever lengths its resident blocks happen
// to draw, and the kernel lasts as long as the busiest CU.  Here the row
// queries' 16-key tiles are cut into equal ranges, one per group of segq =
// KV heads x 16-head groups consecutive waves; wave g of a group attends
// segment g over its group's range, so the segq waves that read the same
// cache pages (one KV head each) run side by side, which keeps DRAM rows open
// for all heads of a page.

// Launched with one block of four waves per CU (one wave per SIMD): fewer
// concurrent page streams keep more DRAM rows open, and more waves per CU
// or a third tile in flight per wave measured no faster.
template <class DT, int D, bool PU, bool F8>
__global__ __launch_bounds__(256) void decode_balanced_kernel(RowArgs a) {
  using M = Mfma<DT>;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  using L = Lds<D>;
  __shared__ __align__(16) unsigned char lds[kWaves * L::kTileBytes];

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t c16 = lane & 15u, j = lane >> 4;
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t hgk = (grp + kHeads - 1) / kHeads;
  const uint32_t segq = a.hkv * hgk;
  const uint32_t groups = a.bal_waves / segq;  // >= 1 (checked by the host)
  const uint32_t w = blockIdx.x * kWaves + wv;
  const uint32_t grp_k = w / segq, g = w % segq;
  if (grp_k >= groups) return;
  bal::Range rg;
  if (!bal::find_range<16>(rg, a, groups, grp_k, w == 0u, lane)) return;

  unsigned char *vt = lds + wv * L::kTileBytes;
  const uint32_t kvh = g / hgk, sub = g % hgk;
  const uint32_t h0 = kvh * grp + sub * kHeads;
  const uint32_t nh = grp - sub * kHeads < kHeads ? grp - sub * kHeads : kHeads;
  constexpr uint32_t EB = F8 ? 1u : 2u;  // bytes per cache element
  const unsigned char *kbase = static_cast<const unsigned char *>(a.k) + uint64_t(kvh) * D * EB;
  const unsigned char *vbase = static_cast<const unsigned char *>(a.v) + uint64_t(kvh) * D * EB;

  bal::Piece pc;
  while (bal::next_piece<16>(rg, a, lane, pc)) {
    const uint32_t tt0 = pc.tt0, tt1 = pc.tt1;
    const uint32_t i = pc.i, seq = pc.seq, n = pc.n;  // found with the range
    const uint32_t lo = window_lo(n, a.window);
    const uint32_t tb = lo / 16u;  // tile tt of the query is grid tile tb + tt
    const uint32_t t_hi = (tb + tt1) * 16u < n ? (tb + tt1) * 16u : n;

    uint4 qb[KS];
    load_q<DT, D>(qb, a, i, h0, nh, lane);
    WaveState<D> st;
    reset_state<D>(st);
    TileMap<PU> map;
    init_map<PU>(map, a, seq, (tb + tt0) * 16u, t_hi, 0u, 1u);
    map.lo = lo;
    stream_tiles<DT, D, PU, F8>(st, map, tt1 - tt0, a, kbase, vbase, qb, vt, a.scale_log2, lane);

    const float lsum = rows4_sum(st.lsum);
    const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;  // v_scale: FP8 value cache
    if (tt0 == 0u && tt1 == pc.ntq) {
      if (c16 < nh) {
        uint16_t *orow = static_cast<uint16_t *>(a.out) + (uint64_t(i) * a.hq + h0 + c16) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          uint2 v2;
          v2.x = M::pack2(st.o[b][0] * inv, st.o[b][1] * inv);
          v2.y = M::pack2(st.o[b][2] * inv, st.o[b][3] * inv);
          *reinterpret_cast<uint2 *>(orow + 16 * b + 4 * j) = v2;
        }
      }
    } else {
      const uint32_t slot = bal::piece_slot(pc, w);
      if (c16 < nh) {
        const uint64_t row = uint64_t(slot) * kHeads + c16;
        float *wo = a.ws_o + row * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) *reinterpret_cast<f32x4_t *>(wo + 16 * b + 4 * j) = st.o[b] * inv;
        if (j == 0) a.ws_lse[row] = st.m + fast_log2(lsum);
      }
    }
  }
}

// Merge of the cut pieces of one (query, head): out = sum_p 2^(lse_p - M)
// o_p / sum_p 2^(lse_p - M), M = max_p lse_p, over the slots of that head's
// units in the groups k0..k1 the query spans.  A unit owns UH heads of one
// KV head (16 for the decode waves, 64 for the MLA blocks); its slots hold
// UH rows.  Queries inside one range were written by the range kernel;
// queries with no tiles get zeros.  One wave per (query, head), four per
// block; lane l owns value elements 4l + 256e .. +3 (dv a multiple of 4, at
// most 1024).  Pieces are taken eight at a time with their lse and partial
// rows loaded together (one round of loads after the range record for up to
// eight pieces), combined online: the running sum is rescaled when a batch
// raises the max.
template <class DT, uint32_t UH>
__global__ __launch_bounds__(256) void merge_balanced_kernel(MergeArgs a) {
  using T = typename DT::T;
  constexpr uint32_t kBatch = 8;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t pair = uint64_t(blockIdx.x) * 4u + wv;
  if (pair >= uint64_t(a.n_queries) * a.hq) return;
  const uint32_t qi = uint32_t(pair / a.hq), h = uint32_t(pair % a.hq);
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t hgk = (grp + UH - 1) / UH;
  const uint32_t segq = a.hkv * hgk;
  const uint32_t g = (h / grp) * hgk + (h % grp) / UH, hl = (h % grp) % UH;
  const uint32_t c0 = a.bal_rec[2u * qi], ntq = a.bal_rec[2u * qi + 1u];
  const uint32_t total_tiles = a.bal_rec[2u * a.n_queries];
  const uint32_t i = a.qlist ? a.qlist[qi] : qi;
  T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * a.dv;
  if (ntq == 0u) {
    for (uint32_t d = lane; d < a.dv; d += 64) out[d] = DT::from_f(0.f);
    return;
  }
  const uint32_t groups = a.bal_waves / segq;
  const uint32_t tpg = total_tiles / groups + (total_tiles % groups != 0u);
  const uint32_t k0 = c0 / tpg, k1 = (c0 + ntq - 1u) / tpg;
  if (k0 == k1) return;  // whole query in one range: already written
  const uint32_t np = k1 - k0 + 1u;
  // piece p: unit u = (k0 + p) segq + g; slot 2u + 1 for p = 0, else 2u
  auto row_of = [&](uint32_t p) -> uint64_t {
    const uint32_t u = (k0 + p) * segq + g;
    const uint32_t slot = p == 0u ? 2u * u + 1u : 2u * u;
    return uint64_t(slot) * UH + hl;
  };
  const uint32_t ne = (a.dv + 255u) / 256u;  // float4 groups per lane
  f32x4_t acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mx = kNoMax, den = 0.f;
  for (uint32_t p0 = 0; p0 < np; p0 += kBatch) {
    const uint32_t pc = np - p0 < kBatch ? np - p0 : kBatch;
    float lse[kBatch];
    f32x4_t ov[kBatch][4];
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      lse[b] = kNoMax;
      if (b < pc) {
        const uint64_t r = row_of(p0 + b);
        lse[b] = a.ws_lse[r];
#pragma unroll
        for (uint32_t e = 0; e < 4; ++e) {
          const uint32_t d = 4u * lane + 256u * e;
          if (e < ne && d < a.dv) ov[b][e] = *reinterpret_cast<const f32x4_t *>(a.ws_o + r * a.dv + d);
        }
      }
    }
    float bm = mx;
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) bm = fmaxf(bm, lse[b]);
    const float sc = fast_exp2(mx - bm);
    den *= sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= sc;
#pragma unroll
    for (uint32_t b = 0; b < kBatch; ++b) {
      if (b < pc) {
        const float w = fast_exp2(lse[b] - bm);
        den += w;
#pragma unroll
        for (uint32_t e = 0; e < 4; ++e)
          if (e < ne && 4u * lane + 256u * e < a.dv) acc[e] += w * ov[b][e];
      }
    }
    mx = bm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (uint32_t e = 0; e < 4; ++e) {
    const uint32_t d = 4u * lane + 256u * e;
    if (e < ne && d < a.dv) {
#pragma unroll
      for (int c = 0; c < 4; ++c) out[d + c] = DT::from_f(acc[e][c] * inv);
    }
  }
}

template <class DT, bool PU, bool F8>
hipError_t launch_d(const RowArgs &a, dim3 grid, hipStream_t st) {
  switch (a.d) {
    case 64: launch_k((decode_mfma_kernel<DT, 64, PU, F8>), grid, dim3(256), 0, st, a); break;
    case 128: launch_k((decode_mfma_kernel<DT, 128, PU, F8>), grid, dim3(256), 0, st, a); break;
    case 256: launch_k((decode_mfma_kernel<DT, 256, PU, F8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <class DT, bool PU, bool F8>
hipError_t launch_bal_d(const RowArgs &a, dim3 grid, hipStream_t st) {
  switch (a.d) {
    case 64: launch_k((decode_balanced_kernel<DT, 64, PU, F8>), grid, dim3(256), 0, st, a); break;
    case 128: launch_k((decode_balanced_kernel<DT, 128, PU, F8>), grid, dim3(256), 0, st, a); break;
    case 256: launch_k((decode_balanced_kernel<DT, 256, PU, F8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <class DT, bool PU>
int bal_blocks_per_cu(uint32_t d) {
  int blocks = 0;
  hipError_t e = hipErrorNotSupported;
  if (d == 64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_balanced_kernel<DT, 64, PU, false>, 256, 0);
  if (d == 128) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_balanced_kernel<DT, 128, PU, false>, 256, 0);
  if (d == 256) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_balanced_kernel<DT, 256, PU, false>, 256, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool rows_mfma_supported(const RowArgs &a, pkv_dtype dt) {
  if (dt != PKV_F16 && dt != PKV_BF16) return false;
  if (a.pdim != 0 || a.d != a.dv || (a.d != 64 && a.d != 128 && a.d != 256)) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v)) return false;
  return true;
}

int rows_mfma_blocks_per_cu(const RowArgs &a, pkv_dtype dt) {
  const uint32_t ps = a.plan.ps;
  const bool pu = (ps & (ps - 1)) == 0 && ps >= 16u;
  int blocks = 0;
  hipError_t e = hipErrorNotSupported;
#define PKV_OCC(DT, D, PU)                                                                  \
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_mfma_kernel<DT, D, PU, false>, \
                                                   256, 0)
  if (dt == PKV_BF16) {
    if (a.d == 64) { if (pu) PKV_OCC(BF16, 64, true); else PKV_OCC(BF16, 64, false); }
    if (a.d == 128) { if (pu) PKV_OCC(BF16, 128, true); else PKV_OCC(BF16, 128, false); }
    if (a.d == 256) { if (pu) PKV_OCC(BF16, 256, true); else PKV_OCC(BF16, 256, false); }
  } else {
    if (a.d == 64) { if (pu) PKV_OCC(F16, 64, true); else PKV_OCC(F16, 64, false); }
    if (a.d == 128) { if (pu) PKV_OCC(F16, 128, true); else PKV_OCC(F16, 128, false); }
    if (a.d == 256) { if (pu) PKV_OCC(F16, 256, true); else PKV_OCC(F16, 256, false); }
  }
#undef PKV_OCC
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

uint64_t rows_mfma_blocks(const RowArgs &a) {
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t hgk = (grp + kHeads - 1) / kHeads;
  return uint64_t(a.n_queries) * a.hkv * hgk * a.splits;
}

hipError_t launch_rows_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint64_t blocks = rows_mfma_blocks(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));
  // page size a power of two >= 16: every 16-token tile lies in one page
  const uint32_t ps = a.plan.ps;
  const bool pu = (ps & (ps - 1)) == 0 && ps >= 16u;
  if (a.kv_fp8) {
    if (dt == PKV_BF16) return pu ? launch_d<BF16, true, true>(a, grid, st) : launch_d<BF16, false, true>(a, grid, st);
    return pu ? launch_d<F16, true, true>(a, grid, st) : launch_d<F16, false, true>(a, grid, st);
  }
  if (dt == PKV_BF16) return pu ? launch_d<BF16, true, false>(a, grid, st) : launch_d<BF16, false, false>(a, grid, st);
  return pu ? launch_d<F16, true, false>(a, grid, st) : launch_d<F16, false, false>(a, grid, st);
}

int balanced_waves_per_cu(uint32_t d, uint32_t ps, pkv_dtype dt) {
  const bool pu = (ps & (ps - 1)) == 0 && ps >= 16u;
  int b;
  if (dt == PKV_BF16) b = pu ? bal_blocks_per_cu<BF16, true>(d) : bal_blocks_per_cu<BF16, false>(d);
  else b = pu ? bal_blocks_per_cu<F16, true>(d) : bal_blocks_per_cu<F16, false>(d);
  return b * kWaves;
}

hipError_t launch_rows_balanced(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  if (a.bal_waves == 0 || a.bal_waves % kWaves != 0) return hipErrorInvalidValue;
  const dim3 grid(a.bal_waves / kWaves);
  const uint32_t ps = a.plan.ps;
  const bool pu = (ps & (ps - 1)) == 0 && ps >= 16u;
  if (a.kv_fp8) {
    if (dt == PKV_BF16) return pu ? launch_bal_d<BF16, true, true>(a, grid, st) : launch_bal_d<BF16, false, true>(a, grid, st);
    return pu ? launch_bal_d<F16, true, true>(a, grid, st) : launch_bal_d<F16, false, true>(a, grid, st);
  }
  if (dt == PKV_BF16) return pu ? launch_bal_d<BF16, true, false>(a, grid, st) : launch_bal_d<BF16, false, false>(a, grid, st);
  return pu ? launch_bal_d<F16, true, false>(a, grid, st) : launch_bal_d<F16, false, false>(a, grid, st);
}

hipError_t launch_merge_balanced(const MergeArgs &a, pkv_dtype dt, uint32_t unit_heads,
                                 hipStream_t st) {
  const uint64_t pairs = uint64_t(a.n_queries) * a.hq;  // one wave each, four per block
  if (pairs == 0) return hipSuccess;
  if (a.dv % 4 != 0 || a.dv > 1024) return hipErrorInvalidValue;
  const uint64_t blocks = (pairs + 3) / 4;
  if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (unit_heads != uint32_t(kHeads) && unit_heads != kMlaBlockHeads) return hipErrorInvalidValue;
  const bool mla = unit_heads == kMlaBlockHeads;
  switch (dt) {
    case PKV_F16:
      if (mla) launch_k((merge_balanced_kernel<F16, kMlaBlockHeads>), grid, dim3(256), 0, st, a);
      else launch_k((merge_balanced_kernel<F16, kHeads>), grid, dim3(256), 0, st, a);
      break;
    case PKV_BF16:
      if (mla) launch_k((merge_balanced_kernel<BF16, kMlaBlockHeads>), grid, dim3(256), 0, st, a);
      else launch_k((merge_balanced_kernel<BF16, kHeads>), grid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
