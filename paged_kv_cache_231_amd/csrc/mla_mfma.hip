// MLA decode kernel on MFMA: absorbed queries against one shared latent head
// plus a position part (ruDNN 0.1.7 `paged_attention` page, `DevicePlan::mla`
// doc), for latent rank 512 and position dim 64.
//
// For one query every q head attends the same cache rows, so scores and the
// output are dense contractions over the latent:
//   S^T[tokens x heads] = latent . q_abs^T + k_pos . q_pos^T   (576-deep)
//   O^T[rank x heads]  += latent^T . P^T                        (token-deep)
// A block owns one (query, split part) and up to 128 heads; each of its
// eight waves owns 16 heads (one MFMA N-tile) with its 512 x 16 output tile
// in registers, so every latent row read from HBM serves all heads.  Latent
// and k_pos rows travel HBM -> LDS directly into a four-stage ring (three
// 16-token tiles ahead), stored with XOR-swizzled 16-byte chunks; the
// latent is read from LDS as the A operand of q.k and, transposed, of the
// value product.  The online softmax is kept in base 2 with lazy
// rescaling.  Split parts write f32 partials that the merge kernel combines.

#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;          // one wave per SIMD
constexpr int kNT = 1;             // 16-head MFMA N-tiles per wave
constexpr int kHeadsPerBlock = kWaves * kNT * 16;
constexpr int kTT = 32;            // tokens per tile (two 16-row M-tiles)
constexpr int kStages = 4;         // LDS ring stages
constexpr int kTableCache = 1024;  // block-table entries cached in LDS
constexpr float kSlack = 8.0f;     // lazy-rescale threshold (log2 units)

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
  // chunk c of latent row r sits in slot c ^ (r & 15) (same 256-byte line);
  // chunk c of position row r in slot c ^ ((r >> 1) & 7)
  static __device__ __forceinline__ uint32_t lat_slot(uint32_t c, uint32_t r) { return c ^ (r & 15u); }
  static __device__ __forceinline__ uint32_t pos_slot(uint32_t c, uint32_t r) { return c ^ ((r >> 1) & 7u); }
};

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (inline assembly: the compiler's wait insertion would otherwise drain the
// ring before every LDS read; the ring's explicit waits order it).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(src)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char *)(p)));
}

__device__ __forceinline__ void settle(const uint4 &x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <class DT, int R, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_kernel(RowArgs a, uint32_t head_groups) {
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
  const uint32_t ps = a.plan.ps;
  const uint64_t span = uint64_t(a.pages_per_split) * ps;
  const uint64_t lo64 = uint64_t(part) * span;
  if (a.splits > 1 && lo64 >= n) return;  // empty part: the merge skips it
  const uint32_t t_lo = uint32_t(lo64 < n ? lo64 : n);
  const uint32_t t_hi = uint32_t(lo64 + span < n ? lo64 + span : n);
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

  // this wave's heads: N-tile nt, column c16 -> head h0 + 16 nt + c16
  const uint32_t h0 = hgi * kHeadsPerBlock + wv * (kNT * 16u);
  uint4 qa[kNT][KS], qp[kNT][KP];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    // columns of heads past hq compute on head 0's query and are not stored
    const uint32_t h = h0 + 16u * nt + c16;
    const uint64_t row = uint64_t(i) * a.hq + (h < a.hq ? h : 0u);
    const T *qrow = static_cast<const T *>(a.q) + row * R;
    const T *prow = static_cast<const T *>(a.qp) + row * P;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[nt][ks] = *reinterpret_cast<const uint4 *>(qrow + 8 * (4 * ks + j));
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) qp[nt][ks] = *reinterpret_cast<const uint4 *>(prow + 8 * (4 * ks + j));
  }
  f32x4_t o[kNT][DB];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int b = 0; b < DB; ++b) o[nt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[kNT], lsum[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    m[nt] = kNoMax;
    lsum[nt] = 0.f;
  }
  const float sl2 = a.scale_log2;
  const T *lat = static_cast<const T *>(a.k);
  const T *kpos = static_cast<const T *>(a.kp);
  __syncthreads();  // table cache ready

  // DMA of tile kt: wave wv loads latent rows 8wv .. 8wv+7 (one whole row
  // per instruction) and position rows 8wv .. 8wv+7 (one instruction, lane
  // l row 8wv + l/8).  Lane l locates row 8wv + l/8; the latent loads take
  // the page and slot of lanes 0, 8, .., 56.  Rows past the end read row 0
  // of page 0; their latent is zeroed before use.
  auto issue = [&](uint32_t kt) {
    unsigned char *stage = lds + (kt % kStages) * L::kStage;
    const uint32_t t0 = t_lo + kt * kTT;
    const uint32_t r = wv * uint32_t(L::kLatPerWave) + (lane >> 3);
    const uint32_t tok = t0 + r;
    const bool ok = tok < t_hi;
    const uint32_t lp = ok ? page_of(tok) : wb;
    const uint32_t slot = ok ? tok - lp * ps : 0u;
    const uint32_t page = ok ? tcache[lp - wb] : 0u;
#pragma unroll
    for (int n2 = 0; n2 < L::kLatPerWave; ++n2) {
      const uint32_t rr = wv * uint32_t(L::kLatPerWave) + n2;
      const uint32_t pg = __builtin_amdgcn_readlane(page, 8 * n2);
      const uint32_t sl = __builtin_amdgcn_readlane(slot, 8 * n2);
      const uint32_t base = pg * uint32_t(a.k_page) + sl * uint32_t(a.k_tok);
      const uint32_t chunk = L::lat_slot(lane, rr);  // slot `lane` holds this chunk
      dma16(lat + base + 8u * chunk, __builtin_amdgcn_readfirstlane(lds_addr(stage + rr * L::kLatRow)));
    }
    const uint32_t chunk = L::pos_slot(lane % L::kPosCPR, r);
    const uint32_t off = page * uint32_t(a.kp_page) + slot * uint32_t(a.kp_tok) + 8u * chunk;
    dma16(kpos + off, __builtin_amdgcn_readfirstlane(lds_addr(stage + L::kLat + 8u * wv * L::kPosRow)));
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

  // Per-lane LDS offsets.  The swizzle only permutes 16-byte chunks inside
  // a 256-byte segment of a row, so each read is a per-lane base (a few
  // registers) plus an immediate segment offset.
  //   q.k:  lane (j, c16) reads chunk 4ks + j of row c16: segment ks >> 2,
  //         in-segment chunk (4 (ks & 3) + j) ^ c16
  //   pos:  chunk 4ks + j of position row c16, slot chunk ^ ((c16 >> 1) & 7)
  //   V^T:  rows vr = 4j + (c16 >> 2) (+16), chunk 2b + ((c16 & 3) >> 1),
  //         8-byte half c16 & 1: segment b >> 3, in-segment chunk
  //         (2 (b & 7) + ((c16 & 3) >> 1)) ^ vr
  const uint32_t qk_row = c16 * L::kLatRow;
  uint32_t qk_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qk_off[u] = 16u * ((4u * u + j) ^ c16);
  const uint32_t pos_row = c16 * L::kPosRow;
  uint32_t pos_off[KP];
#pragma unroll
  for (int ks = 0; ks < KP; ++ks) pos_off[ks] = 16u * L::pos_slot(4u * ks + j, c16);
  const uint32_t vr = 4u * j + (c16 >> 2);
  const uint32_t pv_row = vr * L::kLatRow + 8u * (c16 & 1u);
  uint32_t pv_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) pv_off[u] = 16u * ((2u * u + ((c16 & 3u) >> 1)) ^ (vr & 15u));

  const uint32_t n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTT - 1) / kTT : 0u;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qa[nt][ks]);
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) settle(qp[nt][ks]);
  }
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
    // 16 mt + c16 (A rows), N-tile nt the heads.  Two accumulator chains
    // (even and odd k-steps) per output tile keep the MFMA pipe fed.
    f32x4_t s[2][kNT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4_t acc[2][kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[0][nt] = acc[1][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const unsigned char *lrow = st_lat + mt * (16 * L::kLatRow) + qk_row;
      const unsigned char *prow_l = st_pos + mt * (16 * L::kPosRow) + pos_row;
      // all A operands of this M-tile first (the reads overlap), then the MFMAs
      uint4 ka[KS + KP];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = *reinterpret_cast<const uint4 *>(lrow + qk_off[ks & 3] + 256 * (ks >> 2));
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) ka[KS + ks] = *reinterpret_cast<const uint4 *>(prow_l + pos_off[ks]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[ks & 1][nt] = M::qk(ka[ks], qa[nt][ks], acc[ks & 1][nt]);
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[ks & 1][nt] = M::qk(ka[KS + ks], qp[nt][ks], acc[ks & 1][nt]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) s[mt][nt] = acc[0][nt] + acc[1][nt];
    }

    // online softmax per head; lane (j, c16) holds tokens 16 mt + 4 j + e
    uint4 pb[kNT];
    bool grow = false;
    float alpha[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float x[2][4];
      float mt_max = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = t0 + 16u * mt + 4u * j + e < t_hi;
          x[mt][e] = vis ? s[mt][nt][e] * sl2 : -INFINITY;
          mt_max = fmaxf(mt_max, x[mt][e]);
        }
      mt_max = rows4_max(mt_max);
      const float m_new = mt_max > m[nt] + kSlack ? mt_max : m[nt];
      alpha[nt] = fast_exp2(m[nt] - m_new);
      grow |= m_new != m[nt];
      m[nt] = m_new;
      float p[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[mt][e] = fast_exp2(x[mt][e] - m_new);
      lsum[nt] = lsum[nt] * alpha[nt] + (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                                         ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
      pb[nt].x = M::pack2(p[0][0], p[0][1]);
      pb[nt].y = M::pack2(p[0][2], p[0][3]);
      pb[nt].z = M::pack2(p[1][0], p[1][1]);
      pb[nt].w = M::pack2(p[1][2], p[1][3]);
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int b = 0; b < DB; ++b) o[nt][b] *= alpha[nt];
    }

    // O^T += latent^T . P^T over 32 tokens: K slots 8j .. 8j+3 are tokens
    // 4j .. 4j+3 and slots 8j+4 .. 8j+7 tokens 16+4j .. 16+4j+3, matching
    // the score layout.  Lane (j, c16) reads rows 4j + (c16 >> 2) and
    // 16 + 4j + (c16 >> 2), columns 16b + 4(c16 & 3) .. +3 (transposed).
    const unsigned char *v0 = st_lat + pv_row;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const unsigned char *p0 = v0 + pv_off[b & 7] + 256 * (b >> 3);
      const uint2 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * L::kLatRow);
      const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) o[nt][b] = M::qk(va, pb[nt], o[nt][b]);
    }
    if (kt + kStages - 1 < n_tiles) {
      window_for(kt + kStages - 1);
      issue(kt + kStages - 1);
    }
  }

  // normalise and write: lane holds O^T[d = 16b + 4j + e][head 16 nt + c16]
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const float l_tot = rows4_sum(lsum[nt]);
    const uint32_t h = h0 + 16u * nt + c16;
    if (h >= a.hq) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (a.splits == 1) {
      T *out = static_cast<T *>(a.out) + (uint64_t(i) * a.hq + h) * R;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        uint2 w;
        w.x = M::pack2(o[nt][b][0] * inv, o[nt][b][1] * inv);
        w.y = M::pack2(o[nt][b][2] * inv, o[nt][b][3] * inv);
        *reinterpret_cast<uint2 *>(out + 16 * b + 4 * j) = w;
      }
    } else {
      const uint64_t r = (uint64_t(i) * a.splits + part) * a.hq + h;
      float *wo = a.ws_o + r * R;
#pragma unroll
      for (int b = 0; b < DB; ++b)
        *reinterpret_cast<f32x4_t *>(wo + 16 * b + 4 * j) = o[nt][b] * inv;
      if (j == 0) a.ws_lse[r] = m[nt] + fast_log2(l_tot);
    }
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

hipError_t launch_mla_mfma(const RowArgs &a, pkv_dtype dt, hipStream_t st) {
  const uint32_t hg = (a.hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const uint64_t blocks = mla_mfma_blocks(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));  // a multiple of 8 * hg
  if (dt == PKV_BF16)
    hipLaunchKernelGGL((mla_kernel<BF16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  else
    hipLaunchKernelGGL((mla_kernel<F16, 512, 64>), grid, dim3(256), 0, st, a, hg);
  return hipGetLastError();
}

}  // namespace pkv
