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
// head, 32 q-rows per wave, the N side of 32x32x16 MFMAs.  Keys are walked
// in tiles of 32 rows held in LDS rings.  S^T = K . Q^T puts keys on the M
// side, so a lane holds 16 keys of one q-row; the absolute-position mask
// and an online softmax in base 2 follow, and O^T += V^T . P^T takes V^T
// from transposed LDS reads.  The M rows of the score product are a fixed
// permutation of the tile's key rows, chosen so that a lane's 16
// probabilities are, in order, its own K-slots of the value product: P
// moves between waves only as whole lanes.  Rows are stored unpadded with
// their 16-byte chunks XOR-swizzled by row, which keeps the score reads and
// the transposed value reads free of bank conflicts.  The block table of the
// sequence is cached in LDS.  Blocks that share a (tile, KV head) are
// numbered so they land on one XCD and share its L2.  How the work of a
// block is split between its waves, and how the rings are filled (16-bit
// caches HBM -> LDS directly, FP8 caches widened through registers), is
// described at the kernel.

#include <type_traits>

#include "mfma_common.h"

namespace pkv {

namespace {

constexpr int kPW = 4;             // waves per role in a block (each issues a quarter of the ring loads)
constexpr int kRowsPerBlock = 128; // q-rows per block (32 per wave)
constexpr int kTT = 32;            // key rows per tile
constexpr int kTableCache = 1024;  // block-table entries cached in LDS
// A lane whose 16 probabilities of a tile sum above this (each is then at
// most this) makes the wave move its softmax references to the row maxima.
constexpr float kSumLimit = 256.f;

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <class DT>
struct Mfma32;

template <>
struct Mfma32<BF16> {
  // C(32 x 32) += A(32 x 16) . B(16 x 32), 8 elements per lane
  static __device__ __forceinline__ f32x16_t mma(const uint4 &a, const uint4 &b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // c + both halves of a packed pair
  static __device__ __forceinline__ float add_pair(uint32_t p, float c) {
    const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), one, c, false);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return BF16::pack2(lo, hi); }
};

template <>
struct Mfma32<F16> {
  static __device__ __forceinline__ f32x16_t mma(const uint4 &a, const uint4 &b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float c) {
    const f16x2_t one = {(_Float16)1.f, (_Float16)1.f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p), one, c, false);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const _Float16 a = _Float16(lo), b = _Float16(hi);
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
  }
};

template <int D>
struct PLds {
  static constexpr int kRowB = D * 2;              // bytes per row (unpadded)
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int kTile = kTT * kRowB;        // one K or V tile
  static constexpr int RPW = 1024 / kRowB;         // rows per wave load (64 lanes x 16 B)
  static constexpr int NI = kTT / (RPW * kPW);     // loads per wave per tensor per tile
  // chunk c of row r sits in slot c ^ swz(r)
  static __device__ __forceinline__ uint32_t swz(uint32_t r) {
    return D == 64 ? (r >> 1) & 7u : ((r >> 1) & 7u) | ((r & 1u) << 3);
  }
};

// Key row (0..31 in the tile) behind M row m of the score product.  A lane
// of the 32x32 result holds M rows 8i + 4h + e (i, e = 0..3, h = lane / 32);
// the value product's K-slots of lane half h at step t are its results
// i = 2t, 2t + 1 in order, so K-slot u of step t is M row 16t + 8(u >> 2) +
// 4h + (u & 3).  This permutation makes the four rows one transposed read
// fetches, and the rows 16 lanes read for the score product, fall in
// distinct LDS banks under the swizzle above.
__device__ __forceinline__ uint32_t key_of_mrow(uint32_t m) {
  return (m & 1u) | ((m >> 1) & 1u) << 3 | ((m >> 2) & 1u) << 1 | ((m >> 3) & 1u) << 2 |
         ((m >> 4) & 1u) << 4;
}
// The same for result element 4i + e of lane half 0 (half 1 adds 2).
__host__ __device__ constexpr int key_of_elem(int i, int e) {
  return (e & 1) + 8 * (e >> 1) + 4 * (i & 1) + 16 * (i >> 1);
}

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
// Sum and max of the values of lanes l and l ^ 32 (the swap leaves lane l
// with one of the two in each result, so only symmetric combinations of
// both results are the same in every lane).
__device__ __forceinline__ float halves_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(s[0]), __uint_as_float(s[1]));
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

// The same with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset.
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char *)(p)));
}

// A block-table entry beyond the LDS copy: one load, waited for in the same
// instruction block.  The wait covers every earlier load too (the ring can
// afford it on this path, taken only past kTableCache pages), and the
// compiler never sees a pending load whose registers it might reuse: a load
// it knew about would make it wait for all loads before later LDS reads.
__device__ __forceinline__ uint32_t table_word(const uint32_t *p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Two E4M3 codes (bytes 0, 1 or 2, 3 of x) widened exactly to the query type.
template <class DT>
__device__ __forceinline__ uint32_t widen2(uint32_t x, bool hi);
template <>
__device__ __forceinline__ uint32_t widen2<BF16>(uint32_t x, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen2<F16>(uint32_t x, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
}
// Eight codes (two dwords) widened to one 16-byte chunk of the stage.
template <class DT>
__device__ __forceinline__ uint4 widen8(uint32_t lo, uint32_t hi) {
  return make_uint4(widen2<DT>(lo, false), widen2<DT>(lo, true), widen2<DT>(hi, false), widen2<DT>(hi, true));
}

template <int N>
struct IC {
  static constexpr int value = N;
};

// The kernel.  A block runs eight waves for the same 128 q-rows: waves 0-3
// (score waves) compute S^T = K . Q^T of their 32 q-rows, mask it, run the
// online softmax and hand the packed probabilities and the rescale factor
// to LDS; waves 4-7
// (value waves, wave w + 4 beside score wave w on one SIMD) accumulate
// O^T += V^T . P^T one tile behind and issue every ring load.  A wave's own
// VALU work does not run beside its own MFMAs, but it does beside another
// wave's, so the softmax of one wave hides under the value product of its
// SIMD neighbour, and a wave held at a load issue holds back only itself.
// K and V have rings of three stages each: in interval k (between two block
// barriers) the score waves read K of tile k, the value waves V of tile
// k - 1, and the loads of K of tile k + 2 and V of tile k + 1 are issued.
// Rows no query of the block sees (before the first query's window, past
// the end) are loaded from the first row the block sees, so the ring never
// holds values the probabilities do not zero exactly.  Two blocks fit a CU
// at D = 128 (71 KB of LDS each, at most 128 VGPRs per wave), three at
// D = 64 (47 KB, at most 85 VGPRs).
//
// FP8 caches (E4M3 codes, one byte per element, with a key and a value
// scale) cannot go HBM -> LDS directly: the MFMAs take 16-bit operands.  The
// value waves load each tile's codes into registers two intervals ahead,
// widen them exactly to the query type (every E4M3 value is a bf16 and an
// f16) and store them into the same rings in the same swizzled layout.  The
// key scale is folded into the score scale, the value scale into the
// normalisation.
//
// WIN: a sliding window is in force (without one the block starts at key 0
// and the masks are one-sided).
template <class DT, int D, bool F8, bool WIN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, D == 64 ? 6 : 4))) void prefill_rs_kernel(
    TileArgs a, uint32_t n_sub, uint32_t n_groups) {
  using M = Mfma32<DT>;
  using L = PLds<D>;
  using T = typename DT::T;
  using CT = std::conditional_t<F8, uint8_t, T>;  // cache element: the query type or E4M3 codes
  constexpr int KS = D / 16;  // k-steps of the score product
  constexpr int MB = D / 32;  // 32-row blocks of value dims
  constexpr int NPV = 2 * MB; // value-product MFMAs per tile
  constexpr uint32_t kRS = 3; // ring stages, K and V each
  constexpr uint32_t kTileB = uint32_t(L::kTile);
  constexpr uint32_t kVRing = kRS * kTileB;        // V ring after the K ring
  constexpr uint32_t kPB = 2u * kRS * kTileB;       // probabilities [wave][buf][half][lane] 16 B
  constexpr uint32_t kAB = kPB + 4u * 2u * 2048u;   // rescale factors [wave][buf][lane]
  constexpr uint32_t kIB = kAB + 4u * 2u * 256u;    // 1 / denominator [wave][lane]
  constexpr uint32_t kBytes = kIB + 4u * 256u;
  __shared__ __align__(1024) unsigned char lds[kBytes];
  __shared__ uint32_t tcache[kTableCache];

  // Blocks are dispatched round-robin over the eight XCDs (blockIdx.x % 8).
  // The (tile, KV head) groups are dealt to the XCDs in turn, group g to XCD
  // g % 8, and the n_sub blocks of a group run back to back on its XCD, so
  // they share the group's K/V rows in that XCD's L2.  Dealing groups (not
  // contiguous ranges) spreads every tile's work over all XCDs: tiles of
  // one chunk have similar key counts while chunks differ widely.
  const uint32_t kb = blockIdx.x / 8u;
  const uint32_t group = (kb / n_sub) * 8u + blockIdx.x % 8u;
  if (group >= n_groups) return;
  // the group's sub-blocks longest first (the last queries see the most keys)
  const uint32_t sub = n_sub - 1u - kb % n_sub;
  const uint32_t kvh = group % a.hkv;
  const uint32_t tile = group / a.hkv;

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool vrole = wv >= 4u;
  const uint32_t wq = wv & 3u;  // the wave's 32 q-rows (both roles)
  const uint32_t c32 = lane & 31u, hf = lane >> 5;
  const PlanView &pv = a.plan;
  const uint32_t first = a.tiles[2 * tile], count = a.tiles[2 * tile + 1];
  const uint32_t grp = a.hq / a.hkv;
  const uint32_t qb_n = kRowsPerBlock / grp;
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
  const uint32_t *table = pv.words + pv.table + uint64_t(seq) * pv.W;
  const uint64_t page_elems = a.k_page;
  auto page_of = [&](uint32_t pg) { return uint64_t(pg < pv.N ? pg : 0u) * page_elems; };
  const uint32_t n_lp = (k_end + ps - 1) / ps;
  for (uint32_t e = tid; e < n_lp && e < uint32_t(kTableCache); e += 512) {
    const uint32_t pg = table[e];
    tcache[e] = pg < pv.N ? pg : 0u;
  }

  const uint32_t r = 32u * wq + c32;
  const uint32_t qq = r / grp, hh = r % grp;
  const bool row_ok = r < qb_n * grp && q_lo + qq < q_hi;
  const uint32_t pos = p0 + q_lo + qq;
  const uint32_t pos_min = p0 + q_lo;
  const uint32_t lim = a.causal && pos < k_end - 1u ? pos : k_end - 1u;
  auto win_lo = [&](uint32_t n) { return WIN && n > a.window ? n - a.window : 0u; };
  const uint32_t lo_min = win_lo(a.causal ? pos_min + 1u : k_end);
  const uint32_t lo_max = win_lo(a.causal ? p0 + q_hi : k_end);
  const uint32_t lo_row = a.causal ? win_lo(pos + 1u) : lo_min;
  const uint32_t kt0 = lo_min / kTT;
  const uint32_t n_tiles = (k_end + kTT - 1) / kTT;
  const uint32_t nt = n_tiles - kt0;  // >= 1: the first query sees key lo_min < k_end

  unsigned char *pbw = lds + kPB + wq * 4096u + lane * 16u;              // + buf 2048 + half 1024
  float *abw = reinterpret_cast<float *>(lds + kAB + wq * 512u) + lane;  // + buf 64
  float *ibw = reinterpret_cast<float *>(lds + kIB + wq * 256u) + lane;

  if (!vrole) {
    // ---------------- score waves ----------------
    // This lane's q-row (column c32 of the wave's N block) and its half of
    // the head dims: K-slots of lane half hf at k-step ks are dims
    // (D/2) hf + 8 ks .. +7, for the query operand and the key rows alike.
    uint4 qb[KS];
    {
      const T *qrow = static_cast<const T *>(a.q) +
                      (uint64_t(first + q_lo + qq) * a.hq + kvh * grp + hh) * D + (D / 2) * hf;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[ks] = row_ok ? *reinterpret_cast<const uint4 *>(qrow + 8 * ks) : make_uint4(0, 0, 0, 0);
    }
    block_sync_lds();  // table cache ready (the query loads may still be in flight)
    // LDS byte offsets (within a stage) of this lane's score operand reads:
    // k-step ks reads key row key_of_mrow(c32), chunk (CPR/2) hf + ks.
    uint32_t k_off[KS];
    {
      const uint32_t kr = key_of_mrow(c32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        k_off[ks] = kr * L::kRowB + 16u * ((uint32_t(L::CPR / 2) * hf + ks) ^ L::swz(kr));
    }
    float m = kNoMax, lsum = 0.f;
    const float sl2 = a.scale_log2;
    block_sync_lds();  // B_0: K of the first tile is in the ring

    auto interval = [&](auto j_c, uint32_t kk) {
      constexpr uint32_t J = decltype(j_c)::value;  // == kk mod 6
      constexpr uint32_t ST = J % kRS, BUF = J % 2u;
      const unsigned char *kst = lds + ST * kTileB;
      const uint32_t t0 = (kt0 + kk) * kTT;
      uint4 kbuf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kbuf[ks] = *reinterpret_cast<const uint4 *>(kst + k_off[ks]);
      f32x16_t x;
#pragma unroll
      for (int z = 0; z < 16; ++z) x[z] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) x = M::mma(kbuf[ks], qb[ks], x);
      const bool full = (a.causal ? (t0 + kTT - 1 <= pos_min && t0 + kTT <= k_end)
                                  : (t0 + kTT <= k_end)) && (!WIN || t0 >= lo_max);
      if (!full) {
        const int dl = int(lim) - int(t0) - 2 * int(hf);
        const int dlo = int(lo_row) - int(t0) - 2 * int(hf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[4 * i + e] = key_of_elem(i, e) <= dl && (!WIN || key_of_elem(i, e) >= dlo) ? x[4 * i + e] : -INFINITY;
      }
      uint32_t pk[8];
      float ts = 0.f;
      auto probs = [&]() {
        ts = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0v = fast_exp2(__builtin_fmaf(x[2 * j], sl2, -m));
          const float p1v = fast_exp2(__builtin_fmaf(x[2 * j + 1], sl2, -m));
          pk[j] = M::pack2(p0v, p1v);
          ts = M::add_pair(pk[j], ts);
        }
      };
      probs();
      // Lazy rescaling: the reference moves to the row maxima only when some
      // lane's tile sum passes kSumLimit (so no probability exceeds it);
      // numerator and denominator share the reference, so the result is the
      // same softmax.  The factor goes to the value wave, which scales O
      // before it adds this tile.
      float alpha = 1.f;
      if (__any(ts > kSumLimit)) {
        float lmax = vmax3(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], x[5]), vmax3(x[6], x[7], x[8]));
        lmax = vmax3(lmax, vmax3(x[9], x[10], x[11]), vmax3(x[12], x[13], x[14]));
        lmax = vmax(lmax, x[15]);
        lmax = halves_max(lmax);
        const float m_new = vmax(m, lmax * sl2);
        alpha = fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
        probs();
      }
      lsum += ts;
      *reinterpret_cast<uint4 *>(pbw + BUF * 2048u) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4 *>(pbw + BUF * 2048u + 1024u) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      abw[BUF * 64u] = alpha;
      if (kk + 1u == nt) {
        const float l_tot = halves_sum(lsum);
        *ibw = l_tot > 0.f ? 1.f / l_tot : 0.f;
      }
      block_sync_lds();  // B_{kk+1}
    };
    uint32_t kk = 0;
    for (; kk + 6u <= nt; kk += 6u) {
      interval(IC<0>(), kk);
      interval(IC<1>(), kk + 1u);
      interval(IC<2>(), kk + 2u);
      interval(IC<3>(), kk + 3u);
      interval(IC<4>(), kk + 4u);
      interval(IC<5>(), kk + 5u);
    }
    if (kk < nt) interval(IC<0>(), kk);
    if (kk + 1u < nt) interval(IC<1>(), kk + 1u);
    if (kk + 2u < nt) interval(IC<2>(), kk + 2u);
    if (kk + 3u < nt) interval(IC<3>(), kk + 3u);
    if (kk + 4u < nt) interval(IC<4>(), kk + 4u);
    return;
  }

  // ---------------- value waves ----------------
  const uint32_t tok_elems = uint32_t(a.k_tok);
  const CT *kbase = static_cast<const CT *>(a.k) + uint64_t(kvh) * D;
  const CT *vbase = static_cast<const CT *>(a.v) + uint64_t(kvh) * D;
  // Load n of this wave covers rows RPW (NI wq + n) .. + RPW - 1 of a tile;
  // lane -> row + lane / CPR, LDS slot lane % CPR holding chunk
  // slot ^ swz(row) of the cache row.
  constexpr uint32_t kWaveRows = uint32_t(L::RPW * L::NI);
  uint32_t chunk_el[L::NI], vo[L::NI];
#pragma unroll
  for (int n = 0; n < L::NI; ++n) {
    const uint32_t rr = L::RPW * (L::NI * wq + n) + lane / L::CPR;
    const uint32_t chunk = (lane % L::CPR) ^ L::swz(rr);
    chunk_el[n] = 8u * chunk;
    vo[n] = ((rr - kWaveRows * wq) * tok_elems + 8u * chunk) * uint32_t(sizeof(CT));
  }
  const uint32_t vis_lo = lo_min, vis_hi = k_end;
  // element offset of the cache row of token tok (rows no query of the
  // block sees read row vis_lo instead)
  auto row_off = [&](uint32_t tok) -> uint64_t {
    const uint32_t t = tok >= vis_lo && tok < vis_hi ? tok : vis_lo;
    const uint32_t lp = pow2 ? t >> ps_shift : t / ps;
    const uint32_t slot = t - lp * ps;
    const uint32_t pg = lp < uint32_t(kTableCache) ? tcache[lp] : table_word(table + lp);
    return page_of(pg) + uint64_t(slot) * tok_elems;
  };
  // Fast path: power-of-two pages of at least 8 tokens and a tile whose rows
  // are all seen: a wave's 8 rows are consecutive tokens of one page.
  const bool fast_dma = pow2 && ps >= 8u;
  auto fast_tile = [&](uint32_t j) {
    const uint32_t t0 = (kt0 + j) * kTT;
    return fast_dma && t0 >= vis_lo && t0 + kTT <= vis_hi;
  };
  // (the plan words do not change while a kernel runs: read through the
  // constant address space, a table entry is a scalar load)
  const __attribute__((address_space(4))) uint32_t *ctable =
      (const __attribute__((address_space(4))) uint32_t *)table;
  // the wave's page of tile j (its 8 rows are consecutive tokens of one page)
  auto wave_page = [&](uint32_t j) -> uint32_t {
    const uint32_t tw = __builtin_amdgcn_readfirstlane((kt0 + j) * kTT + kWaveRows * wq);
    return ctable[tw >> ps_shift];
  };
  // loads of tile j (local index) of K (is_v false) or V into its stage;
  // pg: the wave's page of that tile when fast_tile(j)
  auto issue = [&](bool is_v, uint32_t j, uint32_t pg) {
    const uint32_t st_off = (is_v ? kVRing : 0u) + (j % kRS) * kTileB;
    const CT *base = is_v ? vbase : kbase;
    if (fast_tile(j)) {
      const uint32_t tw = (kt0 + j) * kTT + kWaveRows * wq;
      const CT *wb = base + (page_of(pg) + uint64_t(tw & (ps - 1u)) * tok_elems);
#pragma unroll
      for (int n = 0; n < L::NI; ++n) {
        const uint32_t r0 = L::RPW * (L::NI * wq + n);
        dma16s(vo[n], wb, __builtin_amdgcn_readfirstlane(lds_addr(lds + st_off + r0 * L::kRowB)));
      }
    } else {
#pragma unroll
      for (int n = 0; n < L::NI; ++n) {
        const uint32_t r0 = L::RPW * (L::NI * wq + n);
        const uint32_t rr = r0 + lane / L::CPR;
        const uint64_t off = row_off((kt0 + j) * kTT + rr) + chunk_el[n];
        dma16(base + off, __builtin_amdgcn_readfirstlane(lds_addr(lds + st_off + r0 * L::kRowB)));
      }
    }
  };
  // this interval's loads may stay in flight: wait for the rest
  auto wait_all_but = [&](uint32_t groups) {
    if (groups >= 2u) wait_vm<2 * L::NI>();
    else if (groups == 1u) wait_vm<L::NI>();
    else wait_vm<0>();
  };

  // Value product, value block mb, step t, read rr (K-slots 4rr .. 4rr+3):
  // in each 16-lane group, lane 4e + q addresses key row
  // key_of_mrow(16t + 8rr + 4hf + e) and value dims 32mb + 16g + 4q .. +3
  // (g = lane / 16 mod 2); the transposed read hands lane i of the group
  // value dim 32mb + 16g + i of those four rows.  Step t only adds 16 rows,
  // the stage is added per tile.
  uint32_t v_off[MB][2];
  {
    const uint32_t g = (lane >> 4) & 1u, e = (lane >> 2) & 3u, q4 = lane & 3u;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const uint32_t kr = key_of_mrow(8u * rr + 4u * hf + e);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint32_t dv = 32u * mb + 16u * g + 4u * q4;
        v_off[mb][rr] = kVRing + kr * L::kRowB + 16u * ((dv / 8u) ^ L::swz(kr)) + 2u * (dv % 8u);
      }
    }
  }
  auto v_read = [&](const unsigned char *stage, int j) {
    const unsigned char *p = stage + 16 * (j / MB) * L::kRowB;
    const uint2 lo = lds_read_tr16(p + v_off[j % MB][0]), hi = lds_read_tr16(p + v_off[j % MB][1]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  f32x16_t o[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int x = 0; x < 16; ++x) o[b][x] = 0.f;

  // FP8 caches: value-wave thread tv carries codes EPT (tv % 8) .. + EPT - 1
  // of row tv / 8 of a tile, K and V, in one of two register sets; tile j's
  // codes are loaded two intervals before they are widened (exactly: every
  // E4M3 value is a bf16 and an f16) into the tile's K and V stages.  The
  // loads are unconditional (past the last tile they read it again), so the
  // compiler waits only for the set it stores.
  constexpr uint32_t EPT = D / 8;
  const uint32_t tv = tid - 256u;
  const uint32_t f_row = tv >> 3, f_col = (tv & 7u) * EPT;
  uint4 f8k[2], f8v[2];
  // (pg: the wave's page of the tile when it is on the fast path, where a
  // wave's 8 rows are consecutive tokens of one page, as for the DMA)
  auto f8_load = [&](uint32_t j, uint32_t pg, uint4 &rk, uint4 &rv) {
    const uint32_t jj = j < nt ? j : nt - 1u;
    const uint32_t tok = (kt0 + jj) * kTT + f_row;
    const uint64_t off =
        (fast_tile(jj) ? page_of(pg) + uint64_t(tok & (ps - 1u)) * tok_elems : row_off(tok)) + f_col;
    if constexpr (EPT == 16) {
      rk = *reinterpret_cast<const uint4 *>(kbase + off);
      rv = *reinterpret_cast<const uint4 *>(vbase + off);
    } else {
      const uint2 k2 = *reinterpret_cast<const uint2 *>(kbase + off);
      const uint2 v2 = *reinterpret_cast<const uint2 *>(vbase + off);
      rk = make_uint4(k2.x, k2.y, 0, 0);
      rv = make_uint4(v2.x, v2.y, 0, 0);
    }
  };
  auto f8_store = [&](uint32_t j, const uint4 &rk, const uint4 &rv) {
    unsigned char *kr = lds + (j % kRS) * kTileB + f_row * L::kRowB;
    unsigned char *vr = lds + kVRing + (j % kRS) * kTileB + f_row * L::kRowB;
    const uint32_t sw = L::swz(f_row);
    const uint32_t c0 = EPT == 16 ? 2u * (tv & 7u) : (tv & 7u);  // first 8-element chunk
    *reinterpret_cast<uint4 *>(kr + 16u * (c0 ^ sw)) = widen8<DT>(rk.x, rk.y);
    *reinterpret_cast<uint4 *>(vr + 16u * (c0 ^ sw)) = widen8<DT>(rv.x, rv.y);
    if constexpr (EPT == 16) {
      *reinterpret_cast<uint4 *>(kr + 16u * ((c0 + 1u) ^ sw)) = widen8<DT>(rk.z, rk.w);
      *reinterpret_cast<uint4 *>(vr + 16u * ((c0 + 1u) ^ sw)) = widen8<DT>(rv.z, rv.w);
    }
  };

  uint32_t pg_v = 0u, pg_k = 0u;  // pages of the next interval's loads (DMA, fast path)
  // DMA, interval k: loads of K of tile k + 2 and V of tile k + 1 (their
  // stages were last read in interval k - 1); returns the number of tiles
  // issued
  auto loads = [&](uint32_t k) {
    uint32_t n = 0;
    if (k + 2u < nt) { issue(false, k + 2u, pg_k); ++n; }
    if (k + 1u < nt) { issue(true, k + 1u, pg_v); ++n; }
    pg_v = pg_k;
    pg_k = k + 3u < nt && fast_tile(k + 3u) ? wave_page(k + 3u) : 0u;
    return n;
  };
  // the page f8_load needs for tile j (clamped as it clamps); pgf: that of
  // the tile the next interval loads, read one interval ahead
  auto page_f8 = [&](uint32_t j) {
    const uint32_t jj = j < nt ? j : nt - 1u;
    return fast_tile(jj) ? wave_page(jj) : 0u;
  };
  uint32_t pgf = 0u;
  if constexpr (F8) {
    // Prologue: tile 0 into its stages, tiles 1 and 2 into the register
    // sets; interval 0: tile 1 into its stages, tile 3 into its set.
    block_sync_lds();  // table cache ready
    f8_load(0u, page_f8(0u), f8k[0], f8v[0]);
    f8_load(1u, page_f8(1u), f8k[1], f8v[1]);
    f8_store(0u, f8k[0], f8v[0]);
    f8_load(2u, page_f8(2u), f8k[0], f8v[0]);
    block_sync_lds();  // B_0
    if (nt > 1u) f8_store(1u, f8k[1], f8v[1]);
    f8_load(3u, page_f8(3u), f8k[1], f8v[1]);
    pgf = page_f8(4u);
    block_sync_lds();  // B_1
  } else {
    // Prologue: K of tiles 0 and 1 and V of tile 0, then B_0 once all three
    // have landed.  Tiles on the fast path need no table cache and are issued
    // before the barrier that completes it.
    const bool f0 = fast_tile(0), f1 = nt > 1u && fast_tile(1);
    const uint32_t pg0 = f0 ? wave_page(0) : 0u;
    pg_v = f1 ? wave_page(1) : 0u;  // V of tile 1 (interval 0)
    if (f0) {
      issue(false, 0u, pg0);
      issue(true, 0u, pg0);
    }
    if (f1) issue(false, 1u, pg_v);
    block_sync_lds();  // table cache ready
    if (!f0) {
      issue(false, 0u, 0u);
      issue(true, 0u, 0u);
    }
    if (nt > 1u && !f1) issue(false, 1u, 0u);
    pg_k = nt > 2u && fast_tile(2) ? wave_page(2) : 0u;  // K of tile 2 (interval 0)
    wait_vm<0>();
    block_sync_lds();  // B_0
    wait_all_but(loads(0u));
    block_sync_lds();  // B_1
  }

  // interval t + 1: value product of tile t, then the loads
  constexpr int kAhead = 3;
  auto vinterval = [&](auto j_c, uint32_t t) {
    constexpr uint32_t J = decltype(j_c)::value;  // == t mod 6
    constexpr uint32_t ST = J % kRS, BUF = J % 2u;
    const unsigned char *vst = lds + ST * kTileB;
    uint4 vb[kAhead + 1];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) vb[j] = v_read(vst, j);
    const float alpha = abw[BUF * 64u];
    const uint4 pa = *reinterpret_cast<const uint4 *>(pbw + BUF * 2048u);
    const uint4 pb = *reinterpret_cast<const uint4 *>(pbw + BUF * 2048u + 1024u);
    uint32_t n_issued = 0u;
    if constexpr (F8) {
      // interval t + 1: tile t + 2 from its set into its stages, tile t + 4
      // into that set
      if (t + 2u < nt) f8_store(t + 2u, f8k[J % 2u], f8v[J % 2u]);
      if (t + 1u < nt) {
        f8_load(t + 4u, pgf, f8k[J % 2u], f8v[J % 2u]);
        pgf = page_f8(t + 5u);
      }
    } else {
      n_issued = t + 1u < nt ? loads(t + 1u) : 0u;
    }
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < MB; ++b) o[b] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      if (j + kAhead < NPV) vb[(j + kAhead) % (kAhead + 1)] = v_read(vst, j + kAhead);
      o[j % MB] = M::mma(vb[j % (kAhead + 1)], j / MB == 0 ? pa : pb, o[j % MB]);
    }
    if (t + 1u < nt) {
      if constexpr (!F8) wait_all_but(n_issued);
      block_sync_lds();  // B_{t+2}
    }
  };
  uint32_t t = 0;
  for (; t + 6u <= nt; t += 6u) {
    vinterval(IC<0>(), t);
    vinterval(IC<1>(), t + 1u);
    vinterval(IC<2>(), t + 2u);
    vinterval(IC<3>(), t + 3u);
    vinterval(IC<4>(), t + 4u);
    vinterval(IC<5>(), t + 5u);
  }
  if (t < nt) vinterval(IC<0>(), t);
  if (t + 1u < nt) vinterval(IC<1>(), t + 1u);
  if (t + 2u < nt) vinterval(IC<2>(), t + 2u);
  if (t + 3u < nt) vinterval(IC<3>(), t + 3u);
  if (t + 4u < nt) vinterval(IC<4>(), t + 4u);

  if constexpr (F8) wait_vm<0>();  // the register loads past the last tile
  // normalise and write: lane holds O^T[d = 32mb + 8i + 4hf + e][q-row c32]
  // (1 / denominator written by the score wave before the last barrier;
  // FP8: times the value scale)
  const float inv = F8 ? *ibw * a.v_scale : *ibw;
  if (!row_ok) return;
  T *out = static_cast<T *>(a.out) + (uint64_t(first + q_lo + qq) * a.hq + kvh * grp + hh) * D;
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 w;
      w.x = M::pack2(o[b][4 * i] * inv, o[b][4 * i + 1] * inv);
      w.y = M::pack2(o[b][4 * i + 2] * inv, o[b][4 * i + 3] * inv);
      *reinterpret_cast<uint2 *>(out + 32 * b + 8 * i + 4 * hf) = w;
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
  const bool d64 = a.d == 64, win = a.window != 0u;
  // (DT, D, FP8 cache, window) -> kernel
  auto pick = [&](auto dt_c, auto f8_c, auto win_c) {
    using DTT = decltype(dt_c);
    constexpr bool F8 = decltype(f8_c)::value, WIN = decltype(win_c)::value;
    if (d64) launch_k((prefill_rs_kernel<DTT, 64, F8, WIN>), grid, dim3(512), 0, st, a, n_sub, ng);
    else launch_k((prefill_rs_kernel<DTT, 128, F8, WIN>), grid, dim3(512), 0, st, a, n_sub, ng);
  };
  auto pick_win = [&](auto dt_c, auto f8_c) {
    if (win) pick(dt_c, f8_c, std::true_type());
    else pick(dt_c, f8_c, std::false_type());
  };
  auto pick_f8 = [&](auto dt_c) {
    if (a.kv_fp8) pick_win(dt_c, std::true_type());
    else pick_win(dt_c, std::false_type());
  };
  if (dt == PKV_BF16) pick_f8(BF16());
  else pick_f8(F16());
  return hipGetLastError();
}

}  // namespace pkv
