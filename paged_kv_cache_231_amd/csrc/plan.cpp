// Plan encoder and validator (host only).
//
// The ruDNN 0.1.7 `paged_attention` page keeps the schedule as a `HostPlan`
// of u32 words that `DevicePlan::upload` copies to the device once; the word
// layout is not shown there.  This file implements this library's layout,
// spec v1, documented in pkv.h.  Validation happens here, before any launch,
// so kernels can index the cache with the words without further checks.

#include <cstring>
#include <algorithm>
#include <vector>

#include "common.h"

namespace pkv {

namespace {
thread_local const char *g_error = "";
constexpr uint64_t kU32Max = 0xFFFFFFFFull;

uint32_t ceil_div(uint32_t a, uint32_t b) { return a / b + (a % b != 0); }

// Appends the rows and tiles of the queries to `rows` / `tiles` following the
// run rule of spec v1.
void cut_runs(uint32_t q_count, const uint32_t *qseq, const uint32_t *qpos,
              std::vector<uint32_t> *rows, std::vector<uint32_t> *tiles) {
  struct Tile {
    uint32_t first, count;
    uint64_t work;  // sum of (position + 1) over the tile's queries
  };
  std::vector<Tile> found;
  uint32_t a = 0;
  while (a < q_count) {
    uint32_t b = a + 1;
    while (b < q_count && qseq[b] == qseq[a] && qpos[b] == qpos[b - 1] + 1) ++b;
    const uint32_t len = b - a;
    if (len >= PKV_TILE_MIN) {
      for (uint32_t f = a; f < b; f += PKV_TILE_MAX) {
        const uint32_t c = b - f < PKV_TILE_MAX ? b - f : PKV_TILE_MAX;
        found.push_back({f, c, uint64_t(c) * qpos[f] + uint64_t(c) * (c + 1) / 2});
      }
    } else {
      for (uint32_t i = a; i < b; ++i) rows->push_back(i);
    }
    a = b;
  }
  // heaviest first (kernels take tiles in list order), ties by first query
  std::sort(found.begin(), found.end(), [](const Tile &x, const Tile &y) {
    return x.work != y.work ? x.work > y.work : x.first < y.first;
  });
  for (const Tile &t : found) {
    tiles->push_back(t.first);
    tiles->push_back(t.count);
  }
}
}  // namespace

pkv_status fail(pkv_status code, const char *msg) {
  g_error = msg;
  return code;
}
void clear_error() { g_error = ""; }
const char *last_error() { return g_error; }

pkv_status read_layout(const uint32_t *w, size_t n, PlanLayout *L) {
  if (!w || n < PKV_PLAN_HEADER_WORDS) return fail(PKV_EINVAL, "plan shorter than its header");
  if (w[0] != PKV_PLAN_MAGIC || w[1] != PKV_PLAN_VERSION)
    return fail(PKV_EINVAL, "not a spec-v1 plan (magic/version)");
  for (uint32_t i = 9; i < PKV_PLAN_HEADER_WORDS; ++i)
    if (w[i] != 0) return fail(PKV_EINVAL, "reserved plan header words must be zero");
  PlanLayout l;
  l.Q = w[2]; l.S = w[3]; l.W = w[4]; l.ps = w[5]; l.N = w[6]; l.R = w[7]; l.T = w[8];
  const uint64_t total = uint64_t(PKV_PLAN_HEADER_WORDS) + l.S + 2ull * l.Q + l.R +
                         2ull * l.T + uint64_t(l.S) * l.W;
  if (total > kU32Max) return fail(PKV_ERANGE, "plan exceeds u32 word count");
  if (total != n) return fail(PKV_EINVAL, "plan length does not match its header");
  l.lens = PKV_PLAN_HEADER_WORDS;
  l.qseq = l.lens + l.S;
  l.qpos = l.qseq + l.Q;
  l.rows = l.qpos + l.Q;
  l.tiles = l.rows + l.R;
  l.table = l.tiles + 2ull * l.T;
  l.total = total;
  *L = l;
  return PKV_OK;
}

pkv_status validate_plan(const uint32_t *w, size_t n, PlanLayout *out) {
  PlanLayout L;
  pkv_status st = read_layout(w, n, &L);
  if (st != PKV_OK) return st;
  if (L.ps == 0) return fail(PKV_EINVAL, "page size must be positive");
  if (L.S > 0 && L.W == 0) return fail(PKV_EINVAL, "table width must be positive");
  if (uint64_t(L.S) * L.W > kU32Max) return fail(PKV_ERANGE, "block table exceeds u32 indexing");
  const uint32_t *lens = w + L.lens, *qseq = w + L.qseq, *qpos = w + L.qpos;
  for (uint32_t s = 0; s < L.S; ++s)
    if (uint64_t(lens[s]) > uint64_t(L.W) * L.ps)
      return fail(PKV_ESHAPE, "sequence longer than its block-table row");
  for (uint32_t i = 0; i < L.Q; ++i) {
    if (qseq[i] >= L.S) return fail(PKV_EINVAL, "query sequence index out of range");
    if (qpos[i] >= lens[qseq[i]]) return fail(PKV_EINVAL, "query position outside its sequence");
  }
  // Rows and tiles must be exactly what the run rule produces: kernels rely
  // on tiles being consecutive positions of one sequence.
  std::vector<uint32_t> rows, tiles;
  cut_runs(L.Q, qseq, qpos, &rows, &tiles);
  if (rows.size() != L.R || tiles.size() != 2ull * L.T)
    return fail(PKV_EINVAL, "plan rows/tiles do not follow the run rule");
  if (L.R && std::memcmp(rows.data(), w + L.rows, 4ull * L.R) != 0)
    return fail(PKV_EINVAL, "plan rows do not follow the run rule");
  if (L.T && std::memcmp(tiles.data(), w + L.tiles, 8ull * L.T) != 0)
    return fail(PKV_EINVAL, "plan tiles do not follow the run rule");
  for (uint32_t s = 0; s < L.S; ++s) {
    const uint32_t *row = w + L.table + size_t(s) * L.W;
    const uint32_t used = ceil_div(lens[s], L.ps);
    for (uint32_t j = 0; j < L.W; ++j) {
      if (j < used && row[j] >= L.N) return fail(PKV_EINVAL, "block table entry outside the page pool");
      if (j >= used && row[j] != PKV_UNUSED_PAGE)
        return fail(PKV_EINVAL, "unused block table entries must be PKV_UNUSED_PAGE");
    }
  }
  if (out) *out = L;
  return PKV_OK;
}

}  // namespace pkv

namespace pkv {

// Slot keys page * ps + slot of every query's own position (positions are
// inside their sequences and used table entries inside the pool: the plan
// is valid), sorted; a repeated key is a conflict.
pkv_status validate_writes(const uint32_t *w, const PlanLayout &L) {
  std::vector<uint64_t> keys(L.Q);
  for (uint32_t i = 0; i < L.Q; ++i) {
    const uint32_t s = w[L.qseq + i], p = w[L.qpos + i];
    const uint32_t page = w[L.table + size_t(s) * L.W + p / L.ps];
    keys[i] = uint64_t(page) * L.ps + p % L.ps;
  }
  std::sort(keys.begin(), keys.end());
  for (size_t i = 1; i < keys.size(); ++i)
    if (keys[i] == keys[i - 1]) return fail(PKV_EINVAL, "two queries write one cache slot");
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

const char *pkv_last_error(void) { return pkv::last_error(); }

pkv_status pkv_plan_encode(uint32_t S, const uint32_t *lens, uint32_t Q, const uint32_t *qseq,
                           const uint32_t *qpos, uint32_t W, const uint32_t *table, uint32_t ps,
                           uint32_t N, uint32_t *words, size_t *n_words) {
  using namespace pkv;
  clear_error();
  if (!n_words) return fail(PKV_EINVAL, "n_words must not be null");
  if ((S && !lens) || (Q && (!qseq || !qpos)) || (uint64_t(S) * W && !table))
    return fail(PKV_EINVAL, "null schedule array");
  if (ps == 0) return fail(PKV_EINVAL, "page size must be positive");
  if (S > 0 && W == 0) return fail(PKV_EINVAL, "table width must be positive");
  if (uint64_t(S) * W > kU32Max) return fail(PKV_ERANGE, "block table exceeds u32 indexing");
  for (uint32_t s = 0; s < S; ++s)
    if (uint64_t(lens[s]) > uint64_t(W) * ps)
      return fail(PKV_ESHAPE, "sequence longer than its block-table row");
  for (uint32_t i = 0; i < Q; ++i) {
    if (qseq[i] >= S) return fail(PKV_EINVAL, "query sequence index out of range");
    if (qpos[i] >= lens[qseq[i]]) return fail(PKV_EINVAL, "query position outside its sequence");
  }
  std::vector<uint32_t> rows, tiles;
  cut_runs(Q, qseq, qpos, &rows, &tiles);
  const uint64_t total = uint64_t(PKV_PLAN_HEADER_WORDS) + S + 2ull * Q + rows.size() +
                         tiles.size() + uint64_t(S) * W;
  if (total > kU32Max) return fail(PKV_ERANGE, "plan exceeds u32 word count");
  for (uint32_t s = 0; s < S; ++s) {
    const uint32_t used = ceil_div(lens[s], ps);
    for (uint32_t j = 0; j < used; ++j)
      if (table[size_t(s) * W + j] >= N) return fail(PKV_EINVAL, "block table entry outside the page pool");
  }
  const size_t cap = *n_words;
  *n_words = size_t(total);
  if (!words) return PKV_OK;
  if (cap < total) return fail(PKV_EINVAL, "word buffer too small");

  uint32_t *o = words;
  const uint32_t head[PKV_PLAN_HEADER_WORDS] = {PKV_PLAN_MAGIC, PKV_PLAN_VERSION, Q, S, W, ps, N,
                                                uint32_t(rows.size()), uint32_t(tiles.size() / 2)};
  std::memcpy(o, head, sizeof(head)); o += PKV_PLAN_HEADER_WORDS;
  if (S) { std::memcpy(o, lens, 4ull * S); o += S; }
  if (Q) { std::memcpy(o, qseq, 4ull * Q); o += Q; std::memcpy(o, qpos, 4ull * Q); o += Q; }
  if (!rows.empty()) { std::memcpy(o, rows.data(), 4 * rows.size()); o += rows.size(); }
  if (!tiles.empty()) { std::memcpy(o, tiles.data(), 4 * tiles.size()); o += tiles.size(); }
  for (uint32_t s = 0; s < S; ++s) {
    const uint32_t used = ceil_div(lens[s], ps);
    for (uint32_t j = 0; j < W; ++j) *o++ = j < used ? table[size_t(s) * W + j] : PKV_UNUSED_PAGE;
  }
  return PKV_OK;
}

pkv_status pkv_plan_validate(const uint32_t *words, size_t n_words) {
  pkv::clear_error();
  return pkv::validate_plan(words, n_words, nullptr);
}

pkv_status pkv_plan_validate_writes(const uint32_t *words, size_t n_words) {
  pkv::clear_error();
  pkv::PlanLayout L;
  const pkv_status st = pkv::validate_plan(words, n_words, &L);
  if (st != PKV_OK) return st;
  return pkv::validate_writes(words, L);
}

}  // extern "C"
