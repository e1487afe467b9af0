// C ABI of libpkv: plan and workspace objects, argument validation and
// kernel dispatch.
//
// Validation mirrors the checks of the ruDNN 0.1.7 `paged_attention` page
// (`check_tensor`, `bounded`, `execute_attention_into`): every check runs
// before the first launch, so a failing call launches nothing and leaves
// `out` untouched; Q == 0 returns after the checks with no launch.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

struct pkv_plan {
  int device = -1;
  hipStream_t stream = nullptr;
  uint32_t *dev = nullptr;
  std::vector<uint32_t> host;
  pkv::PlanLayout L;
  // per-kernel timing (pkv_plan_timing): event pairs recorded around launches
  struct Rec {
    int kernel;
    hipEvent_t start, stop;
  };
  uint32_t timing = 0;  // mask of timed kernels (1 << pkv_kernel)
  mutable std::vector<Rec> recs;
  mutable std::vector<hipEvent_t> spare;
};

struct pkv_workspace {
  int device = -1;
  hipStream_t stream = nullptr;
  uint32_t queries = 0, heads = 0, dv = 0, splits = 0;  // splits 0: balanced
  float *buf = nullptr;
  size_t bytes = 0;
  // balanced schedule: slot_rows f32 rows of dv (two slots per unit: 16 rows
  // per decode wave, up to max_waves; 64 per MLA block, one block per CU),
  // their lse, then {first tile, tiles} per query and the total
  uint32_t max_waves = 0, cus = 0;
  uint64_t slot_rows = 0;
  float *slot_lse = nullptr;
  uint32_t *rec = nullptr;
};

namespace pkv {
namespace {

constexpr uint64_t kU32Max = 0xFFFFFFFFull;
constexpr float kLog2e = 1.4426950408889634f;

bool u32_elems(std::initializer_list<uint64_t> dims) {
  uint64_t n = 1;
  for (uint64_t d : dims) {
    if (d > kU32Max) return false;
    if (d != 0 && n > kU32Max / d) return false;
    n *= d;
  }
  return n <= kU32Max;
}

// A cache tensor may hold more than 2^32 elements (the kernels address the
// caches with 64-bit offsets); its size in bytes, at four bytes an element
// at most, has to fit in 63 bits.
bool cache_fits(std::initializer_list<uint64_t> dims) {
  unsigned __int128 p = 4;
  for (uint64_t d : dims) {
    p *= d;
    if (p >> 63) return false;
  }
  return true;
}

bool overlaps(const void *a, uint64_t a_bytes, const void *b, uint64_t b_bytes) {
  if (!a || !b || a_bytes == 0 || b_bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

size_t elem_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

pkv_status check_binding(const pkv_plan *plan, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  if (dev != plan->device || stream != plan->stream)
    return fail(PKV_EDEVICE, "call made on another device or stream than the plan");
  return PKV_OK;
}

PlanView view_of(const pkv_plan *p) {
  PlanView v;
  v.words = p->dev;
  v.lens = uint32_t(p->L.lens);
  v.qseq = uint32_t(p->L.qseq);
  v.qpos = uint32_t(p->L.qpos);
  v.table = uint32_t(p->L.table);
  v.W = p->L.W;
  v.ps = p->L.ps;
  v.N = p->L.N;
  return v;
}

pkv_status check_workspace(const pkv_workspace *ws, const pkv_plan *plan, uint32_t heads,
                           uint32_t dv, hipStream_t stream) {
  if (!ws) return PKV_OK;
  if (ws->queries != plan->L.Q || ws->heads != heads || ws->dv != dv || ws->stream != stream ||
      ws->device != plan->device)
    return fail(PKV_EWORKSPACE, "workspace was made for other queries, heads, value dim, device or stream");
  return PKV_OK;
}

pkv_status hip_fail(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "kernel launch failed");
}

// True while `st` is being captured into a graph (or when the query fails).
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

hipEvent_t take_event(const pkv_plan *plan) {
  if (!plan->spare.empty()) {
    hipEvent_t e = plan->spare.back();
    plan->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

}  // namespace
LaunchEvents &launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}
namespace {

// Times the kernel launched inside its scope when the plan's timing is on:
// the launch records a pair of HIP events at the kernel's own start and end
// (launch_k).  A scope that launches nothing records nothing; a stream being
// captured into a graph is not timed.
class Timed {
 public:
  Timed(const pkv_plan *plan, pkv_kernel kernel, hipStream_t st) : plan_(plan) {
    if (!(plan_->timing >> uint32_t(kernel) & 1u)) return;
    if (capturing(st)) return;
    rec_.kernel = int(kernel);
    rec_.start = take_event(plan_);
    rec_.stop = take_event(plan_);
    if (rec_.start && rec_.stop) {
      launch_events() = LaunchEvents{rec_.start, rec_.stop, false};
      on_ = true;
    }
  }
  ~Timed() {
    const bool used = on_ && launch_events().used;
    launch_events() = LaunchEvents{};
    if (used) {
      plan_->recs.push_back(rec_);
    } else {
      if (rec_.start) plan_->spare.push_back(rec_.start);
      if (rec_.stop) plan_->spare.push_back(rec_.stop);
    }
  }

 private:
  const pkv_plan *plan_;
  pkv_plan::Rec rec_{};
  bool on_ = false;
};

// Waves per CU of a balanced launch: one per SIMD.  Fewer concurrent page
// streams keep more DRAM rows open; 8 or 12 waves per CU measured slower.
// An FP8 cache moves half the bytes per tile, so it keeps two waves per SIMD
// to have as many bytes in flight.
constexpr uint32_t kBalancedWavesPerCu = 4;
constexpr uint32_t kBalancedWavesPerCuFp8 = 8;

// Resident waves per CU of the balanced kernel, cached per (dtype, d, page
// uniformity); 0 for shapes it does not take.
int bal_waves_per_cu(uint32_t d, uint32_t ps, pkv_dtype dt) {
  if (dt != PKV_F16 && dt != PKV_BF16) return 0;
  const int di = d == 64 ? 0 : d == 128 ? 1 : d == 256 ? 2 : -1;
  if (di < 0) return 0;
  const int pu = (ps & (ps - 1)) == 0 && ps >= 16u ? 1 : 0;
  static std::atomic<int> cache[2][3][2];
  std::atomic<int> &c = cache[dt == PKV_BF16][di][pu];
  int v = c.load(std::memory_order_relaxed);
  if (v == 0) {
    v = balanced_waves_per_cu(d, ps, dt);
    c.store(v, std::memory_order_relaxed);
  }
  return v;
}

// Waves of a balanced launch, or 0 when the call cannot use the balanced
// schedule (then the rows run unsplit).
uint32_t balanced_waves(const RowArgs &ra, pkv_dtype dt, const pkv_workspace *ws) {
  if (!ws || ws->splits != 0 || ws->max_waves == 0 || ra.pdim != 0) return 0;
  if (!rows_mfma_supported(ra, dt)) return 0;
  // every tile number and k * (tiles per group) must stay below 2^31
  const uint64_t grp = ra.hq / ra.hkv;
  const uint64_t segq = uint64_t(ra.hkv) * ((grp + 15) / 16);
  const uint64_t max_tiles = (uint64_t(ra.plan.W) * ra.plan.ps + 15) / 16;
  if (uint64_t(ra.n_queries) * max_tiles >= (1ull << 31)) return 0;
  const uint64_t per_cu = std::min<uint64_t>(ra.kv_fp8 ? kBalancedWavesPerCuFp8 : kBalancedWavesPerCu,
                                             bal_waves_per_cu(ra.d, ra.plan.ps, dt));
  uint64_t w = std::min<uint64_t>(ws->max_waves, per_cu * ws->cus);
  w -= w % 4;
  if (segq > w) return 0;  // not one group of segq waves
  return uint32_t(w);
}

// Blocks of a balanced MLA launch, or 0 when the call cannot use the
// balanced schedule (then it runs unsplit).
uint32_t mla_balanced(const RowArgs &ra, pkv_dtype dt, const pkv_workspace *ws) {
  if (!ws || ws->splits != 0 || ws->slot_rows == 0 || ra.pdim == 0) return 0;
  if (!mla_mfma_supported(ra, dt)) return 0;
  // every tile number and k * (tiles per group) must stay below 2^31
  const uint64_t max_tiles = (uint64_t(ra.plan.W) * ra.plan.ps + 31) / 32;
  if (uint64_t(ra.n_queries) * max_tiles >= (1ull << 31)) return 0;
  return mla_balanced_blocks(ra, ws->cus, ws->slot_rows);
}

MergeArgs balanced_merge_args(const RowArgs &ra) {
  MergeArgs ma{};
  ma.plan = ra.plan;
  ma.qlist = ra.qlist;
  ma.n_queries = ra.n_queries;
  ma.hq = ra.hq;
  ma.hkv = ra.hkv;
  ma.dv = ra.dv;
  ma.splits = 1;
  ma.pages_per_split = ra.pages_per_split;
  ma.causal = ra.causal;
  ma.ws_o = ra.ws_o;
  ma.ws_lse = ra.ws_lse;
  ma.out = ra.out;
  ma.bal_rec = ra.bal_rec;
  ma.bal_waves = ra.bal_waves;
  return ma;
}

// Set by run_rows when a call took the balanced schedule (the tuner times
// the balanced candidate only when it really runs).
thread_local bool t_ran_balanced = false;

// Launches the row kernel (and the merge when split) over `qlist`.
pkv_status run_rows(const pkv_plan *plan, RowArgs ra, pkv_dtype dt, const pkv_workspace *ws,
                    hipStream_t st) {
  hipError_t e;
  ra.bal_waves = balanced_waves(ra, dt, ws);
  if (ra.bal_waves) {
    t_ran_balanced = true;
    {
      Timed t(plan, PKV_KERNEL_ROWS, st);
      e = launch_rows_balanced(ra, dt, st);
    }
    if (e != hipSuccess) return hip_fail(e);
    Timed t(plan, PKV_KERNEL_MERGE, st);
    return hip_fail(launch_merge_balanced(balanced_merge_args(ra), dt, 16, st));
  }
  ra.bal_waves = mla_balanced(ra, dt, ws);
  if (ra.bal_waves) {
    t_ran_balanced = true;
    {
      Timed t(plan, PKV_KERNEL_MLA, st);
      e = launch_mla_balanced(ra, dt, st);
    }
    if (e != hipSuccess) return hip_fail(e);
    Timed t(plan, PKV_KERNEL_MERGE, st);
    return hip_fail(launch_merge_balanced(balanced_merge_args(ra), dt, kMlaBlockHeads, st));
  }
  if (ra.pdim != 0 && mla_mfma_supported(ra, dt)) {
    if (mla_mfma_blocks(ra) > kU32Max) return fail(PKV_ERANGE, "launch grid exceeds the x-dimension limit");
    Timed t(plan, PKV_KERNEL_MLA, st);
    e = launch_mla_mfma(ra, dt, st);
  } else if (rows_mfma_supported(ra, dt)) {
    if (rows_mfma_blocks(ra) * 256u > kU32Max) return fail(PKV_ERANGE, "launch grid exceeds the x-dimension limit");
    Timed t(plan, PKV_KERNEL_ROWS, st);
    e = launch_rows_mfma(ra, dt, st);
  } else if (ra.kv_fp8) {
    return fail(PKV_ESHAPE, "an FP8 cache needs head_dim == value_dim in {64, 128, 256}");
  } else if (rows_fast_supported(ra, dt)) {
    if (uint64_t(ra.n_queries) * ra.hq * ra.splits * 256u > kU32Max)
      return fail(PKV_ERANGE, "launch grid exceeds the x-dimension limit");
    Timed t(plan, PKV_KERNEL_ROWS, st);
    e = launch_rows_fast(ra, dt, st);
  } else {
    if (uint64_t(ra.n_queries) * ra.hq * ra.splits * 64u > kU32Max)
      return fail(PKV_ERANGE, "launch grid exceeds the x-dimension limit");
    Timed t(plan, ra.pdim ? PKV_KERNEL_MLA : PKV_KERNEL_ROWS, st);
    e = launch_rows_generic(ra, dt, st);
  }
  if (e != hipSuccess) return hip_fail(e);
  if (ws && ra.splits > 1) {
    MergeArgs ma{};
    ma.plan = ra.plan;
    ma.qlist = ra.qlist;
    ma.n_queries = ra.n_queries;
    ma.hq = ra.hq;
    ma.hkv = ra.hkv;
    ma.dv = ra.dv;
    ma.splits = ra.splits;
    ma.pages_per_split = ra.pages_per_split;
    ma.causal = ra.causal;
    ma.window = ra.window;
    ma.ws_o = ra.ws_o;
    ma.ws_lse = ra.ws_lse;
    ma.out = ra.out;
    Timed t(plan, PKV_KERNEL_MERGE, st);
    e = launch_merge(ma, dt, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return PKV_OK;
}

void fill_split(RowArgs *ra, const pkv_plan *plan, pkv_workspace *ws) {
  // a balanced workspace runs the kernels without a balanced schedule unsplit
  const uint32_t splits = ws && ws->splits ? ws->splits : 1u;
  ra->splits = splits;
  const uint32_t W = plan->L.W ? plan->L.W : 1u;
  ra->pages_per_split = W / splits + (W % splits != 0);
  ra->bal_rec = nullptr;
  ra->bal_waves = 0;
  if (ws && ws->splits == 0) {
    ra->ws_o = ws->buf;
    ra->ws_lse = ws->slot_lse;
    ra->bal_rec = ws->rec;
  } else if (ws && splits > 1) {
    ra->ws_o = ws->buf;
    ra->ws_lse = ws->buf + uint64_t(ws->queries) * splits * ws->heads * ws->dv;
  } else {
    ra->ws_o = nullptr;
    ra->ws_lse = nullptr;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

const char *pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

pkv_status pkv_plan_create(const uint32_t *words, size_t n_words, void *stream, pkv_plan **out) {
  clear_error();
  if (!out) return fail(PKV_EINVAL, "out must not be null");
  *out = nullptr;
  PlanLayout L;
  pkv_status st = validate_plan(words, n_words, &L);
  if (st != PKV_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  auto *p = new pkv_plan;
  p->device = dev;
  p->stream = static_cast<hipStream_t>(stream);
  p->host.assign(words, words + n_words);
  p->L = L;
  if (hipMalloc(&p->dev, n_words * sizeof(uint32_t)) != hipSuccess) {
    delete p;
    return fail(PKV_EHIP, "hipMalloc of plan words failed");
  }
  if (hipMemcpyAsync(p->dev, p->host.data(), n_words * sizeof(uint32_t), hipMemcpyHostToDevice,
                     p->stream) != hipSuccess) {
    (void)hipFree(p->dev);
    delete p;
    return fail(PKV_EHIP, "plan upload failed");
  }
  *out = p;
  return PKV_OK;
}

pkv_status pkv_plan_rebind_async(pkv_plan *plan, const uint32_t *words, size_t n_words,
                                 void *stream) {
  clear_error();
  if (!plan) return fail(PKV_EINVAL, "null plan");
  pkv_status st = check_binding(plan, static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  // a copy recorded into a graph would replay the words of capture time
  // while the host copy moved on; rebinding happens between replays
  if (capturing(plan->stream)) return fail(PKV_EINVAL, "plan words cannot change while the stream is captured");
  PlanLayout L;
  st = validate_plan(words, n_words, &L);
  if (st != PKV_OK) return st;
  if (n_words != plan->host.size() || std::memcmp(words + 2, plan->host.data() + 2, 7 * 4) != 0)
    return fail(PKV_ESHAPE, "rebind must keep Q, S, W, ps, N, R and T");
  if (hipMemcpyAsync(plan->dev, words, n_words * sizeof(uint32_t), hipMemcpyHostToDevice,
                     plan->stream) != hipSuccess)
    return fail(PKV_EHIP, "plan rebind copy failed");
  std::memcpy(plan->host.data(), words, n_words * sizeof(uint32_t));
  return PKV_OK;
}

pkv_status pkv_plan_set_word_async(pkv_plan *plan, size_t index, uint32_t value, void *stream) {
  clear_error();
  if (!plan) return fail(PKV_EINVAL, "null plan");
  pkv_status st = check_binding(plan, static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  if (index < PKV_PLAN_HEADER_WORDS || index >= plan->host.size())
    return fail(PKV_EINVAL, "word index outside the plan body");
  // a memset node in a graph would replay one value forever; set words
  // between replays
  if (capturing(plan->stream)) return fail(PKV_EINVAL, "plan words cannot change while the stream is captured");
  const uint32_t old = plan->host[index];
  plan->host[index] = value;
  st = validate_plan(plan->host.data(), plan->host.size(), nullptr);
  if (st != PKV_OK) {
    plan->host[index] = old;
    return st;
  }
  if (hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(plan->dev + index), int(value), 1,
                        plan->stream) != hipSuccess) {
    plan->host[index] = old;
    return fail(PKV_EHIP, "hipMemsetD32Async failed");
  }
  return PKV_OK;
}

pkv_status pkv_plan_header(const pkv_plan *plan, uint32_t *header) {
  clear_error();
  if (!plan || !header) return fail(PKV_EINVAL, "null argument");
  std::memcpy(header, plan->host.data(), PKV_PLAN_HEADER_WORDS * sizeof(uint32_t));
  return PKV_OK;
}

const uint32_t *pkv_plan_device_words(const pkv_plan *plan) { return plan ? plan->dev : nullptr; }

void pkv_plan_destroy(pkv_plan *plan) {
  if (!plan) return;
  if (plan->dev) (void)hipFree(plan->dev);
  for (const auto &r : plan->recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  for (hipEvent_t e : plan->spare) (void)hipEventDestroy(e);
  delete plan;
}

pkv_status pkv_plan_timing_select(pkv_plan *plan, uint32_t kernel_mask) {
  clear_error();
  if (!plan) return fail(PKV_EINVAL, "null plan");
  if (kernel_mask >> (uint32_t(PKV_KERNEL_APPEND) + 1u)) return fail(PKV_EINVAL, "unknown kernel in the mask");
  for (const auto &r : plan->recs) {
    plan->spare.push_back(r.start);
    plan->spare.push_back(r.stop);
  }
  plan->recs.clear();
  plan->timing = kernel_mask;
  return PKV_OK;
}

pkv_status pkv_plan_timing(pkv_plan *plan, int enable) {
  return pkv_plan_timing_select(plan, enable ? (2u << uint32_t(PKV_KERNEL_APPEND)) - 1u : 0u);
}

pkv_status pkv_plan_timing_read(pkv_plan *plan, pkv_kernel kernel, uint32_t *launches,
                                double *total_ms) {
  clear_error();
  if (!plan || !launches || !total_ms) return fail(PKV_EINVAL, "null argument");
  if (int(kernel) < int(PKV_KERNEL_ROWS) || int(kernel) > int(PKV_KERNEL_APPEND))
    return fail(PKV_EINVAL, "unknown kernel");
  uint32_t n = 0;
  double ms = 0.0;
  for (const auto &r : plan->recs) {
    if (r.kernel != int(kernel)) continue;
    float x = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&x, r.start, r.stop) != hipSuccess)
      return fail(PKV_EHIP, "timing event query failed");
    ++n;
    ms += x;
  }
  *launches = n;
  *total_ms = ms;
  return PKV_OK;
}

pkv_status pkv_workspace_create(uint32_t queries, uint32_t heads, uint32_t dv, uint32_t splits,
                                void *stream, pkv_workspace **out) {
  clear_error();
  if (!out) return fail(PKV_EINVAL, "out must not be null");
  *out = nullptr;
  if (splits < 1 || splits > PKV_MAX_SPLITS) return fail(PKV_EINVAL, "split count outside 1..PKV_MAX_SPLITS");
  if (queries == 0 || heads == 0 || dv == 0) return fail(PKV_EINVAL, "workspace dimensions must be positive");
  const uint64_t rows = uint64_t(queries) * splits * heads;
  const uint64_t bytes = rows * (uint64_t(dv) + 1) * sizeof(float);
  if (bytes > PKV_WORKSPACE_LIMIT_BYTES) return fail(PKV_ERANGE, "workspace above PKV_WORKSPACE_LIMIT_BYTES");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  auto *w = new pkv_workspace;
  w->device = dev;
  w->stream = static_cast<hipStream_t>(stream);
  w->queries = queries;
  w->heads = heads;
  w->dv = dv;
  w->splits = splits;
  w->bytes = size_t(bytes);
  if (hipMalloc(&w->buf, w->bytes) != hipSuccess) {
    delete w;
    return fail(PKV_EHIP, "hipMalloc of workspace failed");
  }
  *out = w;
  return PKV_OK;
}

pkv_status pkv_workspace_create_balanced(uint32_t queries, uint32_t heads, uint32_t dv,
                                         void *stream, pkv_workspace **out) {
  clear_error();
  if (!out) return fail(PKV_EINVAL, "out must not be null");
  *out = nullptr;
  if (queries == 0 || heads == 0 || dv == 0) return fail(PKV_EINVAL, "workspace dimensions must be positive");
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return fail(PKV_EHIP, "hipDeviceGetAttribute failed");
  // the most waves a balanced launch uses for any page size or half-precision type
  uint32_t per_cu = 0;
  for (pkv_dtype dt : {PKV_F16, PKV_BF16})
    for (uint32_t ps : {16u, 3u})
      per_cu = std::max<uint32_t>(per_cu, uint32_t(bal_waves_per_cu(dv, ps, dt)));
  per_cu = std::min(per_cu, std::max(kBalancedWavesPerCu, kBalancedWavesPerCuFp8));
  const uint64_t waves = uint64_t(per_cu) * uint32_t(cus);
  // two 16-head slots per decode wave; two 64-head slots per MLA block
  const uint64_t rows = std::max<uint64_t>(2 * waves * 16, 2 * uint64_t(cus) * kMlaBlockHeads);
  const uint64_t bytes = rows * (uint64_t(dv) + 1) * sizeof(float) + (2 * uint64_t(queries) + 1) * 4;
  if (bytes > PKV_WORKSPACE_LIMIT_BYTES) return fail(PKV_ERANGE, "workspace above PKV_WORKSPACE_LIMIT_BYTES");
  auto *w = new pkv_workspace;
  w->device = dev;
  w->stream = static_cast<hipStream_t>(stream);
  w->queries = queries;
  w->heads = heads;
  w->dv = dv;
  w->splits = 0;
  w->max_waves = uint32_t(waves);
  w->cus = uint32_t(cus);
  w->slot_rows = rows;
  w->bytes = size_t(bytes);
  if (hipMalloc(&w->buf, w->bytes) != hipSuccess) {
    delete w;
    return fail(PKV_EHIP, "hipMalloc of workspace failed");
  }
  w->slot_lse = w->buf + rows * dv;
  w->rec = reinterpret_cast<uint32_t *>(w->slot_lse + rows);
  *out = w;
  return PKV_OK;
}

uint32_t pkv_workspace_splits(const pkv_workspace *ws) { return ws ? ws->splits : 0u; }

void pkv_workspace_destroy(pkv_workspace *ws) {
  if (!ws) return;
  if (ws->buf) (void)hipFree(ws->buf);
  delete ws;
}

uint32_t pkv_suggest_splits(const pkv_plan *plan, uint32_t q_heads, uint32_t kv_heads,
                            uint32_t value_dim) {
  if (!plan || plan->L.Q == 0 || plan->L.W == 0) return 1;
  const PlanLayout &L = plan->L;
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, plan->device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // concurrent blocks of the decode kernel for this head size
  RowArgs probe{};
  probe.plan = view_of(plan);
  probe.d = probe.dv = value_dim;
  probe.hq = std::max(1u, q_heads);
  probe.hkv = std::max(1u, kv_heads);
  int per_cu = 2;
  if (value_dim == 64 || value_dim == 128 || value_dim == 256)
    per_cu = rows_mfma_blocks_per_cu(probe, PKV_BF16);
  const double slots = double(cus) * std::max(1, per_cu);
  const uint32_t groups = std::max(1u, kv_heads) *
                          ((std::max(1u, q_heads) / std::max(1u, kv_heads) + 15u) / 16u);

  // visible keys of every query attended one at a time (non-causal bound)
  const uint32_t *w = plan->host.data();
  const bool tiles = L.T > 0;
  const uint32_t nq = tiles ? L.R : L.Q;
  std::vector<uint32_t> len(nq);
  for (uint32_t r = 0; r < nq; ++r) {
    const uint32_t i = tiles ? w[L.rows + r] : r;
    len[r] = w[L.lens + w[L.qseq + i]];
  }

  // Makespan model, in units of "one token row of one KV head": blocks are
  // dispatched in part-major order onto `slots` places and progress at the
  // fair share of the machine's bandwidth, each at most kBoost times that
  // share when the machine is not full; every block costs kOverhead extra;
  // a split adds the merge (its reads and a launch).
  // (one token row = 2 * value_dim half-precision elements; the machine
  // streams ~1.2e4 rows per microsecond, a block's fixed cost is ~2 us at a
  // full machine's fair share and a merge launch ~4 us)
  const double kBoost = 2.0, kOverhead = 64.0, kMergeLaunch = 48000.0;
  const double rate_full = 1.0;  // machine bandwidth, rows per unit time
  const uint32_t cand[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 48, 64, 96, 128, 192, 256};
  uint32_t best_s = 1;
  double best_t = 0.0;
  for (uint32_t s : cand) {
    if (s > L.W || s > PKV_MAX_SPLITS) break;
    const uint64_t per_split = uint64_t(L.Q) * std::max(1u, q_heads) * (uint64_t(value_dim) + 1) * 4;
    if (s > 1 && uint64_t(s) * per_split > PKV_WORKSPACE_LIMIT_BYTES) break;
    const uint64_t pp = L.W / s + (L.W % s != 0);
    const uint64_t span = pp * L.ps;
    // processor sharing with virtual time: every active block advances by
    // the same amount of work per unit of virtual time
    std::vector<double> heap;  // finish points in virtual time (min-heap)
    double now = 0.0, vnow = 0.0;
    uint64_t parts_total = 0;
    auto rate = [&](size_t active) {
      return std::min(kBoost / slots, rate_full / double(active));
    };
    auto advance_one = [&]() {  // finish the earliest block
      std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
      const double v = heap.back();
      now += (v - vnow) / rate(heap.size());
      vnow = v;
      heap.pop_back();
    };
    for (uint32_t part = 0; part < s; ++part) {
      for (uint32_t r = 0; r < nq; ++r) {
        const uint64_t lo = uint64_t(part) * span;
        if (lo >= len[r]) continue;
        const double work = double(std::min<uint64_t>(span, len[r] - lo)) + kOverhead;
        ++parts_total;
        for (uint32_t g = 0; g < groups; ++g) {
          if (heap.size() >= size_t(slots)) advance_one();
          heap.push_back(vnow + work);
          std::push_heap(heap.begin(), heap.end(), std::greater<double>());
        }
      }
    }
    while (!heap.empty()) advance_one();
    double t = now;
    if (s > 1) {
      // merge: read and write every part's rows of every q head (f32, Dv+1
      // words), in units of KV rows of (D + Dv) half-precision elements
      const double merge_rows = double(parts_total) * std::max(1u, q_heads) *
                                (double(value_dim) + 1.0) * 4.0 / (4.0 * value_dim);
      t += merge_rows / rate_full + kMergeLaunch;
    }
    if (best_t == 0.0 || t < best_t * 0.98) {  // prefer fewer parts unless clearly faster
      best_t = t;
      best_s = s;
    }
  }
  return best_s;
}

}  // extern "C"

namespace pkv {
namespace {

pkv_status attention_impl(const pkv_plan *plan, pkv_dtype dtype, bool fp8, const void *q,
                          const void *k, const void *v, void *out, uint32_t hq, uint32_t hkv,
                          uint32_t d, uint32_t dv, float scale, float k_scale, float v_scale,
                          int causal, uint32_t window, pkv_workspace *ws, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!plan) return fail(PKV_EINVAL, "null plan");
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged operands must be F32, F16 or BF16");
  if (hq == 0 || hkv == 0 || hq % hkv != 0 || d == 0 || dv == 0 || d > 1024 || dv > 1024)
    return fail(PKV_ESHAPE, "head counts, head dims or tensor shapes do not fit together");
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PKV_EINVAL, "scale must be finite and positive");
  if (fp8) {
    if (dtype == PKV_F32) return fail(PKV_EINVAL, "an FP8 cache needs F16 or BF16 queries");
    if (d != dv || (d != 64 && d != 128 && d != 256))
      return fail(PKV_ESHAPE, "an FP8 cache needs head_dim == value_dim in {64, 128, 256}");
    if (!std::isfinite(k_scale) || k_scale <= 0.f || !std::isfinite(v_scale) || v_scale <= 0.f)
      return fail(PKV_EINVAL, "FP8 cache scales must be finite and positive");
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
          reinterpret_cast<uintptr_t>(v)) & 15u) != 0)
      return fail(PKV_EINVAL, "an FP8 cache needs 16-byte aligned q, k and v");
  }
  const PlanLayout &L = plan->L;
  if (!u32_elems({L.Q, hq, d}) || !u32_elems({L.Q, hq, dv}) || !cache_fits({L.N, L.ps, hkv, d}) ||
      !cache_fits({L.N, L.ps, hkv, dv}))
    return fail(PKV_ERANGE, "a query or output tensor has more than 2^32 - 1 elements, or a cache 2^63 bytes");
  pkv_status st = check_binding(plan, stream);
  if (st != PKV_OK) return st;
  st = check_workspace(ws, plan, hq, dv, stream);
  if (st != PKV_OK) return st;
  if (L.Q == 0) return PKV_OK;
  const bool have_cache = uint64_t(L.N) * L.ps > 0;
  if (!q || !out || (have_cache && (!k || !v))) return fail(PKV_EINVAL, "null tensor pointer");
  const uint64_t es = elem_size(dtype), ces = fp8 ? 1 : es;  // query / cache element bytes
  const uint64_t out_b = uint64_t(L.Q) * hq * dv * es;
  if (overlaps(out, out_b, q, uint64_t(L.Q) * hq * d * es) ||
      overlaps(out, out_b, k, uint64_t(L.N) * L.ps * hkv * d * ces) ||
      overlaps(out, out_b, v, uint64_t(L.N) * L.ps * hkv * dv * ces))
    return fail(PKV_EINVAL, "output overlaps an input");

  RowArgs ra{};
  ra.plan = view_of(plan);
  ra.hq = hq;
  ra.hkv = hkv;
  ra.d = d;
  ra.dv = dv;
  ra.pdim = 0;
  ra.causal = causal ? 1 : 0;
  ra.window = window;
  ra.scale_log2 = scale * kLog2e * (fp8 ? k_scale : 1.f);
  ra.kv_fp8 = fp8 ? 1u : 0u;
  ra.v_scale = fp8 ? v_scale : 1.f;
  ra.q = q;
  ra.k = k;
  ra.v = v;
  ra.qp = nullptr;
  ra.kp = nullptr;
  ra.k_tok = uint64_t(hkv) * d;
  ra.k_page = ra.k_tok * L.ps;
  ra.v_tok = uint64_t(hkv) * dv;
  ra.v_page = ra.v_tok * L.ps;
  ra.kp_tok = ra.kp_page = 0;
  ra.out = out;
  fill_split(&ra, plan, ws);

  TileArgs ta{};
  ta.plan = ra.plan;
  ta.tiles = plan->dev + L.tiles;
  ta.n_tiles = L.T;
  ta.hq = hq;
  ta.hkv = hkv;
  ta.d = d;
  ta.dv = dv;
  ta.causal = ra.causal;
  ta.window = window;
  ta.scale_log2 = ra.scale_log2;
  ta.kv_fp8 = ra.kv_fp8;
  ta.v_scale = ra.v_scale;
  ta.q = q;
  ta.k = k;
  ta.v = v;
  ta.k_page = ra.k_page;
  ta.k_tok = ra.k_tok;
  ta.v_page = ra.v_page;
  ta.v_tok = ra.v_tok;
  ta.out = out;
  const bool use_tiles = L.T > 0 && tiles_supported(ta, dtype);
  ra.qlist = use_tiles ? plan->dev + L.rows : nullptr;
  ra.n_queries = use_tiles ? L.R : L.Q;

  if (ra.n_queries) {
    st = run_rows(plan, ra, dtype, ws, stream);
    if (st != PKV_OK) return st;
  }
  if (use_tiles) {
    Timed t(plan, PKV_KERNEL_TILES, stream);
    hipError_t e = launch_tiles(ta, dtype, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" {

pkv_status pkv_attention(const pkv_plan *plan, pkv_dtype dtype, const void *q, const void *k,
                         const void *v, void *out, uint32_t hq, uint32_t hkv, uint32_t d,
                         uint32_t dv, float scale, int causal, pkv_workspace *ws, void *stream) {
  clear_error();
  return attention_impl(plan, dtype, false, q, k, v, out, hq, hkv, d, dv, scale, 1.f, 1.f, causal,
                        0u, ws, stream);
}

pkv_status pkv_attention_window(const pkv_plan *plan, pkv_dtype dtype, const void *q,
                                const void *k, const void *v, void *out, uint32_t hq,
                                uint32_t hkv, uint32_t d, uint32_t dv, float scale, int causal,
                                uint32_t window, pkv_workspace *ws, void *stream) {
  clear_error();
  return attention_impl(plan, dtype, false, q, k, v, out, hq, hkv, d, dv, scale, 1.f, 1.f, causal,
                        window, ws, stream);
}

pkv_status pkv_attention_fp8(const pkv_plan *plan, pkv_dtype dtype, const void *q, const void *k,
                             const void *v, void *out, uint32_t hq, uint32_t hkv, uint32_t d,
                             uint32_t dv, float scale, float k_scale, float v_scale, int causal,
                             uint32_t window, pkv_workspace *ws, void *stream) {
  clear_error();
  return attention_impl(plan, dtype, true, q, k, v, out, hq, hkv, d, dv, scale, k_scale, v_scale,
                        causal, window, ws, stream);
}

}  // extern "C"

// Workspace of pkv_attention_noalloc: one array per GPU, in the library's
// device code object (the loader places it; nothing is allocated at call
// time).  Its name is only a host-side stand-in for the device array: host
// code uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char *g_scratch[kMaxDevices] = {};
int g_scratch_cus[kMaxDevices] = {};

// Device address of this device's scratch array and its CU count, resolved
// once per device with that device current; null on failure.
unsigned char *scratch_of(int dev, int *cus) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    int n = 0;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return nullptr;
    g_scratch[dev] = static_cast<unsigned char *>(p);
    g_scratch_cus[dev] = n;
  }
  *cus = g_scratch_cus[dev];
  return g_scratch[dev];
}

}  // namespace
}  // namespace pkv

extern "C" {

pkv_status pkv_attention_noalloc(const pkv_plan *plan, pkv_dtype dtype, const void *q,
                                 const void *k, const void *v, void *out, uint32_t hq,
                                 uint32_t hkv, uint32_t d, uint32_t dv, float scale, int causal,
                                 void *stream) {
  clear_error();
  if (!plan) return fail(PKV_EINVAL, "null plan");
  if (hq == 0 || hkv == 0 || hq % hkv != 0 || d == 0 || dv == 0 || d > 1024 || dv > 1024)
    return fail(PKV_ESHAPE, "head counts, head dims or tensor shapes do not fit together");
  pkv_status st = check_binding(plan, static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  int cus = 0;
  unsigned char *base = scratch_of(plan->device, &cus);
  if (!base) return fail(PKV_EHIP, "resolving the static scratch array failed");
  // layout as a balanced workspace: slot rows of dv f32, their lse, then
  // {first tile, tiles} per query and the total
  const uint64_t rec_bytes = (2ull * plan->L.Q + 1) * 4;
  const uint64_t row_bytes = (uint64_t(dv) + 1) * sizeof(float);
  const uint64_t wave_bytes = 2ull * 16 * row_bytes;  // two 16-head slots per wave
  if (rec_bytes + 4 * wave_bytes > PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERANGE, "too many queries or too large a value dim for the static scratch");
  uint64_t waves = (PKV_NOALLOC_SCRATCH_BYTES - rec_bytes) / wave_bytes;
  uint32_t per_cu = 0;
  for (pkv_dtype dt : {PKV_F16, PKV_BF16})
    for (uint32_t ps : {16u, 3u})
      per_cu = std::max<uint32_t>(per_cu, uint32_t(bal_waves_per_cu(dv, ps, dt)));
  per_cu = std::min(per_cu, kBalancedWavesPerCu);
  waves = std::min<uint64_t>(waves, uint64_t(std::max(per_cu, 1u)) * uint32_t(cus));
  waves -= waves % 4;
  const uint64_t segq = uint64_t(hkv) * ((hq / hkv + 15) / 16);
  if (per_cu && segq > waves)
    return fail(PKV_ERANGE, "the static scratch holds fewer waves than one group of this call");
  pkv_workspace ws;  // a view of the scratch array; owns nothing
  ws.device = plan->device;
  ws.stream = static_cast<hipStream_t>(stream);
  ws.queries = plan->L.Q;
  ws.heads = hq;
  ws.dv = dv;
  ws.splits = 0;
  ws.max_waves = uint32_t(waves);
  ws.cus = uint32_t(cus);
  ws.slot_rows = 2 * waves * 16;
  ws.buf = reinterpret_cast<float *>(base);
  ws.bytes = size_t(ws.slot_rows * row_bytes + rec_bytes);
  ws.slot_lse = ws.buf + ws.slot_rows * dv;
  ws.rec = reinterpret_cast<uint32_t *>(ws.slot_lse + ws.slot_rows);
  return attention_impl(plan, dtype, false, q, k, v, out, hq, hkv, d, dv, scale, 1.f, 1.f, causal,
                        0u, &ws, stream);
}

pkv_status pkv_append(const pkv_plan *plan, pkv_dtype dtype, const void *new_k, const void *new_v,
                      void *k, void *v, void *k_copy, void *v_copy, uint32_t hkv, uint32_t d,
                      uint32_t dv, pkv_append_report *report, void *stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (report) *report = pkv_append_report{0, 0, 0};
  if (!plan) return fail(PKV_EINVAL, "null plan");
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged operands must be F32, F16 or BF16");
  if (hkv == 0 || d == 0 || dv == 0 || d > 1024 || dv > 1024)
    return fail(PKV_ESHAPE, "append needs nonzero head counts and head dims of at most 1024");
  const PlanLayout &L = plan->L;
  if (!u32_elems({L.Q, hkv, d}) || !u32_elems({L.Q, hkv, dv}) || !cache_fits({L.N, L.ps, hkv, d}) ||
      !cache_fits({L.N, L.ps, hkv, dv}))
    return fail(PKV_ERANGE, "a new-row tensor has more than 2^32 - 1 elements, or a cache 2^63 bytes");
  pkv_status st = check_binding(plan, stream);
  if (st != PKV_OK) return st;
  st = validate_writes(plan->host.data(), L);
  if (st != PKV_OK) return st;
  if (L.Q == 0) return PKV_OK;  // a no-op append copies nothing
  if (L.Q > 0x7FFFFFFFu) return fail(PKV_ERANGE, "more than 2^31 - 1 queries to append");
  if (!new_k || !new_v || !k || !v) return fail(PKV_EINVAL, "null tensor pointer");
  const uint64_t es = elem_size(dtype);
  const uint64_t kb = uint64_t(hkv) * d * es, vb = uint64_t(hkv) * dv * es;  // one slot / query
  const uint64_t k_bytes = uint64_t(L.N) * L.ps * kb, v_bytes = uint64_t(L.N) * L.ps * vb;
  const uint64_t nk_bytes = uint64_t(L.Q) * kb, nv_bytes = uint64_t(L.Q) * vb;
  void *kd = k_copy ? k_copy : k, *vd = v_copy ? v_copy : v;
  if (overlaps(kd, k_bytes, vd, v_bytes) || overlaps(k, k_bytes, v, v_bytes))
    return fail(PKV_EINVAL, "K and V caches overlap");
  if ((k_copy && (overlaps(k_copy, k_bytes, k, k_bytes) || overlaps(k_copy, k_bytes, v, v_bytes))) ||
      (v_copy && (overlaps(v_copy, v_bytes, v, v_bytes) || overlaps(v_copy, v_bytes, k, k_bytes))))
    return fail(PKV_EINVAL, "a cache copy overlaps a cache");
  for (const void *src : {new_k, new_v}) {
    const uint64_t sb = src == new_k ? nk_bytes : nv_bytes;
    if (overlaps(src, sb, kd, k_bytes) || overlaps(src, sb, vd, v_bytes))
      return fail(PKV_EINVAL, "new rows overlap a cache they are written to");
  }
  if (overlaps(new_k, nk_bytes, new_v, nv_bytes) && new_k != new_v)
    return fail(PKV_EINVAL, "new K and V rows overlap");

  pkv_append_report rep{0, 0, 0};
  if (k_copy) {
    if (hipMemcpyAsync(k_copy, k, k_bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(PKV_EHIP, "copying the key cache failed");
    rep.key_copied = 1;
    rep.copied_bytes += k_bytes;
  }
  if (v_copy) {
    if (hipMemcpyAsync(v_copy, v, v_bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(PKV_EHIP, "copying the value cache failed");
    rep.value_copied = 1;
    rep.copied_bytes += v_bytes;
  }
  AppendArgs aa{};
  aa.plan = view_of(plan);
  aa.n_queries = L.Q;
  aa.new_k = new_k;
  aa.new_v = new_v;
  aa.k = kd;
  aa.v = vd;
  hipError_t e;
  {
    Timed t(plan, PKV_KERNEL_APPEND, stream);
    e = launch_append(aa, kb, vb, stream);
  }
  if (e != hipSuccess) return hip_fail(e);
  if (report) *report = rep;
  return PKV_OK;
}

pkv_status pkv_mla(const pkv_plan *plan, pkv_dtype dtype, const void *q_abs, const void *q_pos,
                   const void *latent, const void *k_pos, void *out, uint32_t heads, uint32_t rank,
                   uint32_t pos_dim, float scale, int causal, pkv_workspace *ws, void *stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!plan) return fail(PKV_EINVAL, "null plan");
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged operands must be F32, F16 or BF16");
  if (heads == 0 || rank == 0 || rank > 1024)
    return fail(PKV_ESHAPE, "head counts, head dims or tensor shapes do not fit together");
  if (pos_dim == 0 || pos_dim > 256) return fail(PKV_ESHAPE, "position dim must be 1..256 and match between q_pos and k_pos");
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PKV_EINVAL, "scale must be finite and positive");
  const PlanLayout &L = plan->L;
  if (!u32_elems({L.Q, heads, rank}) || !u32_elems({L.Q, heads, pos_dim}) ||
      !cache_fits({L.N, L.ps, 1, rank}) || !cache_fits({L.N, L.ps, 1, pos_dim}))
    return fail(PKV_ERANGE, "a query or output tensor has more than 2^32 - 1 elements, or a cache 2^63 bytes");
  pkv_status st = check_binding(plan, stream);
  if (st != PKV_OK) return st;
  st = check_workspace(ws, plan, heads, rank, stream);
  if (st != PKV_OK) return st;
  if (L.Q == 0) return PKV_OK;
  const bool have_cache = uint64_t(L.N) * L.ps > 0;
  if (!q_abs || !q_pos || !out || (have_cache && (!latent || !k_pos)))
    return fail(PKV_EINVAL, "null tensor pointer");
  const uint64_t es = elem_size(dtype);
  const uint64_t out_b = uint64_t(L.Q) * heads * rank * es;
  if (overlaps(out, out_b, q_abs, uint64_t(L.Q) * heads * rank * es) ||
      overlaps(out, out_b, q_pos, uint64_t(L.Q) * heads * pos_dim * es) ||
      overlaps(out, out_b, latent, uint64_t(L.N) * L.ps * rank * es) ||
      overlaps(out, out_b, k_pos, uint64_t(L.N) * L.ps * pos_dim * es))
    return fail(PKV_EINVAL, "output overlaps an input");

  RowArgs ra{};
  ra.plan = view_of(plan);
  ra.hq = heads;
  ra.hkv = 1;
  ra.d = rank;
  ra.dv = rank;
  ra.pdim = pos_dim;
  ra.v_scale = 1.f;
  ra.causal = causal ? 1 : 0;
  ra.scale_log2 = scale * kLog2e;
  ra.q = q_abs;
  ra.k = latent;
  ra.v = latent;
  ra.qp = q_pos;
  ra.kp = k_pos;
  ra.k_tok = rank;
  ra.k_page = uint64_t(rank) * L.ps;
  ra.v_tok = rank;
  ra.v_page = ra.k_page;
  ra.kp_tok = pos_dim;
  ra.kp_page = uint64_t(pos_dim) * L.ps;
  ra.out = out;
  ra.qlist = nullptr;
  ra.n_queries = L.Q;
  fill_split(&ra, plan, ws);
  return run_rows(plan, ra, dtype, ws, stream);
}

}  // extern "C"

namespace {

// Times `call(ws)` for each candidate split count and returns the fastest;
// fewer splits win unless another count is more than 2% faster.
template <class Call>
pkv_status tune_splits(const pkv_plan *plan, uint32_t heads, uint32_t dv, uint32_t reps,
                       hipStream_t stream, bool try_balanced, Call call, uint32_t *best_out) {
  const PlanLayout &L = plan->L;
  *best_out = 1;
  if (L.Q == 0 || L.W == 0) return PKV_OK;
  reps = std::max(1u, std::min(reps, 100u));
  const uint32_t cand[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
  const uint64_t per_split = uint64_t(L.Q) * heads * (uint64_t(dv) + 1) * sizeof(float);
  uint32_t max_s = 1;
  for (uint32_t c : cand)
    if (c <= L.W && c <= PKV_MAX_SPLITS && uint64_t(c) * per_split <= PKV_WORKSPACE_LIMIT_BYTES) max_s = c;
  pkv_workspace ws;
  ws.device = plan->device;
  ws.stream = stream;
  ws.queries = L.Q;
  ws.heads = heads;
  ws.dv = dv;
  ws.bytes = size_t(uint64_t(max_s) * per_split);
  if (max_s > 1 && hipMalloc(&ws.buf, ws.bytes) != hipSuccess) return fail(PKV_EHIP, "hipMalloc of workspace failed");
  hipEvent_t e0 = nullptr, e1 = nullptr;
  pkv_status st = PKV_OK;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) st = fail(PKV_EHIP, "hipEventCreate failed");
  float best_ms = 0.f;
  for (uint32_t c : cand) {
    if (st != PKV_OK || c > max_s) break;
    ws.splits = c;
    pkv_workspace *w = c > 1 ? &ws : nullptr;
    st = call(w);  // warm-up (and validation)
    if (st != PKV_OK) break;
    if (hipEventRecord(e0, stream) != hipSuccess) { st = fail(PKV_EHIP, "hipEventRecord failed"); break; }
    for (uint32_t r = 0; r < reps && st == PKV_OK; ++r) st = call(w);
    if (st != PKV_OK) break;
    float ms = 0.f;
    if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      st = fail(PKV_EHIP, "timing the candidates failed");
      break;
    }
    if (c == 1 || ms < best_ms * 0.98f) {
      best_ms = ms;
      *best_out = c;
    }
  }
  // the balanced schedule, reported as 0
  pkv_workspace *bw = nullptr;
  if (st == PKV_OK && try_balanced)
    st = pkv_workspace_create_balanced(L.Q, heads, dv, stream, &bw);
  if (st == PKV_OK && bw) {
    t_ran_balanced = false;
    st = call(bw);
    // a call the balanced schedule does not take runs unsplit with this
    // workspace: that candidate was timed already
    const bool applies = t_ran_balanced;
    float ms = 0.f;
    if (st == PKV_OK && applies) {
      if (hipEventRecord(e0, stream) != hipSuccess) st = fail(PKV_EHIP, "hipEventRecord failed");
      for (uint32_t r = 0; r < reps && st == PKV_OK; ++r) st = call(bw);
      if (st == PKV_OK && (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                           hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
        st = fail(PKV_EHIP, "timing the candidates failed");
    }
    // no margin here: the balanced workspace does not grow with the choice,
    // so it wins whenever it measures faster
    if (st == PKV_OK && applies && ms < best_ms) {
      best_ms = ms;
      *best_out = 0;
    }
  }
  if (hipStreamSynchronize(stream) != hipSuccess && st == PKV_OK) st = fail(PKV_EHIP, "hipStreamSynchronize failed");
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (ws.buf) (void)hipFree(ws.buf);
  ws.buf = nullptr;
  pkv_workspace_destroy(bw);
  return st;
}

}  // namespace

extern "C" {

pkv_status pkv_tune_splits(const pkv_plan *plan, pkv_dtype dtype, const void *q, const void *k,
                           const void *v, void *out, uint32_t q_heads, uint32_t kv_heads,
                           uint32_t head_dim, uint32_t value_dim, float scale, int causal,
                           uint32_t reps, void *stream, uint32_t *splits) {
  clear_error();
  if (!plan || !splits) return fail(PKV_EINVAL, "null argument");
  return tune_splits(plan, q_heads, value_dim, reps, static_cast<hipStream_t>(stream), true,
                     [&](pkv_workspace *ws) {
                       return pkv_attention(plan, dtype, q, k, v, out, q_heads, kv_heads, head_dim,
                                            value_dim, scale, causal, ws, stream);
                     },
                     splits);
}

pkv_status pkv_tune_splits_mla(const pkv_plan *plan, pkv_dtype dtype, const void *q_abs,
                               const void *q_pos, const void *latent, const void *k_pos, void *out,
                               uint32_t heads, uint32_t rank, uint32_t pos_dim, float scale,
                               int causal, uint32_t reps, void *stream, uint32_t *splits) {
  clear_error();
  if (!plan || !splits) return fail(PKV_EINVAL, "null argument");
  return tune_splits(plan, heads, rank, reps, static_cast<hipStream_t>(stream), true,
                     [&](pkv_workspace *ws) {
                       return pkv_mla(plan, dtype, q_abs, q_pos, latent, k_pos, out, heads, rank,
                                      pos_dim, scale, causal, ws, stream);
                     },
                     splits);
}

}  // extern "C"
