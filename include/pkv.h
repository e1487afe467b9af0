/*
 * pkv — attention over a paged (block-table) KV cache on MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Every entry point takes plain pointers and sizes; no
 * framework types cross it.  Device buffers are raw device addresses on the
 * current HIP device; `stream` is a hipStream_t passed as `void *` (NULL is
 * the null stream).
 *
 * The operation is the one the ruDNN 0.1.7 `paged_attention` module page
 * states: an immutable, uploaded u32 plan (`DevicePlan::upload`, `HostPlan`),
 * `attention` over packed queries and a paged cache (`DevicePlan::attention`
 * doc), the MLA variant (`DevicePlan::mla` doc), and a reusable split
 * workspace merged through FP32 statistics (`attention_into_split` doc,
 * `SplitWorkspace`).  Kernels read lengths, positions and the block table
 * from the plan's device words, so launches can be captured into a hipGraph
 * and replayed after the words change (boostr 0.1.0 `decode_graph.rs` module
 * doc, sections "Constraints", "Stable-address tensors", "Stream ordering").
 *
 * Errors: every call returns a pkv_status; on failure nothing is launched,
 * no output is written and pkv_last_error() returns a static message for the
 * calling thread (mirroring `PagedAttentionError(&'static str)`).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q/K/V/out (`check_tensor`: F32, F16 or BF16). */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,      /* invalid argument or schedule                        */
  PKV_ESHAPE = 2,      /* shapes disagree (heads, dims, lengths vs table)     */
  PKV_ERANGE = 3,      /* a dimension or element count exceeds u32 indexing  */
  PKV_EDEVICE = 4,     /* plan used on another device or stream              */
  PKV_EWORKSPACE = 5,  /* workspace shape/stream does not match the call     */
  PKV_EHIP = 6         /* a HIP runtime call failed                          */
} pkv_status;

typedef struct pkv_plan pkv_plan;           /* opaque; device words + host copy */
typedef struct pkv_workspace pkv_workspace; /* opaque; f32 split partials      */

/* ------------------------------------------------------------------ plan
 * Plan spec v1: little-endian u32 words (this library's own layout; the page
 * shows a `HostPlan` of u32 words with queries, sequences, table_width,
 * page_size and pages, not the layout).
 *
 *   0       PKV_PLAN_MAGIC
 *   1       PKV_PLAN_VERSION
 *   2..6    Q queries, S sequences, W table width, ps page size, N pages
 *   7       R  row queries (attended one query at a time)
 *   8       T  tiles (runs of consecutive queries of one sequence)
 *   9..15   0
 *   16      lens[S]      tokens in the cache of each sequence
 *   +S      qseq[Q]      sequence of each query
 *   +Q      qpos[Q]      absolute position of each query (< lens[qseq])
 *   +Q      rows[R]      indices of the row queries, ascending
 *   +R      tiles[T][2]  {first query, query count}
 *   +2T     table[S*W]   row-major; entry j of sequence s is the physical
 *                        page of logical token block j when
 *                        j < ceil(lens[s]/ps), else PKV_UNUSED_PAGE
 *
 * Tiles: scanning queries in order, a run is a maximal range of queries of
 * one sequence whose positions increase by one.  Runs of at least
 * PKV_TILE_MIN queries are cut from their first query into tiles of at most
 * PKV_TILE_MAX; queries of shorter runs are rows.  Tiles are listed
 * heaviest first: by decreasing sum of (position + 1) over their queries,
 * ties by increasing first query (kernels start long tiles first).
 *
 * Visible keys of query i: positions 0..qpos[i] when causal (absolute
 * positions, prefill chunks included: `DevicePlan::attention` doc), all
 * lens[qseq[i]] positions otherwise.  Token t of sequence s is slot t % ps of
 * page table[s][t / ps].
 */
#define PKV_PLAN_MAGIC 0x564B5041u
#define PKV_PLAN_VERSION 1u
#define PKV_PLAN_HEADER_WORDS 16u
#define PKV_UNUSED_PAGE 0xFFFFFFFFu
#define PKV_TILE_MIN 8u
#define PKV_TILE_MAX 128u

/* Largest split count of a workspace and largest workspace allocation
 * (`MAX_SPLITS`, `WORKSPACE_LIMIT_BYTES`: names on the page, values ours). */
#define PKV_MAX_SPLITS 256u
#define PKV_WORKSPACE_LIMIT_BYTES (512ull << 20)

/* Validate a schedule and encode its words (host only, no HIP call).
 *   seq_lens[sequences], query_seq[queries], query_pos[queries] (host);
 *   block_table[sequences * table_width] (host, row-major; entries past a
 *   sequence's last used page are ignored).
 *   words: host output of *n_words entries, or NULL to ask for the size.
 *   *n_words: in = capacity, out = words needed (set on success and on
 *   PKV_EINVAL "word buffer too small").
 * Errors: PKV_EINVAL (page_size 0, table_width 0 with sequences, query of a
 * missing sequence, position outside its sequence, used table entry >= pages,
 * small buffer), PKV_ESHAPE (a length above table_width * page_size),
 * PKV_ERANGE (word count or sequences * table_width above u32). */
pkv_status pkv_plan_encode(uint32_t sequences, const uint32_t *seq_lens,
                           uint32_t queries, const uint32_t *query_seq,
                           const uint32_t *query_pos, uint32_t table_width,
                           const uint32_t *block_table, uint32_t page_size,
                           uint32_t pages, uint32_t *words, size_t *n_words);

/* Check that n_words host words are a valid spec-v1 plan (host only). */
pkv_status pkv_plan_validate(const uint32_t *words, size_t n_words);

/* Check the write plan of an append on valid plan words (host only;
 * `validate_writes` on the ruDNN page, shown by name): every query writes
 * the cache slot of its own position, and no two queries may write one
 * physical (page, slot), neither through one (sequence, position) nor
 * through a page two sequences share.  Errors: those of pkv_plan_validate,
 * PKV_EINVAL "two queries write one cache slot". */
pkv_status pkv_plan_validate_writes(const uint32_t *words, size_t n_words);

/* Validate host words, copy them to a new device buffer on `stream` (one
 * H2D copy, `DevicePlan::upload`) and return the plan.  The plan keeps its
 * own host copy, is bound to the current device and to `stream`, and must be
 * used on that stream.  Errors: as pkv_plan_validate, PKV_EHIP. */
pkv_status pkv_plan_create(const uint32_t *words, size_t n_words, void *stream,
                           pkv_plan **out);

/* Replace the plan's words in place, stream-ordered (hipMemcpyAsync on the
 * plan's stream; for a graph replay, call it before hipGraphLaunch on that
 * stream).  The new words must validate and keep header words 2..8 (Q, S, W,
 * ps, N, R, T) unchanged, so every launch grid and captured graph stays
 * valid; lengths, positions, rows, tiles and table entries may change.
 * `words` must stay unchanged until the copy has run (use pinned memory).
 * Not allowed while the plan's stream is being captured (a recorded copy
 * would replay the capture-time words): rebind between replays.
 * Errors: PKV_EINVAL (invalid words, stream under capture), PKV_ESHAPE
 * (header changed), PKV_EDEVICE (other stream/device), PKV_EHIP. */
pkv_status pkv_plan_rebind_async(pkv_plan *plan, const uint32_t *words,
                                 size_t n_words, void *stream);

/* Set one word (index >= 16) with hipMemsetD32Async on the plan's stream:
 * the value travels inside the call, so no host buffer must outlive it
 * (boostr 0.1.0 `DeviceScalars::update` doc).  The plan with the new word
 * must validate (e.g. grow a length only after the table entry of a newly
 * used page is set).  Not allowed while the plan's stream is being
 * captured (a memset node would replay one value): set words between
 * replays.  Errors: PKV_EINVAL (index, invalid plan, stream under capture),
 * PKV_EDEVICE, PKV_EHIP. */
pkv_status pkv_plan_set_word_async(pkv_plan *plan, size_t index, uint32_t value,
                                   void *stream);

/* Copy the plan's 16 header words to `header` (host). */
pkv_status pkv_plan_header(const pkv_plan *plan, uint32_t *header);

/* Device address of the plan words (for callers that rebind from device
 * memory with their own stream-ordered copies). */
const uint32_t *pkv_plan_device_words(const pkv_plan *plan);

/* Free the plan (synchronises the device through hipFree). */
void pkv_plan_destroy(pkv_plan *plan);

/* ------------------------------------------------------------- workspace
 * f32 partials for split-KV: o[queries][splits][heads][dv] followed by
 * lse[queries][splits][heads] (log2-sum-exp2 of the scaled scores).  Split j
 * covers logical pages [j*pp, (j+1)*pp), pp = ceil(W / splits), of each
 * query's block-table row.  Reusable across plans with the same queries,
 * heads, dv and splits on the same stream (`attention_with_workspace` doc);
 * its lifetime is independent of any plan.
 * Errors: PKV_EINVAL (splits outside 1..PKV_MAX_SPLITS, a zero dimension),
 * PKV_ERANGE (above PKV_WORKSPACE_LIMIT_BYTES), PKV_EHIP. */
pkv_status pkv_workspace_create(uint32_t queries, uint32_t heads, uint32_t dv,
                                uint32_t splits, void *stream,
                                pkv_workspace **out);

/* Balanced workspace (this library's schedule; the page's split workspace
 * fixes a part count instead).  pkv_attention with it runs the row queries
 * on the MFMA decode kernel in a balanced schedule: the tile positions (16
 * visible keys) of all row queries, query after query, are cut into equal
 * contiguous ranges, one per group of waves that attend the same keys for
 * the KV heads (and 16-head groups) of the call, so every wave streams the
 * same number of tiles whatever the length mix, and the heads of a page are
 * read side by side.  pkv_mla with it does the same with 32-token tiles and
 * one block per CU as the unit (one range per group of 64-head-group
 * blocks).  The f32 partials of the pieces a range boundary cuts (two slots
 * per unit, one row per head of the unit) are merged by a second kernel.
 * Memory: rows * (dv + 1) f32 + (2 * queries + 1) u32 with rows = max(2 *
 * waves * 16, 2 * CUs * 64), waves = CUs * resident waves per CU of the
 * decode kernel for dv (about 34 MB at dv = 128, 67 MB at dv = 512 on 256
 * CUs).  Calls that the MFMA decode or MLA kernels do not take (f32, head
 * dims other than 64/128/256 or head_dim != value_dim, MLA shapes other
 * than rank 512 with position dim 64, 2^31 or more tile positions, more
 * units per group than the launch has) run unsplit with it.  Same sharing
 * rules as a split workspace: calls that overlap on one workspace race.
 * Errors: PKV_EINVAL (a zero dimension, null out), PKV_ERANGE (above
 * PKV_WORKSPACE_LIMIT_BYTES), PKV_EHIP. */
pkv_status pkv_workspace_create_balanced(uint32_t queries, uint32_t heads,
                                         uint32_t dv, void *stream,
                                         pkv_workspace **out);

/* Split count of a workspace; 0 for a balanced workspace or NULL. */
uint32_t pkv_workspace_splits(const pkv_workspace *ws);
void pkv_workspace_destroy(pkv_workspace *ws);

/* Split count that fills the GPU for a call with these heads over a plan:
 * enough non-empty (query, KV head, part) blocks for several per compute
 * unit, at most PKV_MAX_SPLITS and W, and small enough that the workspace
 * for (plan queries, q_heads, value_dim) stays within
 * PKV_WORKSPACE_LIMIT_BYTES.  A heuristic; any count gives the same result up
 * to rounding.  Returns 1 for a null or empty plan. */
uint32_t pkv_suggest_splits(const pkv_plan *plan, uint32_t q_heads,
                            uint32_t kv_heads, uint32_t value_dim);

/* Measured split choice: runs pkv_attention on the caller's tensors with
 * each candidate split count (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, up
 * to W, PKV_MAX_SPLITS and the workspace limit) `reps` times after one
 * warm-up call, times each candidate with HIP events on `stream`, and
 * writes the fastest count to *splits (a count with more splits must be
 * more than 2% faster to win).  The balanced schedule is the last
 * candidate, reported as 0; it is timed only when the call really runs the
 * balanced kernels (a shape they do not take runs unsplit, which was timed
 * already), and wins when it measures faster than the best count before it
 * (its workspace does not grow with the choice).  Uses
 * temporary workspaces of its own;
 * `out` receives the attention result.  Synchronises the stream; not for
 * use under graph capture.  Errors: those of pkv_attention, PKV_EINVAL for
 * a null plan or splits, PKV_EHIP. */
pkv_status pkv_tune_splits(const pkv_plan *plan, pkv_dtype dtype, const void *q,
                           const void *k, const void *v, void *out,
                           uint32_t q_heads, uint32_t kv_heads, uint32_t head_dim,
                           uint32_t value_dim, float scale, int causal,
                           uint32_t reps, void *stream, uint32_t *splits);

/* The same for pkv_mla (split counts, then the balanced schedule as 0). */
pkv_status pkv_tune_splits_mla(const pkv_plan *plan, pkv_dtype dtype,
                               const void *q_abs, const void *q_pos,
                               const void *latent, const void *k_pos, void *out,
                               uint32_t heads, uint32_t rank, uint32_t pos_dim,
                               float scale, int causal, uint32_t reps,
                               void *stream, uint32_t *splits);

/* ------------------------------------------------------------- attention
 * out[i,h,:] = softmax_t(scale * <q[i,h,:], k_t>) . v_t over the visible
 * keys t of query i, with k_t = k[table[s][t/ps], t%ps, g, :] and
 * g = h / (q_heads / kv_heads) (contiguous GQA groups; no KV repeat).
 *   q   [Q, q_heads, head_dim]               device, dtype
 *   k   [N, ps, kv_heads, head_dim]          device, dtype
 *   v   [N, ps, kv_heads, value_dim]         device, dtype
 *   out [Q, q_heads, value_dim]              device, dtype; must not overlap
 *                                            q, k or v
 * Accumulation is f32.  ws == NULL: unsplit.  Otherwise each query's
 * visible range is split over pkv_workspace_splits(ws) parts whose f32
 * partials are merged on the device, with no host synchronisation.
 * Q == 0 returns PKV_OK with no launch.
 * Errors: PKV_EINVAL (null pointer, bad dtype, scale not finite and > 0,
 * out overlapping an input), PKV_ESHAPE (q_heads % kv_heads, head_dim or
 * value_dim outside 1..1024), PKV_ERANGE (q or out above u32 elements,
 * or a cache above 2^63 bytes: caches are addressed with 64-bit offsets),
 * PKV_EDEVICE, PKV_EWORKSPACE (ws built for other queries/heads/dv/stream),
 * PKV_EHIP (launch failure). */
pkv_status pkv_attention(const pkv_plan *plan, pkv_dtype dtype, const void *q,
                         const void *k, const void *v, void *out,
                         uint32_t q_heads, uint32_t kv_heads, uint32_t head_dim,
                         uint32_t value_dim, float scale, int causal,
                         pkv_workspace *ws, void *stream);

/* Attention with a sliding window (the `window` field of the libmir-cuda
 * decode-attention geometry; the page shows the field, not its use): query
 * i sees only the last `window` of its visible keys, positions
 * [max(0, n - window), n) with n as in pkv_attention; window 0 is
 * pkv_attention.  Decode rows run on the row kernels (split, balanced or
 * unsplit), chunk queries on the chunked-prefill tile kernel, which starts
 * each block at its first query's window and reads nothing before it.
 * Arguments and errors as pkv_attention. */
pkv_status pkv_attention_window(const pkv_plan *plan, pkv_dtype dtype,
                                const void *q, const void *k, const void *v,
                                void *out, uint32_t q_heads, uint32_t kv_heads,
                                uint32_t head_dim, uint32_t value_dim,
                                float scale, int causal, uint32_t window,
                                pkv_workspace *ws, void *stream);

/* Attention over an 8-bit KV cache (the libmir-cuda graph page keeps K and
 * V as byte buffers, `DeviceBuffer<u8>`, next to bf16 queries and outputs;
 * the encoding is not shown).  Each cache element is one OCP FP8 E4M3 byte
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinity, S.1111.111 = NaN), scaled by one f32 per cache:
 *   key = e4m3(k byte) * k_scale, value = e4m3(v byte) * v_scale
 * and the result is that of pkv_attention_window on those keys and values.
 *   q [Q, q_heads, head_dim] and out [Q, q_heads, value_dim]: F16 or BF16
 *   k [N, ps, kv_heads, head_dim], v [N, ps, kv_heads, value_dim]: bytes
 * head_dim == value_dim in {64, 128, 256}; q, k, v 16-byte aligned.  Decode
 * rows run on the decode MFMA kernels (split, balanced or unsplit) and, for
 * head dims 64 and 128, chunk queries on the chunked-prefill tile kernel;
 * both widen the bytes exactly to the query type on their way into LDS (at
 * head dim 256 chunk queries run as rows).  Errors: as
 * pkv_attention; PKV_EINVAL for F32 queries, scales not finite and > 0 or
 * misaligned tensors; PKV_ESHAPE for other head dims. */
pkv_status pkv_attention_fp8(const pkv_plan *plan, pkv_dtype dtype,
                             const void *q, const void *k, const void *v,
                             void *out, uint32_t q_heads, uint32_t kv_heads,
                             uint32_t head_dim, uint32_t value_dim, float scale,
                             float k_scale, float v_scale, int causal,
                             uint32_t window, pkv_workspace *ws, void *stream);

/* ------------------------------------------------------------- no-alloc
 * For callers that cannot allocate device memory at call time (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * pkv_attention with a balanced workspace, except that the workspace is a
 * static device array of PKV_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller still owns
 * q, k, v and out, laid out as for pkv_attention.  Resolving the array's
 * address happens on the first call on a device (hipGetSymbolAddress).
 * The array holds the balanced schedule's slot rows (2 x 16 rows of
 * value_dim + 1 f32 per wave) after the per-query records ((2 Q + 1) u32);
 * the wave count is capped by what fits (1024 waves at value_dim 128 on 256
 * CUs, the same launch as a balanced workspace).  Nothing in it needs to
 * start at zero; every call on one GPU shares that GPU's array and keeps
 * the last call's contents, so calls that overlap on one GPU (two streams,
 * two threads) race.  Shapes the balanced kernels do not take run unsplit,
 * using no scratch.
 * Errors: as pkv_attention; PKV_ERANGE when the queries' records and four
 * waves' slots exceed the array, or when fewer waves fit than one group of
 * the call (KV heads x ceil(G / 16)); PKV_EHIP when the array's address
 * cannot be resolved. */
#define PKV_NOALLOC_SCRATCH_BYTES (32ull << 20)

pkv_status pkv_attention_noalloc(const pkv_plan *plan, pkv_dtype dtype,
                                 const void *q, const void *k, const void *v,
                                 void *out, uint32_t q_heads, uint32_t kv_heads,
                                 uint32_t head_dim, uint32_t value_dim,
                                 float scale, int causal, void *stream);

/* MLA (`DevicePlan::mla` doc): one shared latent head is both key and value;
 * a position part only adds to the score:
 *   x_t = scale * (<q_abs[i,h,:], latent_t> + <q_pos[i,h,:], k_pos_t>)
 *   out[i,h,:] = softmax_t(x) . latent_t                 -> [Q, heads, rank]
 *   q_abs  [Q, heads, rank]      q_pos [Q, heads, pos_dim]
 *   latent [N, ps, 1, rank]      k_pos [N, ps, 1, pos_dim]
 * `scale` comes from the model's QK dimensions, not from rank.  Workspace:
 * none (one pass per query), split (parts merged by log-sum-exp) or
 * balanced (equal ranges of 32-token tiles per group of 64-head blocks, for
 * F16/BF16 with rank 512 and pos_dim 64; other shapes run unsplit with it).
 * Errors: as pkv_attention; PKV_ESHAPE for rank outside 1..1024 or pos_dim
 * outside 1..256. */
pkv_status pkv_mla(const pkv_plan *plan, pkv_dtype dtype, const void *q_abs,
                   const void *q_pos, const void *latent, const void *k_pos,
                   void *out, uint32_t heads, uint32_t rank, uint32_t pos_dim,
                   float scale, int causal, pkv_workspace *ws, void *stream);

/* ------------------------------------------------------------- append
 * Cache append (ruDNN `DevicePlan::append`, `append_with_report`,
 * `CacheAppendReport`): query i stores new_k[i] and new_v[i] (all KV heads)
 * at slot qpos[i] % ps of page table[qseq[i]][qpos[i] / ps] of the caches.
 *   new_k [Q, kv_heads, head_dim], new_v [Q, kv_heads, value_dim]  device
 *   k [N, ps, kv_heads, head_dim], v [N, ps, kv_heads, value_dim]  device
 * k_copy / v_copy: NULL to append in place; otherwise a buffer of the
 * cache's size into which the cache is copied first (device to device, on
 * `stream`) and the append then goes, leaving k / v unchanged (the page's
 * copy-on-write for a cache that is not uniquely owned; which caches are
 * shared is the caller's knowledge here).  report (may be NULL): which
 * caches were copied and the bytes copied.  Q == 0 launches and copies
 * nothing (report all zero).  The write plan is checked on the plan's host
 * words at call time (pkv_plan_validate_writes) before anything is
 * launched.  Captured into a graph, the copies and the append replay with
 * the plan words of replay time; the check ran at capture time.
 * Errors: PKV_EINVAL (null pointer, bad dtype, a conflicting write plan,
 * new rows, caches or copies overlapping each other, K and V caches
 * overlapping), PKV_ESHAPE (a zero head count or dim, a dim above 1024),
 * PKV_ERANGE (a new-row tensor above u32 elements, or a cache above 2^63
 * bytes), PKV_EDEVICE, PKV_EHIP. */
typedef struct {
  uint32_t key_copied;    /* the key cache was copied before the append   */
  uint32_t value_copied;  /* the value cache was copied before the append */
  uint64_t copied_bytes;  /* bytes of the copied caches                    */
} pkv_append_report;

pkv_status pkv_append(const pkv_plan *plan, pkv_dtype dtype, const void *new_k,
                      const void *new_v, void *k, void *v, void *k_copy,
                      void *v_copy, uint32_t kv_heads, uint32_t head_dim,
                      uint32_t value_dim, pkv_append_report *report,
                      void *stream);

/* ------------------------------------------------------------- timing
 * Per-kernel timing, for benchmarks.  While enabled on a plan, every
 * pkv_attention / pkv_mla / pkv_append call with that plan has each kernel
 * it launches record a pair of HIP events at the kernel's own start and end
 * (hipExtLaunchKernel's event arguments: the timestamps belong to the
 * dispatch, on the call's stream, and add no packets between kernels).
 * Kernels: the per-query row kernel (decode rows, split parts, balanced
 * ranges), the chunked-prefill tile kernel, the MLA kernel, the merges
 * (split and balanced), and the cache append.  Enabling clears earlier
 * records.  Calls on a stream that is being captured into a graph are not
 * timed.  Errors: PKV_EINVAL (null plan, unknown kernel, null output),
 * PKV_EHIP (event creation or query failure). */
typedef enum {
  PKV_KERNEL_ROWS = 0,
  PKV_KERNEL_TILES = 1,
  PKV_KERNEL_MLA = 2,
  PKV_KERNEL_MERGE = 3,
  PKV_KERNEL_APPEND = 4
} pkv_kernel;

pkv_status pkv_plan_timing(pkv_plan *plan, int enable);

/* Timing limited to the kernels whose bit (1u << pkv_kernel) is set in
 * kernel_mask; 0 turns timing off, and pkv_plan_timing(plan, 1) is the mask
 * of every kernel.  A timed launch costs a few microseconds of dispatch
 * overhead, so a benchmark times only the kernel it reports.  Enabling
 * clears earlier records.  Errors: PKV_EINVAL (null plan, bits beyond
 * PKV_KERNEL_APPEND). */
pkv_status pkv_plan_timing_select(pkv_plan *plan, uint32_t kernel_mask);

/* Number of recorded launches of `kernel` and their summed duration in
 * milliseconds (waits for the recorded events to complete). */
pkv_status pkv_plan_timing_read(pkv_plan *plan, pkv_kernel kernel,
                                uint32_t *launches, double *total_ms);

/* Static message of the calling thread's last error ("" if none). */
const char *pkv_last_error(void);

/* Library version string. */
const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
