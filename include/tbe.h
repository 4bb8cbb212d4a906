/*
 * tbe.h -- C ABI of libtbe_hip.so, the MI355X (gfx950) Table Batched
 * Embedding hot path.
 *
 * What the library computes (FBTriton TBE page, "Modernizing Table Batched
 * Embeddings with FBTriton", sections "Why redesign a sparse operator?",
 * "Forward", "Backward", "Fewer reads and synchronizations", "Fusion
 * boundaries"; HugeCTR DistributedSlotSparseEmbeddingHash backward
 * walkthrough, steps 1 to 5):
 *
 *   forward   out[b, c_t + d] = (1/L if mean) * sum_{p in bag(t,b)} S[p] * W_t[I[p], d]
 *   backward  per touched row r of table t, once:
 *             g[d] = sum over the row's lookups of S[p] * grad_out[b(p), c_t + d] * (1/L if mean)
 *             M_t[r] += (sum_d g[d]^2) / D_t
 *             W_t[r, d] -= lr * g[d] / (sqrt(M_t[r]) + eps)        (exact row-wise Adagrad)
 *
 * Conventions shared by every entry point
 *  - T tables; table t has R_t rows of width D_t (4 <= D_t <= 1024, D_t % 4 == 0),
 *    sum or mean pooling, weights W_t (device, R_t x D_t row-major, 16-byte
 *    aligned, one storage type for all tables) and row-wise momentum M_t
 *    (device, R_t floats).
 *  - B bags per table, table-major: bag j = t*B + b.  offsets (device, T*B+1
 *    entries, the index type) are CSR: bag j holds lookups
 *    [offsets[j], offsets[j+1]); offsets[0] = 0, non-decreasing,
 *    offsets[T*B] = num_lookups.  indices (device, num_lookups entries) are
 *    rows of the bag's table.  Empty bags pool to 0.
 *  - out and grad_out are [B, Dtot] float32 row-major (device, 16-byte
 *    aligned); table t occupies columns [c_t, c_t + D_t), c_t = sum of the
 *    earlier D.
 *  - per_sample_weights (device float32, num_lookups entries) is optional
 *    (NULL = all ones); each contribution is scaled before grouping by row.
 *  - Index type: TBE_I32 or TBE_I64 for both indices and offsets.  int32 is
 *    accepted only while num_lookups < 2^31 and sum_t R_t < 2^31 (the
 *    linearized row range, FBTriton page, "Forward").
 *  - stream is a hipStream_t (as void*); every entry point except plan
 *    creation only enqueues work on it: no allocation, no host
 *    synchronization, no device-to-host copy.  Counts that only the device
 *    knows (runs, long runs, chunks) stay in the workspace (FBTriton page,
 *    "Fewer reads and synchronizations").
 *  - Ownership: the caller owns every device buffer (weights, momentum,
 *    indices, offsets, per-sample weights, out, grad_out, workspace).  The
 *    plan owns only its small metadata, two side streams and three events
 *    of its own.  A plan is immutable after creation and may be shared by
 *    calls on several streams; a workspace serves one call sequence at a
 *    time.
 *  - Errors: every function returns TBE_OK or a negative code, detected on
 *    the host before anything is enqueued (except TBE_E_HIP, reported from
 *    the launch).  Nothing is printed.  Input contract violations on the
 *    device (offsets not monotone, an index outside [0, R_t)) are not checked
 *    (bounds checks are off by default on the pages) and give undefined
 *    results.
 */
#ifndef TBE_H
#define TBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TBE_OK 0
#define TBE_E_ARG (-1)          /* null / misaligned pointer, negative size, bad enum */
#define TBE_E_UNSUPPORTED (-2)  /* D limits, table count, histogram forced on an ineligible shape */
#define TBE_E_WORKSPACE (-3)    /* workspace too small or not 256-byte aligned */
#define TBE_E_RANGE (-4)        /* int32 indices with num_lookups or sum R_t >= 2^31; sizes >= 2^32 */
#define TBE_E_HIP (-5)          /* the HIP runtime reported an error */
#define TBE_E_ALLOC (-6)        /* plan creation could not allocate */
#define TBE_E_TOO_LARGE (-7)    /* batch too large for the library's static workspace */

/* weight storage types */
#define TBE_F32 0
#define TBE_F16 1
#define TBE_BF16 2
/* index and offset types */
#define TBE_I32 0
#define TBE_I64 1
/* pooling */
#define TBE_SUM 0
#define TBE_MEAN 1

/* tbe_forward flags */
#define TBE_FWD_NO_HIST 0x1u       /* never take the small-table histogram path */
#define TBE_FWD_REQUIRE_HIST 0x2u  /* fail with TBE_E_UNSUPPORTED unless the histogram path applies */
#define TBE_FWD_BALANCE 0x4u       /* generic path: split bag groups into equal pieces (default) */
#define TBE_FWD_NO_BALANCE 0x8u    /* generic path: one whole bag per lane subgroup */
#define TBE_FWD_SAVE_HIST 0x10u    /* tbe_forward_preprocess only: keep the histogram path's row
                                      counts for TBE_BWD_HIST (see there) */
/* tbe_backward_rowwise_adagrad flags */
#define TBE_BWD_PREPROCESSED 0x1u  /* the workspace already holds tbe_preprocess of these inputs */
#define TBE_BWD_FUSED_LONG 0x2u    /* long runs: partials + countdown, last chunk updates (no second launch) */
#define TBE_BWD_CONCURRENT 0x4u    /* run classes on three streams (fork from and join into `stream`) */
#define TBE_BWD_ORDER_CHUNKS 0x8u  /* always walk each table's chunks in bag order (see below) */
#define TBE_BWD_NO_ORDER_CHUNKS 0x10u /* never: walk chunks in list order */
#define TBE_BWD_HIST 0x20u       /* histogram-reuse backward (one small table; see below) */
#define TBE_BWD_CONCURRENT_AUTO 0x40u /* TBE_BWD_CONCURRENT for batches under 64 Mi lookups only */

typedef struct tbe_plan tbe_plan;

/* Byte offsets, inside a workspace, of the preprocessing results (for tests
 * and tools; the layout depends only on the plan, B and num_lookups).
 * Linear row keys are uint32: key = key_base[t] + row, with tables ordered by
 * D bucket, then by table id (tbe_plan_key_bases).  Positions and bag ids are
 * uint32. */
typedef struct {
  size_t sorted_key;   /* num_lookups keys, ascending */
  size_t sorted_bag;   /* num_lookups bag ids j of the sorted lookups; the sort is stable,
                          so equal keys keep lookup-position order */
  size_t sorted_scale; /* num_lookups float S[p]*(1/L if mean) of the sorted lookups; written
                          only with per-sample weights or a mean table */
  size_t run_start;    /* U+1 entries: first sorted slot of each run, then num_lookups */
  size_t run_key;      /* U keys, one per run */
  size_t single_task;  /* n_single uint32x4 {start, row, table, bag}: runs with SL = 1 */
  size_t tiny_task;    /* n_tiny uint32x4 {start, len, row, table}: short runs, 2 <= SL < 32 */
  size_t medium_task;  /* n_medium uint32x4 {start, len, row, table}: short runs, 32 <= SL < 256 */
  size_t long_task;    /* n_long uint32x4 {start, len, row, table}: runs with SL >= 256 */
  size_t long_cbeg;    /* n_long first chunk index of each long run */
  size_t chunk_task;   /* n_chunks uint32x4 {start, len, table, long index}: 256-lookup chunks */
  size_t chunk_perm;   /* n_chunks uint32: chunk list position taken at each walk position when
                          the backward walks chunks in bag order (written by the backward) */
  size_t counters;     /* uint32 {U, n_single, n_tiny, n_medium, n_long, n_chunks, then for
                          each of the five lists its nb+1 per-D-bucket begins} */
  size_t prep_error;   /* uint32, 0 after a good preprocessing; nonzero if a cross-workgroup
                          wait of the scans gave up after its poll limit (results invalid;
                          the backward then writes nothing) */
  size_t hist_counts;  /* B x E uint16 row counts per bag saved by the histogram forward
                          (TBE_FWD_SAVE_HIST; plans with one table of <= 64 rows) */
  /* The hot-row contraction's lists (zero bytes when no table of the plan can
   * take it; written only by a backward that takes it): */
  size_t long_flag;    /* n_long uint32: 1 for a long run that the contraction updated (its
                          chunks are skipped), else 0 */
  size_t dense_rows;   /* T x 128 uint32x4 {start, len, row, long index}: each table's hot rows,
                          the first dense_count[t] entries valid */
  size_t dense_count;  /* T uint32: hot rows per table */
  size_t total;        /* bytes needed */
  int32_t num_buckets; /* nb */
} tbe_ws_views;

/* Create a plan over T tables (host arrays of length T; weights[t] and
 * momentum[t] are device pointers).  Tables are bucketed by next_pow2(D_t)
 * (FBTriton page, "Fewer reads and synchronizations").  The only entry point
 * that allocates (a few KB of device metadata, two default-priority side
 * streams and three events for the backward) and synchronizes.
 * Errors: TBE_E_ARG, TBE_E_UNSUPPORTED (T > 4096, D outside [4, 1024] or not
 * a multiple of 4, R_t < 1), TBE_E_RANGE (sum R_t >= 2^32), TBE_E_ALLOC. */
int tbe_plan_create(tbe_plan** out, int32_t T, const int64_t* rows, const int32_t* dims,
                    const int32_t* pooling, int32_t wdtype, void* const* weights,
                    float* const* momentum);

/* Free the plan's metadata; never touches caller buffers.  NULL is a no-op. */
int tbe_plan_destroy(tbe_plan* plan);

/* Host copy of the linear key base of each table (T entries). */
int tbe_plan_key_bases(const tbe_plan* plan, int64_t* key_base);

/* Bytes of workspace needed for B bags per table and num_lookups lookups
 * (FBTriton page, "Fewer reads and synchronizations": the preprocessing's
 * outputs and counts live in preallocated device memory, so no count is read
 * back to size them; HugeCTR walkthrough, step 3: the sort's temporary
 * storage is sized by a query before the call).  The bound uses only
 * host-known sizes (runs <= N, chunks <= N/256 + long runs).  Errors:
 * TBE_E_ARG, TBE_E_RANGE (num_lookups >= 2^31 - 1). */
int tbe_workspace_size(const tbe_plan* plan, int64_t B, int64_t num_lookups, size_t* bytes);

/* Offsets of the preprocessing results inside such a workspace: the sorted
 * lookups, run starts and keys, and the task lists and their device-resident
 * counts (FBTriton page, "Backward" and "Fewer reads and synchronizations";
 * HugeCTR walkthrough, steps 3 and 4).  Host-side; errors as
 * tbe_workspace_size. */
int tbe_workspace_views(const tbe_plan* plan, int64_t B, int64_t num_lookups,
                        tbe_ws_views* out);

/* Forward pooling (FBTriton page, "Forward"; HugeCTR forward_sum / mean).
 * Writes every element of out[B, Dtot].  Accumulates in float32 for 16-bit
 * weights and in float64 for float32 weights.  A single table with at most
 * 64 rows, 64 <= D <= 128, float16 weights, no per-sample weights and an
 * average bag length >= 64 takes the histogram path (row counts of 16 bags
 * times the table on the matrix cores) unless TBE_FWD_NO_HIST is set.
 * The generic path gives each wave a group of consecutive bags and splits
 * their lookups into equal pieces, one per lane subgroup (a bag cut by the
 * pieces is summed per piece and the parts are added in piece order), or,
 * with TBE_FWD_NO_BALANCE, gives each lane subgroup one bag, summed in
 * lookup order.  TBE_FWD_BALANCE asks for the first explicitly (the default).
 * Both are deterministic (the order of every sum follows from the offsets),
 * and they differ only in the rounding of bags that the pieces cut. */
int tbe_forward(const tbe_plan* plan, int64_t B, int32_t itype, const void* indices,
                const void* offsets, int64_t num_lookups, const float* per_sample_weights,
                float* out, uint32_t flags, void* stream);

/* Forward with fused input checks (FBTriton page, "Forward": bounds checks
 * fused into the forward configurations that can take them, off by default;
 * tbe_validate is the separate pass).  The generic forward (never the
 * histogram path) with every offset and index checked as it is read:
 * offsets are clamped into [0, num_lookups] and, within each wave's group of
 * consecutive bags, made non-decreasing; a lookup whose index lies outside
 * [0, R_t) (an int64 index by its full 64-bit value) reads no row and
 * contributes nothing, while its bag keeps its length for mean pooling.  No
 * access then leaves the inputs and outputs, whatever they hold.  err:
 * device, TBE_VALIDATE_WORDS uint32 with tbe_validate's layout, overwritten
 * (cleared by the call): [0] the TBE_INVALID_* bits found, [1] lookups
 * skipped for an index out of range (each lookup a bag reads; with valid
 * offsets, every bad position once), [2] first bag with a finding, [3] first
 * bad position.  Valid inputs give tbe_forward's output bit for bit (same
 * kernels and sum order) and an error block with no finding.  With offsets
 * out of order, the bags next to them get unspecified but finite sums.
 * Arguments and errors as tbe_forward (TBE_FWD_REQUIRE_HIST:
 * TBE_E_UNSUPPORTED); TBE_E_ARG for a null or misaligned err. */
int tbe_forward_checked(const tbe_plan* plan, int64_t B, int32_t itype, const void* indices,
                        const void* offsets, int64_t num_lookups,
                        const float* per_sample_weights, float* out, uint32_t flags,
                        uint32_t* err, void* stream);

/* Forward and backward preprocessing of the same lookups in one call
 * (FBTriton page, "Backward": the preprocessing can move into the forward).
 * The forward runs on `stream` exactly as tbe_forward; the preprocessing of
 * tbe_preprocess is launched at the same time on one of the plan's side
 * streams (default priority), forked from `stream` before the forward, and
 * `stream` waits for it before any later work.  A tbe_backward(...,
 * TBE_BWD_PREPROCESSED) on `stream` then uses the workspace.  Arguments,
 * ownership and errors as tbe_forward and tbe_preprocess (ws: device, >=
 * tbe_workspace_size bytes, 256-byte aligned).  Calls on one plan are
 * serialized on the host (the fork and join events are the plan's). */
/* TBE_FWD_SAVE_HIST (FBTriton page, "Fusion boundaries": the small-table
 * path saves its histogram in the forward for the backward, which reuses it
 * without fusing the two): for a plan and batch that take the histogram
 * forward and that TBE_BWD_HIST serves (one table of at most 64 rows, D a
 * multiple of 16 from 64 to 128, float16, no per-sample weights, average bag
 * length >= 64; else TBE_E_UNSUPPORTED), the forward also writes every
 * bag's exact row counts (uint16) into ws, and no run preprocessing is
 * launched; a later tbe_backward_rowwise_adagrad(..., TBE_BWD_HIST |
 * TBE_BWD_PREPROCESSED) on the same lookups reads those counts instead of
 * the indices (same bits as without them). */
int tbe_forward_preprocess(const tbe_plan* plan, int64_t B, int32_t itype, const void* indices,
                           const void* offsets, int64_t num_lookups,
                           const float* per_sample_weights, float* out, uint32_t flags, void* ws,
                           size_t ws_bytes, void* stream);

/* Backward preprocessing only (FBTriton page, "Backward": transposition,
 * sort, run-length encoding; classification of runs at SL 256 and task-list
 * compaction with device-resident counts).  Fills the workspace for a later
 * tbe_backward_rowwise_adagrad(..., TBE_BWD_PREPROCESSED) with the same
 * indices, offsets and per-sample weights, in stream order (the contribution
 * scale S[p]*(1/L if mean) is folded in here).  ws: device,
 * >= tbe_workspace_size bytes, 256-byte aligned. */
int tbe_preprocess(const tbe_plan* plan, int64_t B, int32_t itype, const void* indices,
                   const void* offsets, int64_t num_lookups, const float* per_sample_weights,
                   void* ws, size_t ws_bytes, void* stream);

/* Backward with exact row-wise Adagrad applied once per touched row.
 * Preprocesses unless TBE_BWD_PREPROCESSED, then updates each run with
 * SL < 256 in one owning program (a lane subgroup below SL 32, a workgroup
 * from 32 to 255) and runs with SL >= 256 through 256-lookup chunk partial
 * sums plus an update pass (or, with TBE_BWD_FUSED_LONG, each chunk writes
 * its partial with device-coherent write-through atomic stores and counts down
 * the run's remaining chunks, so that the last chunk of a run updates it; no
 * whole-cache fence is used; both give bit-identical weights).  Weights and
 * momentum of touched rows are updated in place;
 * untouched rows are not written.  debug_row_updates (device, nullable): one
 * uint32 per linear key, incremented once per row update.
 * If a cross-workgroup wait of the preprocessing gave up (the workspace's
 * prep_error word is nonzero: a wait exceeded its poll limit, which a
 * correctly working device does not reach), its lists may be spoiled, and
 * every backward kernel returns before writing anything: weights, momentum
 * and debug counters keep their contents, and the caller can read
 * prep_error to learn that the step was skipped.
 * By default every kernel runs on `stream`, one after another.  The run
 * classes own disjoint rows, so with TBE_BWD_CONCURRENT the call forks from
 * `stream` onto the plan's two side streams (medium runs on one, chunks and
 * long-run updates on the other, the rest on `stream`) and joins them back
 * into `stream` before it returns: work enqueued later on `stream` sees
 * every update, and the results are bit-identical to the one-stream order.
 * Calls that share a plan enqueue this fork and join one at a time (a
 * host-side lock).  TBE_BWD_CONCURRENT_AUTO forks only when the batch has
 * fewer than 64 Mi lookups: measured on MI355X, the concurrent classes cut
 * the backward of 2.1 M and 17 M lookup batches by 2% and 5% of the step,
 * but slow a 138 M lookup batch by 15% (the classes compete for the
 * last-level cache).
 * Chunk walk order: the chunks of a table that one XCD takes read about one
 * eighth of the table's grad_out rows; walking them by the bag of their first
 * lookup keeps the rows in use within that XCD's L2.  This is done when
 * grad_out (B x sum D x 4 bytes) exceeds 256 MiB, or always with
 * TBE_BWD_ORDER_CHUNKS, never with TBE_BWD_NO_ORDER_CHUNKS (both: TBE_E_ARG); the order changes
 * no result bit.
 * TBE_BWD_HIST: for a plan with one table of at most 64 rows and D a
 * multiple of 16 up to 128 (else TBE_E_UNSUPPORTED), the weight gradient is
 * computed as one contraction over the bags, grad[e][d] = sum_j C[j][e] *
 * grad_out[j][d] with C the per-bag sums of S[p] * (1/L if mean) of row e's
 * lookups, on the matrix cores (fp32 inputs), then row-wise Adagrad on the
 * rows with a lookup; no run preprocessing (the workspace's run results are
 * neither used nor written).  With TBE_BWD_PREPROCESSED as well, the row
 * counts that tbe_forward_preprocess(..., TBE_FWD_SAVE_HIST) saved in the
 * workspace for this batch (B and num_lookups recorded beside them) replace
 * the indices, for every block of 128 bags whose bags have fewer than 65536
 * lookups; counts saved for another batch are ignored.  Without per-sample
 * weights a coefficient is formed as a float32 count times (1/L if mean) in
 * either case, so the results are bit-identical.  Sums run in another order
 * than the run pipeline's, so the two agree within rounding, not bit for
 * bit. */
int tbe_backward_rowwise_adagrad(const tbe_plan* plan, int64_t B, int32_t itype,
                                 const void* indices, const void* offsets, int64_t num_lookups,
                                 const float* per_sample_weights, const float* grad_out, float lr,
                                 float eps, void* ws, size_t ws_bytes, uint32_t flags,
                                 uint32_t* debug_row_updates, void* stream);

/* tbe_backward_rowwise_adagrad for callers that cannot allocate device
 * memory or hand in a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same preprocessing and
 * kernels, with the workspace in a static device array of the library
 * (TBE_STATIC_WS_BYTES per device, held from the first plan created on the
 * device until the process ends).  The call allocates nothing and calls no
 * allocating routine; the caller still passes every input and output.
 * Arguments as tbe_backward_rowwise_adagrad without ws and ws_bytes; the
 * current device must be the plan's.  Every call on a device shares that
 * device's array and leaves its contents behind (the kernels set up all they
 * read), so calls that overlap on one device (other streams, other plans,
 * other threads) race and must not be issued.  Errors: those of
 * tbe_backward_rowwise_adagrad; TBE_E_ARG with TBE_BWD_PREPROCESSED (no
 * preprocessing result can be handed in); TBE_E_TOO_LARGE when the batch
 * needs more than TBE_STATIC_WS_BYTES of workspace (tbe_workspace_size);
 * TBE_E_HIP if the array's address cannot be resolved. */
#define TBE_STATIC_WS_BYTES (256ull << 20)
int tbe_backward_rowwise_adagrad_noalloc(const tbe_plan* plan, int64_t B, int32_t itype,
                                         const void* indices, const void* offsets,
                                         int64_t num_lookups, const float* per_sample_weights,
                                         const float* grad_out, float lr, float eps,
                                         uint32_t flags, uint32_t* debug_row_updates,
                                         void* stream);

/* Backward with a choice of optimizer epilogue: the same preprocessing and
 * run pipeline as tbe_backward_rowwise_adagrad (which is this call with
 * TBE_OPT_ROWWISE_ADAGRAD), only the per-row update changes.  The plan's
 * momentum[t] buffers hold the optimizer state:
 *  TBE_OPT_ROWWISE_ADAGRAD  R_t floats: M[r] += mean_d g^2,
 *                           w -= lr g / (sqrt(M[r]) + eps);
 *  TBE_OPT_ADAGRAD          element-wise (HugeCTR walkthrough, step 5):
 *                           R_t x D_t floats, row-major, 16-byte aligned:
 *                           A[r][d] += g[d]^2, w[d] -= lr g[d] / (sqrt(A[r][d]) + eps);
 *  TBE_OPT_SGD              w -= lr g; the buffers are not touched.
 * Each touched row is updated once; untouched rows and their state are not
 * written.  TBE_BWD_HIST takes row-wise Adagrad only (else
 * TBE_E_UNSUPPORTED).  Errors: those of tbe_backward_rowwise_adagrad, and
 * TBE_E_ARG for another optimizer code. */
#define TBE_OPT_ROWWISE_ADAGRAD 0
#define TBE_OPT_ADAGRAD 1
#define TBE_OPT_SGD 2
int tbe_backward(const tbe_plan* plan, int64_t B, int32_t itype, const void* indices,
                 const void* offsets, int64_t num_lookups, const float* per_sample_weights,
                 const float* grad_out, int32_t optimizer, float lr, float eps, void* ws,
                 size_t ws_bytes, uint32_t flags, uint32_t* debug_row_updates, void* stream);

/* Input validation and optional repair (FBTriton page, "Forward": the kernels
 * assume their inputs; an optional bounds check and offset repair is a
 * separate pass).  Checks the contract every other entry point assumes:
 * O[0] = 0, O[T*B] = num_lookups, O non-decreasing, offsets in
 * [0, num_lookups], and every index of table t's bags in [0, R_t).  err:
 * device, TBE_VALIDATE_WORDS uint32, overwritten: [0] OR of the
 * TBE_INVALID_* bits found (0: the inputs keep the contract), [1] number of
 * indices out of range (every position once, against the table whose start
 * offset O[t*B], clamped into [0, num_lookups], is the last at or before it),
 * [2] first bag j (table-major) with a finding (the start offset counts as
 * bag 0's, the end offset as the last bag's), [3] first position p of an
 * index out of range (0xffffffff if none).  With TBE_VALIDATE_REPAIR the
 * inputs are then rewritten in place: every index out of range becomes row 0
 * of its table (bags keep their lengths), offsets are clamped into
 * [0, num_lookups] with O[0] = 0 and O[T*B] = num_lookups; offsets out of
 * order are reported, not repaired.  Reads every offset and index once; every
 * access is clamped, so invalid inputs are read safely.  Errors: TBE_E_ARG,
 * TBE_E_RANGE (as tbe_forward), TBE_E_HIP. */
#define TBE_VALIDATE_REPAIR 0x1u
#define TBE_VALIDATE_WORDS 4
#define TBE_INVALID_OFFSET_START 0x1u  /* O[0] != 0 */
#define TBE_INVALID_OFFSET_END 0x2u    /* O[T*B] != num_lookups */
#define TBE_INVALID_OFFSET_ORDER 0x4u  /* some O[j] > O[j+1] */
#define TBE_INVALID_OFFSET_RANGE 0x8u  /* some offset outside [0, num_lookups] */
#define TBE_INVALID_INDEX 0x10u        /* some index outside [0, R_t) */
int tbe_validate(const tbe_plan* plan, int64_t B, int32_t itype, void* indices, void* offsets,
                 int64_t num_lookups, uint32_t* err, uint32_t flags, void* stream);

/* Kernel timing for benchmarks and tools, off by default.  While enabled,
 * every kernel launch of the library carries a start and a stop HIP event
 * bound to the dispatch itself (hipExtLaunchKernel): their difference is the
 * kernel's execution from its dispatch's begin to its end timestamp, the span
 * a kernel trace reports.  Not for use under stream capture.
 * tbe_prof_read waits for the recorded events, writes per-kernel-family
 * totals (name, launches, summed milliseconds) for up to max_kernels
 * families, sets *count to the number of families seen, and clears the
 * records.  names: max_kernels x TBE_PROF_NAME_LEN bytes, NUL-terminated.
 * Both are host-side calls; tbe_prof_read synchronizes on the events. */
#define TBE_PROF_NAME_LEN 32
int tbe_prof_enable(int enable);
int tbe_prof_read(int32_t max_kernels, char* names, int64_t* launches, double* total_ms,
                  int32_t* count);
/* Enqueue `launches` empty kernels (one 64-thread workgroup each) on stream,
 * timed like every library launch while timing is enabled, under the family
 * name "empty": their average is the per-launch floor of a kernel that does
 * nothing. */
int tbe_prof_calibrate(int32_t launches, void* stream);

/* Test knobs, for test suites and tools only: process-wide overrides of the
 * batch sizes from which the library picks the variants it uses on deep
 * batches, so that small inputs can run them against a reference, and of
 * the poll limit of the preprocessing's cross-workgroup waits, so that a
 * wait that gives up can be forced from the host (every kernel still exits
 * normally).  value < 0 restores the default.  Changing a knob while calls
 * are in flight, or between tbe_workspace_size and the calls that use the
 * workspace, is not supported.  Errors: TBE_E_ARG for an unknown knob. */
#define TBE_KNOB_RLE_DEEP_LOOKUPS 1   /* run-length tiles of four 4096-key groups from this
                                         many lookups on (default 8 Mi) */
#define TBE_KNOB_BWD_DEEP_LOOKUPS 2   /* backward gathers with eight lookups in flight and
                                         streamed weight rows from here on (default 64 Mi) */
#define TBE_KNOB_BWD_STREAM_LOOKUPS 3 /* streamed (non-temporal) weight rows in the backward
                                         from here on (default 1 Mi) */
#define TBE_KNOB_WAIT_POLLS 4         /* polls before a look-back wait gives up (default
                                         2^20; 0: a tile with predecessors gives up at once) */
#define TBE_KNOB_DENSE_LOOKUPS 5      /* the hot-row contraction of long runs from this many
                                         lookups on (default 8 Mi) */
int tbe_test_knob(int32_t knob, int64_t value);

/* Static text for a status code. */
const char* tbe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TBE_H */
