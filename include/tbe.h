/*
 * tbe.h -- C ABI of the MI355X (gfx950) table-batched-embedding (TBE) library.
 *
 * One handle covers a set of T embedding tables that live in one flat device
 * buffer, and runs the two halves of the TBE hot path on them:
 *
 *   tbe_forward          pooled lookup over all tables in one launch: every
 *                        bag of row ids is gathered from its table and summed
 *                        (or averaged), optionally scaled per lookup, with fp32
 *                        accumulation whatever the storage dtype.
 *                        kimbodo.com/?p=28372, "What Happened";
 *                        "FBTriton Rewrites Table Batched Embedding"
 *                        (kongchang.com), "Responsibilities of the forward and
 *                        backward passes".
 *   tbe_backward_update  the fused backward: lookups are linearized to
 *                        (table, row) ids, sorted and run-length encoded, the
 *                        upstream gradients of each run are added up (a
 *                        streaming path for short runs, split accumulation for
 *                        runs of 256 lookups or more) and every touched row
 *                        receives exactly one optimizer update.
 *                        kimbodo.com/?p=28372, "What Happened" and "Kimbodo
 *                        Engineering Perspective".
 *
 * The batch format (flat ids + CSR offsets whose last entry is the id count)
 * follows the example call in "Optimizing Recommendation Systems with FBTriton
 * Table Batched Embeddings" (explore.n1n.ai), "Implementation Guide:
 * Integrating TBE".
 *
 * Layouts (all row-major, no padding):
 *   weights   one flat buffer of the storage dtype; table t starts at element
 *             woff_t = sum_{t'<t} rows[t'] * dims[t'] and holds rows[t] rows
 *             of dims[t] elements.
 *   state     row-wise Adagrad only: fp32 [sum_t rows[t]], one value per table
 *             row, indexed by the linear row id roff_t + row
 *             (roff_t = sum_{t'<t} rows[t']).  Must start at 0.
 *   bags      table-major: bag k = t*B + b, B bags per table.
 *   indices   [num_indices] table-local row ids (int32 or int64); num_indices < 2^30.
 *   offsets   [T*B + 1], same integer type as indices; bag k holds
 *             indices[offsets[k] .. offsets[k+1]); offsets[0] = 0 and
 *             offsets[T*B] = num_indices.
 *   per_sample_weights  optional fp32 [num_indices].
 *   output    fp32 [B, sum_t dims[t]]; table t fills columns
 *             [doff_t, doff_t + dims[t]) with doff_t = sum_{t'<t} dims[t'].
 *   grad_output  fp32, same layout as output.
 *
 * Ownership: every buffer is allocated and owned by the caller.  The weights
 * and state pointers given to tbe_create are kept (not copied) and must
 * outlive the handle; so must a forward scratch attached with
 * tbe_set_forward_scratch.  The library allocates only a small per-handle
 * device metadata block (in tbe_create) and frees it in tbe_destroy.
 *
 * Asynchrony: tbe_forward and tbe_backward_update enqueue work on the given
 * HIP stream (a hipStream_t passed as void*, NULL = the null stream) and
 * return without waiting, unless TBE_FLAG_VALIDATE is set.  Host-side argument
 * checks happen first: on any error nothing is enqueued.  Device-side input
 * preconditions (ids in range, offsets monotone and ending at num_indices) are
 * not checked unless TBE_FLAG_VALIDATE is set; violating them is undefined.
 *
 * Graph capture: without TBE_FLAG_VALIDATE and TBE_OPTION_PROFILE, the compute
 * calls only enqueue kernels (no host synchronisation, no allocation, no
 * memset), so they may be captured into a HIP graph on a capturing stream and
 * replayed; a replay gives the same results as the calls made eagerly, bit
 * for bit.  A captured tbe_forward_group and its tbe_backward_update_grouped
 * belong in the same graph (the pairing is checked on the host at capture).
 *
 * Threading: a handle may be used by one host thread at a time.  Two
 * backward_update calls in flight on one handle race on the weights; with
 * TBE_FLAG_SPLIT_BAGS or the count-matrix forward, two forward calls in
 * flight on one handle (on different streams) race on its forward scratch.
 *
 * No C++ exception crosses this interface.  Every function returns a
 * tbe_status; tbe_status_string gives a static description.
 */
#ifndef TBE_H
#define TBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TBE_ABI_VERSION 2

typedef struct tbe_handle tbe_handle;

typedef enum {
  TBE_OK = 0,
  TBE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size or enum, misaligned buffer */
  TBE_ERR_UNSUPPORTED = 2,        /* valid request the library does not handle */
  TBE_ERR_INDEX_OUT_OF_RANGE = 3, /* TBE_FLAG_VALIDATE found a bad id or offsets array */
  TBE_ERR_WORKSPACE_TOO_SMALL = 4,
  TBE_ERR_HIP = 5,                /* a HIP runtime call or kernel launch failed */
  TBE_ERR_OUT_OF_MEMORY = 6,      /* metadata allocation failed */
  TBE_ERR_DEVICE_WAIT = 7         /* a device-side wait gave up: that backward update was
                                     skipped (see tbe_check_device_status) */
} tbe_status;

typedef enum { TBE_F32 = 0, TBE_F16 = 1, TBE_BF16 = 2 } tbe_dtype;       /* table storage */
typedef enum { TBE_I32 = 0, TBE_I64 = 1 } tbe_index_dtype;                /* indices and offsets */
typedef enum { TBE_POOL_SUM = 0, TBE_POOL_MEAN = 1 } tbe_pooling;
typedef enum { TBE_OPT_SGD = 0, TBE_OPT_ROWWISE_ADAGRAD = 1 } tbe_optimizer;

enum {
  /* Check ids and offsets on the device before touching any output or
   * weight; the call then waits for the stream and returns
   * TBE_ERR_INDEX_OUT_OF_RANGE on a bad batch. */
  TBE_FLAG_VALIDATE = 1u,
  /* Never use the count-matrix (MFMA) forward (the default: on MI355X the
   * gather forward measured faster at every qualifying workload tried). */
  TBE_FLAG_NO_HISTOGRAM = 2u,
  /* Use the count-matrix forward for every table; tbe_create fails with
   * TBE_ERR_UNSUPPORTED if a table does not qualify. */
  TBE_FLAG_FORCE_HISTOGRAM = 4u,
  /* Use the count-matrix forward for the tables that qualify and the gather
   * forward for the others (per call: only when there are no per-sample
   * weights).  Qualifying: fp16/bf16 storage, E_t <= 1024, D_t <= 256 and a
   * multiple of 16, rows 16-byte aligned in the flat weights.  Source:
   * kimbodo.com/?p=28372, "What Happened" (small tables that qualify use a
   * histogram and tensor-core path). */
  TBE_FLAG_HISTOGRAM = 8u,
  /* Skew balancing (off by default): a bag of more than 128 lookups pools its
   * first 128 in the forward's own pass and its other 128-lookup segments
   * in parallel waves, whose sums are then added to the bag's output in
   * segment order (deterministic; the fp32 rounding order differs from the
   * unsplit sum).  The segment sums go to the caller's forward scratch
   * (tbe_set_forward_scratch, about 64 MB); a call whose lookups could need
   * more segments than it holds pools its bags unsplit.  Source: kimbodo.com/?p=28372,
   * "Kimbodo Engineering Perspective" (load imbalance across lookups). */
  TBE_FLAG_SPLIT_BAGS = 16u,
  /* Count-matrix backward (off by default): for every bag b of table t, its
   * gradient row is added to each row r its lookups hit, as the dense product
   * Gamma_t = C_t^T G_t on the matrix cores (C_t the bag-by-row count
   * matrix, G_t the table's columns of grad_output, scaled by 1/L for mean
   * pooling), with G split exactly into three bf16 parts so the products are
   * exact and the sums fp32 in a fixed order; then one optimizer update per
   * row that a lookup touched.  No sort: the counts replace the grouping.
   * Every table must have at most 1024 rows and a dim that is a multiple of
   * 16 up to 256, else tbe_create fails with TBE_ERR_UNSUPPORTED; calls with
   * per-sample weights take the sort path.  tbe_forward_group then only pools
   * (there is no grouping to make) and records the batch for
   * tbe_backward_update_grouped.  Extends kimbodo.com/?p=28372, "What
   * Happened" (a histogram and tensor-core path for small tables, shown there
   * for the forward) to the backward. */
  TBE_FLAG_COUNT_BACKWARD = 32u
};

typedef struct {
  int32_t num_tables;      /* T >= 1 */
  const int64_t* rows;     /* host [T], rows[t] >= 1, sum < 2^31 */
  const int32_t* dims;     /* host [T], 1 <= dims[t] <= 1024 */
  int32_t weight_dtype;    /* tbe_dtype */
  int32_t pooling;         /* tbe_pooling */
  int32_t optimizer;       /* tbe_optimizer */
  uint32_t flags;          /* TBE_FLAG_* */
} tbe_config;

/* Optional output of tbe_backward_update: the grouping it computed.  Device
 * buffers with room for num_indices entries; num_unique is one int32. */
typedef struct {
  int32_t* unique_ids;     /* ascending linear row ids roff_t + row */
  int32_t* run_lengths;    /* lookups per unique id */
  int32_t* num_unique;     /* U */
} tbe_runs;

/* Tuning / test knobs for tbe_set_option. */
typedef enum {
  /* Runs with at least this many lookups take the split-accumulation path
   * (default 256).  Changes only the fp32 summation order. */
  TBE_OPTION_LONG_RUN_THRESHOLD = 1,
  /* 1: every kernel the calls launch records its own start and end in a pair
   * of HIP events (hipExtLaunchKernelGGL), readable with tbe_stage_times;
   * 0 (default): off. */
  TBE_OPTION_PROFILE = 2,
  /* How the backward groups lookups by (table, row) id ("Kimbodo Engineering
   * Perspective": transpose, sort, run-length encoding).
   * 0 (default): when the batch sorts in two radix digits (at most 2^20
   *    lookups, ids of 11 to 20 bits), one pass on the high digit and then a
   *    bucket-local sort with the run-length encoding in the same kernel;
   *    otherwise as 1.
   * 1: LSD radix passes, then a separate run-length-encoding kernel.
   * Both give the same order (stable on the id), so results are bit-identical.
   * Other values: TBE_ERR_INVALID_ARGUMENT. */
  TBE_OPTION_SORT = 3,
  /* Polls a workgroup of the backward's grouping makes while it waits for an
   * earlier one (the sort's and the run-length encoding's look-backs) before
   * it gives up (default 2^20, far beyond any wait seen; 0 to 2^31 - 1).  A
   * wait that gives up never faults or hangs: the call finishes, updates no
   * weight and no state, reports num_unique = -1 in its runs, and marks the
   * handle (tbe_check_device_status).  0 makes every such wait give up at
   * once, which only serves to test that path. */
  TBE_OPTION_SPIN_LIMIT = 4,
  /* The pooled lookup of small tables ("What Happened": the same gather and
   * pooling, with the rows read from the CU's local memory).
   * 1 (default): when some tables qualify (fp16/bf16 storage, rows of 3 to 8
   *    16-byte chunks, at most 128 KB with rows padded to 4 or 8 chunks) and a
   *    call without TBE_FLAG_SPLIT_BAGS has at least 16 x the largest such E_t
   *    lookups per table and short enough bags (a mean of at most 16 lookups;
   *    8 with per-sample weights and rows of 5 to 8 chunks), every workgroup
   *    of those tables stages its table in LDS once and pools its bags from
   *    there; the other tables take the gather kernel.
   * 0: every table takes the gather kernel.
   * Both give the same bits.  Other values: TBE_ERR_INVALID_ARGUMENT. */
  TBE_OPTION_LDS_FORWARD = 5
} tbe_option;

/* Create a handle.  Validates the configuration (host only; nothing is
 * allocated when it fails), computes the table layout and copies a small
 * metadata block to the current device.  weights: device, flat, storage
 * dtype, 16-byte aligned.  optim_state: device fp32 [sum rows], required for
 * row-wise Adagrad, ignored (may be NULL) for SGD. */
tbe_status tbe_create(const tbe_config* config, void* weights, float* optim_state,
                      tbe_handle** out);

/* Release the handle's metadata.  Waits for nothing; the caller must not
 * destroy a handle whose work is still running.  NULL is a no-op. */
void tbe_destroy(tbe_handle* handle);

/* Device scratch of the forward's opt-in paths, which the caller provides:
 * the count-matrix forward's transposed copy of its tables (TBE_FLAG_HISTOGRAM,
 * TBE_FLAG_FORCE_HISTOGRAM; rewritten by every forward call that takes that
 * path) and the split bags' segment sums (TBE_FLAG_SPLIT_BAGS).  *bytes = 0
 * when the handle uses neither path: its forward calls need no scratch. */
tbe_status tbe_forward_scratch_size(const tbe_handle* handle, size_t* bytes);

/* Attach a caller-owned device buffer of at least tbe_forward_scratch_size
 * bytes, 256-byte aligned, for the later forward calls on the handle (kept,
 * not copied: it must stay valid until it is replaced, detached with NULL and
 * 0, or the handle destroyed).  Its contents need no initialisation and are
 * undefined after a call.  While a handle that needs scratch has none, its
 * forward calls return TBE_ERR_WORKSPACE_TOO_SMALL and enqueue nothing.
 * Errors: TBE_ERR_INVALID_ARGUMENT (null handle, misaligned buffer, NULL with
 * bytes != 0), TBE_ERR_WORKSPACE_TOO_SMALL (bytes below the size). */
tbe_status tbe_set_forward_scratch(tbe_handle* handle, void* scratch, size_t bytes);

/* Pooled forward.  B >= 0 bags per table; num_indices >= 0.  B == 0 is a
 * no-op; bags without ids produce zeros (also under mean pooling). */
tbe_status tbe_forward(tbe_handle* handle, int32_t B, const void* indices, const void* offsets,
                       int32_t index_dtype, int64_t num_indices,
                       const float* per_sample_weights, float* output, void* stream);

/* Gradient of the loss with respect to the per-sample weights: for every
 * lookup i of bag k = (t, b), grad_psw[i] = s_k * <grad_output[b, doff_t :
 * doff_t + D_t], W_t[x_i]>, with s_k = 1 (sum) or 1 / L_k (mean).  The pages
 * take per-sample weights in the forward (kimbodo.com/?p=28372, "What
 * Happened"); the forward is linear in them, which gives this gradient.  It
 * reads the weights, so call it before tbe_backward_update changes them.
 * grad_output: device fp32 [B, sum D]; grad_psw: device fp32 [num_indices],
 * written.  Errors as tbe_forward. */
tbe_status tbe_psw_grad(tbe_handle* handle, int32_t B, const void* indices, const void* offsets,
                        int32_t index_dtype, int64_t num_indices, const float* grad_output,
                        float* grad_psw, void* stream);

/* Bytes of device workspace tbe_backward_update needs for this batch shape. */
tbe_status tbe_backward_workspace_size(const tbe_handle* handle, int32_t B, int64_t num_indices,
                                       size_t* bytes);

/* Fused backward + optimizer update of the handle's weights (and state).
 * lr: learning rate; eps: Adagrad epsilon (ignored for SGD).  workspace:
 * device, 256-byte aligned, at least tbe_backward_workspace_size bytes; its
 * contents on entry do not matter.  runs: optional (NULL for none). */
tbe_status tbe_backward_update(tbe_handle* handle, int32_t B, const void* indices,
                               const void* offsets, int32_t index_dtype, int64_t num_indices,
                               const float* per_sample_weights, const float* grad_output,
                               float lr, float eps, void* workspace, size_t workspace_bytes,
                               const tbe_runs* runs, void* stream);

/* tbe_backward_update for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the workspace
 * taken from a static device array of TBE_STATIC_SCRATCH_BYTES inside the
 * library (one per GPU, held until the process ends) instead of a caller
 * buffer.  Allocates nothing, neither device nor host memory, and records no
 * kernel timings (TBE_OPTION_PROFILE does not apply).  A batch whose
 * tbe_backward_workspace_size exceeds TBE_STATIC_SCRATCH_BYTES gets
 * TBE_ERR_WORKSPACE_TOO_SMALL with nothing enqueued.  Every call on one GPU,
 * from any handle, uses that GPU's one array: calls that overlap in time on
 * one GPU (several streams, or host threads) race on it and give undefined
 * results; calls ordered on one stream are fine.  Other arguments and errors
 * as tbe_backward_update; TBE_ERR_HIP if the array's address could not be
 * found. */
#define TBE_STATIC_SCRATCH_BYTES (64u << 20)
tbe_status tbe_backward_update_no_alloc(tbe_handle* handle, int32_t B, const void* indices,
                                        const void* offsets, int32_t index_dtype,
                                        int64_t num_indices, const float* per_sample_weights,
                                        const float* grad_output, float lr, float eps,
                                        const tbe_runs* runs, void* stream);

/* Forward plus the backward's grouping of the same batch.  kimbodo.com/?p=28372,
 * "Kimbodo Engineering Perspective": the transpose, sort and run-length
 * encoding of the backward can be done during the forward (an option that is
 * off by default there).  On `stream`: the workspace is cleared, the batch
 * is pooled (as tbe_forward) and linearized (for batches of at most 2^20
 * lookups in one launch, the linearize workgroups running beside the pooled
 * lookup; one after the other above that); then the sort and the run-length
 * encoding of the batch follow, into `workspace` (sized by
 * tbe_backward_workspace_size, 256-byte aligned).  With TBE_FLAG_VALIDATE the
 * ids are checked before anything is queued.  Arguments and errors as
 * tbe_forward, plus TBE_ERR_WORKSPACE_TOO_SMALL.  The handle records the call
 * by its workspace (up to 64 such records, oldest dropped first), so several
 * forward_group calls on different workspaces may precede their backward
 * calls.  The workspace must then go, unchanged and with the same batch
 * buffers (ids, offsets, per-sample weights, B, num_indices, index dtype), to
 * one tbe_backward_update_grouped call; the long-run threshold and sort
 * options in force at this call are the ones used there.  The pair gives the
 * same output, weights and state as tbe_forward + tbe_backward_update, bit
 * for bit. */
tbe_status tbe_forward_group(tbe_handle* handle, int32_t B, const void* indices,
                             const void* offsets, int32_t index_dtype, int64_t num_indices,
                             const float* per_sample_weights, float* output, void* workspace,
                             size_t workspace_bytes, void* stream);

/* tbe_backward_update without the grouping: uses the one a tbe_forward_group
 * call on the same batch left in `workspace` (same arguments and errors as
 * tbe_backward_update; the result is bit-identical).  Returns
 * TBE_ERR_INVALID_ARGUMENT, with nothing enqueued, when the handle holds no
 * grouping of this workspace, or when its batch buffers, B, num_indices or
 * index dtype differ from that forward_group call's.  Each grouping serves one
 * backward call; a plain tbe_backward_update or a new tbe_forward_group on the
 * same workspace discards it. */
tbe_status tbe_backward_update_grouped(tbe_handle* handle, int32_t B, const void* indices,
                                       const void* offsets, int32_t index_dtype,
                                       int64_t num_indices, const float* per_sample_weights,
                                       const float* grad_output, float lr, float eps,
                                       void* workspace, size_t workspace_bytes,
                                       const tbe_runs* runs, void* stream);

/* Device-side failures of backward calls since the last check.  Waits for
 * `stream` (all work queued on it, hipStream_t as void*), then reads and
 * clears the handle's mark: TBE_ERR_DEVICE_WAIT if a backward call's wait gave
 * up since the last check (TBE_OPTION_SPIN_LIMIT; that call left weights and
 * state untouched), else TBE_OK.  With TBE_FLAG_VALIDATE every backward call
 * makes this check itself before it returns. */
tbe_status tbe_check_device_status(tbe_handle* handle, void* stream);

/* Set a tbe_option (see above). */
tbe_status tbe_set_option(tbe_handle* handle, int32_t option, int64_t value);

/* With TBE_OPTION_PROFILE on: waits for the recorded events, then writes, for
 * every kernel launched by the calls made since the last read (in launch
 * order, at most capacity), its duration in milliseconds (from the kernel's
 * start to its end, host gaps excluded) to ms and the kernel's static name to
 * names (may be NULL); *count receives the number written.  The recorded
 * events are then dropped. */
tbe_status tbe_stage_times(tbe_handle* handle, float* ms, const char** names, int32_t capacity,
                           int32_t* count);

const char* tbe_status_string(tbe_status status);
int32_t tbe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TBE_H */
