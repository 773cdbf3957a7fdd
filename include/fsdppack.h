/*
 * fsdppack.h -- C ABI of libfsdppack: FSDP2's mixed-dtype gradient pack for
 * reduce-scatter, the write-back of a reduce-scatter output into sharded
 * gradients, and the all-gather copy-in / copy-out, on AMD MI355X (gfx950).
 *
 * What the calls compute (web pages on FSDP2 per-parameter mixed precision):
 *  - "PyTorch adds per-parameter mixed precision to FSDP2" (ainewsletter.today),
 *    paragraph 2: gradients of one fully_shard unit arrive in mixed compute
 *    dtypes (BF16, FP32); they are chunked and padded and cast straight into a
 *    single buffer of the reduction dtype, one bucket (and one reduce-scatter)
 *    per effective reduction dtype.  Paragraph 1: the all-gather copy-in
 *    groups staging copies by (source, target) dtype and keeps one all-gather
 *    per unit.
 *  - "The unit you wrapped" (kernels.rudrite.com), shard and padding
 *    paragraphs: a rank's piece is a contiguous row-major slice, and
 *    right-hand padding gives every rank the same size.
 *  - "Mixed-Precision Training" (NeMo AutoModel docs), table "Storage Dtype
 *    Compared to Compute Dtype": param_dtype is the compute dtype the
 *    all-gather delivers, reduce_dtype the dtype of the gradient reduction,
 *    the storage dtype that of the resident sharded parameter.
 *
 * Layout (W = world size, a layout parameter only; no collective is issued):
 *  - Parameter t is viewed as [dim0, inner].  Rank r's chunk is rows
 *    [r*c, (r+1)*c) with c = ceil(dim0 / W), i.e. flat elements
 *    [r*P, r*P + P) with P = c * inner; elements past numel = dim0 * inner
 *    are padding (+0).
 *  - Reduce-scatter input of a bucket: a row-major [W, S] array of the bucket's
 *    reduction dtype, S = sum of the members' P; member t occupies columns
 *    [O_t, O_t + P_t) of every row, O_t the exclusive prefix sum of P in
 *    unit order.
 *  - All-gather buffer: a row-major [W, B]-byte array; parameter t's P_t
 *    elements in its param dtype start at byte A_t of each row (A_0 = 0, every
 *    A_t and B a multiple of 16, parameters in unit order, gap bytes zero).
 *
 * Conventions:
 *  - dtype codes: FSDPPACK_BF16 (bfloat16), FSDPPACK_FP32 (IEEE binary32).
 *    bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest, ties to even,
 *    keeps subnormals, overflows to infinity, and turns a NaN into a quiet
 *    NaN with the same sign and top payload bits.
 *  - Data pointers are device pointers owned by the caller; each must be
 *    aligned to its element size.  Pointer arrays (grads, shards, params) are
 *    host arrays with one entry per parameter, indexed by parameter (unit
 *    order); they are read during the call only.  An entry may be NULL only
 *    where it is never dereferenced (a parameter with zero elements, or one
 *    outside the bucket being packed).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every compute
 *    call enqueues one kernel launch on it (none when there is nothing to
 *    write) and returns without waiting; argument errors are reported
 *    synchronously and enqueue nothing.
 *  - Every call returns FSDPPACK_OK (0) or a negative error code, and on
 *    error leaves a message for fsdppack_last_error() (per thread).  No
 *    exception crosses the ABI.
 *  - A plan is immutable after creation and may be shared by threads and
 *    streams; its device tables are uploaded on the first compute call that
 *    needs them (a synchronous copy) on the device current at that time, and
 *    the plan may only be used on that device afterwards.
 *  - Per-call pointer arrays reach the kernel in one of two ways.  Up to 64
 *    entries travel in the launch's own arguments: nothing is uploaded or
 *    cached, so a call with new pointers (gradients allocated afresh every
 *    backward) costs the same as one with known pointers.  Larger arrays use
 *    device tables cached by content, 16 per operation (per bucket for the
 *    pack): a call whose set is cached uses its table; a call with a new set
 *    of up to 960 entries passes it in the launch arguments and then uploads
 *    it asynchronously on `stream`, behind its launch, for the next call
 *    with that set, unless the table it would replace is still being
 *    uploaded (then the set is not cached: the call never waits).  A larger
 *    new set is uploaded before its launch; when it replaces the least
 *    recently used table the call waits on the host for that table's own
 *    earlier upload only.  A replacement makes `stream` wait on the device
 *    for work other streams had enqueued when they used the table (no
 *    device-wide synchronisation); calls with a cached set record no event
 *    and upload nothing.  A stream passed to a compute call must stay valid
 *    until the plan is destroyed.
 *  - A launch's grid is bounded by the hardware's 32-bit work-item counts:
 *    the planner rejects (EINVAL) a unit whose launches would need more
 *    workgroups (about 128 GiB written by one launch).
 */
#ifndef FSDPPACK_H
#define FSDPPACK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fsdppack_dtype {
    FSDPPACK_DTYPE_NONE = 0,   /* reduce_dtype only: "unset", use the grad dtype */
    FSDPPACK_BF16 = 1,
    FSDPPACK_FP32 = 2
};

enum fsdppack_status {
    FSDPPACK_OK = 0,
    FSDPPACK_EINVAL = -1,  /* bad argument: NULL, out-of-range index, misaligned pointer, bad size */
    FSDPPACK_EDTYPE = -2,  /* unsupported dtype code */
    FSDPPACK_ENOMEM = -3,  /* host or device allocation failed */
    FSDPPACK_EHIP = -4,    /* a HIP runtime call failed (the message names it) */
    FSDPPACK_ESTATE = -5   /* plan destroyed or corrupt, or used on another device */
};

/* One parameter of a fully_shard unit.  dim0 >= 0, inner >= 1 when dim0 > 0
 * (a 0-d tensor is dim0 = 1, inner = 1).  grad_dtype: the dtype its gradient
 * arrives in.  reduce_dtype: the policy's reduction dtype, or
 * FSDPPACK_DTYPE_NONE for "same as the gradient".  storage_dtype: dtype of
 * the resident sharded parameter (copy-in source).  param_dtype: compute
 * dtype delivered by the all-gather (copy-in target, copy-out dtype). */
typedef struct fsdppack_param_desc {
    int64_t dim0;
    int64_t inner;
    int32_t grad_dtype;
    int32_t reduce_dtype;
    int32_t storage_dtype;
    int32_t param_dtype;
} fsdppack_param_desc;

typedef struct fsdppack_plan fsdppack_plan;   /* opaque, library-owned */

/* Plan one unit ("PyTorch adds per-parameter mixed precision to FSDP2",
 * paragraph 2: one bucket, and one reduce-scatter, per effective reduction
 * dtype; "The unit you wrapped", padding paragraphs: equal right-padded rank
 * chunks): bucket the n parameters by effective reduction dtype
 * (reduce_dtype if set, else grad_dtype; buckets in order of first
 * appearance, members in unit order) and compute P, O, S per bucket and the
 * all-gather offsets A and row size B.  Host work only (no HIP call).
 * params: n descriptors (host).  world: W >= 1.  *out_plan receives a new
 * plan owned by the caller until fsdppack_plan_destroy.
 * Errors: EINVAL (NULL, n < 0, W < 1, negative sizes, sizes whose byte
 * counts overflow int64), EDTYPE (unknown dtype code), ENOMEM. */
int fsdppack_plan_buckets(const fsdppack_param_desc *params, int32_t n, int32_t world,
                          fsdppack_plan **out_plan);

/* Plan one unit in the FSDP1 flat-parameter layout ("The unit you wrapped",
 * the auto_wrap_policy and padding paragraphs): the n parameters, flattened
 * and concatenated in unit order, form one flat parameter of N elements
 * (parameter t at flat offset F_t), padded to W*c, c = ceil(N / W); rank r
 * holds flat positions [r*c, (r+1)*c).  The unit needs one effective
 * reduction dtype and one param dtype; gradient and storage dtypes may differ
 * per parameter.  The plan has one bucket (none when n = 0), and the compute
 * calls take the flat meaning:
 *  - pack_reduce_scatter_input: out ([W, c], the reduction dtype) = the
 *    concatenated gradients cast, +0 past N;
 *  - reduce_scatter_copy_out, all_gather_copy_in: the per-parameter entries
 *    are parameter t's piece on the rank (the part of [F_t, F_t + numel_t)
 *    inside the rank's positions, in the storage dtype; NULL allowed when
 *    empty); rs_out is the rank's c reduced elements; the copy-in writes the
 *    rank's row (c elements of the param dtype, +0 past N) of ag_out;
 *  - all_gather_copy_out: ag is the gathered flat parameter, W*c elements of
 *    the param dtype; parameter t is its elements [F_t, F_t + numel_t).
 * Introspection: plan_bucket gives S = c, P_t = numel_t and O_t = F_t;
 * plan_all_gather_layout gives B = c * size(param dtype) bytes (no rounding),
 * P_t = numel_t and A_t = F_t * size(param dtype).
 * Errors: as fsdppack_plan_buckets, and EDTYPE when the parameters' effective
 * reduction dtypes or param dtypes differ. */
int fsdppack_plan_buckets_flat(const fsdppack_param_desc *params, int32_t n, int32_t world,
                               fsdppack_plan **out_plan);

/* Number of buckets and parameters of a plan. */
int fsdppack_plan_info(const fsdppack_plan *plan, int32_t *num_buckets, int32_t *num_params,
                       int32_t *world);

/* Describe bucket `bucket`: its reduction dtype, row length S, and its
 * nmembers parameter indices with their P and O (arrays owned by the plan,
 * valid until it is destroyed).  Any output pointer may be NULL. */
int fsdppack_plan_bucket(const fsdppack_plan *plan, int32_t bucket, int32_t *reduce_dtype,
                         int64_t *S, int32_t *nmembers, const int32_t **members,
                         const int64_t **P, const int64_t **O);

/* All-gather layout: row bytes B, and per parameter (unit order) P and the
 * byte offset A within a row (arrays owned by the plan).  Any output pointer
 * may be NULL. */
int fsdppack_plan_all_gather_layout(const fsdppack_plan *plan, int64_t *B, const int64_t **P,
                                    const int64_t **A);

/* Fused reduce-scatter pack of one bucket (the _chunk_cat.out-style op that
 * "PyTorch adds per-parameter mixed precision to FSDP2" (ainewsletter.today),
 * paragraphs 2-3, describes: gradients chunked, padded and cast in one pass
 * into the bucket's reduction dtype, with no pre-cast temporaries; rank
 * chunks and right-hand padding as in "The unit you wrapped", padding
 * paragraphs):
 *   out[r*S + O_t + j] = cast(grads[t][r*P_t + j])  if r*P_t + j < numel_t,
 *                      = +0                          otherwise,
 * for every member t, rank r < W and j < P_t, cast = the member's grad dtype
 * to the bucket's reduction dtype.  grads: n host entries (by parameter
 * index) of device pointers to contiguous gradients of numel_t elements;
 * only the bucket's members are read.  out: device buffer of W*S elements of
 * the reduction dtype, fully overwritten.  One kernel launch on `stream`.
 * Errors: EINVAL (bucket out of range, NULL or misaligned pointer), ESTATE,
 * EHIP, ENOMEM. */
int fsdppack_pack_reduce_scatter_input(const fsdppack_plan *plan, int32_t bucket,
                                       const void *const *grads, void *out, void *stream);

/* The same fused reduce-scatter pack, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): it allocates nothing.  The kernel reads the
 * bucket's pack tables from a library-owned device scratch of 1 MiB per GPU,
 * held until the process ends, and the pointers travel in the launch
 * arguments; the plan's own device tables are neither used nor created.
 * The plan lays its tables out for the scratch when it is built: every
 * bucket's in one image when they fit together, else one image per bucket.
 * A call copies its image there (one hipMemcpyAsync from the plan's host
 * memory, on `stream`) only when the scratch does not already hold it;
 * when it does but the copy that put it there may still be running, the
 * call's stream waits for that copy on the device (hipStreamWaitEvent).  At
 * its first call on a device it looks up the scratch's address and creates
 * the event that marks those copies (make that first call outside stream
 * capture).  Under stream capture the copy is recorded into the graph ahead
 * of the kernel, so every replay brings its own tables; from then on every
 * call on that device copies, since a replay may have replaced what the
 * scratch held.  A graph holding such a call reads the plan's host image at
 * each replay: it must not be replayed once the plan is destroyed.
 * Destroying a plan that this entry point copied from synchronises the
 * device.  Same arguments, result and
 * errors as fsdppack_pack_reduce_scatter_input, and also EINVAL when the
 * bucket has more than 960 members or its tables exceed the scratch (about
 * 13 000 column-map stretches).  Every call on a GPU shares that GPU's
 * scratch: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race, so a caller orders them. */
int fsdppack_pack_reduce_scatter_input_noalloc(const fsdppack_plan *plan, int32_t bucket,
                                               const void *const *grads, void *out, void *stream);

/* All-gather copy-in ("PyTorch adds per-parameter mixed precision to FSDP2",
 * paragraph 1: the copy-in casts each local shard to its target dtype and
 * keeps a single all-gather per unit) for rank `rank` (0 <= rank < W): row
 * `rank` of ag_out
 * (a device [W, B]-byte buffer) receives each parameter's padded local shard
 * cast from its storage dtype to its param dtype at byte A_t; the row's gap
 * bytes are written as zero, the other rows are not touched.  shards: n host
 * entries of device pointers to P_t elements each (storage dtype).  The
 * (storage, param) dtype pairs all run in the same single launch.
 * Errors: EINVAL, ESTATE, EHIP, ENOMEM. */
int fsdppack_all_gather_copy_in(const fsdppack_plan *plan, int32_t rank, const void *const *shards,
                                void *ag_out, void *stream);

/* All-gather copy-out ("The unit you wrapped": the layer's full shape only
 * returns once the unit is gathered; the right-hand padding exists only for
 * the even split and is dropped): rebuild every full parameter from the
 * gathered [W, B]-byte buffer ag, dropping padding:
 *   params[t][r*P_t + j] = element j of parameter t's segment in row r,
 *   for j < min(P_t, numel_t - r*P_t).
 * params: n host entries of device pointers to numel_t elements each
 * (param dtype), fully overwritten.  Errors: EINVAL, ESTATE, EHIP, ENOMEM. */
int fsdppack_all_gather_copy_out(const fsdppack_plan *plan, const void *ag, void *const *params,
                                 void *stream);

/* Reduce-scatter output write-back for rank `rank` (0 <= rank < W): the step
 * after the bucket's reduce-scatter, where each rank keeps the gradient slice
 * of the parameters it owns ("The unit you wrapped", the paragraphs on the
 * collectives FSDP issues), in the resident parameter's dtype ("Mixed-
 * Precision Training": reduce_dtype only sets how gradients are summed; the
 * gradient buffer follows the resident parameter dtype):
 *   shard_grads[t][j] = cast(div(rs_out[O_t + j]))   for j < min(P_t, numel_t - rank*P_t)
 * for every member t of the bucket.  rs_out: device pointer to the rank's
 * reduced row, S elements of the bucket's reduction dtype (row `rank` of a
 * reduce-scatter of the packed [W, S] input), read only.  div: when
 * divide_factor is not 1, the element divided by divide_factor in the
 * reduction dtype (a correctly rounded binary32 division, then rounded once
 * to bfloat16 when that is the reduction dtype; a NaN is not divided and gets
 * the quiet bit); cast: the reduction dtype to the member's storage dtype.
 * shard_grads: n host entries (by parameter index) of device pointers to the
 * rank chunk's real elements (storage dtype), overwritten; entries of
 * non-members, and of members with no real element on this rank, are not read
 * and may be NULL.  divide_factor must be finite and > 0.  One kernel launch
 * on `stream`.  Errors: EINVAL (bucket or rank out of range, bad
 * divide_factor, NULL or misaligned pointer), ESTATE, EHIP, ENOMEM. */
int fsdppack_reduce_scatter_copy_out(const fsdppack_plan *plan, int32_t bucket, int32_t rank,
                                     const void *rs_out, float divide_factor, void *const *shard_grads,
                                     void *stream);

/* The write-back of every bucket of the unit in one launch: for each bucket
 * b, exactly what fsdppack_reduce_scatter_copy_out(plan, b, rank, rs_outs[b],
 * divide_factor, shard_grads, stream) writes (same passages: each rank keeps
 * the gradient slice of the parameters it owns, "The unit you wrapped"; the
 * gradient follows the resident parameter dtype, "Mixed-Precision
 * Training").  A unit whose parameters reduce in two dtypes has two buckets,
 * each with its own reduce-scatter; once both are done, this call writes
 * every sharded gradient at the cost of one launch instead of one per
 * bucket.  rs_outs: one host entry per bucket (in bucket order) of a device
 * pointer to the rank's reduced row of that bucket (S_b elements of its
 * reduction dtype), read only.  shard_grads: n host entries by parameter
 * index, as for the per-bucket call (NULL allowed where the rank has no real
 * element).  With one bucket (and for a flat plan) this is the per-bucket
 * call on bucket 0.  One kernel launch on `stream` when there is anything to
 * write.  Errors: EINVAL (rank out of range, bad divide_factor, NULL or
 * misaligned pointer), ESTATE, EHIP, ENOMEM. */
int fsdppack_reduce_scatter_copy_out_all(const fsdppack_plan *plan, int32_t rank, const void *const *rs_outs,
                                         float divide_factor, void *const *shard_grads, void *stream);

/* Free a plan and its device tables.  Synchronises the device first if the
 * plan was ever used there (no kernel may still read its tables) or the
 * allocation-free pack copied from it (no copy may still read its host
 * images).  NULL is a no-op. */
void fsdppack_plan_destroy(fsdppack_plan *plan);

/* Message of the last failed call on this thread ("" if none). */
const char *fsdppack_last_error(void);

/* Kernel timing: the next compute call made on this thread stamps
 * `start_event` and `stop_event` (hipEvent_t, created by the caller with
 * timing enabled; either may be NULL) at its kernel's start and end, so
 * hipEventElapsedTime gives that kernel's exact execution time.  The next
 * compute call takes the events whether it launches or not: a call with
 * nothing to write, or one rejected for its arguments, clears them without
 * stamping them.  For benchmarks and profilers. */
int fsdppack_time_next_launch(void *start_event, void *stop_event);

/* Library-wide counters since load (for tests and tracing): counters[0] =
 * kernel launches, [1] = pointer-table uploads, [2] = pointer-table reuses,
 * [3] = plan device-table uploads, [4] = pointer tables replaced by a new set,
 * [5] = cross-stream waits enqueued at such a replacement, [6] = launches
 * whose pointers travelled in the launch arguments, [7] = host waits for a
 * replaced table's previous upload (the only waits a compute call makes; no
 * compute call synchronises the device), [8] = copies of pack tables into
 * the allocation-free pack's scratch.  The first min(n, 9) entries are
 * written. */
int fsdppack_counters(int64_t *counters, int32_t n);

/* Measurement aid: launch a kernel that does nothing, with `workgroups`
 * workgroups of `threads` threads (1..1024, a multiple of 64) on `stream`.
 * Its duration is the floor under which no launch of that grid can go (the
 * dispatch of its workgroups and the launch's fixed cost), the yardstick for
 * the small copy-in and write-back launches.  Errors: EINVAL (workgroups < 1,
 * bad threads, or workgroups * threads >= 2^32), EHIP. */
int fsdppack_empty_launch(int32_t workgroups, int32_t threads, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDPPACK_H */
