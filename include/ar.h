/*
 * ar.h -- ring / tree collectives over N rank buffers held in ONE GPU's HBM.
 *
 * C ABI of libar.so (HIP kernels for gfx950 / MI355X).  N logical ranks are N
 * separate device buffers of `count` elements each; a "send" from rank r to
 * rank d is a read of r's buffer and a write (or read-modify-write) of d's.
 *
 * Sources, cited by page title and section:
 *   [L09] "第09讲：网络通信基础与集合通信 Collective 原语直觉" (Lecture 09,
 *         collective primitives): 3.1 Broadcast, 3.4 reduction operators,
 *         3.5 AllReduce, 3.6 ReduceScatter, 3.7 AllGather, 3.9 AllReduce =
 *         ReduceScatter + AllGather, 4.2-4.4 ring, 5.2 double binary tree.
 *   [CH4] "4. 通信模式：集合通信（AllReduce、AllGather等）原理与实现"
 *         (Chapter 4, communication patterns): 4.3.1 ring, 4.3.2 tree.
 *   [SCR] "从零实现集合通信" (Collectives from scratch): section "two-pass
 *         ring allreduce" (两趟实现 ring allreduce) and its cost table.
 *
 * Conventions shared by every collective below
 * --------------------------------------------
 * bufs    HOST array of `nranks` DEVICE pointers; bufs[r] is rank r's buffer
 *         of `count` contiguous elements of `dtype`.  Every buffer must be
 *         aligned to the element size, and no two buffers may overlap.  When
 *         every buffer is 16-byte aligned the kernels move 16-byte packs;
 *         otherwise they move one element at a time, with the same
 *         arithmetic in the same order (identical results, lower speed).  The
 *         caller allocates and owns every buffer; the library never
 *         allocates user memory and keeps no pointer after returning (the
 *         pointers travel inside kernel arguments).
 * nranks  N, 1 <= N <= AR_MAX_RANKS.
 * count   T, elements per rank.  Chunk layout: C = ceil(T/N), chunk c =
 *         [c*C, min(T, (c+1)*C)); only trailing chunks are short, and a chunk
 *         is empty when c*C >= T.  Rank c owns chunk c.
 * stream  a hipStream_t (NULL = the null stream of the
 *         calling thread's current device, which must then be the device
 *         that holds the buffers; a non-null stream carries its device).  Calls are
 *         asynchronous and stream-ordered: they enqueue kernels and return;
 *         the library never synchronises.  Completion is observed through
 *         the stream.  All buffers are updated IN PLACE.
 * Arithmetic (the receiver stores `local (+) incoming`, as in the pages'
 *         per-hop in-place add [L09 7.1][CH4 4.3.1]):
 *           AR_INT32    two's-complement wrap-around for SUM and PROD;
 *           AR_FLOAT32  one IEEE binary32 operation, round to nearest even,
 *                       subnormals kept, never fused or reassociated;
 *           AR_BFLOAT16 widen both to binary32, apply the op, round back to
 *                       bfloat16 to nearest even after EVERY hop (a NaN
 *                       stays a NaN; its payload bits are unspecified);
 *           MAX / MIN   keep the local value unless the incoming one compares
 *                       strictly greater / smaller.
 *         The ring calls reproduce the ring's order per element exactly
 *         (chunk c folds ranks c+1, c+2, ..., c); the tree call reproduces the
 *         binomial double tree's pairing.  Results are therefore bit-exact
 *         and independent of the implementation chosen by ar_set_impl().
 * Errors  argument errors are reported synchronously BEFORE anything is
 *         enqueued, so such a call has no effect:
 *           AR_ERROR_INVALID_ARGUMENT  bufs or an entry NULL; nranks out of
 *               range; a pointer not aligned to the element size; two buffer
 *               ranges overlapping; count * element size overflowing; root
 *               out of range; unknown dtype or op;
 *           AR_ERROR_UNSUPPORTED       a valid request this build lacks;
 *           AR_ERROR_HIP               a kernel launch failed; the hipError_t
 *               is kept for ar_last_hip_error().  With the step
 *               implementation (or a fused ring or tree AllReduce that runs
 *               as two launches) the launches before the failing one may
 *               already be enqueued, so the buffers are then unspecified.  (Faults
 *               during execution surface at the caller's next
 *               synchronisation.)
 *         count == 0 or nranks == 1 is a valid no-op (AR_SUCCESS, nothing
 *         enqueued); with count == 0 the entries of bufs are not inspected
 *         (an empty tensor may have a NULL data pointer).
 * Counters every successful call adds the logical inter-rank bytes of its
 *         schedule (each transfer of k elements adds k * element size to the
 *         sender's `sent` and the receiver's `recv`) and its schedule steps
 *         to process-wide counters, whatever implementation runs.
 * Debug   with the environment variable AR_DEBUG set (and not "0") when the
 *         library loads, every call with work to do first builds the logical
 *         schedule it follows and checks it: every transfer inside the
 *         buffers and between two distinct ranks, no transfer of a step
 *         writing what another one of the step reads or writes [the ring's
 *         within-step disjointness, L09 4.3], the documented step count, and
 *         per-rank bytes equal to what the counters add.  A violation, which
 *         would be a defect of this library, is printed to stderr and aborts
 *         the process; nothing of that call is enqueued.
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <stdint.h>

/* The HIP stream handle, declared as HIP's runtime API declares it (an
 * opaque pointer), so that this header needs no HIP include; including
 * <hip/hip_runtime_api.h> before or after it is fine. */
typedef struct ihipStream_t* hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 64
#define AR_VERSION 1

typedef enum {
  AR_SUCCESS = 0,
  AR_ERROR_INVALID_ARGUMENT = 1,
  AR_ERROR_UNSUPPORTED = 2,
  AR_ERROR_HIP = 3
} ar_status_t;

/* AR_BFLOAT16_ACC32: bfloat16 buffers ("bf16 with fp32 accumulation").  The
 * reductions (ring AllReduce and ReduceScatter, tree AllReduce, Reduce)
 * carry float32 partials from hop to hop in the schedule's own order and
 * round to bfloat16 once, at the end; a partial cannot live in a bfloat16
 * buffer between kernel launches, so these reductions run fused under either
 * implementation.  Copies (AllGather, Broadcast, Scatter, Gather, AllToAll)
 * are bfloat16 copies.  Elements count 2 bytes in every byte counter. */
typedef enum {
  AR_INT32 = 0,
  AR_FLOAT32 = 1,
  AR_BFLOAT16 = 2,
  AR_BFLOAT16_ACC32 = 3
} ar_dtype_t;

/* The reduction operators listed in [L09 3.4]. */
typedef enum { AR_SUM = 0, AR_PROD = 1, AR_MAX = 2, AR_MIN = 3 } ar_op_t;

typedef enum {
  AR_RING_ALLREDUCE = 0,
  AR_REDUCE_SCATTER = 1,
  AR_ALLGATHER = 2,
  AR_BROADCAST = 3,
  AR_TREE_ALLREDUCE = 4,
  AR_REDUCE = 5,
  AR_SCATTER = 6,
  AR_GATHER = 7,
  AR_ALLTOALL = 8
} ar_collective_t;

/* How a collective is executed; results are bit-identical either way.
 *   AR_IMPL_FUSED  one pass: every element's N inputs are read once, folded
 *                  in the schedule's order (tiles staged through LDS, the
 *                  partials in registers), and the result is written once
 *                  per destination rank; the copies (AllGather, Broadcast)
 *                  read each element once and write it into every other
 *                  rank, one destination rank per pass.  The AllReduces of
 *                  12 or more ranks and 384 MiB or more of inputs run as two
 *                  such launches (see ar_ring_allreduce, ar_tree_allreduce).
 *   AR_IMPL_STEP   the schedule literally: one kernel launch per ring step or
 *                  tree round, each applying all of that step's transfers. */
typedef enum { AR_IMPL_FUSED = 0, AR_IMPL_STEP = 1 } ar_impl_t;

/* Ring AllReduce [L09 3.5, 3.9, 4.3][CH4 4.3.1][SCR two-pass ring]:
 * ReduceScatter then AllGather.  Afterwards every bufs[r] holds, at element
 * i of chunk c, the fold x[c+1][i] (+) ... (+) x[c][i] taken in ring order
 * (each hop: the receiving rank's own value (+) the incoming partial).
 * AR_IMPL_FUSED: one fold storing into every rank; from 12 ranks and 384 MiB
 * of inputs (nranks * count * element size) up, the fused ReduceScatter and
 * then the fused AllGather (two launches, the same bits, faster there). */
ar_status_t ar_ring_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream);

/* Ring ReduceScatter [L09 3.6][SCR two-pass ring, first pass]: N-1 steps; at
 * step t rank r forwards chunk (r-t-1) mod N to rank r+1, which stores
 * own (+) incoming.  Afterwards chunk r of bufs[r] holds the full reduction of
 * chunk r (same fold as ar_ring_allreduce).  The contents of the other chunks
 * of every buffer are UNSPECIFIED afterwards (partials or inputs, depending
 * on the implementation). */
ar_status_t ar_reduce_scatter(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream);

/* Ring AllGather [L09 3.7][SCR two-pass ring, second pass]: the input of
 * rank r is chunk r of bufs[r] (its other chunks are ignored and
 * overwritten); N-1 steps, at step t rank r forwards chunk (r-t) mod N to
 * rank r+1, which overwrites.  Afterwards every buffer holds every rank's
 * chunk. */
ar_status_t ar_allgather(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                         hipStream_t stream);

/* Broadcast [L09 3.1][SCR cost table: T bytes over a log2 N tree]: every
 * bufs[r] ends equal to bufs[root].  Schedule (and counters): a binomial tree
 * on roles (r - root) mod N, ceil(log2 N) rounds. */
ar_status_t ar_broadcast(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                         hipStream_t stream);

/* Double-binary-tree AllReduce [L09 5.2][CH4 4.3.2][SCR cost table:
 * 2 log2 N steps].  Two binomial trees reduce toward role 0 and broadcast
 * back, each over half the data: tree 0 handles elements [0, ceil(T/2)) with
 * role == rank, tree 1 handles [ceil(T/2), T) with role == N-1-rank.  Reduce
 * round k: role q (q mod 2^(k+1) == 0, q + 2^k < N) stores
 * own (+) value of role q + 2^k.  Every bufs[r] ends with role 0's result.
 * AR_IMPL_FUSED: one fold storing into every rank; from 12 ranks and 384 MiB
 * of inputs up, the two trees' folds stored into their roots (rank 0, rank
 * N-1) and then both halves fanned out from there (two launches, the same
 * bits, faster there). */
ar_status_t ar_tree_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream);

/* ---- rooted primitives ------------------------------------------------------ */

/* Reduce to `root` [L09 3.4]: bufs[root] ends with the reduction of every
 * rank's buffer; every other buffer keeps its data.  Order: the reduce
 * rounds of a binomial tree on roles (rank - root) mod N over the whole
 * buffer (the rounds of ar_tree_allreduce [L09 5.2]): round k, role q
 * (q mod 2^(k+1) == 0, q + 2^k < N) stores own (+) value of role q + 2^k;
 * the partials live in registers, never in a rank buffer.  One fused kernel
 * runs under either implementation.  Counters: each non-root rank sends its
 * buffer once to its parent; ceil(log2 N) steps.  root out of range ->
 * AR_ERROR_INVALID_ARGUMENT. */
ar_status_t ar_reduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, ar_op_t op,
                      int root, hipStream_t stream);

/* Scatter from `root` [L09 3.2]: chunk c of bufs[root] (the ring chunk
 * layout above) is copied into chunk c of bufs[c] for every c != root; every
 * other element of every buffer is unchanged.  One step of N-1 direct
 * transfers. */
ar_status_t ar_scatter(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                       hipStream_t stream);

/* Gather to `root` [L09 3.3]: chunk c of bufs[c] is copied into chunk c of
 * bufs[root] for every c != root, so the root holds every rank's shard in
 * rank order; the other buffers are unchanged.  One step of N-1 direct
 * transfers. */
ar_status_t ar_gather(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                      hipStream_t stream);

/* AllToAll [L09 3.8, lab 4 in 7.4]: every buffer is N equal blocks of
 * count/N elements; block j of bufs[i] is meant for rank j, which receives
 * it in block i (recv[j][i] = send[i][j], a transpose across ranks).  Block
 * i of bufs[i] stays in place.  count must be a multiple of nranks
 * (otherwise AR_ERROR_INVALID_ARGUMENT).  One step: each rank sends and
 * receives (N-1) blocks.  One kernel swaps block j of rank i with block i of
 * rank j for every pair i < j, under either implementation. */
ar_status_t ar_alltoall(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                        hipStream_t stream);

/* ---- size-based choice between ring and tree ----------------------------- */

/* AllReduce that picks the ring or the double tree by message size [L09 5.3:
 * NCCL runs the tree for small messages and the ring for large ones][SCR
 * exercises: ring vs tree at 1 KB, 1 MB and 16 MB].  It predicts the time of
 * both under the current implementation (ar_set_impl) with the cost model
 * below and runs ar_ring_allreduce or ar_tree_allreduce, whichever is lower
 * (the ring on a tie).  Arguments, errors and counters are those of the call
 * it runs; its result is that call's result bit for bit. */
ar_status_t ar_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                         ar_op_t op, hipStream_t stream);

/* The collective ar_allreduce would run (AR_RING_ALLREDUCE or
 * AR_TREE_ALLREDUCE) for these arguments under the current implementation.
 * Host only. */
ar_status_t ar_allreduce_choice(int nranks, size_t count, ar_dtype_t dtype,
                                ar_collective_t* choice);

/* Kernel launches and HBM bytes of one call of `coll` under `impl` with these
 * arguments, as the library will run it: AR_IMPL_FUSED is one launch moving
 * every input once and every output once (2 N T s for an AllReduce), except
 * the AllReduces from 12 ranks and 384 MiB of inputs, which are two launches
 * moving (2 N + 1) T s; AR_IMPL_STEP is one launch per schedule step moving
 * 3 bytes per element of every reduce transfer (read both sides, write one)
 * and 2 per element of every copy transfer.  Reduce and AllToAll run their
 * one kernel, Scatter and Gather their one step (root 0), under either;
 * bfloat16 with float32 partials runs its reductions fused.  0 launches and
 * 0 bytes when nranks == 1.  AR_ERROR_INVALID_ARGUMENT for an out-of-range
 * argument or a NULL output pointer.  Host only. */
ar_status_t ar_launch_plan(ar_collective_t coll, ar_impl_t impl, int nranks, size_t count,
                           ar_dtype_t dtype, int* launches, uint64_t* hbm_bytes);

/* Cost model, the single-GPU form of the pages' alpha-beta model [L09 1.3,
 * 7.3]: predicted microseconds of one call
 *     = launches * alpha_us + hbm_bytes / (gbps * 1e3)
 * with launches and hbm_bytes those of ar_launch_plan.  One (alpha_us, gbps)
 * pair is kept per (collective, implementation); the defaults are fitted to
 * the message-size sweep measured on MI355X.  Host only. */
ar_status_t ar_predict_time(ar_collective_t coll, ar_impl_t impl, int nranks, size_t count,
                            ar_dtype_t dtype, double* microseconds);
ar_status_t ar_set_cost_model(ar_collective_t coll, ar_impl_t impl, double alpha_us,
                              double gbps);
ar_status_t ar_get_cost_model(ar_collective_t coll, ar_impl_t impl, double* alpha_us,
                              double* gbps);

/* ---- host-only helpers: no GPU work, usable without a GPU ---------------- */

/* C = ceil(count / nranks); 0 if nranks < 1. */
size_t ar_chunk_size(int nranks, size_t count);

/* Bounds [*begin, *end) of chunk `chunk`; AR_ERROR_INVALID_ARGUMENT if nranks
 * or chunk is out of range or an output pointer is NULL. */
ar_status_t ar_chunk_range(int nranks, size_t count, int chunk, size_t* begin, size_t* end);

/* Logical bytes each rank sends and receives in one call of `coll` with these
 * arguments ([SCR cost table]; e.g. 2T(N-1)/N per rank for the ring when N
 * divides T).  sent and recv are caller arrays of nranks uint64_t.  `root`
 * is used for AR_BROADCAST, AR_REDUCE, AR_SCATTER and AR_GATHER only;
 * AR_ALLTOALL needs count to be a multiple of nranks. */
ar_status_t ar_expected_bytes(ar_collective_t coll, int nranks, size_t count, ar_dtype_t dtype,
                              int root, uint64_t* sent, uint64_t* recv);

/* Schedule steps of one call: 2(N-1) ring AllReduce, N-1 ReduceScatter and
 * AllGather, ceil(log2 N) Broadcast and Reduce, 2 ceil(log2 N) tree
 * AllReduce, 1 Scatter, Gather and AllToAll (0 for every collective when
 * N == 1); -1 on a bad argument. */
int ar_expected_steps(ar_collective_t coll, int nranks);

/* Process-wide cumulative counters since load or the last reset [SCR
 * exercises: per-rank byte counter].  Copies the first nranks entries
 * (0 <= nranks <= AR_MAX_RANKS) of the logical bytes each rank sent and
 * received into sent / recv (either may be NULL).  Thread-safe. */
ar_status_t ar_counters_read(int nranks, uint64_t* sent, uint64_t* recv);
/* Total schedule steps counted since load or the last reset. */
uint64_t ar_counters_steps(void);
void ar_counters_reset(void);

/* Process-wide choice of implementation for subsequent calls (initially
 * AR_IMPL_FUSED, or AR_IMPL_STEP when the environment variable AR_IMPL is
 * "step" at load).  Thread-safe. */
ar_status_t ar_set_impl(ar_impl_t impl);
ar_impl_t ar_get_impl(void);

/* Static description of a status code. */
const char* ar_status_string(ar_status_t status);

/* hipError_t of this thread's most recent AR_ERROR_HIP (0 if none). */
int ar_last_hip_error(void);

/* AR_VERSION of the loaded library. */
int ar_version(void);

/* ---- testing ---------------------------------------------------------------- */

/* For callers' tests of their AR_ERROR_HIP handling (the error path of the
 * "Errors" paragraph above, which a healthy GPU never takes): the k-th kernel
 * launch the library attempts from now on (k >= 1; a collective call makes
 * one launch, or one per step with AR_IMPL_STEP, or two for the two-launch
 * AllReduces, and none when it is a no-op) reports hipErrorLaunchFailure
 * instead of being enqueued.  That call then returns AR_ERROR_HIP with nothing more enqueued,
 * ar_last_hip_error() gives hipErrorLaunchFailure on its thread, the
 * launches it made before stay enqueued, and the counters are not updated.
 * The injection is spent by that launch; k == 0 disarms it.  Process-wide;
 * host only; AR_ERROR_INVALID_ARGUMENT for k < 0. */
ar_status_t ar_debug_fail_launch(int k);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
