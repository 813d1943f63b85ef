/*
 * ar.h -- C ABI of libar: all-reduce, reduce-scatter and all-gather over n
 * logical ranks whose buffers all live in one MI355X's HBM.
 *
 * What the calls compute (sources: the "NCCL all-reduce" post on
 * rakshithvasudev.github.io, sections "What all-reduce promises", "The ring,
 * exactly as the kernel runs it", "The double binary tree" and "How NCCL
 * picks: a cost model, not a threshold"; and "FSDP collectives 101" on the
 * same site, sections "All-gather: everyone shows their piece", "Why backward
 * needs a different collective" and "DDP's all-reduce, chopped in half"):
 *
 *   all-reduce      every rank contributes one same-shaped buffer; the
 *                   buffers are combined element-wise and every rank ends with
 *                   the identical result.  It runs as reduce-scatter (each
 *                   rank finishes one chunk) followed by all-gather (the
 *                   finished chunks circulate unchanged).
 *   reduce-scatter  every rank contributes n*R elements; rank r keeps the
 *                   combined slice r (R elements).
 *   all-gather      every rank contributes R elements; every rank receives
 *                   the concatenation of all pieces, in rank order.  No
 *                   arithmetic: outputs are bit copies.
 *
 * Ops: sum, prod, min, max, avg.  avg pre-scales every floating-point
 * contribution by fp32(1/n) as it is read; for int32 the finished sum is
 * divided by n once (truncating toward zero) where the chunk completes.
 * int32 sum and prod wrap modulo 2^32.  bf16/fp16 values are combined in fp32
 * and rounded (to nearest even) back to the storage type after every hop.
 *
 * Reduction order (the hop order of the ring): chunk c of an all-reduce is
 * finished at rank c; its chain starts with rank c+1's contribution and adds
 * ranks c+2, ..., c in turn (indices mod n), the incoming partial being the
 * left operand.  The fused and ring schedules both follow this order, so
 * their floating-point results are identical bit for bit.  The tree schedule
 * reduces up the bit-trick binary tree rooted at rank 0 (own value first,
 * then the children in ascending rank order) and broadcasts back down.
 * The dtree schedule (all-reduce only) is the double binary tree: the first
 * u*floor(V/2) elements (u, V below) are reduced up and broadcast down the
 * tree above, the rest up its complement, whose leaves are the first tree's
 * interior ranks: the mirror image (rank v in the place of rank n-1-v) when n
 * is even, the same tree shifted by one rank (rank v in the place of rank
 * v-1) when n is odd; each tree combines own value first, then the children
 * in ascending rank order, and its root applies the postOp.
 * The split schedule (all-reduce only) is the fused single pass with every
 * rank combined at once, in the aligned pairwise order over rank indices:
 * ranks [lo, lo+len) combine as [lo, lo+h) (+) [lo+h, lo+len), h the largest
 * power of two below len, the lower ranks being the left operand; every
 * contribution enters as a storage-type value (float avg pre-scaled), every
 * combine is rounded to the storage type, int32 avg divides the total once.
 * Its floating-point sums therefore differ from the ring's in the last bits
 * (integer results, min and max are the same under every schedule).
 * All-reduce chunks are cut in 16-byte units:
 *   u = 16 / element size, V = ceil(count / u),
 *   chunk c = [u*floor(c*V/n), u*floor((c+1)*V/n)) clamped to count.
 * Reduce-scatter and all-gather use the equal split of R elements per rank.
 *
 * Buffers and ownership: ``sendbufs`` and ``recvbufs`` are HOST arrays of n
 * DEVICE pointers, one buffer per logical rank, all on the current HIP device.
 * The caller owns the arrays and the buffers; the library reads the two
 * arrays during the call only (they are copied by value into the kernel
 * arguments) and allocates no device memory on any call.  Buffers must be
 * aligned to their element size; 16-byte alignment of every pointer selects
 * the vector paths.  All-reduce buffers that all sit at one 16-byte phase
 * (every address the same mod 16, e.g. views at one offset of per-rank flat
 * buffers) run the vector kernels from the first 16-byte boundary, the few
 * elements around it element-wise; reduce-scatter and all-gather do the same
 * when all inputs share one phase and all outputs share one (possibly another)
 * phase, and when R * element size is not a multiple of 16.  At mixed phases
 * with every pointer 4-byte aligned (always so for 4-byte elements),
 * all-reduces in ring order (AR_SCHED_RING, AR_SCHED_FUSED), reduce-scatters
 * and all-gathers of pieces of whole words run vector kernels on the pointers
 * as given (a 16-byte access needs only 4-byte alignment), the last count mod
 * lanes elements (the ends of each slice or piece) element-wise.  Other alignments take an element-wise
 * path.  Every path gives identical results.  Reading
 * through aligned 16-byte vectors, the reduce-scatter and all-gather may read
 * (never write) the rest of the 16-byte blocks that hold an input buffer's
 * first and last bytes.
 *
 * Aliasing: send buffers may alias one another (they are only read).
 *   all-reduce      in place when recvbufs[r] == sendbufs[r];
 *   reduce-scatter  in place when recvbufs[r] == sendbufs[r] + r*R elements;
 *   all-gather      in place when sendbufs[r] == recvbufs[r] + r*R elements.
 * Any other overlap between a receive range and another buffer's range is
 * rejected with AR_ERR_INVALID_ARG.
 *
 * Ordering: calls are asynchronous and ordered on ``stream`` (a hipStream_t;
 * NULL is the default stream).  AR_OK means the work was enqueued; results are
 * valid once the stream reaches that point.  Faults during execution surface
 * at the caller's next synchronisation.
 *
 * Errors: every call validates its arguments before launching anything and
 * returns a status code; nothing is printed (unless AR_DEBUG=1 is set in the
 * environment, which logs one line per planned call to stderr) and no
 * exception crosses the ABI.  count == 0 returns AR_OK without a launch.
 *
 * Environment: AR_SCHEDULE=auto|ring|tree|fused|split|dtree forces a schedule for calls
 * made with AR_SCHED_AUTO; AR_CALIB=<path> names the cost-model calibration
 * file (default: calib_gfx950.txt beside the library); AR_GRID=<n> overrides
 * the number of workgroups per launch.
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 128

typedef enum {
    AR_OK = 0,
    AR_ERR_INVALID_ARG = 1,   /* null pointer, n out of range, bad enum, overlapping buffers */
    AR_ERR_UNSUPPORTED = 2,   /* schedule not legal for this collective (tree, split, dtree for RS/AG) */
    AR_ERR_ALIGNMENT = 3,     /* a pointer not aligned to the element size */
    AR_ERR_HIP = 4            /* the HIP runtime reported an error (launch, device query) */
} ar_status_t;

typedef enum { AR_FLOAT32 = 0, AR_BFLOAT16 = 1, AR_FLOAT16 = 2, AR_INT32 = 3 } ar_dtype_t;
typedef enum { AR_SUM = 0, AR_PROD = 1, AR_MIN = 2, AR_MAX = 3, AR_AVG = 4 } ar_op_t;
typedef enum {
    AR_SCHED_AUTO = 0,
    AR_SCHED_RING = 1,
    AR_SCHED_TREE = 2,
    AR_SCHED_FUSED = 3,
    AR_SCHED_SPLIT = 4,
    AR_SCHED_DTREE = 5
} ar_sched_t;
typedef enum { AR_COLL_ALLREDUCE = 0, AR_COLL_REDUCE_SCATTER = 1, AR_COLL_ALL_GATHER = 2 } ar_coll_t;

/* Numerics of a floating-point reduction: the two accuracy trades named in
 * "FSDP collectives 101" (bf16 reductions accumulate in bf16 along the way,
 * which grows lossy with the number of ranks, hence reducing in fp32; fp16
 * averages split the divisor across pre- and post-scaling).  A zeroed struct
 * (or NULL) is the behaviour of ar_allreduce / ar_reduce_scatter. */
typedef enum {
    AR_ACC_STORAGE = 0,  /* every partial rounded to the storage type when it leaves a hop */
    AR_ACC_FP32 = 1      /* bf16 / fp16: partials stay fp32 and the result is rounded once where it
                          * completes; same bytes moved.  Only the fused schedule keeps partials in
                          * registers: other schedules return AR_ERR_UNSUPPORTED and AUTO picks fused.
                          * No effect for fp32 / int32. */
} ar_acc_t;
typedef enum {
    AR_AVG_PRESCALE = 0, /* float avg: every contribution times fp32(1/n) as it is read */
    AR_AVG_SPLIT = 1     /* float avg: every contribution times 1/p as read, p = 2^e with e the least
                          * integer such that 4^e >= n (a power of two near sqrt(n), so the pre-scale is
                          * exact), and the finished sum divided by n/p in fp32 before the final
                          * rounding: fewer underflows than 1/n, fewer overflows than sum-then-divide.
                          * Every schedule.  No effect for int32 or other ops. */
} ar_avg_t;
typedef struct {
    ar_acc_t acc;
    ar_avg_t avg;
} ar_numerics_t;

/* Result of the cost model, indexed by ar_sched_t (entry 0, AUTO, is unused).
 * predicted_us[s] = launch_us[s] + step_us[s] * steps[s] + bytes[s] / bandwidth[s]
 * for every legal schedule s; ``chosen`` is the legal schedule with the
 * smallest prediction (ties go to the lower enum value), except that the
 * fused schedule is chosen whenever its prediction is within 3 % of the
 * smallest (one-pass schedules moving the same bytes differ by less than the
 * spread between measurements). */
typedef struct {
    ar_sched_t chosen;
    unsigned legal_mask;        /* bit s set when schedule s is legal for the call */
    int steps[6];               /* dependent steps: ring 2(n-1) (n-1 for RS/AG), tree and dtree 2*depth, fused 1, split 1 */
    double bytes[6];            /* algorithmic HBM bytes the schedule moves */
    double predicted_us[6];     /* cost-model time; 0 for illegal schedules */
} ar_plan_t;

/* All-reduce ``count`` elements per rank.
 *   sendbufs[r], recvbufs[r]: device buffers of count elements (r = 0..n-1)
 *   n in [1, AR_MAX_RANKS]; sched = AR_SCHED_AUTO lets ar_plan choose.
 * Source: "NCCL all-reduce", sections "What all-reduce promises" and "The
 * ring, exactly as the kernel runs it" (ring), "The double binary tree"
 * (tree), "When the switch does the math" (one read and one write per byte:
 * the model for the fused single pass; every rank combined at once in an
 * order the switch leaves open: the split schedule). */
ar_status_t ar_allreduce(const void *const *sendbufs, void *const *recvbufs, size_t count,
                         ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched, hipStream_t stream);

/* All-reduce with explicit numerics (``numerics`` NULL: the defaults, as
 * ar_allreduce).  AR_ERR_INVALID_ARG for values outside the enums;
 * AR_ERR_UNSUPPORTED when the forced schedule cannot honour them. */
ar_status_t ar_allreduce_ex(const void *const *sendbufs, void *const *recvbufs, size_t count,
                            ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched,
                            const ar_numerics_t *numerics, hipStream_t stream);

/* Reduce-scatter: sendbufs[r] holds n*recvcount elements, recvbufs[r]
 * receives recvcount elements (slice r of the combined result).
 * Source: "FSDP collectives 101", section "Why backward needs a different
 * collective"; the ring's reduce-scatter half. Schedules: ring, fused
 * (tree, split and dtree: AR_ERR_UNSUPPORTED). */
ar_status_t ar_reduce_scatter(const void *const *sendbufs, void *const *recvbufs, size_t recvcount,
                              ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched, hipStream_t stream);

/* Reduce-scatter with explicit numerics (as ar_allreduce_ex).  FSDP's
 * "reduce in fp32" for bf16 gradients without moving fp32 bytes:
 * AR_ACC_FP32 reads and writes bf16 and keeps the partials in fp32. */
ar_status_t ar_reduce_scatter_ex(const void *const *sendbufs, void *const *recvbufs, size_t recvcount,
                                 ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched,
                                 const ar_numerics_t *numerics, hipStream_t stream);

/* All-gather: sendbufs[r] holds sendcount elements, recvbufs[r] receives
 * n*sendcount elements (x_0 || x_1 || ... || x_{n-1}).
 * Source: "FSDP collectives 101", section "All-gather: everyone shows their
 * piece"; the ring's all-gather half. Schedules: ring, fused
 * (tree, split and dtree: AR_ERR_UNSUPPORTED). */
ar_status_t ar_all_gather(const void *const *sendbufs, void *const *recvbufs, size_t sendcount,
                          ar_dtype_t dtype, int n, ar_sched_t sched, hipStream_t stream);

/* Cost model only (host, no GPU needed): fills *out for the call that
 * (coll, count, dtype, op, n) describes; ``count`` is the per-rank count of
 * ar_allreduce, the recvcount of ar_reduce_scatter or the sendcount of
 * ar_all_gather.  Source: "NCCL all-reduce", section "How NCCL picks: a cost
 * model, not a threshold" (time = latency + bytes / bandwidth, argmin per
 * call, no threshold). */
ar_status_t ar_plan(ar_coll_t coll, size_t count, ar_dtype_t dtype, ar_op_t op, int n, ar_plan_t *out);

/* Parent of rank v in the tree schedule's bit-trick binary tree over n ranks
 * (-1 for the root, rank 0, or for v outside [0, n)).  Host only.
 * Source: "NCCL all-reduce", section "The double binary tree". */
int ar_tree_parent(int n, int v);

/* Parent of rank v in tree ``which`` of the dtree schedule (0: the tree of
 * ar_tree_parent; 1: its complement, the mirror image for even n or the
 * one-rank shift for odd n); -1 for that tree's root or for v outside
 * [0, n).  Host only.  Source: "NCCL all-reduce", section "The double binary
 * tree" (a second tree with the roles of leaves and interior ranks swapped). */
int ar_dtree_parent(int n, int which, int v);

/* Human-readable name of a status code (static storage). */
const char *ar_status_string(ar_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* AR_H */
