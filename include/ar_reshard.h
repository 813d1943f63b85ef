/*
 * ar_reshard.h -- C ABI of libar's M-to-N layout reshard: M source ranks hold
 * a global tensor in one layout, N destination ranks need it in another, and
 * every rank is a buffer in one MI355X's HBM.
 *
 * Source: "NCCL M2N: A Layout- and Topology-Aware Collective for Distributed
 * Tensor Resharding" (arxiv.org/html/2610.07516):
 *
 *   layout (§IV)   L = (S, M, p): a global shape S, a process mesh M of
 *                  D_0 x D_1 slots anchored at base rank r_0, and one
 *                  placement per mesh axis, Shard(d) or Replicate.  Slot
 *                  (i_0, i_1) is communicator rank r_0 + i_0*D_1 + i_1
 *                  (Eq. (1)); its local shard spans, along tensor dimension d,
 *                  [floor(i_k*S_d/D_k), floor((i_k+1)*S_d/D_k)) when axis k
 *                  shards d and [0, S_d) otherwise (Eq. (2)).  A local buffer
 *                  holds its shard contiguously in row-major order.
 *   reshard (§IV)  when the call completes every destination slot holds the
 *                  local shard of S its layout prescribes.
 *   schedule (§V-A)  for each source and destination the per-dimension
 *                  overlap [max(l), min(u)); empty overlaps are skipped;
 *                  replicated source copies collapse to one owner (here: the
 *                  lowest slot holding the shard; other replicas are never
 *                  read and may be passed as NULL).
 *   leaders (§V-B) per destination shard j with q_j contributions (ordered
 *                  by source shard) and rho replicas per domain, every
 *                  replica of the first domain takes floor(q_j/rho) of them
 *                  and the first q_j mod rho one more.
 *
 * Routes (all produce identical bytes; they differ in HBM traffic):
 *   FLAT   one copy per (source, destination) transfer: every contribution
 *          is read once per destination replica (2 * r * B bytes for r
 *          replicas of a B-byte payload);
 *   HIER   the hierarchical route with every replica in one domain: each
 *          contribution is copied once into its leader replica, then every
 *          leader's regions are copied to the other replicas ((2 + r) * B);
 *   FUSED  each contribution is read once and written to all r replicas of
 *          its destination shard in the same pass ((1 + r) * B): on one GPU
 *          the leader's local fan-out needs no intermediate copy.
 *   AUTO   the cost model's choice: launches * launch cost + bytes / measured
 *          bandwidth (fused on one GPU, where all replicas share one HBM).
 *
 * Scope: tensors of 1 to 3 dimensions, meshes of 1 or 2 axes with at most
 * 128 slots, any placement in which no tensor dimension is sharded by two
 * axes; element sizes 1, 2, 4, 8 or 16 bytes (a reshard only moves bytes, so
 * any type of that size).  Shard sizes need not divide evenly (Eq. (2)).
 *
 * Buffers and ownership: ``src_bufs`` (one entry per source mesh slot, in
 * slot order = communicator rank - r_0) and ``dst_bufs`` (one per
 * destination slot) are HOST arrays of DEVICE pointers on the current HIP
 * device; the caller owns arrays and buffers, the library reads the arrays
 * during the call only and allocates no device memory.  Pointers must be
 * aligned to the element size; a call whose addresses, row lengths and
 * strides are all multiples of 16 bytes uses 16-byte vectors, any other call
 * an element-wise path with the same result.  No destination buffer may
 * overlap another destination buffer or a source buffer that is read
 * (AR_ERR_INVALID_ARG).
 *
 * Ordering: asynchronous on ``stream``; AR_OK means the work was enqueued.
 * Errors: arguments are validated before any launch; status codes only.
 * A tensor with no elements returns AR_OK without a launch.
 */
#ifndef AR_RESHARD_H
#define AR_RESHARD_H

#include "ar.h"

#ifdef __cplusplus
extern "C" {
#endif

#define AR_RESHARD_MAX_DIMS 3
#define AR_RESHARD_MAX_MESH_DIMS 2
#define AR_RESHARD_MAX_SLOTS 128
#define AR_REPLICATE (-1)

/* One endpoint layout (S, M, p) of §IV. */
typedef struct {
    int ndim;                                   /* tensor dimensions, 1..3 */
    long long shape[AR_RESHARD_MAX_DIMS];       /* global shape S, every S_d >= 0 */
    int mesh_ndim;                              /* mesh axes, 1..2 */
    int mesh[AR_RESHARD_MAX_MESH_DIMS];         /* D_k >= 1; product <= AR_RESHARD_MAX_SLOTS */
    int placement[AR_RESHARD_MAX_MESH_DIMS];    /* AR_REPLICATE, or d in [0, ndim) for Shard(d) */
    int base_rank;                              /* r_0 of Eq. (1); names ranks in plans only */
} ar_layout_t;

typedef enum { AR_ROUTE_AUTO = 0, AR_ROUTE_FLAT = 1, AR_ROUTE_HIER = 2, AR_ROUTE_FUSED = 3 } ar_route_t;

/* One §V-A transfer: the box [lo, hi) (global coordinates, per tensor
 * dimension; unused dimensions hold [0, 1)) that source rank ``src_rank``
 * contributes to destination rank ``dst_rank``; ``leader_rank`` is the
 * replica of dst_rank's shard that receives the contribution first in the
 * hierarchical route (§V-B). */
typedef struct {
    int src_rank;
    int dst_rank;
    int leader_rank;
    long long lo[AR_RESHARD_MAX_DIMS];
    long long hi[AR_RESHARD_MAX_DIMS];
    long long bytes;
} ar_transfer_t;

/* Plan summary; arrays indexed by ar_route_t (entry 0, AUTO, unused). */
typedef struct {
    ar_route_t chosen;          /* the cost model's route */
    int n_transfers;            /* §V-A transfers (source owner, destination slot) */
    int n_sources;              /* owner source slots (replicas collapsed) */
    int n_shards;               /* distinct destination shards K */
    int max_replicas;           /* most replicas of one destination shard */
    long long unique_bytes;     /* B: one copy of every destination shard */
    double bytes[4];            /* HBM bytes each route moves */
    int launches[4];            /* kernel launches each route needs */
    double predicted_us[4];     /* launches * launch_us + bytes / bandwidth */
} ar_reshard_plan_t;

/* Eq. (2) and Eq. (1): the local shard of mesh slot ``slot`` under
 * ``layout`` as [lo[d], hi[d]) per tensor dimension (AR_RESHARD_MAX_DIMS
 * entries each; unused dimensions [0, 1)), and its communicator rank in
 * ``*rank`` when ``rank`` is not NULL.  A local buffer of that slot holds
 * prod(hi - lo) elements.  AR_ERR_INVALID_ARG for a malformed layout or a
 * slot outside [0, D_0 * D_1); AR_ERR_UNSUPPORTED as ar_reshard_plan. */
ar_status_t ar_layout_shard(const ar_layout_t *layout, int slot, long long *lo, long long *hi, int *rank);

/* Plan a reshard from ``src`` to ``dst`` for elements of ``elem_size`` bytes,
 * with the destination replicas of every shard split evenly over ``domains``
 * domains (leaders come from the first; 1 = every replica local, the
 * arrangement ar_reshard runs).  Fills ``out`` and, when ``transfers`` is not
 * NULL, up to ``max_transfers`` transfers in (source owner slot, destination
 * slot) order; out->n_transfers is the full count.  Host only: no GPU needed.
 * AR_ERR_INVALID_ARG for malformed layouts, different global shapes, a
 * domain count that does not divide every shard's replica count;
 * AR_ERR_UNSUPPORTED for a tensor dimension sharded by two axes or an
 * element size outside {1, 2, 4, 8, 16}. */
ar_status_t ar_reshard_plan(const ar_layout_t *src, const ar_layout_t *dst, size_t elem_size, int domains,
                            ar_reshard_plan_t *out, ar_transfer_t *transfers, int max_transfers);

/* Run the reshard on ``stream`` with ``route`` (AR_ROUTE_AUTO: the cost
 * model's choice).  ``src_bufs[s]`` must be valid for every owner source slot
 * (NULL allowed for the other replicas); ``dst_bufs[t]`` for every
 * destination slot; NULL is also allowed for any slot whose shard has no
 * elements (Eq. (2) gives empty shards when D_k > S_d).  Errors as
 * ar_reshard_plan, plus AR_ERR_INVALID_ARG for a NULL buffer that is needed
 * or overlapping buffers, AR_ERR_ALIGNMENT for a pointer not aligned to
 * elem_size, AR_ERR_HIP for a failed launch. */
ar_status_t ar_reshard(const void *const *src_bufs, void *const *dst_bufs, const ar_layout_t *src,
                       const ar_layout_t *dst, size_t elem_size, ar_route_t route, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AR_RESHARD_H */
