// tree_reg.hip -- the tree and double-tree schedules for n <= 16, evaluated in
// registers in one pass.
//
// The tree schedule's result at every element is one expression over the n
// contributions, fixed by the tree: each rank's partial is pre(own) combined
// with its first child's partial, then its second child's ("NCCL all-reduce"
// post, section "The double binary tree"; partials rounded to the storage type
// at every combine), the root's partial is finished and broadcast.  On one GPU
// the up and down phases are memory traffic only, so a lane loads the n
// vectors of its position, evaluates that expression with the shape folded in
// at compile time (tree_shape.hpp, the same functions that build the host's
// shape), and stores the root's value to every rank: every byte read once and
// written once, as in the fused pass, instead of staging partials level by
// level through LDS.  The double tree takes the first tree over vectors
// [0, g.split) and the second over [g.split2, Vfull): grid y picks the range,
// so the choice is uniform per workgroup.  Bit-identical to the LDS-staged
// kernels (and the oracle's trees).
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"
#include "fused_common.hpp"
#include "tree_shape.hpp"

namespace ar {

template <int NR, int WHICH> struct ConstTree {
    static constexpr TreeTopo T = tree_topo(NR, WHICH);
};

// Partials of the ranks post[I], post[I+1], ... (children before parents).
template <int DT, int OP, int NR, int WHICH, int I>
__device__ __forceinline__ void tree_up(const u32x4 (&raw)[NR], Pack<DT> (&val)[NR], float s) {
    if constexpr (I < NR) {
        constexpr int r = ConstTree<NR, WHICH>::T.post[I];
        constexpr int c0 = ConstTree<NR, WHICH>::T.child[r][0];
        constexpr int c1 = ConstTree<NR, WHICH>::T.child[r][1];
        val[r] = first<DT, OP>(unpack<DT>(raw[r]), s);
        if constexpr (c0 >= 0) merge<DT, OP>(val[r], val[c0]);
        if constexpr (c1 >= 0) merge<DT, OP>(val[r], val[c1]);
        tree_up<DT, OP, NR, WHICH, I + 1>(raw, val, s);
    }
}

template <int DT, int OP, int NR, int WHICH>
__device__ __forceinline__ u32x4 tree_value(const u32x4 (&raw)[NR], const Geometry &g) {
    Pack<DT> val[NR];
    tree_up<DT, OP, NR, WHICH, 0>(raw, val, g.s);
    constexpr int root = ConstTree<NR, WHICH>::T.root;
    finish<DT, OP>(val[root], NR, g);
    return pack<DT>(val[root]);
}

template <int DT, int OP, int NR, bool DUAL>
__global__ __launch_bounds__(kFusedThreads) void tree_reg_kernel(const RankTableFor<NR> t, const Geometry g) {
    const bool second = DUAL && blockIdx.y == 1;
    const long long lo = second ? g.split2 : 0;
    const long long hi = (DUAL && !second) ? g.split : g.Vfull;
    const TileSpan ts = aligned_tile(lo, hi, (long long)blockIdx.x, g.ref, kFusedTile);
    if (ts.lo >= ts.hi) return;
    bool ok;
    const unsigned lane_off = tile_lane(ts, ts.start + threadIdx.x, ok);
    const long long base = ts.lo * 16;
    u32x4 raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        raw[r] = __builtin_nontemporal_load((const u32x4 *)((const char *)t.src[r] + base + lane_off));
    __builtin_amdgcn_sched_barrier(0);                       // every load issued before the first combine
    u32x4 w;
    if (second) w = tree_value<DT, OP, NR, 1>(raw, g);
    else w = tree_value<DT, OP, NR, 0>(raw, g);
    if (!ok) return;
#pragma unroll
    for (int r = 0; r < NR; ++r) __builtin_nontemporal_store(w, (u32x4 *)((char *)t.dst[r] + base + lane_off));
}

hipError_t launch_tree_reg_allreduce(bool dual, int dt, int op, const RankTable &t, const Geometry &g, int lds,
                                     hipStream_t s) {
    if (g.n < 2 || g.n > 16) return hipErrorInvalidValue;
    const long long len = dual ? (g.split > g.Vfull - g.split2 ? g.split : g.Vfull - g.split2) : g.Vfull;
    if (len <= 0) return hipSuccess;
    const dim3 grid((unsigned)aligned_tiles(len, kFusedTile), dual ? 2u : 1u);
    return dispatch(dt, op, [&](auto D, auto O) {
        return by_ranks(g.n, [&](auto R) {
            constexpr int NR = decltype(R)::value;
            if constexpr (NR == 0) {
                return hipErrorInvalidValue;
            } else {
                const RankTableFor<NR> tn = narrow<NR>(t);
                if (dual)
                    return launch(tree_reg_kernel<decltype(D)::value, decltype(O)::value, NR, true>, grid,
                                  dim3(kFusedThreads), (size_t)lds, s, tn, g);
                return launch(tree_reg_kernel<decltype(D)::value, decltype(O)::value, NR, false>, grid,
                              dim3(kFusedThreads), (size_t)lds, s, tn, g);
            }
        });
    });
}

}  // namespace ar
