// tree_fast.hpp -- the tree schedule's compile-time-n kernels (every n from
// 2 to 16), shared by the two translation units that instantiate them
// (tree.hip: n <= 8, tree_hi.hip: n = 9..16), so both compile in parallel.
//
// A window is W vectors at the same offset of every rank buffer.  NR * TPR
// threads, TPR per rank (TPR = 256 / the power of two at or above NR), each
// holding K = 8 vectors of its rank, so a thread keeps 8 loads in flight (the
// tree gives each rank one load per vector, so without K the window would be
// one HBM round trip for 16 bytes per thread).  LDS: one partial per rank and
// vector, NR * W * 16 bytes (at most 32 KB).  One workgroup per window.
#pragma once

#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

constexpr int kTreeK = 8;

template <int NR> struct TreeFastShape {
    static constexpr int P2 = NR <= 2 ? 2 : (NR <= 4 ? 4 : (NR <= 8 ? 8 : 16));
    static constexpr int TPR = kThreads / P2;      // threads per rank
    static constexpr int W = TPR * kTreeK;         // vectors per rank per window
    static constexpr int T = NR * TPR;             // threads per workgroup
};

// Vectors per rank in one window of the compile-time-n tree kernels.
inline long long tree_fast_window(int n) {
    const int p2 = n <= 2 ? 2 : (n <= 4 ? 4 : (n <= 8 ? 8 : 16));
    return (long long)(kThreads / p2) * kTreeK;
}

template <int DT, int OP, int NR>
__device__ __forceinline__ void tree_window_fast(const RankTable &t, const TreeShape &tree, const Geometry &g,
                                                 long long lo, long long hi, long long win, u32x4 *slot) {
    constexpr int TPR = TreeFastShape<NR>::TPR;
    constexpr int W = TreeFastShape<NR>::W;
    const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    const long long pos0 = lo + win * W + sub;
    u32x4 own[kTreeK];
    bool ok[kTreeK];
#pragma unroll
    for (int k = 0; k < kTreeK; ++k) {
        const long long v = pos0 + (long long)k * TPR;
        ok[k] = v < hi;
        own[k] = ld_stream(t.src[r], ok[k] ? v : lo);          // past hi: a valid, ignored load
    }
    __builtin_amdgcn_sched_barrier(0);
    const int d = tree.depth[r], root = tree.root;
    const int ch0 = tree.child[r][0], ch1 = tree.child[r][1], par = tree.parent[r];
    for (int lev = tree.max_depth; lev >= 0; --lev) {          // up: deepest level first
        if (d == lev) {
#pragma unroll
            for (int k = 0; k < kTreeK; ++k) {
                if (!ok[k]) continue;
                const int i = sub + k * TPR;
                Pack<DT> acc = first<DT, OP>(unpack<DT>(own[k]), g.s);
                if (ch0 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[ch0 * W + i]));
                if (ch1 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[ch1 * W + i]));
                if (r == root) finish<DT, OP>(acc, NR, g);
                slot[r * W + i] = pack<DT>(acc);
            }
        }
        __syncthreads();
    }
    for (int lev = 0; lev <= tree.max_depth; ++lev) {          // down: root first
        if (d == lev) {
#pragma unroll
            for (int k = 0; k < kTreeK; ++k) {
                if (!ok[k]) continue;
                const int i = sub + k * TPR;
                const u32x4 val = (r == root) ? slot[r * W + i] : slot[par * W + i];
                slot[r * W + i] = val;
                st_stream(t.dst[r], pos0 + (long long)k * TPR, val);
            }
        }
        __syncthreads();
    }
}

template <int DT, int OP, int NR, bool DUAL>
__global__ __launch_bounds__(kThreads) void tree_allreduce_fast(const RankTable t, const TreeShape tree0,
                                                                const TreeShape tree1, const Geometry g) {
    constexpr int W = TreeFastShape<NR>::W;
    __shared__ u32x4 slot[NR * W];
    const long long first = DUAL ? (g.split + W - 1) / W : (long long)gridDim.x;   // windows of the first tree
    const long long win = blockIdx.x;
    if (win < first) tree_window_fast<DT, OP, NR>(t, tree0, g, 0, DUAL ? g.split : g.Vfull, win, slot);
    else tree_window_fast<DT, OP, NR>(t, tree1, g, g.split, g.Vfull, win - first, slot);
}

// Launch the compile-time kernel for n in [LO, HI] (n must be in the range).
template <int LO, int HI, bool DUAL>
hipError_t launch_tree_fast_range(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                                  const Geometry &g, int lds, hipStream_t s) {
    if constexpr (LO > HI) {
        return hipErrorInvalidValue;
    } else {
        if (g.n != LO) return launch_tree_fast_range<LO + 1, HI, DUAL>(dt, op, t, tree, tree2, g, lds, s);
        constexpr long long W = TreeFastShape<LO>::W;
        const long long windows =
            DUAL ? (g.split + W - 1) / W + (g.Vfull - g.split + W - 1) / W : (g.Vfull + W - 1) / W;
        const dim3 blocks((unsigned)windows);
        return dispatch(dt, op, [&](auto D, auto O) {
            return launch(tree_allreduce_fast<decltype(D)::value, decltype(O)::value, LO, DUAL>, blocks,
                          dim3(TreeFastShape<LO>::T), (size_t)lds, s, t, tree, tree2, g);
        });
    }
}

// n = 9..16, instantiated in tree_hi.hip.
hipError_t launch_tree_fast_hi(bool dual, int dt, int op, const RankTable &t, const TreeShape &tree,
                               const TreeShape &tree2, const Geometry &g, int lds, hipStream_t s);

}  // namespace ar
