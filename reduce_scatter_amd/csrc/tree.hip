// tree.hip -- the log-step tree schedule, staged through LDS.
//
// The "NCCL all-reduce" post (rakshithvasudev.github.io), section "The double
// binary tree": ranks form a binary tree built by a bit trick (a rank's lowest
// set bit fixes its depth; its parent clears that bit and sets the next one
// up, falling back to just clearing it at the edge of the range).  Data is
// reduced from the leaves up to the root, every node adding its own
// contribution to what its children deliver, and the result is broadcast back
// down, every node keeping a copy.  2 * depth dependent steps instead of the
// ring's 2(n-1).
//
// These LDS-staged kernels serve n > 16 (and n <= 16 under AR_TREE_STAGED=1);
// up to 16 ranks tree_reg.hip evaluates the same trees in registers in one
// pass, with the same results.
//
// One workgroup runs the whole tree for a window of W vectors at the same
// offset of every rank buffer.  Item (rank v, vector w) holds rank v's
// contribution; LDS holds one partial per rank.  Up phase, deepest level
// first: partial(v) = own(v), then each child's partial in ascending rank
// order; the root applies the postOp.  Down phase, root first: each rank
// copies its parent's final value and stores it.  A workgroup barrier
// separates the levels.  All of a rank's loads are issued at the start
// (nothing they read depends on the tree), so the levels only wait on LDS.
//
// The double binary tree (same section: a second tree with the roles of
// leaves and interior ranks swapped, and half of every buffer sent up each)
// uses the same kernels with two host-built shapes: the windows of the first
// half take the first tree, those of the second half its complement.  On one
// GPU there are no per-rank links to balance, so it costs what the single tree
// costs; its results differ from the single tree's in the second half.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// One window of the generic kernel: vectors [pos0, pos0 + W) of every rank,
// clipped to hi, reduced up ``tree`` and broadcast down it.
template <int DT, int OP>
__device__ __forceinline__ void tree_window(const RankTable &t, const TreeShape &tree, const Geometry &g,
                                            long long pos0, long long hi, const int *r, const int *w, int cnt,
                                            u32x4 *slot) {
    const int n = g.n, W = g.W;
    u32x4 own[kItemsPerThread];
    bool ok[kItemsPerThread];
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        ok[k] = k < cnt && pos0 + w[k] < hi;
        if (ok[k]) own[k] = ld_stream(t.src[r[k]], pos0 + w[k]);
    }
    // up: deepest level first
    for (int d = tree.max_depth; d >= 0; --d) {
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            if (!ok[k] || tree.depth[r[k]] != d) continue;
            const int v = r[k];
            Pack<DT> acc = first<DT, OP>(unpack<DT>(own[k]), g.s);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int ch = tree.child[v][e];
                if (ch >= 0) merge<DT, OP>(acc, unpack<DT>(slot[ch * W + w[k]]));
            }
            if (v == tree.root) finish<DT, OP>(acc, n, g);
            slot[v * W + w[k]] = pack<DT>(acc);
        }
        __syncthreads();
    }
    // down: the root keeps its value; each level copies from its parent
    for (int d = 0; d <= tree.max_depth; ++d) {
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            if (!ok[k] || tree.depth[r[k]] != d) continue;
            const int v = r[k];
            const u32x4 val = (v == tree.root) ? slot[v * W + w[k]] : slot[tree.parent[v] * W + w[k]];
            slot[v * W + w[k]] = val;
            st_stream(t.dst[v], pos0 + w[k], val);
        }
        __syncthreads();
    }
}

// Any n: a persistent grid walks the windows.  A single tree takes the
// windows of [0, Vfull); the double tree (DUAL) takes the windows of
// [0, g.split) up the first tree and those of [g.split2, Vfull) up the second.
template <int DT, int OP, bool DUAL>
__global__ __launch_bounds__(kThreads) void tree_allreduce_kernel(const RankTable t, const TreeShape tree0,
                                                                  const TreeShape tree1, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    u32x4 *slot = (u32x4 *)lds;
    int r[kItemsPerThread], w[kItemsPerThread], cnt = 0;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        const int q = threadIdx.x + k * kThreads;
        r[k] = 0;
        w[k] = 0;
        if (q < n * W) {
            r[k] = q / W;
            w[k] = q - r[k] * W;
            cnt = k + 1;
        }
    }
    const long long first = DUAL ? (g.split + W - 1) / W : g.windows;     // windows of the first tree
    for (long long win = blockIdx.x; win < g.windows; win += gridDim.x) {
        if (win < first) tree_window<DT, OP>(t, tree0, g, win * W, DUAL ? g.split : g.Vfull, r, w, cnt, slot);
        else tree_window<DT, OP>(t, tree1, g, g.split2 + (win - first) * W, g.Vfull, r, w, cnt, slot);
    }
}


template <bool DUAL>
hipError_t launch_trees(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                        const Geometry &g, int grid, hipStream_t s) {
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(tree_allreduce_kernel<decltype(D)::value, decltype(O)::value, DUAL>, dim3(grid), dim3(kThreads),
                      (size_t)g.n * g.W * 16, s, t, tree, tree2, g);
    });
}

hipError_t launch_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                 int grid, hipStream_t s) {
    return launch_trees<false>(dt, op, t, tree, tree, g, grid, s);
}

hipError_t launch_dtree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                                  const Geometry &g, int grid, hipStream_t s) {
    return launch_trees<true>(dt, op, t, tree, tree2, g, grid, s);
}

}  // namespace ar
