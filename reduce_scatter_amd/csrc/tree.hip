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
#include <cstdlib>

#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// A thread's items are fixed for the whole kernel (item q = rank q / W,
// vector q % W), so each item's place in a tree -- depth, parent and children
// -- is read from the shape in the kernel arguments once, into one register
// per item: depth | parent << 8 | child0 << 16 | child1 << 24, each field a
// signed byte (-1 = none).  Looking the shape up by the item's rank on every
// level instead was a memory round trip per level (measured on MI355X at 72
// ranks: 0.8-0.9 TB/s for both staged kernels).
struct ItemShape {
    int code[kItemsPerThread];
    int root;
};

__device__ __forceinline__ int field(int code, int f) { return (int)(signed char)((unsigned)code >> (8 * f)); }

__device__ __forceinline__ ItemShape item_shape(const TreeShape &tree, const int *r, int cnt) {
    ItemShape s;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        const int v = k < cnt ? r[k] : 0;
        s.code[k] = (int)((unsigned)(unsigned char)(k < cnt ? tree.depth[v] : -1) |
                          (unsigned)(unsigned char)tree.parent[v] << 8 | (unsigned)(unsigned char)tree.child[v][0] << 16 |
                          (unsigned)(unsigned char)tree.child[v][1] << 24);
    }
    s.root = tree.root;
    return s;
}

// One up level: at depth d, partial(v) = own(v), then each child's partial in
// ascending rank order; the root applies the postOp.
template <int DT, int OP>
__device__ __forceinline__ void up_level(const ItemShape &sh, const Geometry &g, int d, const int *r, const int *w,
                                         const bool *ok, const u32x4 *own, u32x4 *slot) {
    const int W = g.W;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        if (!ok[k] || field(sh.code[k], 0) != d) continue;
        const int v = r[k];
        Pack<DT> acc = first<DT, OP>(unpack<DT>(own[k]), g.s);
        const int c0 = field(sh.code[k], 2), c1 = field(sh.code[k], 3);
        if (c0 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[c0 * W + w[k]]));
        if (c1 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[c1 * W + w[k]]));
        if (v == sh.root) finish<DT, OP>(acc, g.n, g);
        slot[v * W + w[k]] = pack<DT>(acc);
    }
}

// One down level: at depth d the root keeps its value and every other rank
// copies its parent's; each stores its value to its output.
__device__ __forceinline__ void down_level(void *const *dst, const ItemShape &sh, const Geometry &g, int d,
                                           long long pos0, const int *r, const int *w, const bool *ok, u32x4 *slot) {
    const int W = g.W;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        if (!ok[k] || field(sh.code[k], 0) != d) continue;
        const int v = r[k];
        const int p = v == sh.root ? v : field(sh.code[k], 1);
        const u32x4 val = slot[p * W + w[k]];
        slot[v * W + w[k]] = val;
        st_stream(dst[k], pos0 + w[k], val);
    }
}

// The items of thread ``tid`` among nthreads: item k is (rank r[k], vector
// w[k]) of the window; returns how many of the kItemsPerThread exist.
__device__ __forceinline__ int items_of(int tid, int nthreads, int n, int W, int *r, int *w) {
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        const int q = tid + k * nthreads;
        r[k] = 0;
        w[k] = 0;
        if (q < n * W) {
            r[k] = q / W;
            w[k] = q - r[k] * W;
            cnt = k + 1;
        }
    }
    return cnt;
}

// Each item's rank pointers, read from the kernel arguments once (indexed by
// a per-lane rank, each read is a memory access).
__device__ __forceinline__ void item_pointers(const RankTable &t, const int *r, const void **src, void **dst) {
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        src[k] = t.src[r[k]];
        dst[k] = t.dst[r[k]];
    }
}

// Window ``win`` of the schedule: its first vector, the range [lo, hi) it is
// clipped to, and which tree it takes.  Windows sit on a grid of W vectors
// from vector 0 (W a multiple of 8: whole 128-byte lines); the double tree
// sends the windows from ``first`` on up the second tree, the first of them
// starting at split2 rounded down to the grid.
struct TreeWindow {
    long long pos0, lo, hi;
    bool second;
};
template <bool DUAL>
__device__ __forceinline__ TreeWindow tree_window_at(const Geometry &g, long long win, long long first) {
    TreeWindow x;
    x.second = DUAL && win >= first;
    x.pos0 = x.second ? g.split2 - g.split2 % g.W + (win - first) * g.W : win * g.W;
    x.lo = x.second ? g.split2 : 0;
    x.hi = DUAL && !x.second ? g.split : g.Vfull;
    return x;
}
__device__ __forceinline__ bool in_window(const TreeWindow &x, long long v) { return v >= x.lo && v < x.hi; }

// ---------------------------------------------------------------------------
// Level by level: one workgroup runs the whole tree for a window of W vectors
// at the same offset of every rank buffer, up levels deepest first, then down
// levels root first, a workgroup barrier after each.  All of a rank's loads
// are issued at the start (nothing they read depends on the tree), so the
// levels only wait on LDS.  A persistent grid walks the windows.
// ---------------------------------------------------------------------------
template <int DT, int OP, bool DUAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void tree_allreduce_kernel(const RankTable t, const TreeShape tree0,
                                                                  const TreeShape tree1, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4 *slot = (u32x4 *)lds;
    int r[kItemsPerThread], w[kItemsPerThread];
    const int cnt = items_of(threadIdx.x, kThreads, g.n, g.W, r, w);
    const void *src[kItemsPerThread];
    void *dst[kItemsPerThread];
    item_pointers(t, r, src, dst);
    const ItemShape sh0 = item_shape(tree0, r, cnt);
    const ItemShape sh1 = DUAL ? item_shape(tree1, r, cnt) : sh0;
    const int depth = tree0.max_depth > tree1.max_depth ? tree0.max_depth : tree1.max_depth;
    const long long first = DUAL ? (g.split + g.W - 1) / g.W : g.windows;   // windows of the first tree
    for (long long win = blockIdx.x; win < g.windows; win += gridDim.x) {
        const TreeWindow x = tree_window_at<DUAL>(g, win, first);
        const ItemShape &sh = x.second ? sh1 : sh0;
        u32x4 own[kItemsPerThread];
        bool ok[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            ok[k] = k < cnt && in_window(x, x.pos0 + w[k]);
            if (ok[k]) own[k] = ld_stream(src[k], x.pos0 + w[k]);
        }
        for (int d = depth; d >= 0; --d) {
            up_level<DT, OP>(sh, g, d, r, w, ok, own, slot);
            __syncthreads();
        }
        for (int d = 0; d <= depth; ++d) {
            down_level(dst, sh, g, d, x.pos0, r, w, ok, slot);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Concurrent up and down teams (same section of the post: a tree block splits
// into a team that reduces chunk w+1 up the tree while another broadcasts
// chunk w down it).  The workgroup is two teams of kThreads threads over two
// LDS window buffers: in iteration i the up team reduces the workgroup's
// window i into one buffer while the down team broadcasts window i-1 from the
// other.  Both walk their tree one level per step (the up team deepest level
// first, the down team root first), so a window costs depth+1 workgroup
// barriers instead of 2*(depth+1), and the up team's loads of window i+1
// (issued one iteration ahead) and the down team's stores overlap the other
// team's levels.  Every combine is the level-by-level kernel's, in the same
// order, so the results are identical.
// ---------------------------------------------------------------------------
template <int DT, int OP, bool DUAL>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(4))) void tree_team_kernel(
    const RankTable t, const TreeShape tree0, const TreeShape tree1, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    const bool up = threadIdx.x < kThreads;                     // uniform per wavefront
    int r[kItemsPerThread], w[kItemsPerThread];
    const int cnt = items_of(up ? (int)threadIdx.x : (int)threadIdx.x - kThreads, kThreads, n, W, r, w);
    const ItemShape sh0 = item_shape(tree0, r, cnt);
    const ItemShape sh1 = DUAL ? item_shape(tree1, r, cnt) : sh0;
    const int depth = tree0.max_depth > tree1.max_depth ? tree0.max_depth : tree1.max_depth;
    const long long first = DUAL ? (g.split + W - 1) / W : g.windows;   // windows of the first tree
    const long long b = blockIdx.x, G = gridDim.x;
    const long long mine = g.windows > b ? (g.windows - b + G - 1) / G : 0;   // this workgroup's windows
    u32x4 *const buf[2] = {(u32x4 *)lds, (u32x4 *)lds + n * W};

    // The teams run loops of their own with the same number of barriers: (mine + 1) iterations of depth + 1
    // steps (the up team has no window in the last iteration, the down team none in the first).  Keeping
    // the up team's loads and the down team's stores in separate code lets a wait for one window's loads
    // leave the next window's in flight.
    if (up) {
        const void *src[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) src[k] = t.src[r[k]];
        // Every load is issued (an item outside the range reads vector 0 of its rank and is not used), so
        // the number of loads in flight is fixed and the wait for the older window counts exactly.
        auto load = [&](long long i, u32x4 *own, bool *ok) {
            const TreeWindow x = tree_window_at<DUAL>(g, b + i * G, first);
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                ok[k] = i < mine && k < cnt && in_window(x, x.pos0 + w[k]);
                own[k] = ld_stream(src[k], ok[k] ? x.pos0 + w[k] : 0);
            }
        };
        auto reduce = [&](long long i, const u32x4 *own, const bool *ok) {
            const TreeWindow x = tree_window_at<DUAL>(g, b + i * G, first);
            const ItemShape &sh = x.second ? sh1 : sh0;
            u32x4 *const slot = buf[i & 1];
            for (int s = 0; s <= depth; ++s) {
                up_level<DT, OP>(sh, g, depth - s, r, w, ok, own, slot);
                __syncthreads();
            }
        };
        u32x4 ownA[kItemsPerThread], ownB[kItemsPerThread];
        bool okA[kItemsPerThread], okB[kItemsPerThread];
        load(0, ownA, okA);
        for (long long i = 0; i <= mine; i += 2) {
            load(i + 1, ownB, okB);                              // one window ahead
            reduce(i, ownA, okA);
            if (i + 1 > mine) break;
            load(i + 2, ownA, okA);
            reduce(i + 1, ownB, okB);
        }
    } else {
        void *dst[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) dst[k] = t.dst[r[k]];
        for (long long i = 0; i <= mine; ++i) {
            const TreeWindow x = tree_window_at<DUAL>(g, b + (i - 1) * G, first);
            bool ok[kItemsPerThread];
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) ok[k] = i >= 1 && k < cnt && in_window(x, x.pos0 + w[k]);
            const ItemShape &sh = x.second ? sh1 : sh0;
            u32x4 *const slot = buf[(i + 1) & 1];                // window i-1
            for (int s = 0; s <= depth; ++s) {
                down_level(dst, sh, g, s, x.pos0, r, w, ok, slot);
                __syncthreads();
            }
        }
    }
}

// AR_TREE_TEAMS=0 selects the level-by-level kernel instead (read on every
// launch, so one process can compare the two).
static bool tree_teams() {
    const char *e = getenv("AR_TREE_TEAMS");
    return !(e && *e == '0');
}

template <bool DUAL>
hipError_t launch_trees(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                        const Geometry &g, int cus, hipStream_t s) {
    // residency: a team workgroup is 8 waves of at most 128 VGPRs (two per
    // compute unit), a level-by-level one 4 waves (four per compute unit); a
    // larger persistent grid would leave the extra workgroups to start only
    // after the resident ones have walked all their windows
    if (tree_teams())
        return dispatch(dt, op, [&](auto D, auto O) {
            return launch(tree_team_kernel<decltype(D)::value, decltype(O)::value, DUAL>,
                          dim3(grid_for(g.windows, cus, 2)), dim3(2 * kThreads), (size_t)2 * g.n * g.W * 16, s, t,
                          tree, tree2, g);
        });
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(tree_allreduce_kernel<decltype(D)::value, decltype(O)::value, DUAL>,
                      dim3(grid_for(g.windows, cus, 4)), dim3(kThreads), (size_t)g.n * g.W * 16, s, t, tree, tree2, g);
    });
}

hipError_t launch_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                 int cus, hipStream_t s) {
    return launch_trees<false>(dt, op, t, tree, tree, g, cus, s);
}

hipError_t launch_dtree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                                  const Geometry &g, int cus, hipStream_t s) {
    return launch_trees<true>(dt, op, t, tree, tree2, g, cus, s);
}

}  // namespace ar
