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
// Past 16 ranks (and up to 16 under AR_TREE_STAGED=1) a launch first tries
// the streaming in-order walk of tree_stream.hip, one pass with the same
// results; these LDS-staged kernels take the trees it cannot hold (the double
// tree's shifted second tree at 127 ranks) and every tree under
// AR_TREE_STREAM=0.  Up to 16 ranks tree_reg.hip evaluates the same trees in
// registers in one pass, with the same results.
//
// A workgroup runs the whole tree for a window of W vectors at the same offset
// of every rank buffer.  Item (rank v, vector w) holds rank v's contribution;
// LDS holds one partial per rank.  Up phase, deepest level first: partial(v) =
// own(v), then each child's partial in ascending rank order; the root applies
// the postOp.  Down phase, root first: each rank copies its parent's final
// value and stores it.  A workgroup barrier separates the levels.
//
// Two kernels: level by level (one team walks the window up, then down), and
// concurrent up and down teams (same section of the post: a tree block splits
// into a team that reduces chunk w+1 up the tree while another broadcasts
// chunk w down it).
//
// The double binary tree (same section: a second tree with the roles of
// leaves and interior ranks swapped, and half of every buffer sent up each)
// is one streaming launch for both halves where the walk holds both trees
// (and they need the same LDS), else one launch per half and shape, each
// streamed or staged.  On one GPU
// there are no per-rank links to balance, so it costs what the single tree
// costs; its results differ from the single tree's in the second half.
#include <cstdlib>

#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// The vectors one launch covers, [lo, hi), in windows of W vectors on a grid
// from ``base`` (lo rounded down to a multiple of W, so windows are whole
// 128-byte lines of every buffer; only the first may be partial).
struct TreeRange {
    long long lo, hi, base, windows;
};

// A thread's items are fixed for the whole kernel.  Item q is vector q % W of
// rank post[q / W], post listing the ranks deepest level first, so the items
// of one level are contiguous and a wavefront mostly holds ranks of a single
// depth: on every level step the other wavefronts skip their LDS work
// entirely.  (With item q on rank q / W, every wavefront held ranks of every
// depth and issued its LDS instructions on every step, mostly with few lanes
// active; measured on MI355X at 72 ranks that cost a third of the time.)
// Each item's place in the tree -- depth, parent, children -- is read once
// into one register: depth | parent << 8 | child0 << 16 | child1 << 24, each
// field a signed byte (-1 = none).  Looked up by rank on every level instead,
// it was a memory round trip per level (0.8-0.9 TB/s at 72 ranks).
struct Items {
    int r[kItemsPerThread], w[kItemsPerThread], code[kItemsPerThread];
    int cnt, root;
};

__device__ __forceinline__ int field(int code, int f) { return (int)(signed char)((unsigned)code >> (8 * f)); }

__device__ __forceinline__ Items items_of(const TreeShape &tree, int tid, int nthreads, int n, int W) {
    Items it;
    it.cnt = 0;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        const int q = tid + k * nthreads;
        const bool has = q < n * W;
        const int v = has ? tree.post[q / W] : 0;
        it.r[k] = v;
        it.w[k] = has ? q % W : 0;
        if (has) it.cnt = k + 1;
        it.code[k] = (int)((unsigned)(unsigned char)(has ? tree.depth[v] : -1) |
                           (unsigned)(unsigned char)tree.parent[v] << 8 | (unsigned)(unsigned char)tree.child[v][0] << 16 |
                           (unsigned)(unsigned char)tree.child[v][1] << 24);
    }
    it.root = tree.root;
    return it;
}

// One up level: at depth d, partial(v) = own(v), then each child's partial in
// ascending rank order; the root applies the postOp.
template <int DT, int OP>
__device__ __forceinline__ void up_level(const Items &it, const Geometry &g, int d, const bool *ok, const u32x4 *own,
                                         u32x4 *slot) {
    const int W = g.W;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        if (!ok[k] || field(it.code[k], 0) != d) continue;
        const int v = it.r[k];
        Pack<DT> acc = first<DT, OP>(unpack<DT>(own[k]), g.s);
        const int c0 = field(it.code[k], 2), c1 = field(it.code[k], 3);
        if (c0 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[c0 * W + it.w[k]]));
        if (c1 >= 0) merge<DT, OP>(acc, unpack<DT>(slot[c1 * W + it.w[k]]));
        if (v == it.root) finish<DT, OP>(acc, g.n, g);
        slot[v * W + it.w[k]] = pack<DT>(acc);
    }
}

// One down level: at depth d the root keeps its value and every other rank
// copies its parent's; each stores its value to its output.
__device__ __forceinline__ void down_level(void *const *dst, const Items &it, const Geometry &g, int d, long long pos0,
                                           const bool *ok, u32x4 *slot) {
    const int W = g.W;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        if (!ok[k] || field(it.code[k], 0) != d) continue;
        const int v = it.r[k];
        const int p = v == it.root ? v : field(it.code[k], 1);
        const u32x4 val = slot[p * W + it.w[k]];
        slot[v * W + it.w[k]] = val;
        st_stream(dst[k], pos0 + it.w[k], val);
    }
}

// ---------------------------------------------------------------------------
// Level by level: up levels deepest first, then down levels root first, a
// workgroup barrier after each.  All of a window's loads are issued before
// its first level.  A persistent grid walks the windows.
// ---------------------------------------------------------------------------
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void tree_allreduce_kernel(
    const RankTable t, const TreeShape tree, const Geometry g, const TreeRange rg) {
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4 *slot = (u32x4 *)lds;
    const Items it = items_of(tree, threadIdx.x, kThreads, g.n, g.W);
    const void *src[kItemsPerThread];
    void *dst[kItemsPerThread];
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        src[k] = t.src[it.r[k]];
        dst[k] = t.dst[it.r[k]];
    }
    const int depth = tree.max_depth;
    for (long long win = blockIdx.x; win < rg.windows; win += gridDim.x) {
        const long long pos0 = rg.base + win * g.W;
        u32x4 own[kItemsPerThread];
        bool ok[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            const long long v = pos0 + it.w[k];
            ok[k] = k < it.cnt && v >= rg.lo && v < rg.hi;
            if (ok[k]) own[k] = ld_stream(src[k], v);
        }
        for (int d = depth; d >= 0; --d) {
            up_level<DT, OP>(it, g, d, ok, own, slot);
            __syncthreads();
        }
        for (int d = 0; d <= depth; ++d) {
            down_level(dst, it, g, d, pos0, ok, slot);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Concurrent up and down teams.  The workgroup is two teams of kThreads
// threads over two LDS window buffers: in iteration i the up team reduces the
// workgroup's window i into one buffer while the down team broadcasts window
// i-1 from the other.  Both walk their tree one level per step (the up team
// deepest level first, the down team root first), so a window costs depth+1
// workgroup barriers instead of 2*(depth+1), and the up team's loads of window
// i+1 (issued one iteration ahead) and the down team's stores overlap the
// other team's levels.  Every combine is the level-by-level kernel's, in the
// same order, so the results are identical.
// ---------------------------------------------------------------------------
template <int DT, int OP>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(4))) void tree_team_kernel(
    const RankTable t, const TreeShape tree, const Geometry g, const TreeRange rg) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    const bool up = threadIdx.x < kThreads;                     // uniform per wavefront
    const Items it = items_of(tree, up ? (int)threadIdx.x : (int)threadIdx.x - kThreads, kThreads, n, W);
    const int depth = tree.max_depth;
    const long long b = blockIdx.x, G = gridDim.x;
    const long long mine = rg.windows > b ? (rg.windows - b + G - 1) / G : 0;   // this workgroup's windows
    u32x4 *const buf[2] = {(u32x4 *)lds, (u32x4 *)lds + n * W};

    // The teams run loops of their own with the same number of barriers: (mine + 1) iterations of depth + 1
    // steps (the up team has no window in the last iteration, the down team none in the first).  Keeping
    // the up team's loads and the down team's stores in separate code lets a wait for one window's loads
    // leave the next window's in flight.
    if (up) {
        const void *src[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) src[k] = t.src[it.r[k]];
        // Every load is issued (an item outside the range reads vector lo of its rank and is not used), so
        // the number of loads in flight is fixed and the wait for the older window counts exactly.
        auto load = [&](long long i, u32x4 *own, bool *ok) {
            const long long pos0 = rg.base + (b + i * G) * W;
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                const long long v = pos0 + it.w[k];
                ok[k] = i < mine && k < it.cnt && v >= rg.lo && v < rg.hi;
                own[k] = ld_stream(src[k], ok[k] ? v : rg.lo);
            }
        };
        auto reduce = [&](long long i, const u32x4 *own, const bool *ok) {
            u32x4 *const slot = buf[i & 1];
            for (int s = 0; s <= depth; ++s) {
                up_level<DT, OP>(it, g, depth - s, ok, own, slot);
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
        for (int k = 0; k < kItemsPerThread; ++k) dst[k] = t.dst[it.r[k]];
        for (long long i = 0; i <= mine; ++i) {
            const long long pos0 = rg.base + (b + (i - 1) * G) * W;    // window i-1 (none when i = 0)
            bool ok[kItemsPerThread];
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                const long long v = pos0 + it.w[k];
                ok[k] = i >= 1 && k < it.cnt && v >= rg.lo && v < rg.hi;
            }
            u32x4 *const slot = buf[(i + 1) & 1];
            for (int s = 0; s <= depth; ++s) {
                down_level(dst, it, g, s, pos0, ok, slot);
                __syncthreads();
            }
        }
    }
}

// Which staged kernel: the teams up to 32 ranks, level by level beyond.
// Measured on MI355X (fp32, in place, TB/s teams / level by level): 17 ranks
// at 128 MB per rank 5.13 / 4.43, 33 ranks at 64 MB 3.87 / 3.86, 72 ranks at
// 25 MB 2.76 / 3.13.  AR_TREE_TEAMS=1 or 0 forces one (read on every launch,
// so one process can compare the two).
static bool tree_teams(int n) {
    const char *e = getenv("AR_TREE_TEAMS");
    if (e && (*e == '0' || *e == '1')) return *e == '1';
    return n <= 32;
}

// One launch over the vectors [lo, hi) with one tree shape.
static hipError_t launch_tree_range(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                    long long lo, long long hi, int cus, hipStream_t s) {
    hipError_t streamed;                                       // in-order trees: one streaming pass (tree_stream.hip)
    if (launch_tree_stream_range(dt, op, t, tree, g, lo, hi, s, &streamed)) return streamed;
    TreeRange rg;
    rg.lo = lo;
    rg.hi = hi;
    rg.base = lo - lo % g.W;
    rg.windows = hi > rg.base ? (hi - rg.base + g.W - 1) / g.W : 0;
    if (rg.windows <= 0 || lo >= hi) return hipSuccess;
    // residency: a team workgroup is 8 waves of at most 128 VGPRs (two per
    // compute unit), a level-by-level one 4 waves (four per compute unit); a
    // larger persistent grid would leave the extra workgroups to start only
    // after the resident ones have walked all their windows
    if (tree_teams(g.n))
        return dispatch(dt, op, [&](auto D, auto O) {
            return launch(tree_team_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid_for(rg.windows, cus, 2)),
                          dim3(2 * kThreads), (size_t)2 * g.n * g.W * 16, s, t, tree, g, rg);
        });
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(tree_allreduce_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid_for(rg.windows, cus, 4)),
                      dim3(kThreads), (size_t)g.n * g.W * 16, s, t, tree, g, rg);
    });
}

hipError_t launch_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                 int cus, hipStream_t s) {
    return launch_tree_range(dt, op, t, tree, g, 0, g.Vfull, cus, s);
}

hipError_t launch_dtree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                                  const Geometry &g, int cus, hipStream_t s) {
    hipError_t streamed;                                       // both halves in one streaming launch
    if (launch_dtree_stream(dt, op, t, tree, tree2, g, 0, g.split, g.split2, g.Vfull, s, &streamed)) return streamed;
    const hipError_t e = launch_tree_range(dt, op, t, tree, g, 0, g.split, cus, s);
    if (e != hipSuccess) return e;
    return launch_tree_range(dt, op, t, tree2, g, g.split2, g.Vfull, cus, s);
}

}  // namespace ar
