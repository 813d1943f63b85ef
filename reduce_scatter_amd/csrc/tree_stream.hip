// tree_stream.hip -- the tree schedule past 16 ranks in one streaming pass.
//
// The "NCCL all-reduce" post (rakshithvasudev.github.io), section "The double
// binary tree": every rank's partial is its own contribution combined with
// its children's partials (ascending rank order), the root's is the result,
// and the result is broadcast back to every rank.  In the bit-trick tree every
// subtree covers a contiguous run of ranks and a node with two children has
// one below and one above it.  So the ranks can be visited in ascending order
// with a stack of partials, as an in-order walk:
//
//   at rank v:  acc = pre(own(v)); if v has a child below, acc (+)= pop()
//               if v has a child above: push(acc)            (pending)
//               else: repeat ``cascade`` times acc = pop() (+) acc, push(acc)
//
// where ``cascade`` counts the ancestors whose upper child the finished
// subtree is.  The double tree's second tree is the mirror image for even n
// (again in order) and the first tree shifted by one rank for odd n: walked
// from rank 1 up to n-1 and then rank 0, it is in order too, except that a
// node whose children are rank 0 and another rank must combine rank 0's
// subtree first although the walk finishes it last.  Such a node leaves its
// other child's partial on the stack under its own pending one, and the
// cascade level that completes it pops both, in rank order.  Every combine is
// the staged kernels', in the same order, so the results are identical (the
// host runs each program on node ids and refuses any that would not reproduce
// the tree).  After the last rank the stack holds the root's partial; the
// postOp is applied and the value stored to every rank.  The double tree's two
// halves, each with its own program, share one launch where they need the
// same LDS.
//
// One wavefront per tile of 64*U vectors on an address-aligned grid, U per
// lane spaced by the wavefront width: each load is one 1 KB run of one rank,
// and a tile reads U KB of each rank in turn, the loads of the next D-1 ranks
// in flight while one is combined (D register buffers in rotation).  The
// stack lives in LDS, one region per wavefront at least the program's depth
// (below 96 ranks a larger reservation caps the wavefronts per compute unit):
// its depth is a uniform value, so a push or a pop is one LDS access per
// vector at a uniform offset, each lane to its own words (held in registers
// instead, the slots needed a branch per slot on every access, which the
// register allocator answered with copies and spills at one wave per SIMD).
#include <cstdlib>
#include <type_traits>

#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// The tile shape by rank count, measured on MI355X (fp32 sum, in place, per
// cent of 8 TB/s).  Below 96 ranks, 2 vectors per lane with 4 buffers, and a
// 48 KB LDS reservation per wavefront (three per compute unit: more waves
// means more concurrent rank streams and worse DRAM locality; with 60 VGPRs
// nothing else limits them): 17 ranks at 128 MB per rank 76-77, 33 at 64 MB
// 73, 48 at 32 MB 70, 63 at 32 MB 69, 72 at 25 MB 65 (no reservation: 66, 64,
// -, -, 60; 32 KB: 77, 72, 68, 66, 62; 56 KB: 64, 66, 66, 67, 64).  From 96
// ranks, for 4-byte types, 8 vectors per lane with 2 buffers (8 KB runs of
// each rank; the stack alone reserves 48-56 KB): 100 ranks at 16 MB 62-65
// against 59-61, 128 at 8 MB 70-72 against 54-59.  2-byte types keep the
// narrow shape there (their partials take twice the registers: bf16 at 128
// ranks and 32 MB 65 against 55, at 100 ranks 60 against 57, at 128 ranks and
// 8 MB 51.5 against 53).  Other shapes measured (2 vectors with 3 buffers, 4
// with 2-4, 4 waves per workgroup) were no better anywhere.
constexpr int kStreamWideRanks = 96;
constexpr size_t kStreamNarrowLds = 48 << 10;

// Launches under 1 MB per rank keep the staged kernels.  A wavefront walks
// the n ranks one after another, so a small call costs about n dependent load
// rounds (measured: 9 us at 17 ranks, 49 at 72, 86 at 128, fp32 sum), while
// the staged kernels load every rank at once and scale with n times the
// bytes; both grow with n, so the crossover is about the same per-rank size
// everywhere (staged / streamed, us: 72 ranks at 256 KB 25 / 51, at 1 MB 89 /
// 53; 128 ranks at 512 KB per launch 157 / 175, at 1 MB 338 / 112; 33 ranks at
// 256 KB 11 / 15, at 1 MB 28 / 18).
constexpr long long kStreamMinBytes = 1 << 20;
// Stack slots: enough for every tree of both schedules up to 128 ranks except
// the shifted tree at 127 ranks (8), which keeps the staged kernels.
constexpr int kStreamSlots = 7;

// Step v visits rank (first + v) mod n: bit 0, combine the child visited
// before it (pop); bit 1, a child still to come (push pending); bits 2-4, the
// cascade count; bit 5 + k, cascade level k also pops the partial its node
// left under its pending one and combines it after the finished subtree.
// (Whole words: the kernel reads them with scalar loads, which unlike vector
// loads do not wait behind the next rank's loads in flight.)
struct TreeProgram {
    uint32_t op[kTableRanks];
    int first;
};

// One launch's work: one range of frame vectors, or the double tree's two
// halves, each range with its own program.  The grid holds range 0's tiles,
// then range 1's, so the halves share one launch and its drain.
struct StreamWork {
    TreeProgram prog[2];
    long long lo[2], hi[2];
    long long tiles0;          // grid tiles of range 0
};

template <int U> __device__ __forceinline__ void stream_load(u32x4 (&b)[U], const void *src, long long base,
                                                         const unsigned (&off)[U]) {
    const char *p = (const char *)src + base;
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = __builtin_nontemporal_load((const u32x4 *)(p + off[u]));
}

// The stack of partials, in the storage type (every combine already rounds
// to it, so packing is exact): 16 bytes per vector whatever the type, slot k
// of vector u at lds[(k * U + u) * 64] from the lane's own word.  (Slot 0 in
// registers instead, one LDS slot less per wavefront, measured -8 to +14
// points depending on the rank count: not kept.)
template <int U> struct Stack {
    u32x4 *lds;
    __device__ __forceinline__ u32x4 get(int k, int u) const { return lds[(k * U + u) * kFusedThreads]; }
    __device__ __forceinline__ void put(int k, int u, const u32x4 &v) { lds[(k * U + u) * kFusedThreads] = v; }
};

// One step of the walk on the rank whose vectors ``b`` holds.
template <int DT, int OP, int U>
__device__ __forceinline__ void stream_step(const u32x4 (&b)[U], int op, Stack<U> &st, int &sp, float s) {
    Pack<DT> acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = first<DT, OP>(unpack<DT>(b[u]), s);
    if (op & 1) {                                              // the child visited before: its finished partial
        --sp;
#pragma unroll
        for (int u = 0; u < U; ++u) merge<DT, OP>(acc[u], unpack<DT>(st.get(sp, u)));
    }
    if (!(op & 2)) {                                           // the subtree is finished
        const int levels = (op >> 2) & 7;
        for (int k = 0; k < levels; ++k) {                     // ... and with it each ancestor's later child
            --sp;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                Pack<DT> a = unpack<DT>(st.get(sp, u));
                merge<DT, OP>(a, acc[u]);
                acc[u] = a;
            }
            if ((op >> (5 + k)) & 1) {                         // the ancestor's other child, the higher rank
                --sp;
#pragma unroll
                for (int u = 0; u < U; ++u) merge<DT, OP>(acc[u], unpack<DT>(st.get(sp, u)));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) st.put(sp, u, pack<DT>(acc[u]));
    ++sp;                                                      // pending (child to come) or finished
}

template <int DT, int OP, int U, int D>
__global__ __launch_bounds__(kFusedThreads) void tree_stream_kernel(const RankTable t, const StreamWork wk,
                                                                    const Geometry g) {
    constexpr long long T = (long long)kFusedThreads * U;
    extern __shared__ u32x4 stream_stack[];
    const int n = g.n;
    const long long b = blockIdx.x;
    const int h = b < wk.tiles0 ? 0 : 1;                       // uniform: this workgroup's range
    const TreeProgram &prog = wk.prog[h];
    const TileSpan ts = aligned_tile(wk.lo[h], wk.hi[h], h ? b - wk.tiles0 : b, g.ref, T);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + threadIdx.x + u * kFusedThreads, ok[u]);
    const long long base = ts.lo * 16;
    Stack<U> st;
    st.lds = stream_stack + threadIdx.x;
    int sp = 0;                                                // uniform: the same program for every lane

    // Step v visits rank (first + v) mod n; buffer v % D holds it.
    const int f = prog.first;
    const auto rank_of = [&](int v) { return f + v < n ? f + v : f + v - n; };
    u32x4 buf[D][U];
#pragma unroll
    for (int k = 0; k + 1 < D; ++k)                            // (past n, a harmless re-read of rank n-1: a load
        stream_load<U>(buf[k], t.src[rank_of(k < n ? k : n - 1)], base, off);   // under a branch cost copies)
    // Whole rounds in which every next rank exists, so every load is issued
    // unconditionally and each step waits only for its own buffer (loads
    // under a branch make the wait counts conservative: a step then waited
    // for all loads in flight); then at most 2D - 2 steps of tail.
    int v = 0;
    for (; v + 2 * D - 2 < n; v += D) {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            stream_load<U>(buf[(k + D - 1) % D], t.src[rank_of(v + k + D - 1)], base, off);
            stream_step<DT, OP, U>(buf[k], (int)prog.op[v + k], st, sp, g.s);
        }
    }
#pragma unroll
    for (int k = 0; k < 2 * D - 2; ++k) {
        if (v + k < n) {
            if (v + k + D - 1 < n) stream_load<U>(buf[(k + D - 1) % D], t.src[rank_of(v + k + D - 1)], base, off);
            stream_step<DT, OP, U>(buf[k % D], (int)prog.op[v + k], st, sp, g.s);
        }
    }

    Pack<DT> root[U];
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        root[u] = unpack<DT>(st.get(0, u));
        finish<DT, OP>(root[u], n, g);
        w[u] = pack<DT>(root[u]);
    }
    for (int r = 0; r < n; ++r) {
        char *p = (char *)t.dst[r] + base;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) __builtin_nontemporal_store(w[u], (u32x4 *)(p + off[u]));
    }
}

// The stream program of a tree walked from rank ``first``, or false when the
// walk would not reproduce the tree.  The program is run on node ids: every
// stack entry is a rank's pending partial or a finished subtree's, and every
// pop must deliver exactly the one the tree combines there, children in
// ascending rank order after the node's own value.  The walk must end with the
// root's finished subtree alone on the stack and never hold more than
// kStreamSlots partials.
static bool tree_program(const TreeShape &tree, int n, int first, TreeProgram &prog, int &depth) {
    if (n < 1 || n > kTableRanks || first < 0 || first >= n) return false;
    int pos[kTableRanks];
    for (int v = 0; v < n; ++v) pos[(first + v) % n] = v;
    int stack[kTableRanks + 1];                                // a rank's finished subtree, + kTableRanks if pending
    int sp = 0;
    depth = 0;
    const auto pop = [&](int want) { return sp > 0 && stack[--sp] == want; };
    for (int v = 0; v < n; ++v) {
        const int r = (first + v) % n;
        const int c0 = tree.child[r][0], c1 = tree.child[r][1];  // ascending rank order
        int before = -1, after = -1;
        for (const int c : {c0, c1}) {
            if (c < 0) continue;
            int &side = pos[c] < v ? before : after;
            if (side >= 0) return false;
            side = c;
        }
        const bool keep = before >= 0 && after >= 0 && after == c0;   // the later child combines first
        int code = 0, levels = 0;
        if (before >= 0 && !keep) {
            if (!pop(before)) return false;
            code |= 1;
        }
        if (after >= 0) {
            if (keep && !(sp > 0 && stack[sp - 1] == before)) return false;
            stack[sp++] = r + kTableRanks;
            code |= 2;
        } else {
            int x = r;
            for (int p = tree.parent[x]; p >= 0 && pos[p] < pos[x]; x = p, p = tree.parent[x]) {
                if (levels >= 7 || !pop(p + kTableRanks)) return false;
                if (tree.child[p][0] == x && tree.child[p][1] >= 0) {   // p kept its other child's partial
                    if (!pop(tree.child[p][1])) return false;
                    code |= 1 << (5 + levels);
                }
                ++levels;
            }
            stack[sp++] = x;
        }
        if (sp > kStreamSlots) return false;
        if (sp > depth) depth = sp;
        prog.op[v] = (uint32_t)(code | levels << 2);
    }
    if (sp != 1 || stack[0] != tree.root) return false;
    for (int v = n; v < kTableRanks; ++v) prog.op[v] = 0;
    prog.first = first;
    return true;
}

// AR_TREE_STREAM=0 keeps the LDS-staged kernels for every tree; =1 streams
// every tree the walk holds at any size; unset, launches of 1 MB per rank and
// more stream.  Read on every launch, so one process can compare the kernels.
static int tree_stream_mode() {
    const char *e = getenv("AR_TREE_STREAM");
    if (e && (*e == '0' || *e == '1')) return *e - '0';
    return 2;
}

// The walk over ``halves`` ranges, range h of the vectors [lo[h], hi[h]) up
// ``*trees[h]``, in one launch; false (nothing launched) when a range is under
// the size threshold or a tree is not one the walk holds.
static bool launch_stream(int dt, int op, const RankTable &t, const TreeShape *const *trees, int halves,
                          const Geometry &g, const long long *lo, const long long *hi, hipStream_t s,
                          hipError_t *err) {
    const int mode = tree_stream_mode();
    if (mode == 0) return false;
    StreamWork wk;
    int depth = 0, depths[2] = {0, 0};
    bool any = false;
    for (int h = 0; h < 2; ++h) {
        wk.lo[h] = h < halves ? lo[h] : 0;
        wk.hi[h] = h < halves && hi[h] > lo[h] ? hi[h] : wk.lo[h];
        if (wk.hi[h] == wk.lo[h]) continue;
        if (mode == 2 && (wk.hi[h] - wk.lo[h]) * 16 < kStreamMinBytes) return false;
        int d = 0;
        // the first tree and the mirror image walk from rank 0, the shifted tree from rank 1
        if (!(tree_program(*trees[h], g.n, 0, wk.prog[h], d) || tree_program(*trees[h], g.n, 1, wk.prog[h], d)))
            return false;
        depth = d > depth ? d : depth;
        depths[h] = d;
        any = true;
    }
    if (!any) return false;
    // Two ranges share a launch only where they need the same LDS: with the
    // 8 KB runs the reservation is the stack's depth, and one launch at the deeper
    // half's depth cut the other half's wavefronts per compute unit (128 ranks,
    // 8 MB per rank, depths 7 and 6: 69-70 % in one launch, 75 % in two);
    // below 96 the 48 KB reservation is the same for both, and one launch
    // gained 1-4 points (17, 33 and 72 ranks) over two.
    const bool wide = g.n >= kStreamWideRanks && (dt == F32 || dt == I32);
    if (halves == 2 && wide && depths[0] && depths[1] && depths[0] != depths[1]) return false;
    const auto go = [&](auto Uc, auto Dc, size_t lds) {
        constexpr int U = decltype(Uc)::value, D = decltype(Dc)::value;
        const long long T = (long long)kFusedThreads * U;
        wk.tiles0 = wk.hi[0] > wk.lo[0] ? aligned_tiles(wk.hi[0] - wk.lo[0], T) : 0;
        const long long tiles = wk.tiles0 + (wk.hi[1] > wk.lo[1] ? aligned_tiles(wk.hi[1] - wk.lo[1], T) : 0);
        if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
        const size_t stack = (size_t)depth * U * kFusedThreads * 16;
        return dispatch(dt, op, [&](auto Dt, auto O) {
            constexpr int DT = decltype(Dt)::value;
            if constexpr (U == 8 && Lanes<DT>::value == 8) return hipErrorInvalidValue;   // never chosen (above)
            else
                return launch(tree_stream_kernel<DT, decltype(O)::value, U, D>, dim3((unsigned)tiles),
                              dim3(kFusedThreads), stack > lds ? stack : lds, s, t, wk, g);
        });
    };
    if (wide)
        *err = go(std::integral_constant<int, 8>(), std::integral_constant<int, 2>(), (size_t)0);
    else
        *err = go(std::integral_constant<int, 2>(), std::integral_constant<int, 4>(), kStreamNarrowLds);
    return true;
}

bool launch_tree_stream_range(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                              long long lo, long long hi, hipStream_t s, hipError_t *err) {
    const TreeShape *trees[1] = {&tree};
    return launch_stream(dt, op, t, trees, 1, g, &lo, &hi, s, err);
}

bool launch_dtree_stream(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                         const Geometry &g, long long lo0, long long hi0, long long lo1, long long hi1, hipStream_t s,
                         hipError_t *err) {
    const TreeShape *trees[2] = {&tree, &tree2};
    const long long lo[2] = {lo0, lo1}, hi[2] = {hi0, hi1};
    return launch_stream(dt, op, t, trees, 2, g, lo, hi, s, err);
}

}  // namespace ar
