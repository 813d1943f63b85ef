// ar_kernels.hpp -- kernel argument blocks and launcher entry points (host
// side of the kernels).  The pointer tables travel by value in the kernel
// arguments, so a launch needs no device-side table and no allocation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

constexpr int kTableRanks = 128;

// One pointer pair per rank, by value in the kernel arguments.  Kernels built
// for a compile-time rank count NR take a table of exactly NR entries
// (RankTableFor<NR>): the runtime copies every kernel argument on every
// launch, and the full 128-rank table (2 KB) cost about 1.4 us of host time
// per launch on MI355X (4.1 against 2.7 us for a kernel with one int argument).
// CAP = 0 is the full table of kTableRanks entries (the any-n kernels').
template <int CAP> struct RankTableN {
    static constexpr int kCap = CAP > 0 ? CAP : kTableRanks;
    const void *src[kCap];
    void *dst[kCap];
};
using RankTable = RankTableN<0>;
template <int NR> using RankTableFor = RankTableN<NR>;

// The first entries of ``t`` as the table a kernel for NR ranks takes.
template <int NR> inline RankTableFor<NR> narrow(const RankTable &t) {
    RankTableFor<NR> r;
    for (int i = 0; i < RankTableFor<NR>::kCap; ++i) {
        r.src[i] = t.src[i];
        r.dst[i] = t.dst[i];
    }
    return r;
}

// Geometry of one collective call, in 16-byte vectors of the element type.
//   all-reduce:     chunk c = vectors [floor(c*V/n), floor((c+1)*V/n)) of
//                   every rank buffer; full vectors are [0, Vfull).
//   reduce-scatter: chunk c = vectors [c*Rv, (c+1)*Rv) of every input;
//                   output slice of rank r = vectors [0, Rv).
//   all-gather:     piece k = vectors [0, Rv) of input k, landing at
//                   [k*Rv, (k+1)*Rv) of every output.
struct Geometry {
    long long V;        // all-reduce: ceil(count / lanes)
    long long q;        // all-reduce: V / n
    int rem;            // all-reduce: V % n (chunk c starts at c*q + floor(c*rem/n))
    long long Vfull;    // all-reduce: count / lanes (vectors with no tail)
    long long Rv;       // reduce-scatter / all-gather: vectors per slice
    long long windows;  // work units along a chunk (tiles or LDS windows)
    int n;
    int W;              // ring/tree: vectors per rank in one LDS window
    float s;            // fp32(1/n), the float avg pre-scale
    long long ref;      // fused / split: address / 16 of the buffer whose alignment cuts the tiles
    long long split;    // double tree: vectors [0, split) go up the first tree, [split2, Vfull) up the second
    long long split2;   //   (split2 = split, or split + 1 in the shifted frame below)
    int shift;          // all-reduce in the shifted frame (every buffer at one 16-byte phase, vectors counted
                        // from the first 16-byte boundary): 1, and chunk c's vectors end one early, the
                        // vector across each chunk boundary going to the element-wise kernel; else 0
    float post_div;     // split float avg: the finished sum is divided by n / p (0: no post-division)
    int acc32;          // bf16 / fp16 partials kept in fp32, rounded once (the fused schedule)
    long long slice_bytes;  // phased reduce-scatter / all-gather: bytes per slice or piece
    long long in_off;       // phased: byte offset of the first input byte past the (16-byte aligned) table pointer
    long long out_off;      // phased: byte offset of output vector 0 past the caller's output pointer
    long long last_off;     // phased: offset (from the table pointer) of the last 16-byte block holding input
    int ar_chunks;          // phased reduce-scatter: slice c is all-reduce chunk c (vectors [floor(c*V/n),
                            // floor((c+1)*V/n)) of every rank, from q and rem), stored to dst[c] at its offset
    int phased_words;       // phased reduce-scatter, compile-time n: 0 funnel loads, 1 word-aligned loads where
                            // the phase is not whole words, 2 word-aligned loads everywhere (any n: always);
                            // set to 2 by the caller for pointers at mixed phases (4-byte aligned), else
                            // chosen at launch; phased all-gather: 2 for pointers at mixed phases (one
                            // word-aligned load per vector), else the funnel
};

// Tiles are cut on a grid aligned to absolute T-vector boundaries of a
// reference buffer (vector v of the range sits at address (ref + v) * 16): the
// first tile of a range may be partial, every later one covers a whole
// aligned run.  Measured on MI355X: a 16-byte misalignment of the rank buffers
// costs the one-vector-per-lane kernels about a quarter of their bandwidth
// when tiles follow the range start instead.
struct TileSpan {
    long long start;    // first vector of the aligned tile (may lie before lo)
    long long lo, hi;   // the tile's vectors inside the range: [lo, hi), empty when lo >= hi
};

__host__ __device__ inline TileSpan aligned_tile(long long lo, long long hi, long long j, long long ref, long long T) {
    const long long a = (ref + lo) & (T - 1);                 // T is a power of two
    TileSpan s;
    s.start = lo - a + j * T;
    s.lo = s.start > lo ? s.start : lo;
    s.hi = s.start + T < hi ? s.start + T : hi;
    return s;
}

// Vector v of an aligned tile: its byte offset from the tile's first in-range
// vector, and whether it is in range (a lane outside re-reads an in-range
// vector and drops the result, so no load needs a branch).
__device__ __forceinline__ unsigned tile_lane(const TileSpan &ts, long long v, bool &ok) {
    ok = v >= ts.lo && v < ts.hi;
    const long long c = v < ts.lo ? ts.lo : (v >= ts.hi ? ts.hi - 1 : v);
    return (unsigned)(c - ts.lo) * 16u;
}

// Tiles needed for a range of len vectors, whatever its alignment.
inline long long aligned_tiles(long long len, long long T) { return len > 0 ? (len + T - 1) / T + 1 : 0; }

// A tree schedule's shape, host-built: depth, parent and up to two children
// per rank (-1 = none, in ascending rank order), the root, and post[] listing
// the ranks children-first.
struct TreeShape {
    int8_t depth[kTableRanks];
    int8_t parent[kTableRanks];
    int8_t child[kTableRanks][2];
    uint8_t post[kTableRanks];
    int max_depth;
    int root;
};

// Launchers.  dt / op use the ar_dtype_t / ar_op_t numbering.  ``grid`` is
// the number of workgroups (already clamped to the work available).
// Vector paths (every pointer 16-byte aligned):
// Fused kernels launch one workgroup per tile (g.windows tiles per chunk, n
// chunks); ``lds`` is the dynamic LDS each workgroup reserves (a residency cap).
hipError_t launch_fused_allreduce(int dt, int op, const RankTable &t, const Geometry &g, int lds, hipStream_t s);
// The reduce-scatter sizes its grid itself (tiles of 64 vectors, 128 above 16
// ranks).
hipError_t launch_fused_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, int lds, hipStream_t s);
hipError_t launch_fused_all_gather(const RankTable &t, const Geometry &g, int lds, hipStream_t s);
// Phased forms: slices of g.slice_bytes bytes in inputs at one 16-byte phase
// (table pointers aligned down to 16 bytes, the data g.in_off bytes in) into
// outputs at one phase (table pointers advanced g.out_off bytes to a 16-byte
// boundary).  They write every whole 16-byte vector of that output frame
// (reduce-scatter: g.Rv per output; all-gather: those wholly inside each piece,
// tiles on the grid of g.ref), reading the inputs through aligned pairs of
// vectors; the elements outside go through launch_elem_reduce_scatter and
// launch_elem_all_gather_edges.
hipError_t launch_fused_reduce_scatter_phased(int dt, int op, const RankTable &t, const Geometry &g, int lds,
                                              hipStream_t s);
hipError_t launch_fused_all_gather_phased(const RankTable &t, const Geometry &g, int lds, hipStream_t s);
hipError_t launch_allreduce_halves(int dt, int op, const RankTable &t, const Geometry &g, int lds_rs, int lds_ag,
                                   hipStream_t s);
// Fused pass in the aligned pairwise order over ranks (all-reduce only): one
// workgroup of ceil(n / K) waves per 64-vector tile of [0, Vfull).
hipError_t launch_split_allreduce(int dt, int op, const RankTable &t, const Geometry &g, hipStream_t s);
// Ring / staged tree: ``grid`` sizes the persistent launch of the any-n
// kernels; the compile-time-n ring kernels launch one workgroup per window and
// reserve ``lds`` bytes of dynamic LDS (a residency cap, as for the fused
// kernels).
hipError_t launch_ring_allreduce(int dt, int op, const RankTable &t, const Geometry &g, int grid, int lds,
                                 hipStream_t s);
hipError_t launch_ring_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, int grid, int lds,
                                      hipStream_t s);
hipError_t launch_ring_all_gather(const RankTable &t, const Geometry &g, int grid, int lds, hipStream_t s);
// Tree and double tree for n <= 16 in one register pass (shapes fixed at
// compile time; dual: the first tree over [0, g.split), the second over
// [g.split, Vfull)); ``lds`` as for the fused kernels.
hipError_t launch_tree_reg_allreduce(bool dual, int dt, int op, const RankTable &t, const Geometry &g, int lds,
                                     hipStream_t s);
// Staged trees (windows of g.W vectors, a multiple of 8): one shape over all
// of [0, Vfull); double tree: ``tree`` over vectors [0, g.split) and
// ``tree2`` over [g.split2, Vfull), one launch each.  The launcher sizes its
// persistent grids from the device's compute units ``cus``.
// The tree schedule over vectors [lo, hi) in one streaming pass when the tree
// is an in-order tree (returns true and the launch status in *err); false
// leaves the call to the LDS-staged kernels.
bool launch_tree_stream_range(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                              long long lo, long long hi, hipStream_t s, hipError_t *err);
// Both halves of the double tree, [lo0, hi0) up ``tree`` and [lo1, hi1) up
// ``tree2``, in one streaming launch when the walk holds both (as above).
bool launch_dtree_stream(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                         const Geometry &g, long long lo0, long long hi0, long long lo1, long long hi1, hipStream_t s,
                         hipError_t *err);
hipError_t launch_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                 int cus, hipStream_t s);
hipError_t launch_dtree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const TreeShape &tree2,
                                  const Geometry &g, int cus, hipStream_t s);
// Workgroups for a persistent launch over ``units`` work units: per_cu per
// compute unit (AR_GRID overrides), at most ``units``.
int grid_for(long long units, int cus, int per_cu);
// Element-wise paths (any alignment, and the all-reduce tail), elements
// [e_begin, e_end) of every rank buffer / slice:
hipError_t launch_elem_ring_allreduce(int dt, int op, const RankTable &t, const Geometry &g, long long e_begin,
                                      long long e_end, hipStream_t s);
// The ring-order remainder of a shifted-frame all-reduce (every chunk's head,
// boundary-straddling vector and the tail), ``t`` the callers' pointers.
hipError_t launch_elem_ring_gaps(int dt, int op, const RankTable &t, const Geometry &g, long long head,
                                 long long count, hipStream_t s);
hipError_t launch_elem_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                      long long e_begin, long long e_end, hipStream_t s);
hipError_t launch_elem_split_allreduce(int dt, int op, const RankTable &t, const Geometry &g, long long e_begin,
                                       long long e_end, hipStream_t s);
// Elements [0, a) and [b, R) of every reduce-scatter slice (a = b = 0: all).
hipError_t launch_elem_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, long long R,
                                      long long a, long long b, hipStream_t s);
hipError_t launch_elem_all_gather(int elem_bytes, const RankTable &t, const Geometry &g, long long R, hipStream_t s);
// The elements of every all-gather piece outside the 16-byte output vectors
// the phased kernel writes (at most 15 bytes at each end of a piece).
hipError_t launch_elem_all_gather_edges(int elem_bytes, const RankTable &t, const Geometry &g, long long R,
                                        hipStream_t s);

// Threads per workgroup for every vector kernel.
constexpr int kThreads = 256;
// Fused kernels: one wavefront per workgroup, one 16-byte vector per lane.
constexpr int kFusedThreads = 64;
constexpr int kFusedTile = kFusedThreads;
// Default dynamic-LDS reservation of a fused workgroup, in KB, per collective
// (caps the resident workgroups per CU; see fused.hip and api.cpp).  The
// all-reduce's reservation grows with the rank count (indexed by n <= 16):
// every resident wave has 2n DRAM streams open, and the best number of
// resident waves per CU falls as n grows, to about 50 / n (20 at n = 2, 13 at
// n = 4, 6 at n = 8, 4 at n = 16; measured on MI355X at 128 MB - 1 GB per
// rank, every n from 2 to 16; n = 2 and 4 re-swept at 256 MB per rank in two
// passes: 8 KB at n = 2 79.2-79.9 % of peak against 77.2-77.5 % at 6 KB, 12 KB
// at n = 4 82.8-83.1 % against 81.0-81.7 % at 14 KB; n = 3, 5-7, 12 and 16 at
// their best already).
constexpr int kFusedLdsAllReduceByN[17] = {0, 0, 8, 10, 12, 16, 20, 22, 24, 28, 32, 34, 36, 38, 40, 40, 40};
// The reduce-scatter (n loads, one store per lane) and the all-gather (one
// load, n stores) likewise, from the same kind of sweep (128 MB per rank on
// the big side): reduce-scatter best at 0 KB for n = 2, 14 KB for n = 6-8,
// 22-26 KB for n = 12-16 (6.4-6.7 TB/s).  The all-gather (ordinary input
// loads) runs best with about 30 / (n + 1) resident waves per CU: 14 KB (11
// per CU) at n = 2, 26 KB (6) at n = 4, 34 KB (4) at n = 6-7, 48 KB (3) at
// n = 8-14, 64 KB (2) from n = 15 on, 24, 32 and 72 included (7.0-7.5 TB/s up
// to n = 16, 6.9 at 32, 6.1 at 72).  (64 KB at n = 8 measured 0.9 points
// faster for calls back to back but 9 points slower for a single call, and
// slower for the phased all-gather, which shares the reservation.)
constexpr int kFusedLdsReduceScatterByN[17] = {0, 0, 0, 6, 10, 12, 14, 14, 14, 16, 18, 20, 22, 22, 24, 24, 24};
constexpr int kFusedLdsAllGatherByN[17] = {0, 0, 14, 18, 26, 30, 34, 34, 48, 48, 48, 48, 48, 48, 48, 64, 64};
constexpr int kFusedLdsAllReduceKB = 0;      // n > 16 (the wide kernel): every cap from 10 to 64 KB measured slower
constexpr int kFusedLdsReduceScatterKB = 48;   // n > 16, two vectors per lane (3 workgroups per CU)
constexpr int kFusedLdsAllGatherKB = 64;
constexpr double kCacheBytes = 256.0 * 1024 * 1024;   // the Infinity Cache (MALL) of MI355X
constexpr int kGatherStreamLds = 36 * 1024;          // all-gather cap once its pieces outgrow that cache
// Default dynamic-LDS reservation of the compile-time-n ring workgroups, in
// KB (on top of their static LDS).
constexpr int kRingLdsKB = 0;
// The all-reduce ring by n, where fewer resident windows kept DRAM access
// local: 24 KB at n = 3, 32 KB at n = 4, 48 KB at n = 5-8, none at n = 2 and
// past 8, where every cap measured level or slower.  Measured on MI355X, fp32,
// 128-256 MB per rank, % of peak in two passes over separate processes:
// n = 3 76.1 -> 77.9 (24 KB), n = 4 76.8 -> 78.9 (32 KB, against 48), n = 5
// 69.5 -> 70.7-71.3 (48 KB), n = 8 70.2 -> 74.3 (48 KB); n = 2 uncapped 79-80
// (a cap cost it up to 38 points); n = 12 level at every cap.
constexpr int kRingLdsAllReduceByN[17] = {0, 0, 0, 24, 32, 48, 48, 48, 48, 0, 0, 0, 0, 0, 0, 0, 0};
constexpr int kRingLdsAllGatherKB = 0;
// Ring/tree kernels: at most this many (rank, vector) items per thread.
constexpr int kItemsPerThread = 4;

}  // namespace ar
