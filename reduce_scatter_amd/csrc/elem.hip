// elem.hip -- element-wise paths: the same arithmetic, in the same order, as
// the vector kernels, one element per thread.  Used for buffers that are not
// 16-byte aligned, reduce-scatter / all-gather slices that are not whole
// 16-byte vectors, and the all-reduce tail (the last count mod lanes
// elements).  Identical results first; loads are batched so the paths are
// not latency-bound.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

constexpr int kElemGridCap = 2048;

static int elem_grid(long long work) {
    long long b = (work + kThreads - 1) / kThreads;
    return (int)(b < 1 ? 1 : (b > kElemGridCap ? kElemGridCap : b));
}

// Element e's chain in the hop order of chunk c: ranks c+1, ..., c (mod n).
// Loads go out in batches of 8 before the batch is combined (a load per hop,
// each waited for before the next, had left the element-wise paths
// latency-bound); lanes past n re-read rank c's element and ignore it.
template <int DT, int OP>
__device__ __forceinline__ typename Pack<DT>::T chain1(const RankTable &t, int n, int c, long long e, float s,
                                                       bool keep32) {
    constexpr int B = 8;
    typename Pack<DT>::T acc{};
    for (int k0 = 0; k0 < n; k0 += B) {
        typename Pack<DT>::T v[B];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
            const int k = k0 + kk < n ? k0 + kk : n - 1;
            int r = c + 1 + k;
            r = r >= n ? r - n : r;
            r = r >= n ? r - n : r;
            v[kk] = load1<DT>(t.src[r], e);
        }
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
            if (k0 + kk >= n) break;
            acc = (k0 + kk == 0) ? first1<DT, OP>(v[kk], s, keep32) : hop1<DT, OP>(acc, v[kk], s, keep32);
        }
    }
    return acc;
}

// All-reduce in ring hop order.  Chunk c (grid y) covers the elements of its
// 16-byte units [floor(c*V/n), floor((c+1)*V/n)); this launch does the part of
// it inside [e0, e1).  The chunk index is uniform across a workgroup, so the
// rank pointers stay in scalar registers (an index computed per element had
// made every pointer a per-lane load).
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_ring_allreduce_kernel(const RankTable t, const Geometry g,
                                                                      long long e0, long long e1) {
    const int n = g.n;
    const int c = (int)blockIdx.y;
    constexpr long long u = Lanes<DT>::value;
    long long lo = u * ((long long)c * g.q + (g.rem ? (long long)((unsigned)(c * g.rem) / (unsigned)n) : 0));
    long long hi = u * ((long long)(c + 1) * g.q + (g.rem ? (long long)((unsigned)((c + 1) * g.rem) / (unsigned)n) : 0));
    lo = lo > e0 ? lo : e0;
    hi = hi < e1 ? hi : e1;
    for (long long e = lo + blockIdx.x * (long long)kThreads + threadIdx.x; e < hi;
         e += (long long)gridDim.x * kThreads) {
        typename Pack<DT>::T acc = chain1<DT, OP>(t, n, c, e, g.s, g.acc32);
        acc = finish1<DT, OP>(acc, n, g);
        for (int r = 0; r < n; ++r) store1<DT>(t.dst[r], e, acc);
    }
}

// The element-wise remainder of an all-reduce in ring hop order whose vectors
// ran in the shifted frame (every buffer at one 16-byte phase; g.Vfull whole
// vectors counted from element ``head``, chunk c taking frame vectors
// [B_c, min(B_{c+1} - 1, Vfull))): chunk c (grid y) minus those vectors, i.e.
// its first ``head`` elements, the vector that straddles its end, and the tail
// after the last whole frame vector.  ``t`` holds the callers' pointers.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_ring_gaps_kernel(const RankTable t, const Geometry g,
                                                                 long long head, long long count) {
    const int n = g.n;
    const int c = (int)blockIdx.y;
    constexpr long long u = Lanes<DT>::value;
    const long long b0 = (long long)c * g.q + (g.rem ? (long long)((unsigned)(c * g.rem) / (unsigned)n) : 0);
    const long long b1 = (long long)(c + 1) * g.q + (g.rem ? (long long)((unsigned)((c + 1) * g.rem) / (unsigned)n) : 0);
    const long long lo = u * b0;
    const long long hi = u * b1 < count ? u * b1 : count;
    const long long fe = b1 - 1 < g.Vfull ? b1 - 1 : g.Vfull;       // frame vectors [b0, fe) were done
    const long long s0 = head + u * b0, s1 = fe > b0 ? head + u * fe : s0;
    const long long a1 = s0 < hi ? s0 : hi;                          // piece 1: [lo, a1)
    const long long a2 = s1 > lo ? s1 : lo;                          // piece 2: [a2, hi)
    const long long len1 = a1 > lo ? a1 - lo : 0, len2 = hi > a2 ? hi - a2 : 0;
    for (long long i = threadIdx.x; i < len1 + len2; i += kThreads) {
        const long long e = i < len1 ? lo + i : a2 + (i - len1);
        typename Pack<DT>::T acc = chain1<DT, OP>(t, n, c, e, g.s, g.acc32);
        acc = finish1<DT, OP>(acc, n, g);
        for (int r = 0; r < n; ++r) store1<DT>(t.dst[r], e, acc);
    }
}

// All-reduce in tree order: ranks are visited children-first (tree.post), so
// every child's partial is final before its parent combines it.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_tree_allreduce_kernel(const RankTable t, const TreeShape tree,
                                                                      const Geometry g, long long e0, long long e1) {
    const int n = g.n;
    typename Pack<DT>::T part[kTableRanks];
    for (long long e = e0 + blockIdx.x * (long long)kThreads + threadIdx.x; e < e1;
         e += (long long)gridDim.x * kThreads) {
        for (int i = 0; i < n; ++i) {
            const int v = tree.post[i];
            typename Pack<DT>::T acc = first1<DT, OP>(load1<DT>(t.src[v], e), g.s);
            for (int q = 0; q < 2; ++q) {
                const int ch = tree.child[v][q];
                if (ch >= 0) {
                    if constexpr (DT == I32) acc = combine<DT, OP>(acc, part[ch]);
                    else acc = round_to<DT>(combine<DT, OP>(acc, part[ch]));
                }
            }
            part[v] = acc;
        }
        const typename Pack<DT>::T root = finish1<DT, OP>(part[tree.root], n, g);
        for (int v = 0; v < n; ++v) store1<DT>(t.dst[v], e, root);
    }
}

// Reduce-scatter: output element i of rank c (grid y) = chunk c's chain over
// inputs c*R + i of ranks c+1, ..., c; elements [0, a) and [b, R) of every
// slice (the vector kernels did [a, b)).
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_reduce_scatter_kernel(const RankTable t, const Geometry g,
                                                                      long long R, long long a, long long b) {
    const int n = g.n;
    const int c = (int)blockIdx.y;
    const long long len = a + (R - b);
    for (long long j = blockIdx.x * (long long)kThreads + threadIdx.x; j < len; j += (long long)gridDim.x * kThreads) {
        const long long i = j < a ? j : b + (j - a);
        const typename Pack<DT>::T acc = chain1<DT, OP>(t, n, c, (long long)c * R + i, g.s, g.acc32);
        store1<DT>(t.dst[c], i, finish1<DT, OP>(acc, n, g));
    }
}

// All-gather: bit copies of 2- or 4-byte elements; piece k is grid y.
template <typename E>
__global__ __launch_bounds__(kThreads) void elem_all_gather_kernel(const RankTable t, const Geometry g, long long R) {
    const int n = g.n;
    const int k = (int)blockIdx.y;
    for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < R; i += (long long)gridDim.x * kThreads) {
        const E v = ((const E *)t.src[k])[i];
        for (int r = 0; r < n; ++r) ((E *)t.dst[r])[(long long)k * R + i] = v;
    }
}

// The elements of all-gather piece k (grid y) outside the output frame's
// 16-byte vectors that lie wholly inside the piece: [0, head) and [tail, R) of
// the piece, where the piece covers frame bytes [b0, b0 + Rb), b0 = k*Rb -
// g.out_off, Rb = R * e.
template <typename E>
__global__ __launch_bounds__(kFusedThreads) void elem_all_gather_edges_kernel(const RankTable t, const Geometry g,
                                                                             long long R) {
    const int n = g.n;
    const int k = (int)blockIdx.y;
    const long long e = (long long)sizeof(E);
    const long long b0 = (long long)k * R * e - g.out_off, b1 = b0 + R * e;   // the piece's frame bytes
    const long long o0 = (b0 + 15) >> 4, o1 = b1 >> 4;               // its whole 16-byte vectors [o0, o1)
    long long head = R, tail = R;
    if (o1 > o0) {
        head = (o0 * 16 - b0) / e;
        tail = (o1 * 16 - b0) / e;
    }
    for (long long i = threadIdx.x; i < R - tail + head; i += kFusedThreads) {
        const long long q = i < head ? i : tail + (i - head);
        const E v = ((const E *)t.src[k])[q];
        for (int r = 0; r < n; ++r) ((E *)t.dst[r])[(long long)k * R + q] = v;
    }
}

// Workgroups along one chunk / slice / piece of ``len`` elements, with n of
// them side by side (grid y).
static dim3 elem_grid2(long long len, int n) {
    long long x = (len + kThreads - 1) / kThreads;
    const long long cap = (kElemGridCap * 4 + n - 1) / n;
    x = x < 1 ? 1 : (x > cap ? cap : x);
    return dim3((unsigned)x, (unsigned)n);
}

hipError_t launch_elem_ring_allreduce(int dt, int op, const RankTable &t, const Geometry &g, long long e0,
                                      long long e1, hipStream_t s) {
    if (e1 <= e0) return hipSuccess;
    const long long chunk = (e1 - e0 + g.n - 1) / g.n + 16;     // at most this many elements of [e0, e1) per chunk
    const dim3 grid = elem_grid2(chunk < e1 - e0 ? chunk : e1 - e0, g.n);
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_ring_allreduce_kernel<decltype(D)::value, decltype(O)::value>, grid, dim3(kThreads), 0, s, t,
                      g, e0, e1);
    });
}

hipError_t launch_elem_ring_gaps(int dt, int op, const RankTable &t, const Geometry &g, long long head,
                                 long long count, hipStream_t s) {
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_ring_gaps_kernel<decltype(D)::value, decltype(O)::value>, dim3(1, (unsigned)g.n),
                      dim3(kThreads), 0, s, t, g, head, count);
    });
}

hipError_t launch_elem_tree_allreduce(int dt, int op, const RankTable &t, const TreeShape &tree, const Geometry &g,
                                      long long e0, long long e1, hipStream_t s) {
    if (e1 <= e0) return hipSuccess;
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_tree_allreduce_kernel<decltype(D)::value, decltype(O)::value>, dim3(elem_grid(e1 - e0)), dim3(kThreads), 0, s, t, tree, g, e0, e1);
    });
}

hipError_t launch_elem_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, long long R,
                                      long long a, long long b, hipStream_t s) {
    if (a + (R - b) <= 0) return hipSuccess;
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value>, elem_grid2(a + (R - b), g.n),
                      dim3(kThreads), 0, s, t, g, R, a, b);
    });
}

hipError_t launch_elem_all_gather_edges(int elem_bytes, const RankTable &t, const Geometry &g, long long R,
                                        hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const dim3 grid(1, (unsigned)g.n);
    if (elem_bytes == 4) return launch(elem_all_gather_edges_kernel<uint32_t>, grid, dim3(kFusedThreads), 0, s, t, g, R);
    return launch(elem_all_gather_edges_kernel<uint16_t>, grid, dim3(kFusedThreads), 0, s, t, g, R);
}

hipError_t launch_elem_all_gather(int elem_bytes, const RankTable &t, const Geometry &g, long long R, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const dim3 grid = elem_grid2(R, g.n);
    if (elem_bytes == 4) return launch(elem_all_gather_kernel<uint32_t>, grid, dim3(kThreads), 0, s, t, g, R);
    return launch(elem_all_gather_kernel<uint16_t>, grid, dim3(kThreads), 0, s, t, g, R);
}

}  // namespace ar
