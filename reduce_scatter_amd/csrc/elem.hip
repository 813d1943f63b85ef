// elem.hip -- element-wise paths: the same arithmetic, in the same order, as
// the vector kernels, one element per thread.  Used for buffers that are not
// 16-byte aligned and for the all-reduce tail (the last count mod lanes
// elements).  Throughput is not a goal here; identical results are.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

constexpr int kElemGridCap = 2048;

static int elem_grid(long long work) {
    long long b = (work + kThreads - 1) / kThreads;
    return (int)(b < 1 ? 1 : (b > kElemGridCap ? kElemGridCap : b));
}

// All-reduce in ring hop order.  Element e lies in vector e / lanes, which
// lies in chunk c = ((vec+1)*n - 1) / V (the chunk whose 16-byte-unit range
// [floor(c*V/n), floor((c+1)*V/n)) contains it).
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_ring_allreduce_kernel(const RankTable t, const Geometry g,
                                                                      long long e0, long long e1) {
    const int n = g.n;
    for (long long e = e0 + blockIdx.x * (long long)kThreads + threadIdx.x; e < e1;
         e += (long long)gridDim.x * kThreads) {
        const long long vec = e / Lanes<DT>::value;
        const int c = (int)(((vec + 1) * n - 1) / g.V);
        typename Pack<DT>::T acc = first1<DT, OP>(load1<DT>(t.src[add_mod(c, 1 % n, n)], e), g.s, g.acc32);
        for (int k = 2; k <= n; ++k) {
            int r = c + k;
            r = r >= n ? r - n : r;
            r = r >= n ? r - n : r;
            acc = hop1<DT, OP>(acc, load1<DT>(t.src[r], e), g.s, g.acc32);
        }
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

// Reduce-scatter: output element i of rank r = chunk r's chain over inputs
// r*R + i of ranks r+1, ..., r.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_reduce_scatter_kernel(const RankTable t, const Geometry g,
                                                                      long long R) {
    const int n = g.n;
    const long long total = (long long)n * R;
    for (long long q = blockIdx.x * (long long)kThreads + threadIdx.x; q < total;
         q += (long long)gridDim.x * kThreads) {
        const int c = (int)(q / R);
        const long long i = q - (long long)c * R;
        const long long e = (long long)c * R + i;
        typename Pack<DT>::T acc = first1<DT, OP>(load1<DT>(t.src[add_mod(c, 1 % n, n)], e), g.s, g.acc32);
        for (int k = 2; k <= n; ++k) {
            int r = c + k;
            r = r >= n ? r - n : r;
            r = r >= n ? r - n : r;
            acc = hop1<DT, OP>(acc, load1<DT>(t.src[r], e), g.s, g.acc32);
        }
        store1<DT>(t.dst[c], i, finish1<DT, OP>(acc, n, g));
    }
}

// All-gather: bit copies of 2- or 4-byte elements.
template <typename E>
__global__ __launch_bounds__(kThreads) void elem_all_gather_kernel(const RankTable t, const Geometry g, long long R) {
    const int n = g.n;
    const long long total = (long long)n * R;
    for (long long q = blockIdx.x * (long long)kThreads + threadIdx.x; q < total;
         q += (long long)gridDim.x * kThreads) {
        const int k = (int)(q / R);
        const long long i = q - (long long)k * R;
        const E v = ((const E *)t.src[k])[i];
        for (int r = 0; r < n; ++r) ((E *)t.dst[r])[(long long)k * R + i] = v;
    }
}

hipError_t launch_elem_ring_allreduce(int dt, int op, const RankTable &t, const Geometry &g, long long e0,
                                      long long e1, hipStream_t s) {
    if (e1 <= e0) return hipSuccess;
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_ring_allreduce_kernel<decltype(D)::value, decltype(O)::value>, dim3(elem_grid(e1 - e0)), dim3(kThreads), 0, s, t, g, e0, e1);
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
                                      hipStream_t s) {
    if (R <= 0) return hipSuccess;
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value>, dim3(elem_grid((long long)g.n * R)), dim3(kThreads), 0, s, t, g, R);
    });
}

hipError_t launch_elem_all_gather(int elem_bytes, const RankTable &t, const Geometry &g, long long R, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const dim3 grid(elem_grid((long long)g.n * R));
    if (elem_bytes == 4) return launch(elem_all_gather_kernel<uint32_t>, grid, dim3(kThreads), 0, s, t, g, R);
    return launch(elem_all_gather_kernel<uint16_t>, grid, dim3(kThreads), 0, s, t, g, R);
}

}  // namespace ar
