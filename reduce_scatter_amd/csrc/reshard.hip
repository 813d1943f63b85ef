// reshard.hip -- the copy kernel of the M-to-N layout reshard.
//
// Every workgroup is one wavefront and copies one tile of one row of one
// segment: U vectors of VB bytes per lane (U * kReshardThreads per tile, the
// lanes adjacent for each u), all read before the first store, then stored to
// each of the segment's destinations (the fused route's one read and r
// writes per byte).  Work units are numbered segment by segment, row by row,
// tile by tile, so consecutive workgroups walk each row in address order.
#include "reshard_kernels.hpp"

namespace ar {

template <int VB> struct VecOf;
template <> struct VecOf<16> { typedef unsigned int T __attribute__((ext_vector_type(4))); };
template <> struct VecOf<8> { typedef unsigned int T __attribute__((ext_vector_type(2))); };
template <> struct VecOf<4> { typedef unsigned int T; };
template <> struct VecOf<2> { typedef unsigned short T; };
template <> struct VecOf<1> { typedef unsigned char T; };

template <int VB, int U>
__global__ __launch_bounds__(kReshardThreads) void reshard_copy_kernel(const ReshardArgs a) {
    typedef typename VecOf<VB>::T V;
    const long long unit = (long long)blockIdx.x;
    int k = 0;
    while (k + 1 < a.nseg && a.seg[k + 1].unit0 <= unit) ++k;         // uniform scan over <= 24 segments
    const ReshardSeg &g = a.seg[k];
    // a launch has fewer than 2^31 work units, so 32-bit divisions suffice
    const unsigned local = (unsigned)(unit - g.unit0);
    const unsigned r = local / (unsigned)g.tiles;                      // row of the segment
    const unsigned tile = local - r * (unsigned)g.tiles;
    const unsigned i0 = r / (unsigned)g.n1;
    const unsigned i1 = r - i0 * (unsigned)g.n1;
    const char *src = g.src + g.src_off + (long long)i0 * g.src_s0 + (long long)i1 * g.src_s1;
    const long long d = g.dst_off + (long long)i0 * g.dst_s0 + (long long)i1 * g.dst_s1;
    // vector u of this lane: byte col[u] of the row, lanes adjacent for every u;
    // a lane past the row's end re-reads the row's last vector and stores nothing
    const long long base = (long long)tile * (kReshardThreads * U * VB) + (long long)threadIdx.x * VB;
    long long col[U];
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        col[u] = base + (long long)u * (kReshardThreads * VB);
        const long long c = col[u] < g.row ? col[u] : g.row - VB;
        v[u] = __builtin_nontemporal_load((const V *)(src + c));
    }
    __builtin_amdgcn_sched_barrier(0);                                 // every load issued before the stores
    for (int j = 0; j < g.dst_count; ++j) {
        char *dp = (char *)a.dst[g.dst_first + j] + d;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (col[u] < g.row) __builtin_nontemporal_store(v[u], (V *)(dp + col[u]));
    }
}

template <int VB>
hipError_t launch_vb(const ReshardArgs &a, dim3 grid, int u, int lds, hipStream_t s) {
    void *args[] = {(void *)&a};
    const dim3 block(kReshardThreads);
    switch (u) {
    case 1: return hipLaunchKernel((const void *)reshard_copy_kernel<VB, 1>, grid, block, args, (size_t)lds, s);
    case 2: return hipLaunchKernel((const void *)reshard_copy_kernel<VB, 2>, grid, block, args, (size_t)lds, s);
    case 4: return hipLaunchKernel((const void *)reshard_copy_kernel<VB, 4>, grid, block, args, (size_t)lds, s);
    case 8: return hipLaunchKernel((const void *)reshard_copy_kernel<VB, 8>, grid, block, args, (size_t)lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reshard(const ReshardArgs &a, long long units, int vb, int u, int lds, hipStream_t s) {
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffffLL || a.nseg < 1 || a.nseg > kReshardSegs) return hipErrorInvalidValue;
    const dim3 grid((unsigned)units);
    switch (vb) {
    case 16: return launch_vb<16>(a, grid, u, lds, s);
    case 8: return launch_vb<8>(a, grid, u, lds, s);
    case 4: return launch_vb<4>(a, grid, u, lds, s);
    case 2: return launch_vb<2>(a, grid, u, lds, s);
    case 1: return launch_vb<1>(a, grid, u, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
