// reshard.hip -- the copy kernel of the M-to-N layout reshard.
//
// Every workgroup is one wavefront and copies one tile of one row of one
// segment: kReshardThreads vectors of VB bytes, one per lane, read once from
// the segment's source and stored to each of its destinations (the fused
// route's one read and r writes per byte, the same access pattern as the
// fused all-gather).  Work units are numbered segment by segment, row by row,
// tile by tile, so consecutive workgroups walk each row in address order.
#include "reshard_kernels.hpp"

namespace ar {

template <int VB> struct VecOf;
template <> struct VecOf<16> { typedef unsigned int T __attribute__((ext_vector_type(4))); };
template <> struct VecOf<8> { typedef unsigned int T __attribute__((ext_vector_type(2))); };
template <> struct VecOf<4> { typedef unsigned int T; };
template <> struct VecOf<2> { typedef unsigned short T; };
template <> struct VecOf<1> { typedef unsigned char T; };

template <int VB>
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
    const long long col = (long long)tile * (kReshardThreads * VB) + (long long)threadIdx.x * VB;
    if (col >= g.row) return;                                          // past the row's end (last tile)
    const char *sp = g.src + g.src_off + (long long)i0 * g.src_s0 + (long long)i1 * g.src_s1 + col;
    const V v = __builtin_nontemporal_load((const V *)sp);
    const long long d = g.dst_off + (long long)i0 * g.dst_s0 + (long long)i1 * g.dst_s1 + col;
    for (int j = 0; j < g.dst_count; ++j)
        __builtin_nontemporal_store(v, (V *)((char *)a.dst[g.dst_first + j] + d));
}

hipError_t launch_reshard(const ReshardArgs &a, long long units, int vb, int lds, hipStream_t s) {
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffffLL || a.nseg < 1 || a.nseg > kReshardSegs) return hipErrorInvalidValue;
    const dim3 grid((unsigned)units), block(kReshardThreads);
    void *args[] = {(void *)&a};
    switch (vb) {
    case 16: return hipLaunchKernel((const void *)reshard_copy_kernel<16>, grid, block, args, (size_t)lds, s);
    case 8: return hipLaunchKernel((const void *)reshard_copy_kernel<8>, grid, block, args, (size_t)lds, s);
    case 4: return hipLaunchKernel((const void *)reshard_copy_kernel<4>, grid, block, args, (size_t)lds, s);
    case 2: return hipLaunchKernel((const void *)reshard_copy_kernel<2>, grid, block, args, (size_t)lds, s);
    case 1: return hipLaunchKernel((const void *)reshard_copy_kernel<1>, grid, block, args, (size_t)lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
