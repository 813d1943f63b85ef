// fused_rs.hip -- the fused reduce-scatter: one pass in the ring's hop order.
//
// Output vector v of rank c is chunk c's reduction over input vectors
// c*Rv + v of ranks c+1, ..., c: every input byte is read once and every output
// byte written once ((n + 1) * R * e bytes per rank), with results
// bit-identical to the ring schedule.  One workgroup is one wavefront and
// handles one tile of 64*U vectors of one slice, U per lane spaced by the
// wavefront width; the grid is x = tile, y = slice, so the dispatcher walks the
// tiles slice by slice in address order.  Above 16 ranks (the any-n kernel)
// U = 2: two 1 KB runs per rank and twice the loads in flight per lane, under a
// tighter residency cap, measured on MI355X at 128 MB per rank: 6.6-6.7 TB/s at
// n = 24, 32 and 72 against 6.3-6.5 with U = 1.  Up to 16 ranks U = 2 or 4
// never beat U = 1 at its best cap (6.2-6.7 TB/s), so those kernels keep U = 1.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"
#include "fused_common.hpp"

namespace ar {

template <int DT, int OP, int NR, int U>
__global__ __launch_bounds__(kFusedThreads) void fused_reduce_scatter_kernel(const RankTableFor<NR> t, const Geometry g) {
    const int n = NR > 0 ? NR : g.n;
    const int c = (int)blockIdx.y;
    // tiles follow the alignment of the n input slices (slice c of the reference input)
    const TileSpan ts = aligned_tile(0, g.Rv, (long long)blockIdx.x, g.ref + (long long)c * g.Rv, kFusedTile * U);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + threadIdx.x + u * kFusedTile, ok[u]);
    Pack<DT> acc[U];
    chain<DT, OP, NR, U>(t, n, c, ((long long)c * g.Rv + ts.lo) * 16, off, g.s, g.acc32, acc);
    char *p = (char *)t.dst[c] + ts.lo * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        finish<DT, OP>(acc[u], n, g);
        __builtin_nontemporal_store(pack<DT>(acc[u]), (u32x4 *)(p + off[u]));
    }
}

hipError_t launch_fused_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, int lds,
                                       hipStream_t s) {
    if (g.Rv <= 0) return hipSuccess;
    if (g.n > 16) {
        const dim3 grid((unsigned)aligned_tiles(g.Rv, (long long)kFusedTile * 2), (unsigned)g.n);
        return dispatch(dt, op, [&](auto D, auto O) {
            return launch(fused_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value, 0, 2>, grid,
                          dim3(kFusedThreads), (size_t)lds, s, t, g);
        });
    }
    const dim3 grid((unsigned)aligned_tiles(g.Rv, kFusedTile), (unsigned)g.n);
    return dispatch(dt, op, [&](auto D, auto O) {
        return by_ranks(g.n, [&](auto R) {
            return launch(fused_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value, decltype(R)::value, 1>,
                          grid, dim3(kFusedThreads), (size_t)lds, s, narrow<decltype(R)::value>(t), g);
        });
    });
}

}  // namespace ar
