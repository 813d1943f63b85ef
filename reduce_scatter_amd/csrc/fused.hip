// fused.hip -- the fused single-pass schedule.
//
// Every input byte is read once and every output byte written once (2*n*S
// bytes for an all-reduce of S bytes per rank): the model is the in-switch
// reduction of the "NCCL all-reduce" post (rakshithvasudev.github.io, section
// "When the switch does the math": one load that returns the combined value,
// one store that lands on every rank), done here by the GPU that holds all the
// rank buffers.  Each 16-byte vector is combined in the ring's hop order for
// its chunk (chunk c: ranks c+1, c+2, ..., c), so the results are bit-identical
// to the ring schedule.
//
// Work decomposition: a tile is kFusedTile vectors of one chunk; tiles of
// different chunks interleave (tile t -> chunk t mod n) so that concurrently
// running workgroups stream from different offsets.  A persistent grid walks
// the tiles.  Per thread, the loads of up to kRankBatch ranks are issued
// before the first is combined, so up to kUnroll * kRankBatch 16-byte loads
// are in flight per lane.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// Byte offset of the start of tile j of a chunk starting at vector ``vbeg``.
__device__ __forceinline__ long long tile_vec(long long vbeg, long long j) { return vbeg + j * kFusedTile; }

template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void fused_allreduce_kernel(const RankTable t, const Geometry g) {
    const int n = g.n;
    const long long tiles = g.windows * n;
    for (long long tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int c = (int)(tile % n);
        const long long j = tile / n;
        const long long vbeg = ((long long)c * g.V) / n;
        long long vend = ((long long)(c + 1) * g.V) / n;
        if (vend > g.Vfull) vend = g.Vfull;
        const long long v0 = tile_vec(vbeg, j);
        if (v0 >= vend) continue;
        const long long byte0 = v0 * 16;
        unsigned off[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const unsigned lane_vec = threadIdx.x + u * kThreads;
            ok[u] = v0 + lane_vec < vend;
            off[u] = lane_vec * 16u;
        }
        Pack<DT> acc[kUnroll];
        for (int k0 = 0; k0 < n; k0 += kRankBatch) {
            u32x4 raw[kUnroll][kRankBatch];
#pragma unroll
            for (int kk = 0; kk < kRankBatch; ++kk) {
                if (k0 + kk < n) {
                    int r = c + 1 + k0 + kk;
                    r = r >= n ? r - n : r;
                    r = r >= n ? r - n : r;
                    const char *p = (const char *)t.src[r] + byte0;
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
                        if (ok[u]) raw[u][kk] = __builtin_nontemporal_load((const u32x4 *)(p + off[u]));
                }
            }
#pragma unroll
            for (int kk = 0; kk < kRankBatch; ++kk) {
                if (k0 + kk < n) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) {
                        if (!ok[u]) continue;
                        Pack<DT> x = unpack<DT>(raw[u][kk]);
                        if (k0 + kk == 0) acc[u] = first<DT, OP>(x, g.s);
                        else hop<DT, OP>(acc[u], x, g.s);
                    }
                }
            }
        }
        u32x4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!ok[u]) continue;
            post<DT, OP>(acc[u], n);
            w[u] = pack<DT>(acc[u]);
        }
        for (int r = 0; r < n; ++r) {
            char *p = (char *)t.dst[r] + byte0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (ok[u]) __builtin_nontemporal_store(w[u], (u32x4 *)(p + off[u]));
        }
    }
}

// Reduce-scatter: output vector v of rank r is chunk r's reduction over
// input vectors r*Rv + v of ranks r+1, ..., r.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void fused_reduce_scatter_kernel(const RankTable t, const Geometry g) {
    const int n = g.n;
    const long long tiles = g.windows * n;
    for (long long tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int c = (int)(tile % n);
        const long long j = tile / n;
        const long long v0 = j * kFusedTile;       // within the slice
        if (v0 >= g.Rv) continue;
        const long long in_byte0 = ((long long)c * g.Rv + v0) * 16;
        const long long out_byte0 = v0 * 16;
        unsigned off[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const unsigned lane_vec = threadIdx.x + u * kThreads;
            ok[u] = v0 + lane_vec < g.Rv;
            off[u] = lane_vec * 16u;
        }
        Pack<DT> acc[kUnroll];
        for (int k0 = 0; k0 < n; k0 += kRankBatch) {
            u32x4 raw[kUnroll][kRankBatch];
#pragma unroll
            for (int kk = 0; kk < kRankBatch; ++kk) {
                if (k0 + kk < n) {
                    int r = c + 1 + k0 + kk;
                    r = r >= n ? r - n : r;
                    r = r >= n ? r - n : r;
                    const char *p = (const char *)t.src[r] + in_byte0;
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
                        if (ok[u]) raw[u][kk] = __builtin_nontemporal_load((const u32x4 *)(p + off[u]));
                }
            }
#pragma unroll
            for (int kk = 0; kk < kRankBatch; ++kk) {
                if (k0 + kk < n) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) {
                        if (!ok[u]) continue;
                        Pack<DT> x = unpack<DT>(raw[u][kk]);
                        if (k0 + kk == 0) acc[u] = first<DT, OP>(x, g.s);
                        else hop<DT, OP>(acc[u], x, g.s);
                    }
                }
            }
        }
        char *p = (char *)t.dst[c] + out_byte0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!ok[u]) continue;
            post<DT, OP>(acc[u], n);
            __builtin_nontemporal_store(pack<DT>(acc[u]), (u32x4 *)(p + off[u]));
        }
    }
}

// All-gather: input vector v of piece k is read once and written to vector
// k*Rv + v of every output.  Pure assembly, no arithmetic.
__global__ __launch_bounds__(kThreads) void fused_all_gather_kernel(const RankTable t, const Geometry g) {
    const int n = g.n;
    const long long tiles = g.windows * n;
    for (long long tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int k = (int)(tile % n);
        const long long j = tile / n;
        const long long v0 = j * kFusedTile;
        if (v0 >= g.Rv) continue;
        const long long in_byte0 = v0 * 16;
        const long long out_byte0 = ((long long)k * g.Rv + v0) * 16;
        unsigned off[kUnroll];
        bool ok[kUnroll];
        u32x4 w[kUnroll];
        const char *src = (const char *)t.src[k] + in_byte0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const unsigned lane_vec = threadIdx.x + u * kThreads;
            ok[u] = v0 + lane_vec < g.Rv;
            off[u] = lane_vec * 16u;
            if (ok[u]) w[u] = __builtin_nontemporal_load((const u32x4 *)(src + off[u]));
        }
        for (int r = 0; r < n; ++r) {
            char *p = (char *)t.dst[r] + out_byte0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (ok[u]) __builtin_nontemporal_store(w[u], (u32x4 *)(p + off[u]));
        }
    }
}

hipError_t launch_fused_allreduce(int dt, int op, const RankTable &t, const Geometry &g, int grid, hipStream_t s) {
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(fused_allreduce_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid), dim3(kThreads), 0, s, t, g);
    });
}

hipError_t launch_fused_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, int grid,
                                       hipStream_t s) {
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(fused_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid), dim3(kThreads), 0, s, t, g);
    });
}

hipError_t launch_fused_all_gather(const RankTable &t, const Geometry &g, int grid, hipStream_t s) {
    return launch(fused_all_gather_kernel, dim3(grid), dim3(kThreads), 0, s, t, g);
}

}  // namespace ar
