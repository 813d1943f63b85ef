// ring.hip -- the ring schedule, staged through LDS.
//
// The "NCCL all-reduce" post (rakshithvasudev.github.io), section "The ring,
// exactly as the kernel runs it": the buffer is split into n chunks; in the
// reduce-scatter half every rank receives a running total from its
// predecessor, adds its own contribution and passes it on, so chunk c's total
// is complete after n-1 hops at the rank that owns it (the completing step
// applies the postOp and keeps the result); in the all-gather half the
// finished chunks are forwarded unchanged for n-1 more hops, each rank keeping
// a copy.  Chunks are cut into slices that flow independently (section "Why a
// 100 GB all-reduce doesn't OOM": a fixed window per connection, never a
// message-sized buffer).
//
// On one GPU the ranks are buffers.  A workgroup runs the whole ring for one
// window of W vectors at the same offset inside each of the n chunks (a
// "channel"): a (rank r, vector w) item stands for rank r's share of that
// window.  The wire between rank r and rank r+1 is one LDS slot per chunk:
// at step p rank r adds its contribution to the running total of chunk
// (r-1-p) mod n held in LDS, and a workgroup barrier is the hop to the next
// rank.  Each rank's loads for step p+1 are issued before step p's LDS work,
// so HBM latency overlaps the barriers.  HBM traffic is the same 2*n*S bytes
// as the fused pass: every input vector is read once, every output written
// once; the running totals never leave LDS.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

namespace ar {

// Per-thread view of its (rank, vector-in-window) items.
struct Items {
    int count;                         // items this thread owns (<= kItemsPerThread)
    int r[kItemsPerThread];
    int w[kItemsPerThread];
};

__device__ __forceinline__ Items make_items(int n, int W) {
    Items it;
    it.count = 0;
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
        const int q = threadIdx.x + k * kThreads;
        it.r[k] = 0;
        it.w[k] = 0;
        if (q < n * W) {
            it.r[k] = q / W;
            it.w[k] = q - it.r[k] * W;
            it.count = k + 1;
        }
    }
    return it;
}

// mod n for a in [-2n, 2n)
__device__ __forceinline__ int wrap(int a, int n) {
    a = a < 0 ? a + n : a;
    a = a < 0 ? a + n : a;
    return a >= n ? a - n : a;
}

// All-reduce.  LDS: slot[c * W + w] (16 bytes each) and the chunk bounds.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void ring_allreduce_kernel(const RankTable t, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    u32x4 *slot = (u32x4 *)lds;
    long long *vb = (long long *)(lds + (size_t)n * W * 16);     // chunk c = [vb[c], vb[c+1])
    for (int c = threadIdx.x; c <= n; c += kThreads) {
        long long b = ((long long)c * g.V) / n;
        vb[c] = b < g.Vfull ? b : g.Vfull;
    }
    __syncthreads();
    const Items it = make_items(n, W);

    for (long long win = blockIdx.x; win < g.windows; win += gridDim.x) {
        const long long pos0 = win * W;
        // reduce-scatter half: steps p = 0..n-1; at step p rank r handles chunk (r-1-p) mod n
        u32x4 cur[kItemsPerThread], nxt[kItemsPerThread];
        bool ok_cur[kItemsPerThread], ok_nxt[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            ok_cur[k] = false;
            if (k < it.count) {
                const int c = wrap(it.r[k] - 1, n);
                const long long v = vb[c] + pos0 + it.w[k];
                ok_cur[k] = v < vb[c + 1];
                if (ok_cur[k]) cur[k] = ld_stream(t.src[it.r[k]], v);
            }
        }
        for (int p = 0; p < n; ++p) {
            // issue the next step's loads first
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                ok_nxt[k] = false;
                if (k < it.count && p + 1 < n) {
                    const int c = wrap(it.r[k] - 2 - p, n);
                    const long long v = vb[c] + pos0 + it.w[k];
                    ok_nxt[k] = v < vb[c + 1];
                    if (ok_nxt[k]) nxt[k] = ld_stream(t.src[it.r[k]], v);
                }
            }
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                if (!ok_cur[k]) continue;
                const int c = wrap(it.r[k] - 1 - p, n);
                u32x4 *sl = &slot[c * W + it.w[k]];
                Pack<DT> own = unpack<DT>(cur[k]);
                Pack<DT> acc;
                if (p == 0) {
                    acc = first<DT, OP>(own, g.s);                 // send: own contribution alone
                } else {
                    acc = unpack<DT>(*sl);                         // recvReduceSend
                    hop<DT, OP>(acc, own, g.s);
                }
                if (p == n - 1) {                                  // chunk c == r completes here
                    finish<DT, OP>(acc, n, g);
                    st_stream(t.dst[it.r[k]], vb[c] + pos0 + it.w[k], pack<DT>(acc));
                }
                *sl = pack<DT>(acc);
            }
            __syncthreads();                                       // the hop to rank r+1
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                cur[k] = nxt[k];
                ok_cur[k] = ok_nxt[k];
            }
        }
        // all-gather half: at step p rank r receives finished chunk (r-1-p) mod n and keeps it
        for (int p = 0; p < n - 1; ++p) {
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                if (k >= it.count) continue;
                const int c = wrap(it.r[k] - 1 - p, n);
                const long long v = vb[c] + pos0 + it.w[k];
                if (v < vb[c + 1]) st_stream(t.dst[it.r[k]], v, slot[c * W + it.w[k]]);
            }
        }
        __syncthreads();                                           // slots are reused by the next window
    }
}

// Reduce-scatter: the reduce half only; chunk c = input vectors [c*Rv, (c+1)*Rv).
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void ring_reduce_scatter_kernel(const RankTable t, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    u32x4 *slot = (u32x4 *)lds;
    const Items it = make_items(n, W);
    for (long long win = blockIdx.x; win < g.windows; win += gridDim.x) {
        const long long pos0 = win * W;
        u32x4 cur[kItemsPerThread], nxt[kItemsPerThread];
        bool ok[kItemsPerThread];
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            ok[k] = k < it.count && pos0 + it.w[k] < g.Rv;        // same position in every chunk
            if (ok[k]) cur[k] = ld_stream(t.src[it.r[k]], (long long)wrap(it.r[k] - 1, n) * g.Rv + pos0 + it.w[k]);
        }
        for (int p = 0; p < n; ++p) {
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k)
                if (ok[k] && p + 1 < n)
                    nxt[k] = ld_stream(t.src[it.r[k]], (long long)wrap(it.r[k] - 2 - p, n) * g.Rv + pos0 + it.w[k]);
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                if (!ok[k]) continue;
                const int c = wrap(it.r[k] - 1 - p, n);
                u32x4 *sl = &slot[c * W + it.w[k]];
                Pack<DT> own = unpack<DT>(cur[k]);
                Pack<DT> acc;
                if (p == 0) {
                    acc = first<DT, OP>(own, g.s);
                } else {
                    acc = unpack<DT>(*sl);
                    hop<DT, OP>(acc, own, g.s);
                }
                if (p == n - 1) {
                    finish<DT, OP>(acc, n, g);
                    st_stream(t.dst[it.r[k]], pos0 + it.w[k], pack<DT>(acc));
                } else {
                    *sl = pack<DT>(acc);
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) cur[k] = nxt[k];
        }
    }
}

// All-gather: the gather half only.  Every rank keeps its own piece, then the
// pieces are forwarded around the ring for n-1 steps.
__global__ __launch_bounds__(kThreads) void ring_all_gather_kernel(const RankTable t, const Geometry g) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = g.n, W = g.W;
    u32x4 *slot = (u32x4 *)lds;
    const Items it = make_items(n, W);
    for (long long win = blockIdx.x; win < g.windows; win += gridDim.x) {
        const long long pos0 = win * W;
#pragma unroll
        for (int k = 0; k < kItemsPerThread; ++k) {
            if (k >= it.count || pos0 + it.w[k] >= g.Rv) continue;
            const int r = it.r[k];
            const u32x4 x = ld_stream(t.src[r], pos0 + it.w[k]);
            slot[r * W + it.w[k]] = x;
            st_stream(t.dst[r], (long long)r * g.Rv + pos0 + it.w[k], x);          // keep my own piece
        }
        __syncthreads();
        for (int p = 0; p < n - 1; ++p) {
#pragma unroll
            for (int k = 0; k < kItemsPerThread; ++k) {
                if (k >= it.count || pos0 + it.w[k] >= g.Rv) continue;
                const int c = wrap(it.r[k] - 1 - p, n);                            // received from r-1
                st_stream(t.dst[it.r[k]], (long long)c * g.Rv + pos0 + it.w[k], slot[c * W + it.w[k]]);
            }
        }
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------
// Compile-time rank counts (every n = NR from 2 to 16): one (rank, vector) item
// per thread, W vectors per rank per window (RingShape), and every step's
// load issued before the first step runs (a rank's contributions do not
// depend on the running totals, only the LDS work does), so a window costs
// about one HBM round trip plus n barriers.  One workgroup per window, windows
// in address order.  Window j of a chunk (or slice, or piece) is the j-th
// W-vector run of an address-aligned grid (the reference buffer's, as for the
// fused tiles), so chunks whose starts are not W-vector multiples still read
// and write whole 1 KB runs; every rank computes the same window of every
// chunk, which is all the LDS exchange needs.
// ---------------------------------------------------------------------------
template <int NR> __device__ __forceinline__ int wrap_c(int a) { return (a + NR) % NR; }

// Window shape: W vectors per rank, each wavefront holding one rank's share
// of the window (64 threads per rank) or, with two items per thread, two
// ranks' shares (ranks rr and rr + R2, R2 = ceil(n/2) wavefronts).
// Workgroups stay at 512 threads or fewer.  Measured on MI355X (% of peak):
//   * up to 8 ranks, W = 64 (1 KB runs), one item per thread;
//   * 9-16 ranks, W = 32 (512-byte runs), one item per thread.  W = 64 with
//     one item per thread (1024-thread workgroups) ran slower (16 ranks int32
//     at 64 MB per rank 64.9 -> 55.2, 12 ranks fp32 at 128 MB 66.8 -> 50.5:
//     fewer windows resident per compute unit, and each window's 2(n-1)
//     barriers span 16 wavefronts);
//   * the all-reduce at 16 ranks: W = 64 with two items per thread (16 int32
//     at 1 GB per rank 61 -> 68, fp32 at 64 MB 71 -> 73).  The same shape lost
//     4-10 points for the all-reduce at 10-14 ranks and 4 for the all-gather
//     at 16, and left the reduce-scatter level, so only this case has it.
template <int NR, bool AR> struct RingShape {
    static constexpr int IPT = (AR && NR == 16) ? 2 : 1;      // items (ranks) per thread
    static constexpr int W = (IPT == 2 || NR <= 8) ? 64 : 32;
    static constexpr int R2 = (NR + IPT - 1) / IPT;            // rows of W threads (rank shares)
    static constexpr int T = R2 * W;
};

// chunk c of an all-reduce in vectors: [start(c), min(start(c+1), Vfull))
__device__ __forceinline__ long long ring_chunk_start(int c, const Geometry &g) {
    const long long b = (long long)c * g.q;
    return g.rem ? b + (long long)((unsigned)(c * g.rem) / (unsigned)g.n) : b;
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__((RingShape<NR, true>::T)) void ring_allreduce_fast(const RankTableFor<NR> t, const Geometry g) {
    using RS = RingShape<NR, true>;
    constexpr int W = RS::W, IPT = RS::IPT, R2 = RS::R2;
    __shared__ u32x4 slot[NR * W];                 // the wire: one slot per chunk and vector
    const int rr = threadIdx.x / W, w = threadIdx.x % W;
    u32x4 raw[IPT][NR];
    long long vv[IPT][NR];
    bool ok[IPT][NR];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool has = rr + i * R2 < NR;         // no second item for the last wavefront at odd n
        const int r = has ? rr + i * R2 : 0;
#pragma unroll
        for (int p = 0; p < NR; ++p) {             // step p: rank r handles chunk (r-1-p) mod n
            const int c = wrap_c<NR>(r - 1 - p);
            long long e = ring_chunk_start(c + 1, g) - g.shift;
            e = e < g.Vfull ? e : g.Vfull;
            // window blockIdx.x of chunk c, cut on the W-vector grid of rank 0's output addresses
            const TileSpan ts = aligned_tile(ring_chunk_start(c, g), e, blockIdx.x, g.ref, W);
            const long long v = ts.start + w;
            ok[i][p] = has && v >= ts.lo && v < ts.hi;
            vv[i][p] = ok[i][p] ? v : 0;           // an always-valid address for lanes outside the chunk
            raw[i][p] = ld_stream(t.src[r], vv[i][p]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // reduce-scatter half: send, n-2 x receive-reduce-send, receive-reduce-copy-send with the postOp
#pragma unroll
    for (int p = 0; p < NR; ++p) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int r = rr + i * R2;
            const int c = wrap_c<NR>(r - 1 - p);
            if (!ok[i][p]) continue;
            Pack<DT> acc;
            if (p == 0) {
                acc = first<DT, OP>(unpack<DT>(raw[i][p]), g.s);
            } else {
                acc = unpack<DT>(slot[c * W + w]);
                hop<DT, OP>(acc, unpack<DT>(raw[i][p]), g.s);
            }
            if (p == NR - 1) {                     // chunk r completes here: postOp, keep it
                finish<DT, OP>(acc, NR, g);
                st_stream(t.dst[r], vv[i][p], pack<DT>(acc));
            }
            slot[c * W + w] = pack<DT>(acc);
        }
        __syncthreads();                           // the hop to rank r+1
    }
    // all-gather half: at step p rank r receives finished chunk (r-1-p) mod n and keeps it
#pragma unroll
    for (int p = 0; p < NR - 1; ++p) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int r = rr + i * R2;
            const int c = wrap_c<NR>(r - 1 - p);
            if (ok[i][p]) st_stream(t.dst[r], vv[i][p], slot[c * W + w]);
        }
    }
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__((RingShape<NR, false>::T)) void ring_reduce_scatter_fast(const RankTableFor<NR> t, const Geometry g) {
    using RS = RingShape<NR, false>;
    constexpr int W = RS::W, IPT = RS::IPT, R2 = RS::R2;
    __shared__ u32x4 slot[NR * W];
    const int rr = threadIdx.x / W, w = threadIdx.x % W;
    u32x4 raw[IPT][NR];
    long long vpos[IPT][NR];
    bool ok[IPT][NR];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool has = rr + i * R2 < NR;
        const int r = has ? rr + i * R2 : 0;
#pragma unroll
        for (int p = 0; p < NR; ++p) {
            const int c = wrap_c<NR>(r - 1 - p);
            // window blockIdx.x of slice c, cut on the W-vector grid of rank 0's input addresses
            const TileSpan ts = aligned_tile(0, g.Rv, blockIdx.x, g.ref + (long long)c * g.Rv, W);
            const long long v = ts.start + w;
            ok[i][p] = has && v >= ts.lo && v < ts.hi;
            vpos[i][p] = ok[i][p] ? v : 0;
            raw[i][p] = ld_stream(t.src[r], (long long)c * g.Rv + vpos[i][p]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < NR; ++p) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int r = rr + i * R2;
            const int c = wrap_c<NR>(r - 1 - p);
            if (!ok[i][p]) continue;
            Pack<DT> acc;
            if (p == 0) {
                acc = first<DT, OP>(unpack<DT>(raw[i][p]), g.s);
            } else {
                acc = unpack<DT>(slot[c * W + w]);
                hop<DT, OP>(acc, unpack<DT>(raw[i][p]), g.s);
            }
            if (p == NR - 1) {
                finish<DT, OP>(acc, NR, g);
                st_stream(t.dst[r], vpos[i][p], pack<DT>(acc));
            } else {
                slot[c * W + w] = pack<DT>(acc);
            }
        }
        __syncthreads();
    }
}

template <int NR>
__global__ __launch_bounds__((RingShape<NR, false>::T)) void ring_all_gather_fast(const RankTableFor<NR> t, const Geometry g) {
    using RS = RingShape<NR, false>;
    constexpr int W = RS::W, IPT = RS::IPT, R2 = RS::R2;
    __shared__ u32x4 slot[NR * W];
    const int rr = threadIdx.x / W, w = threadIdx.x % W;
    // window blockIdx.x of piece k, cut on the W-vector grid of rank 0's output addresses
    auto at = [&](int k, bool &ok) {
        const TileSpan ts = aligned_tile(0, g.Rv, blockIdx.x, g.ref + (long long)k * g.Rv, W);
        const long long v = ts.start + w;
        ok = v >= ts.lo && v < ts.hi;
        return v;
    };
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int r = rr + i * R2;
        if (r >= NR) continue;
        bool mine_ok;
        const long long mine = at(r, mine_ok);
        if (mine_ok) {
            const u32x4 x = ((const u32x4 *)t.src[r])[mine];   // an ordinary load, as the fused all-gather's input
            slot[r * W + w] = x;
            st_stream(t.dst[r], (long long)r * g.Rv + mine, x);            // keep my own piece
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NR - 1; ++p) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int r = rr + i * R2;
            if (r >= NR) continue;
            const int c = wrap_c<NR>(r - 1 - p);                          // received from rank r-1
            bool ok;
            const long long v = at(c, ok);
            if (ok) st_stream(t.dst[r], (long long)c * g.Rv + v, slot[c * W + w]);
        }
    }
}

// Windows of the fast kernels (one workgroup each): enough aligned W-vector
// windows for the longest chunk or slice, whatever its alignment.
long long ring_fast_windows(const Geometry &g, bool allreduce) {
    const long long W = ((allreduce && g.n == 16) || g.n <= 8) ? 64 : 32;      // RingShape<n, allreduce>::W
    const long long len = allreduce ? (g.V + g.n - 1) / g.n : g.Rv;
    return aligned_tiles(len, W);
}

// Measured on MI355X (fp32, 128 MB per rank): the persistent any-n kernels
// ran at 2.8-3.3 TB/s for n = 3, 5, 6, 7 and 12, against 5.1-5.6 TB/s for the
// compile-time kernels at n = 4, 8 and 16; every n up to 16 now has its own.
bool ring_fast_ranks(int n) { return n >= 2 && n <= 16; }

template <int NR, typename F> hipError_t ring_by_ranks_from(int n, F &&f) {
    if constexpr (NR >= 16) {
        return f(std::integral_constant<int, 16>{});
    } else {
        if (n == NR) return f(std::integral_constant<int, NR>{});
        return ring_by_ranks_from<NR + 1>(n, f);
    }
}
template <typename F> hipError_t ring_by_ranks(int n, F &&f) { return ring_by_ranks_from<2>(n, f); }

static size_t ring_lds_bytes(const Geometry &g, bool bounds) {
    return (size_t)g.n * g.W * 16 + (bounds ? ((size_t)g.n + 1) * sizeof(long long) : 0);
}

hipError_t launch_ring_allreduce(int dt, int op, const RankTable &t, const Geometry &g, int grid, int lds,
                                 hipStream_t s) {
    if (ring_fast_ranks(g.n)) {
        const dim3 blocks((unsigned)ring_fast_windows(g, true));
        return dispatch(dt, op, [&](auto D, auto O) {
            return ring_by_ranks(g.n, [&](auto R) {
                return launch(ring_allreduce_fast<decltype(D)::value, decltype(O)::value, decltype(R)::value>,
                              blocks, dim3(RingShape<decltype(R)::value, true>::T), (size_t)lds, s,
                              narrow<decltype(R)::value>(t), g);
            });
        });
    }
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(ring_allreduce_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid), dim3(kThreads),
                      ring_lds_bytes(g, true), s, t, g);
    });
}

hipError_t launch_ring_reduce_scatter(int dt, int op, const RankTable &t, const Geometry &g, int grid, int lds,
                                      hipStream_t s) {
    if (ring_fast_ranks(g.n)) {
        const dim3 blocks((unsigned)ring_fast_windows(g, false));
        return dispatch(dt, op, [&](auto D, auto O) {
            return ring_by_ranks(g.n, [&](auto R) {
                return launch(ring_reduce_scatter_fast<decltype(D)::value, decltype(O)::value, decltype(R)::value>,
                              blocks, dim3(RingShape<decltype(R)::value, false>::T), (size_t)lds, s,
                              narrow<decltype(R)::value>(t), g);
            });
        });
    }
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(ring_reduce_scatter_kernel<decltype(D)::value, decltype(O)::value>, dim3(grid),
                      dim3(kThreads), ring_lds_bytes(g, false), s, t, g);
    });
}

hipError_t launch_ring_all_gather(const RankTable &t, const Geometry &g, int grid, int lds, hipStream_t s) {
    if (ring_fast_ranks(g.n)) {
        const dim3 blocks((unsigned)ring_fast_windows(g, false));
        return ring_by_ranks(g.n, [&](auto R) {
            return launch(ring_all_gather_fast<decltype(R)::value>, blocks, dim3(RingShape<decltype(R)::value, false>::T),
                          (size_t)lds, s, narrow<decltype(R)::value>(t), g);
        });
    }
    return launch(ring_all_gather_kernel, dim3(grid), dim3(kThreads), ring_lds_bytes(g, false), s, t, g);
}

}  // namespace ar
