// split.hip -- the fused single pass with the ranks split across the waves of
// a workgroup and combined in a fixed pairwise order.
//
// The model is the in-switch reduction of the "NCCL all-reduce" post
// (rakshithvasudev.github.io, section "When the switch does the math"): one
// load returns the value combined over every rank and one store lands it on
// every rank, so every input byte is read once and every output byte written
// once (2*n*S bytes for S bytes per rank), and no rank waits for another's
// partial.  The post leaves the order of the switch's additions open; here it
// is the aligned binary tree over rank indices: ranks [lo, lo+len) combine as
// [lo, lo+h) (+) [lo+h, lo+len) with h the largest power of two below len,
// the lower ranks being the left operand.  Each contribution enters as a
// storage-type value (float avg pre-scales it by fp32(1/n)), every combine is
// computed in fp32 (int32: wrapping) and rounded to the storage type, and the
// int32 avg divides the total by n once.  The chain of dependent combines is
// ceil(log2 n) long instead of the ring order's n-1, which is what matters
// when there are many ranks and little data per rank.
//
// Work decomposition: a workgroup owns one tile of 64 16-byte vectors at the
// same offset of every rank buffer (no chunks: the order does not depend on
// the position).  Wave w holds the aligned block of K ranks [w*K, w*K+K); its
// lanes read 64 consecutive vectors of each of those ranks (one coalesced
// 1 KB run per rank), all K loads in flight before the first combine.  The K
// contributions are combined in registers (the low levels of the tree), the
// waves' partials meet in LDS (the high levels), every wave finishes the tree
// for the tile and stores the result to its own K ranks.  K is the smallest
// power of two that keeps the workgroup at 16 waves or fewer.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"

#include <cstdlib>

namespace ar {

// Aligned pairwise combination of a sequence of partials, fed left to right:
// st[l] holds the partial of the latest complete aligned block of 2^l inputs.
// Adding input number i merges it with st[l] for every trailing one bit of i
// (the block on the left is the left operand).  ``finish`` combines what is
// left for a count of c inputs: the blocks of c's set bits, the lowest-ranked
// (highest bit) leftmost.  Every index is a compile-time constant once the
// callers' loops are unrolled, so the stack stays in registers.
template <int DT, int OP, int L> struct PairStack {
    Pack<DT> st[L];

    template <int I, int l = 0> __device__ __forceinline__ void push(Pack<DT> v) {
        if constexpr (l < L - 1 && ((I >> l) & 1)) {
            merge<DT, OP>(st[l], v);
            push<I, l + 1>(st[l]);
        } else {
            st[l] = v;
        }
    }

    __device__ __forceinline__ Pack<DT> finish(int c) {
        Pack<DT> acc = st[0];
        bool have = false;
#pragma unroll
        for (int l = 0; l < L; ++l) {
            if (!((c >> l) & 1)) continue;
            if (have) {
                merge<DT, OP>(st[l], acc);
                acc = st[l];
            } else {
                acc = st[l];
                have = true;
            }
        }
        return acc;
    }
};

template <int N> struct Log2Ceil { static constexpr int value = N <= 1 ? 0 : 1 + Log2Ceil<(N + 1) / 2>::value; };
template <> struct Log2Ceil<1> { static constexpr int value = 0; };

constexpr int kSplitMaxWaves = 16;

template <int I, int K, int DT, int OP, int L>
__device__ __forceinline__ void push_ranks(PairStack<DT, OP, L> &ps, const u32x4 *raw, int stride, int valid,
                                           float s) {
    if constexpr (I < K) {
        if (I < valid) {
            ps.template push<I>(first<DT, OP>(unpack<DT>(raw[I * stride]), s));
            push_ranks<I + 1, K>(ps, raw, stride, valid, s);
        }
    }
}

template <int I, int DT, int OP, int L>
__device__ __forceinline__ void push_waves(PairStack<DT, OP, L> &ps, const u32x4 *part, int stride, int valid) {
    if constexpr (I < kSplitMaxWaves) {
        if (I < valid) {
            ps.template push<I>(unpack<DT>(part[I * stride]));
            push_waves<I + 1>(ps, part, stride, valid);
        }
    }
}

// One workgroup per tile of 64*U vectors; lane l of every wave owns vectors
// l, l+64, ..., l+64*(U-1) of the tile, so each load instruction of a wave
// is one 1 KB run of one rank and a wave reads U KB of each of its ranks.
// Phase 1: all K*U loads in flight, then each of the U vectors' K
// contributions combined in registers and stored to LDS (one partial per
// wave).  Phase 2: each tile vector's partials are combined once, by one
// thread, the postOp applied, the result written back to LDS.  Phase 3: every
// wave stores the finished tile to its own ranks.
template <int DT, int OP, int K, int U, int CAP>
__global__ __launch_bounds__(kFusedThreads *kSplitMaxWaves) void split_allreduce_kernel(const RankTableN<CAP> t,
                                                                                        const Geometry g) {
    constexpr int T = kFusedThreads * U;                        // vectors per tile
    __shared__ u32x4 part[kSplitMaxWaves * T];                  // part[w * T + v]
    const int n = g.n;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));     // wave index (uniform)
    const int lane = (int)(threadIdx.x & 63);
    const int waves = (int)(blockDim.x >> 6);
    const int r0 = w * K;                                       // this wave's ranks: [r0, min(r0 + K, n))
    const int mine = min(K, n - r0);                            // >= 1: the block has ceil(n / K) waves
    const TileSpan ts = aligned_tile(0, g.Vfull, blockIdx.x, g.ref, T);   // non-empty: the grid has no spare tile
    const long long base = ts.lo * 16;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + lane + u * kFusedThreads, ok[u]);

    u32x4 raw[K * U];                                           // raw[k * U + u]
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const char *p = (const char *)t.src[k < mine ? r0 + k : r0 + mine - 1] + base;   // past n: ignored
#pragma unroll
        for (int u = 0; u < U; ++u) raw[k * U + u] = __builtin_nontemporal_load((const u32x4 *)(p + off[u]));
    }
    __builtin_amdgcn_sched_barrier(0);                          // every load issued before the first combine
#pragma unroll
    for (int u = 0; u < U; ++u) {
        PairStack<DT, OP, Log2Ceil<K>::value + 1> lo;
        push_ranks<0, K>(lo, raw + u, U, mine, g.s);
        part[w * T + u * kFusedThreads + lane] = pack<DT>(lo.finish(mine));
    }
    __syncthreads();

    for (int v = (int)threadIdx.x; v < T; v += (int)blockDim.x) {
        PairStack<DT, OP, Log2Ceil<kSplitMaxWaves>::value + 1> hi;
        push_waves<0>(hi, part + v, T, waves);
        Pack<DT> acc = hi.finish(waves);
        finish<DT, OP>(acc, n, g);
        part[v] = pack<DT>(acc);                                // only this thread touches index v here
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const u32x4 out = part[u * kFusedThreads + lane];
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (k < mine) __builtin_nontemporal_store(out, (u32x4 *)((char *)t.dst[r0 + k] + base + off[u]));
    }
}

// Element-wise form (buffers not 16-byte aligned, and the count mod lanes
// tail): one element per thread, the same aligned pairwise order over all n
// ranks, with the block stack indexed at run time.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void elem_split_allreduce_kernel(const RankTable t, const Geometry g,
                                                                        long long e_begin, long long e_end) {
    typedef typename Pack<DT>::T T;
    const long long i = e_begin + (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= e_end) return;
    const int n = g.n;
    T st[8];                                                    // n <= 128: blocks of up to 2^7 ranks
    for (int r = 0; r < n; ++r) {
        T v = first1<DT, OP>(load1<DT>(t.src[r], i), g.s);
        int l = 0;
        for (; (r >> l) & 1; ++l) v = merge1<DT, OP>(st[l], v);
        st[l] = v;
    }
    T acc = st[0];
    bool have = false;
    for (int l = 0; l < 8; ++l) {
        if (!((n >> l) & 1)) continue;
        acc = have ? merge1<DT, OP>(st[l], acc) : st[l];
        have = true;
    }
    acc = finish1<DT, OP>(acc, n, g);
    for (int r = 0; r < n; ++r) store1<DT>(t.dst[r], i, acc);
}

// Ranks per wave: the smallest power of two with ceil(n / K) <= 16 waves
// (AR_SPLIT_K raises it: 2, 4, 8 or 16).
int split_ranks_per_wave(int n) {
    static const int env = [] {
        const char *e = getenv("AR_SPLIT_K");
        const int v = e ? atoi(e) : 0;
        return (v == 2 || v == 4 || v == 8 || v == 16) ? v : 0;
    }();
    int k = 1;
    while ((n + k - 1) / k > kSplitMaxWaves) k *= 2;
    // from 17 to 64 ranks fewer, fuller waves: 4 ranks per wave, one vector per lane, a 32 KB residency
    // cap (measured on MI355X at 25 MB per rank in place, n = 17, 24, 32, 48: +1-12 % over 2 ranks per wave
    // uncapped, in three pairs of runs); past 64 the same change measured level or slower
    const int pref = (n > 16 && n <= 64) ? 4 : 1;
    k = k < pref ? pref : k;
    return k < env ? env : k;
}

// Vectors per lane and rank (AR_SPLIT_U overrides: 1, 2 or 4).  Measured on
// MI355X: 2 (2 KB runs per rank, twice the bytes in flight) is best up to 16
// ranks (n = 8, 256 MB per rank: 6.15 TB/s against 5.62 with 1); past 16
// ranks, where a wave holds 4 or more ranks' loads, 1 is best (n = 72, 25 MB
// per rank: 5.51 TB/s against 5.20 with 2).
int split_vectors_per_lane(int K, int n) {
    static const int env = [] {
        const char *e = getenv("AR_SPLIT_U");
        const int v = e ? atoi(e) : 0;
        return (v == 1 || v == 2 || v == 4) ? v : 0;
    }();
    if (env) return (K >= 8 && env == 4) ? 2 : (K == 16 ? 1 : env);
    return (K >= 8 || n > 16) ? 1 : 2;      // past 16 ranks K is 4 or more
}

// Dynamic LDS a split workgroup reserves beyond its static partials (a
// residency cap: 32 KB from 17 to 64 ranks, none otherwise; AR_SPLIT_LDS_KB
// overrides).
int split_lds_bytes(int n) {
    static const int v = [] {
        const char *e = getenv("AR_SPLIT_LDS_KB");
        const long kb = e ? atol(e) : -1;
        return kb < 0 ? -1 : (int)(kb > 128 ? 128 : kb) * 1024;
    }();
    if (v >= 0) return v;
    return (n > 16 && n <= 64) ? 32 * 1024 : 0;
}

// The rank table goes in at 16 entries for n <= 16 (256 bytes of kernel
// arguments instead of 2 KB: the split kernel serves the small calls, where
// the launch's host time is the call's cost).
template <int DT, int OP, int K, int CAP>
hipError_t launch_split_cap(int U, const RankTableN<CAP> &t, const Geometry &g, dim3 grid, dim3 block, size_t lds,
                            hipStream_t s) {
    switch (U) {
    case 1: return launch(split_allreduce_kernel<DT, OP, K, 1, CAP>, grid, block, lds, s, t, g);
    case 2:
        if constexpr (K < 16) return launch(split_allreduce_kernel<DT, OP, K, 2, CAP>, grid, block, lds, s, t, g);
        return hipErrorInvalidValue;
    default:
        if constexpr (K < 8) return launch(split_allreduce_kernel<DT, OP, K, 4, CAP>, grid, block, lds, s, t, g);
        return hipErrorInvalidValue;
    }
}

template <int DT, int OP, int K>
hipError_t launch_split_u(int U, const RankTable &t, const Geometry &g, dim3 block, hipStream_t s) {
    const long long T = (long long)kFusedThreads * U;
    const dim3 grid((unsigned)((((g.ref & (T - 1)) + g.Vfull) + T - 1) / T));       // tiles of the aligned grid
    const size_t lds = (size_t)split_lds_bytes(g.n);
    if (g.n <= 16) return launch_split_cap<DT, OP, K, 16>(U, narrow<16>(t), g, grid, block, lds, s);
    return launch_split_cap<DT, OP, K, 0>(U, t, g, grid, block, lds, s);
}

hipError_t launch_split_allreduce(int dt, int op, const RankTable &t, const Geometry &g, hipStream_t s) {
    const int K = split_ranks_per_wave(g.n);
    const int U = split_vectors_per_lane(K, g.n);
    const dim3 block((unsigned)(((g.n + K - 1) / K) * kFusedThreads));
    return dispatch(dt, op, [&](auto D, auto O) {
        constexpr int DT = decltype(D)::value, OP = decltype(O)::value;
        switch (K) {
        case 1: return launch_split_u<DT, OP, 1>(U, t, g, block, s);
        case 2: return launch_split_u<DT, OP, 2>(U, t, g, block, s);
        case 4: return launch_split_u<DT, OP, 4>(U, t, g, block, s);
        case 8: return launch_split_u<DT, OP, 8>(U, t, g, block, s);
        case 16: return launch_split_u<DT, OP, 16>(U, t, g, block, s);
        default: return hipErrorInvalidValue;
        }
    });
}

hipError_t launch_elem_split_allreduce(int dt, int op, const RankTable &t, const Geometry &g, long long e_begin,
                                       long long e_end, hipStream_t s) {
    const long long elems = e_end - e_begin;
    if (elems <= 0) return hipSuccess;
    const dim3 grid((unsigned)((elems + kThreads - 1) / kThreads));
    return dispatch(dt, op, [&](auto D, auto O) {
        return launch(elem_split_allreduce_kernel<decltype(D)::value, decltype(O)::value>, grid, dim3(kThreads), 0,
                      s, t, g, e_begin, e_end);
    });
}

}  // namespace ar
