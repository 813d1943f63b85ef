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
// Work decomposition (measured on MI355X, see the design notes): one
// workgroup is ONE wavefront and handles one tile of kFusedTile = 64
// 16-byte vectors of one chunk, one vector per lane; the grid has one
// workgroup per tile, in chunk-major order, so the hardware dispatcher keeps
// the set of tiles in flight compact in address space.  Each lane issues the
// loads of up to NB ranks before combining the first, then the n stores.
// Workgroups reserve dynamic LDS they never touch: the reservation caps how
// many are resident per CU (6 with 24 KB of the 160 KB per CU), which keeps
// the number of concurrently open DRAM streams low.  That cap, not maximum
// occupancy, lifts this 2n-stream read/write pattern from ~71 % to ~77-79 %
// of peak HBM bandwidth on gradient-like data.
#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"
#include "fused_common.hpp"

namespace ar {

// The grid is 2-D: x = tile within the chunk, y = chunk, so the dispatcher
// walks tiles chunk by chunk in address order and no division is needed.
__device__ __forceinline__ void tile_coords(int &c, long long &j) {
    c = (int)blockIdx.y;
    j = (long long)blockIdx.x;
}

template <int NR, class TAB>
__device__ __forceinline__ void store_all(const TAB &t, int n, long long base, unsigned lane_off, u32x4 w) {
    if constexpr (NR > 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
            __builtin_nontemporal_store(w, (u32x4d *)((char *)t.dst[r] + base + lane_off));
    } else {
        for (int r = 0; r < n; ++r) __builtin_nontemporal_store(w, (u32x4d *)((char *)t.dst[r] + base + lane_off));
    }
}

// Start of all-reduce chunk c in vectors, floor(c*V/n), as c*q + floor(c*rem/n)
// with q = V / n and rem = V % n (host-computed): no 64-bit division and no
// table fetch stands between a workgroup's start and its first load.
__device__ __forceinline__ long long chunk_start(int c, const Geometry &g) {
    const long long b = (long long)c * g.q;
    return g.rem ? b + (long long)((unsigned)(c * g.rem) / (unsigned)g.n) : b;
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kFusedThreads) void fused_allreduce_kernel(const RankTableFor<NR> t, const Geometry g) {
    const int n = NR > 0 ? NR : g.n;
    int c;
    long long j;
    tile_coords(c, j);
    long long vend = chunk_start(c + 1, g) - g.shift;
    vend = vend < g.Vfull ? vend : g.Vfull;
    const TileSpan ts = aligned_tile(chunk_start(c, g), vend, j, g.ref, kFusedTile);
    if (ts.lo >= ts.hi) return;                               // past the chunk's end: nothing in this tile
    bool ok;
    const unsigned lane_off = tile_lane(ts, ts.start + threadIdx.x, ok);
    const unsigned off[1] = {lane_off};
    Pack<DT> acc[1];
    chain<DT, OP, NR, 1>(t, n, c, ts.lo * 16, off, g.s, g.acc32, acc);
    if (!ok) return;
    finish<DT, OP>(acc[0], n, g);
    store_all<NR>(t, n, ts.lo * 16, lane_off, pack<DT>(acc[0]));
}

// Many ranks (n > 16): with 2n streams per tile, DRAM locality comes from
// long runs per stream, so each lane owns U vectors of the tile spaced by the
// wavefront width (a 64*U-vector tile: 16 KB per rank for 4-byte types, 8 KB
// for 2-byte types, which need twice the registers per vector) and the ranks
// are walked two at a time, each rank's U loads issued as one run before the
// next rank's (left to the scheduler, the two ranks' loads alternate vector by
// vector).  Measured at n = 72 with 25 MB per rank: 65 % of peak HBM
// bandwidth, against 53 % for one vector per lane.
//
// A chunk's tiles are whole except its first and last.  A whole tile takes
// the lean path (every lane's vectors in range, byte offsets lane*16 + u*1024
// folded into the scalar rank pointer); the edge tiles take the clamped path,
// with in-tile positions in 32 bits and the range checks as one bit mask, so
// both fit a wavefront in 256 registers and two wavefronts share a SIMD.
// Every tile of a 72-rank call is resident at once, so the call lasts as long
// as its slowest tile: the edge tiles keep the two-rank batches.  Measured at
// n = 72, 25 MB per rank, fp32 in place: with 64-bit range checks on every
// tile the kernel needed 260 registers (one wavefront per SIMD) and ran 62 %
// of peak.
template <int DT> struct WideTile {
    static constexpr int U = (DT == BF16 || DT == F16) ? 8 : 16;
    static constexpr int B = 2;
};

template <int DT, int OP, bool KEEP32>
__device__ __forceinline__ void wide_whole_tile(const RankTable &t, int n, int c, long long base, const Geometry &g) {
    constexpr int U = WideTile<DT>::U, B = WideTile<DT>::B;
    const unsigned lane = threadIdx.x * 16u;
    Pack<DT> acc[U];
    for (int k0 = 0; k0 < n; k0 += B) {
        const char *ptr[B];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) ptr[kk] = (const char *)t.src[hop_rank(c, k0 + kk < n ? k0 + kk : n - 1, n)] + base;
        __builtin_amdgcn_sched_barrier(0);                     // the batch's rank pointers before its loads
        u32x4 raw[B][U];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                raw[kk][u] = __builtin_nontemporal_load((const u32x4d *)(ptr[kk] + u * kFusedThreads * 16 + lane));
            __builtin_amdgcn_sched_barrier(0);                 // one rank's run issued whole before the next
        }
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
            if (k0 + kk >= n) break;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (k0 + kk == 0) acc[u] = first<DT, OP, KEEP32>(unpack<DT>(raw[kk][u]), g.s);
                else hop<DT, OP, KEEP32>(acc[u], unpack<DT>(raw[kk][u]), g.s);
            }
        }
    }
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        finish<DT, OP>(acc[u], n, g);
        w[u] = pack<DT>(acc[u]);
    }
    for (int r = 0; r < n; ++r) {
        char *p = (char *)t.dst[r] + base;
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(w[u], (u32x4d *)(p + u * kFusedThreads * 16 + lane));
    }
}

template <int DT, int OP, bool KEEP32>
__device__ __forceinline__ void wide_edge_tile(const RankTable &t, int n, int c, const TileSpan &ts, const Geometry &g) {
    constexpr int U = WideTile<DT>::U, B = WideTile<DT>::B;
    // positions inside the tile in 32 bits: the in-range part is [lo, hi) of [0, 64*U)
    const int lo = (int)(ts.lo - ts.start), hi = (int)(ts.hi - ts.start);
    unsigned off[U];
    unsigned okm = 0;                                          // bit u: vector u of this lane is in range
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = (int)threadIdx.x + u * kFusedThreads;
        okm |= (unsigned)(v >= lo && v < hi) << u;
        off[u] = (unsigned)((v < lo ? lo : (v >= hi ? hi - 1 : v)) - lo) * 16u;
    }
    const long long base = ts.lo * 16;
    Pack<DT> acc[U];
    for (int k0 = 0; k0 < n; k0 += B) {
        const char *ptr[B];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) ptr[kk] = (const char *)t.src[hop_rank(c, k0 + kk < n ? k0 + kk : n - 1, n)] + base;
        __builtin_amdgcn_sched_barrier(0);
        u32x4 raw[B][U];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
#pragma unroll
            for (int u = 0; u < U; ++u) raw[kk][u] = __builtin_nontemporal_load((const u32x4d *)(ptr[kk] + off[u]));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
            if (k0 + kk >= n) break;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (k0 + kk == 0) acc[u] = first<DT, OP, KEEP32>(unpack<DT>(raw[kk][u]), g.s);
                else hop<DT, OP, KEEP32>(acc[u], unpack<DT>(raw[kk][u]), g.s);
            }
        }
    }
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        finish<DT, OP>(acc[u], n, g);
        w[u] = pack<DT>(acc[u]);
    }
    for (int r = 0; r < n; ++r) {
        char *p = (char *)t.dst[r] + base;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((okm >> u) & 1u) __builtin_nontemporal_store(w[u], (u32x4d *)(p + off[u]));
    }
}

// A tile across the boundary of chunks c and c+1 holds the end of chunk c
// (hop order c+1, c+2, ..., c) and the start of chunk c+1 (c+2, ..., c, c+1):
// the same ranks, one step apart.  So one workgroup walks the rank sequence
// c+1, ..., c, c+1 (n+1 loads) over the whole tile: lanes of chunk c take
// steps 0..n-1, lanes of chunk c+1 steps 1..n, each its own chunk's exact
// order.  Measured at n = 72, 25 MB per rank (chunk boundaries off the tile
// grid): two partial-tile workgroups per boundary, each as long as a whole
// tile, had held the kernel at 64-65 % of peak against 68-70 % with the
// boundaries on the grid.
template <int DT, int OP, bool KEEP32>
__device__ __forceinline__ void wide_shared_tile(const RankTable &t, int n, int c, long long ts, long long b,
                                                 const Geometry &g) {
    constexpr int U = WideTile<DT>::U, B = WideTile<DT>::B;
    const unsigned lane = threadIdx.x * 16u;
    const long long base = ts * 16;
    const int bb = (int)(b - ts);                              // chunk c+1 starts at vector bb of the tile
    unsigned upper = 0, skip = 0;                              // bit u: vector u of this lane is chunk c+1's;
#pragma unroll                                                 // ... is the shifted frame's vector b-1 (no chunk's)
    for (int u = 0; u < U; ++u) {
        const int v = (int)threadIdx.x + u * kFusedThreads;
        upper |= (unsigned)(v >= bb) << u;
        skip |= (unsigned)(g.shift != 0 && v == bb - 1) << u;
    }
    Pack<DT> acc[U];
    {                                                          // steps 0 and 1
        const char *p0 = (const char *)t.src[hop_rank(c, 0, n)] + base;
        const char *p1 = (const char *)t.src[hop_rank(c, 1, n)] + base;
        __builtin_amdgcn_sched_barrier(0);
        u32x4 r0[U], r1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r0[u] = __builtin_nontemporal_load((const u32x4d *)(p0 + u * kFusedThreads * 16 + lane));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) r1[u] = __builtin_nontemporal_load((const u32x4d *)(p1 + u * kFusedThreads * 16 + lane));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Pack<DT> lower = first<DT, OP, KEEP32>(unpack<DT>(r0[u]), g.s);
            hop<DT, OP, KEEP32>(lower, unpack<DT>(r1[u]), g.s);
            const Pack<DT> up = first<DT, OP, KEEP32>(unpack<DT>(r1[u]), g.s);
            const bool sel = (upper >> u) & 1u;
#pragma unroll
            for (int e = 0; e < Pack<DT>::K; ++e) acc[u].v[e] = sel ? up.v[e] : lower.v[e];   // per lane, no memory
        }
    }
    for (int k0 = 2; k0 < n; k0 += B) {                        // steps 2..n-1: every lane
        const char *ptr[B];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) ptr[kk] = (const char *)t.src[hop_rank(c, k0 + kk < n ? k0 + kk : n - 1, n)] + base;
        __builtin_amdgcn_sched_barrier(0);
        u32x4 raw[B][U];
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                raw[kk][u] = __builtin_nontemporal_load((const u32x4d *)(ptr[kk] + u * kFusedThreads * 16 + lane));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < B; ++kk) {
            if (k0 + kk >= n) break;
#pragma unroll
            for (int u = 0; u < U; ++u) hop<DT, OP, KEEP32>(acc[u], unpack<DT>(raw[kk][u]), g.s);
        }
    }
    {                                                          // step n: chunk c+1's last hop (rank c+1)
        const char *pn = (const char *)t.src[hop_rank(c, n, n)] + base;
        __builtin_amdgcn_sched_barrier(0);
        u32x4 rn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) rn[u] = __builtin_nontemporal_load((const u32x4d *)(pn + u * kFusedThreads * 16 + lane));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Pack<DT> h = acc[u];
            hop<DT, OP, KEEP32>(h, unpack<DT>(rn[u]), g.s);
            const bool sel = (upper >> u) & 1u;
#pragma unroll
            for (int e = 0; e < Pack<DT>::K; ++e) acc[u].v[e] = sel ? h.v[e] : acc[u].v[e];
        }
    }
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        finish<DT, OP>(acc[u], n, g);
        w[u] = pack<DT>(acc[u]);
    }
    for (int r = 0; r < n; ++r) {
        char *p = (char *)t.dst[r] + base;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (!((skip >> u) & 1u)) __builtin_nontemporal_store(w[u], (u32x4d *)(p + u * kFusedThreads * 16 + lane));
    }
}

// Chunk geometry of the wide kernel, shared by the host (the grid) and the
// device.  Chunk c is frame vectors [lo, hi): the floor cut, less the shifted
// frame's last vector, clamped to Vfull.  c * rem < 128 * 128 fits 32 bits.
__host__ __device__ inline long long wide_chunk_start(int c, const Geometry &g) {
    const long long b = (long long)c * g.q;
    return g.rem ? b + (long long)((unsigned)(c * g.rem) / (unsigned)g.n) : b;
}

__host__ __device__ inline void wide_chunk(int c, const Geometry &g, long long &lo, long long &hi) {
    lo = wide_chunk_start(c, g);
    hi = wide_chunk_start(c + 1, g) - g.shift;
    hi = hi < g.Vfull ? hi : g.Vfull;
}

// Tiles of the ref-aligned T-vector grid that overlap [lo, hi).
__host__ __device__ inline long long wide_tiles(const Geometry &g, long long lo, long long hi, long long T) {
    return hi > lo ? (g.ref + hi + T - 1) / T - (g.ref + lo) / T : 0;
}

// Whether the tile across the boundary of chunks c and c+1 is one shared
// unit: whole, inside [0, Vfull), holding vectors of both chunks and of no
// other.  ts: its first vector.
__host__ __device__ inline bool wide_shared(int c, const Geometry &g, long long T, long long &ts) {
    if (c + 1 >= g.n) return false;
    const long long b = wide_chunk_start(c + 1, g);
    const long long m = (g.ref + b) & (T - 1);
    if (m <= g.shift) return false;                            // on the grid, or chunk c's part of it is empty
    ts = b - m;
    long long lo, hi, lo1, hi1;
    wide_chunk(c, g, lo, hi);
    wide_chunk(c + 1, g, lo1, hi1);
    return ts >= lo && ts + T <= hi1;
}

// The wide kernel's grid is one workgroup per unit, numbered in address
// order: a unit is one tile of one chunk, except that a shared boundary tile
// (above) is one unit, counted with the lower chunk; first[c] is the number
// of units before chunk c.  Workgroups are dealt to the 8 XCDs round robin,
// and every unit of a 72-rank call is resident at once, so the busiest XCD
// sets the time: a grid of n rows of equal length, the shorter chunks' rows
// padded with empty workgroups, left some XCDs 5 % more tiles than others
// (measured at n = 72, 25 MB per rank: 65 % of peak against 69 % for the same
// tiles without the holes).
struct WidePieces {
    unsigned first[kTableRanks + 1];
};

template <int DT, int OP, bool KEEP32>
__device__ __forceinline__ void fused_allreduce_wide(const RankTable &t, const Geometry &g, const WidePieces &pc) {
    constexpr long long T = (long long)kFusedThreads * WideTile<DT>::U;
    const unsigned p = blockIdx.x;
    int lo = 0, hi = g.n;                                      // the chunk c with first[c] <= p < first[c+1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pc.first[mid] <= p) lo = mid;
        else hi = mid;
    }
    const int c = lo;
    long long cl, ch, ts;
    wide_chunk(c, g, cl, ch);
    long long j = (long long)(p - pc.first[c]);
    if (c > 0 && wide_shared(c - 1, g, T, ts)) ++j;            // the first tile went with chunk c-1
    if (j == wide_tiles(g, cl, ch, T) - 1 && wide_shared(c, g, T, ts)) {
        wide_shared_tile<DT, OP, KEEP32>(t, g.n, c, ts, wide_chunk_start(c + 1, g), g);
        return;
    }
    const TileSpan tsp = aligned_tile(cl, ch, j, g.ref, T);
    if (tsp.lo >= tsp.hi) return;
    if (tsp.lo == tsp.start && tsp.hi == tsp.start + T) wide_whole_tile<DT, OP, KEEP32>(t, g.n, c, tsp.lo * 16, g);
    else wide_edge_tile<DT, OP, KEEP32>(t, g.n, c, tsp, g);
}

template <int DT, int OP>
__global__ __launch_bounds__(kFusedThreads) void fused_allreduce_wide_kernel(const RankTable t, const Geometry g,
                                                                             const WidePieces pc) {
    if constexpr (DT == BF16 || DT == F16) {
        if (g.acc32) {
            fused_allreduce_wide<DT, OP, true>(t, g, pc);
            return;
        }
    }
    fused_allreduce_wide<DT, OP, false>(t, g, pc);
}

// All-gather: input vector v of piece k is read once and written to vector
// k*Rv + v of every output.  Pure assembly, no arithmetic.  The input is read
// with an ordinary load and the outputs written non-temporally: measured on
// MI355X, a non-temporal input load cost this one-load, n-store pattern
// 6-14 % (n = 8 bf16, 16 Mi elements per piece: 6.4 against 7.2 TB/s), while
// the reduce-scatter and the all-reduce (n loads per store) ran best with
// non-temporal loads and stores.  A tile is 64*U vectors, U per lane spaced by
// the wavefront width.  Measured on MI355X at 256 MB out per rank: U = 2 ran
// 6.4-7.3 TB/s at every n from 2 to 12, against 5.3-6.2 for n = 3, 5, 6, 7 and
// 12 with U = 1 (level at n = 2 and 8, 3 % lower at n = 4); 16 ranks and the
// one-rank copy ran 5 % faster with U = 1; past 16 ranks (n = 17, 24, 32, 72
// at 64 and 256 MB out per rank) U = 2 averaged 6.1-6.8 against 5.5-6.4 TB/s.
int gather_vectors_per_lane(int n) { return (n >= 2 && n != 16) ? 2 : 1; }

template <int NR, int U>
__global__ __launch_bounds__(kFusedThreads) void fused_all_gather_kernel(const RankTableFor<NR> t, const Geometry g) {
    const int n = NR > 0 ? NR : g.n;
    int k;
    long long j;
    tile_coords(k, j);
    // tiles follow the alignment of the n outputs (piece k of the reference output)
    const TileSpan ts = aligned_tile(0, g.Rv, j, g.ref + (long long)k * g.Rv, kFusedTile * U);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + threadIdx.x + u * kFusedTile, ok[u]);
    const char *p = (const char *)t.src[k] + ts.lo * 16;
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *(const u32x4 *)(p + off[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (ok[u]) store_all<NR>(t, n, ((long long)k * g.Rv + ts.lo) * 16, off[u], w[u]);
}

// Units of the wide (n > 16) all-reduce kernel, first[c] per chunk (see
// WidePieces).  Returns the total, or -1 past the grid's x limit.
long long wide_pieces(int dt, const Geometry &g, WidePieces &pc) {
    const long long T = kFusedThreads * ((dt == BF16 || dt == F16) ? WideTile<BF16>::U : WideTile<F32>::U);
    long long total = 0, ts;
    for (int c = 0; c < g.n; ++c) {
        pc.first[c] = (unsigned)total;
        long long lo, hi;
        wide_chunk(c, g, lo, hi);
        total += wide_tiles(g, lo, hi, T) - ((c > 0 && wide_shared(c - 1, g, T, ts)) ? 1 : 0);
        if (total > 0x7fffffffLL) return -1;
    }
    for (int c = g.n; c <= kTableRanks; ++c) pc.first[c] = (unsigned)total;
    return total;
}

hipError_t launch_fused_allreduce(int dt, int op, const RankTable &t, const Geometry &g, int lds, hipStream_t s) {
    if (g.n > 16) {
        WidePieces pc;
        const long long pieces = wide_pieces(dt, g, pc);
        if (pieces < 0) return hipErrorInvalidValue;
        if (pieces == 0) return hipSuccess;
        return dispatch(dt, op, [&](auto D, auto O) {
            return launch(fused_allreduce_wide_kernel<decltype(D)::value, decltype(O)::value>, dim3((unsigned)pieces),
                          dim3(kFusedThreads), (size_t)lds, s, t, g, pc);
        });
    }
    const dim3 grid((unsigned)g.windows, (unsigned)g.n);
    return dispatch(dt, op, [&](auto D, auto O) {
        return by_ranks(g.n, [&](auto R) {
            return launch(fused_allreduce_kernel<decltype(D)::value, decltype(O)::value, decltype(R)::value>, grid,
                          dim3(kFusedThreads), (size_t)lds, s, narrow<decltype(R)::value>(t), g);
        });
    });
}

hipError_t launch_fused_all_gather(const RankTable &t, const Geometry &g, int lds, hipStream_t s) {
    if (g.Rv <= 0) return hipSuccess;
    const int U = gather_vectors_per_lane(g.n);
    const dim3 grid((unsigned)aligned_tiles(g.Rv, (long long)kFusedTile * U), (unsigned)g.n);
    return by_ranks(g.n, [&](auto R) {
        constexpr int NR = decltype(R)::value;
        if (U == 2) return launch(fused_all_gather_kernel<NR, 2>, grid, dim3(kFusedThreads), (size_t)lds, s, narrow<NR>(t), g);
        return launch(fused_all_gather_kernel<NR, 1>, grid, dim3(kFusedThreads), (size_t)lds, s, narrow<NR>(t), g);
    });
}

}  // namespace ar
