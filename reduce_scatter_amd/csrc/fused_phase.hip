// fused_phase.hip -- the fused reduce-scatter and all-gather for slices whose
// byte length is not a multiple of 16.
//
// Reduce-scatter input slice c of every rank starts c*R*e bytes into a
// 16-byte-aligned buffer, so with R*e not a multiple of 16 the slices sit at
// different phases within 16-byte vectors, while every output is aligned.
// Each lane reads its 16 input bytes either as the two aligned vectors around
// them, assembled by a funnel shift (funnel16), or as one load from the word
// boundary at or below them (4-byte alignment is enough for a 16-byte global
// load), shifted by whole bytes only where the phase is not whole words (the
// phase is the same for every rank of a slice, so either choice is uniform
// across the workgroup); it combines the n contributions in the ring hop
// order exactly as the aligned kernel does and stores one aligned output
// vector.  (A first form loaded the second vector only for a non-zero
// phase; that branch made the compiler wait for each rank's pair before
// issuing the next, and n = 16 ran at 3.1 TB/s.)  The all-gather is the mirror image: aligned input pieces,
// output pieces at phase k*R*e mod 16, each lane assembling the 16 input bytes
// that land in one whole output vector.  The elements of the partial vectors
// at the slice edges go through the element-wise kernels.  The second vector
// of a pair is the neighbour lane's first, served by the cache; only the line
// past a tile's end is fetched twice (by this tile and the next, which runs on
// another XCD), so the larger the tile, the closer the fetched bytes come to
// the algorithmic ones.
#include <cstdlib>
#include <cstring>

#include "ar_device.hpp"
#include "ar_kernels.hpp"
#include "dispatch.hpp"
#include "fused_common.hpp"

namespace ar {

// The vector of lane + 1, and ``last`` in lane 63: lane 0's value is replaced
// by ``last`` and the wavefront rotated left by one lane (ds_bpermute: each
// lane reads another lane's register through the LDS crossbar, no LDS
// memory).  The exchange runs with every lane active: a lane reading from a
// lane that is switched off gets zero, and selecting ``last`` after the read
// let the compiler switch lane 63 off for it (lane 62 then read zeros).
__device__ __forceinline__ u32x4 next_lane(u32x4 v, u32x4 last, bool first_lane) {
    const int src = (int)((((threadIdx.x & 63u) + 1u) & 63u) << 2);   // byte address of lane + 1 mod 64
    const u32x4 w = first_lane ? last : v;
    u32x4 r;
    r.x = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)w.x);
    r.y = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)w.y);
    r.z = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)w.z);
    r.w = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)w.w);
    return r;
}

// Lane 0's vector, in every lane.
__device__ __forceinline__ u32x4 lane0(u32x4 v) {
    u32x4 r;
    r.x = (unsigned)__builtin_amdgcn_readlane((int)v.x, 0);
    r.y = (unsigned)__builtin_amdgcn_readlane((int)v.y, 0);
    r.z = (unsigned)__builtin_amdgcn_readlane((int)v.z, 0);
    r.w = (unsigned)__builtin_amdgcn_readlane((int)v.w, 0);
    return r;
}

// Combine the n ranks' 16 bytes at byte ``base + lane_off[u] + ph`` (u < U;
// ``base`` a multiple of 16, the same for the whole workgroup, and so is the
// phase ``ph``) in the hop order of chunk c into acc[u].  Each lane loads the
// two aligned vectors that hold its bytes, every load of the chain issued
// before the first combine; the second vector of a lane is its neighbour's
// first (a cache hit, except past the last lane of a run).  CLAMP (the tiles
// at the input's end only, a uniform choice): the second vector at ``base +
// hi_off[u]``, hi_off = lane_off + 16 clamped to the input's last 16-byte
// block (past it the second vector is only reached with ph = 0, where it is
// not used).  Elsewhere it is addressed as the first plus 16: measured on
// MI355X, the clamp's separate address on every tile cost the n = 8 bf16
// reduce-scatter 13 % (5.5 -> 4.8 TB/s).  Compile-time n only (past 16 ranks
// the word-aligned chain below runs).
//
// NEXT (whole tiles away from the input's end only; a uniform choice): lane l's
// second vector is lane l+1's first, taken from its register (next_lane),
// lane 63's is lane 0's first of the next run, or for the last run one more
// load at the same address in every lane (one line): each rank costs U + 1
// load instructions instead of 2U, and the cache serves one request per line
// instead of two.  Measured on MI355X with R - 1 elements per slice, 256 MB in
// per rank: n = 8 fp32 72.1 -> 76.3-76.6 % of peak, n = 16 bf16 72.6 -> 74 %,
// n = 8 bf16 and n = 3 level.  The phased all-gather measured level or slower
// with it and keeps both loads.
template <int DT, int OP, int NR, bool KEEP32, bool CLAMP, int U, bool NEXT = false>
__device__ __forceinline__ void chain_phased(const RankTableFor<NR> &t, int c, long long base,
                                             const unsigned (&lane_off)[U], const unsigned (&hi_off)[U], unsigned ph,
                                             float s, Pack<DT> (&acc)[U]) {
    static_assert(NR > 0, "past 16 ranks the word-aligned chain runs");
    static_assert(!(NEXT && CLAMP), "the register neighbour needs the unclamped layout");
    if constexpr (NEXT) {
        const bool lane0_ = (threadIdx.x & 63u) == 0u;
        const void *ptr[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) ptr[k] = t.src[hop_rank(c, k, NR)];
        __builtin_amdgcn_sched_barrier(0);
        u32x4 lo[NR][U], ex[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const char *p = (const char *)ptr[k] + base;
#pragma unroll
            for (int u = 0; u < U; ++u) lo[k][u] = __builtin_nontemporal_load((const u32x4 *)(p + lane_off[u]));
            ex[k] = *(const u32x4 *)(p + kFusedTile * U * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const u32x4 hi = next_lane(lo[k][u], u + 1 < U ? lane0(lo[k][u + 1 < U ? u + 1 : u]) : ex[k], lane0_);
                const Pack<DT> x = unpack<DT>(funnel16(lo[k][u], hi, ph));
                if (k == 0) acc[u] = first<DT, OP, KEEP32>(x, s);
                else hop<DT, OP, KEEP32>(acc[u], x, s);
            }
        }
    } else {
        const void *ptr[NR];                 // every rank pointer's scalar load issued before the vector loads
#pragma unroll
        for (int k = 0; k < NR; ++k) ptr[k] = t.src[hop_rank(c, k, NR)];
        __builtin_amdgcn_sched_barrier(0);
        u32x4 lo[NR][U], hi[NR][U];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const char *p = (const char *)ptr[k] + base + lane_off[u];
                lo[k][u] = __builtin_nontemporal_load((const u32x4 *)p);
                hi[k][u] = CLAMP ? *(const u32x4 *)(p - lane_off[u] + hi_off[u]) : *(const u32x4 *)(p + 16);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[u] = first<DT, OP, KEEP32>(unpack<DT>(funnel16(lo[0][u], hi[0][u], ph)), s);
#pragma unroll
            for (int k = 1; k < NR; ++k) hop<DT, OP, KEEP32>(acc[u], unpack<DT>(funnel16(lo[k][u], hi[k][u], ph)), s);
        }
    }
}

// The 16 bytes that start b bytes into v (b < 4), the last b of them from nx,
// the word after v (v_alignbyte_b32 per word).
__device__ __forceinline__ u32x4 shift_words(u32x4 v, unsigned nx, unsigned b) {
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(v.y, v.x, b);
    r.y = __builtin_amdgcn_alignbyte(v.z, v.y, b);
    r.z = __builtin_amdgcn_alignbyte(v.w, v.z, b);
    r.w = __builtin_amdgcn_alignbyte(nx, v.w, b);
    return r;
}

// The word w of lane + 1, and ``last`` in lane 63 (as next_lane, one word).
__device__ __forceinline__ unsigned next_word(unsigned w, unsigned last, bool first_lane) {
    const int src = (int)((((threadIdx.x & 63u) + 1u) & 63u) << 2);
    return (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)(first_lane ? last : w));
}

// Word-aligned form of the chain: each lane loads its 16 input bytes from the
// word boundary at or just below them, ``wbase + lane_off[u]`` (wbase = the
// tile's first input byte rounded down to a word, uniform; b = the bytes it
// was rounded by, uniform), so a rank costs one load per vector, as in the
// aligned kernel, and 4-byte types need no shift at all.  Only with b != 0
// (2-byte types at a slice whose phase is an odd number of elements: NX) the
// last b bytes come from the next word: from the next lane's register on whole
// tiles (XCHG: lane 63's from lane 0 of the next run, or for the last run one
// dword load at the tile's end, the same address in every lane), else from a
// dword load.  Every byte read lies in the word holding the lane's first input
// byte through the word holding its last, so no load passes the input's last
// 16-byte block and no clamp is needed.
template <int DT, int OP, int NR, bool KEEP32, int U, bool NX, bool XCHG, class TAB>
__device__ __forceinline__ void chain_words(const TAB &t, int n, int c, long long wbase,
                                            const unsigned (&lane_off)[U], unsigned b, float s, Pack<DT> (&acc)[U]) {
    static_assert(!(XCHG && !NX), "the exchange only supplies the word after the vector");
    static_assert(!(XCHG && NR == 0), "the any-n chain loads the word");
    if constexpr (NR > 0) {
        const bool lane0_ = (threadIdx.x & 63u) == 0u;
        const void *ptr[NR];                 // every rank pointer's scalar load issued before the vector loads
#pragma unroll
        for (int k = 0; k < NR; ++k) ptr[k] = t.src[hop_rank(c, k, NR)];
        __builtin_amdgcn_sched_barrier(0);
        u32x4 v[NR][U];
        unsigned nx[NR][U], ex[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const char *p = (const char *)ptr[k] + wbase;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v[k][u] = __builtin_nontemporal_load((const u32x4d *)(p + lane_off[u]));
                if constexpr (NX && !XCHG) nx[k][u] = *(const unsigned *)(p + lane_off[u] + 16);
            }
            if constexpr (XCHG) ex[k] = *(const unsigned *)(p + kFusedTile * U * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                u32x4 w = v[k][u];
                if constexpr (XCHG) {
                    const unsigned last =
                        u + 1 < U ? (unsigned)__builtin_amdgcn_readlane((int)v[k][u + 1 < U ? u + 1 : u].x, 0) : ex[k];
                    w = shift_words(w, next_word(v[k][u].x, last, lane0_), b);
                } else if constexpr (NX) {
                    w = shift_words(w, nx[k][u], b);
                }
                const Pack<DT> x = unpack<DT>(w);
                if (k == 0) acc[u] = first<DT, OP, KEEP32>(x, s);
                else hop<DT, OP, KEEP32>(acc[u], x, s);
            }
        }
    } else {
        static_assert(U == 1, "the any-n chain takes one vector per lane");
        constexpr int B = 8;
        for (int k0 = 0; k0 < n; k0 += B) {
            u32x4 v[B];
            unsigned nx[B];
#pragma unroll
            for (int kk = 0; kk < B; ++kk) {
                const int k = k0 + kk < n ? k0 + kk : n - 1;                 // past n: a valid, ignored load
                const char *p = (const char *)t.src[hop_rank(c, k, n)] + wbase + lane_off[0];
                v[kk] = __builtin_nontemporal_load((const u32x4d *)p);
                if constexpr (NX) nx[kk] = *(const unsigned *)(p + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < B; ++kk) {
                if (k0 + kk >= n) break;
                u32x4 w = v[kk];
                if constexpr (NX) w = shift_words(w, nx[kk], b);
                const Pack<DT> x = unpack<DT>(w);
                if (k0 + kk == 0) acc[0] = first<DT, OP, KEEP32>(x, s);
                else hop<DT, OP, KEEP32>(acc[0], x, s);
            }
        }
    }
}

// Reduce-scatter: grid x = tiles of output vectors, y = slice c.  Output
// vector o of rank c (16 bytes at g.out_off + 16*o of the caller's output) is
// chunk c's chain over the same element positions of input slice c of ranks
// c+1, ..., c: bytes g.in_off + c*Rb + 16*o from the aligned table pointers (Rb
// = g.slice_bytes bytes per slice, g.Rv whole output vectors).  Tiles follow
// output c's alignment: its writes are the ones a cache line split between two
// workgroups would cost; the reads sit at the slice's phase whatever the
// tiling.  Both loads of a lane stay in 16-byte blocks that hold input bytes
// (the second is clamped to the last one).  A tile is 64*U output vectors, U
// per lane spaced by the wavefront width, so each load instruction covers one
// 1 KB run and only the last run's second vectors reach past the tile (into a
// line the next tile, on another XCD's L2, fetches again).  U = 2 up to 8
// ranks: measured on MI355X with R - 1 elements per slice (256 MB in per
// rank, n = 8), 5.87 against 5.53 TB/s for bf16 and 5.74 against 5.55 for
// fp32; level at n = 4 and 16, so 16 ranks and more keep U = 1.
template <int NR> struct PhasedTile {
    static constexpr int U = (NR > 0 && NR <= 8) ? 2 : 1;
};

// Start of all-reduce chunk c in vectors, floor(c*V/n), as c*q + floor(c*rem/n).
__device__ __forceinline__ long long ar_chunk_lo(int c, const Geometry &g) {
    const long long b = (long long)c * g.q;
    return g.rem ? b + (long long)((unsigned)(c * g.rem) / (unsigned)g.n) : b;
}

template <int DT, int OP, int NR, bool KEEP32>
__device__ __forceinline__ void rs_phased(const RankTableFor<NR> &t, const Geometry &g) {
    constexpr int U = PhasedTile<NR>::U;
    const int n = NR > 0 ? NR : g.n;
    const int c = (int)blockIdx.y;
    // a workgroup of blockDim.x / 64 wavefronts takes that many consecutive tiles, one per wavefront
    const long long j = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const unsigned lane = threadIdx.x & 63u;
    long long lo = 0, hi = g.Rv;
    if (g.ar_chunks) {                                       // all-reduce chunk c, at its own offset
        lo = ar_chunk_lo(c, g);
        hi = ar_chunk_lo(c + 1, g) - g.shift;               // shifted frame: the vector across the end is not c's
        hi = hi < g.Vfull ? hi : g.Vfull;
    }
    const TileSpan ts = aligned_tile(lo, hi, j, (long long)((uintptr_t)t.dst[c] >> 4), kFusedTile * U);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + lane + u * kFusedTile, ok[u]);
    const long long a = g.ar_chunks ? ts.lo * 16 : g.in_off + (long long)c * g.slice_bytes + ts.lo * 16;  // first input byte
    const long long rel = g.last_off - (a & ~15LL);                             // last block, from the tile base
    Pack<DT> acc[U];
    const bool whole = ts.lo == ts.start && ts.hi == ts.start + kFusedTile * U;
    const unsigned b = (unsigned)(a & 3);                       // 0 for 4-byte types (element-aligned inputs)
    if (NR == 0 || g.phased_words == 2 || (g.phased_words == 1 && b != 0)) {
        if (Lanes<DT>::value == 4 || b == 0) {
            chain_words<DT, OP, NR, KEEP32, U, false, false>(t, n, c, a & ~3LL, off, 0u, g.s, acc);
        } else if constexpr (Lanes<DT>::value == 8) {
            if (NR > 0 && whole)
                chain_words<DT, OP, NR, KEEP32, U, true, (NR > 0)>(t, n, c, a & ~3LL, off, b, g.s, acc);
            else
                chain_words<DT, OP, NR, KEEP32, U, true, false>(t, n, c, a & ~3LL, off, b, g.s, acc);
        }
    } else if constexpr (NR > 0) {
        if (whole && rel >= 16 * (kFusedTile * U + 1)) {        // the neighbour's vector from its register
            chain_phased<DT, OP, NR, KEEP32, false, U, true>(t, c, a & ~15LL, off, off, (unsigned)(a & 15), g.s, acc);
        } else if (rel >= 16 * (kFusedTile * U + 1)) {   // no lane's second vector can pass the input's last block
            chain_phased<DT, OP, NR, KEEP32, false, U>(t, c, a & ~15LL, off, off, (unsigned)(a & 15), g.s, acc);
        } else {                             // the input's last tiles: the second load clamped (a uniform branch)
            unsigned hi_off[U];
#pragma unroll
            for (int u = 0; u < U; ++u) hi_off[u] = (long long)off[u] + 16 < rel ? off[u] + 16u : (unsigned)rel;
            chain_phased<DT, OP, NR, KEEP32, true, U>(t, c, a & ~15LL, off, hi_off, (unsigned)(a & 15), g.s, acc);
        }
    }
    char *p = (char *)t.dst[c] + ts.lo * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        finish<DT, OP>(acc[u], n, g);
        __builtin_nontemporal_store(pack<DT>(acc[u]), (u32x4d *)(p + off[u]));
    }
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__(8 * kFusedThreads) void fused_reduce_scatter_phased_kernel(const RankTableFor<NR> t,
                                                                                       const Geometry g) {
    if constexpr (DT == BF16 || DT == F16) {
        if (g.acc32) {
            rs_phased<DT, OP, NR, true>(t, g);
            return;
        }
    }
    rs_phased<DT, OP, NR, false>(t, g);
}

// All-gather: grid x = tiles of output vectors, y = piece k.  Piece k covers
// bytes [b0, b0 + Rb) of the output frame (b0 = k*Rb - g.out_off); its whole
// frame vectors are [ceil(b0/16), floor((b0 + Rb)/16)), vector o holding the
// piece's input bytes 16*o - b0 (g.in_off more from the aligned table
// pointer).  Tiles follow the outputs' alignment (g.ref); the second load is
// clamped as above.  Tiles of 64*U vectors as in the reduce-scatter, U = 2
// for every n from 2 on: measured on MI355X with R - 1 elements per piece at
// 256 MB out per rank, 7.14-7.16 against 6.5-6.7 TB/s at n = 8 (bf16 and
// fp32), 5.8-6.3 against 5.0-5.3 at n = 9, 6.0 against 4.7-4.8 at n = 24 and
// 4.7-5.2 against 4.0-4.3 at n = 17; level at n = 4, 16 and 72, and at 64 MB.
int phased_gather_vectors_per_lane(int n) { return n >= 2 ? 2 : 1; }

template <int NR, int U>
__global__ __launch_bounds__(kFusedThreads) void fused_all_gather_phased_kernel(const RankTableFor<NR> t,
                                                                                const Geometry g) {
    const int n = NR > 0 ? NR : g.n;
    const int k = (int)blockIdx.y;
    const long long b0 = (long long)k * g.slice_bytes - g.out_off;      // piece k's first byte in the output frame
    const TileSpan ts =
        aligned_tile((b0 + 15) >> 4, (b0 + g.slice_bytes) >> 4, (long long)blockIdx.x, g.ref, kFusedTile * U);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + threadIdx.x + u * kFusedTile, ok[u]);
    const long long in = g.in_off + ts.lo * 16 - b0;                      // the tile's first input byte
    u32x4 w[U];
    if (g.phased_words == 2) {
        // pointers at mixed phases, every one and the piece length whole words (the caller checked): the
        // input bytes of every frame vector start at a 4-byte-aligned address, one load each
        const char *p = (const char *)t.src[k] + in;
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = *(const u32x4d *)(p + off[u]);
    } else {
        const long long rel = g.last_off - (in & ~15LL);
        const char *p = (const char *)t.src[k] + (in & ~15LL);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned hi_off = (long long)off[u] + 16 < rel ? off[u] + 16u : (unsigned)rel;
            const u32x4 lo = *(const u32x4 *)(p + off[u]);                // ordinary loads, as the aligned
            const u32x4 hi = *(const u32x4 *)(p + hi_off);                // all-gather reads its input
            w[u] = funnel16(lo, hi, (unsigned)(in & 15));
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const long long out = ts.lo * 16 + off[u];                        // in the output frame
        if constexpr (NR > 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) __builtin_nontemporal_store(w[u], (u32x4d *)((char *)t.dst[r] + out));
        } else {
            for (int r = 0; r < n; ++r) __builtin_nontemporal_store(w[u], (u32x4d *)((char *)t.dst[r] + out));
        }
    }
}

// The all-gather half of an all-reduce run as reduce-scatter then
// all-gather: chunk c (grid y), finished in rank c's output by the
// reduce-scatter half, copied to every other rank's output at the same
// offset.  Tiles of 64*U vectors follow rank 0's output (g.ref); the loads are
// ordinary (the chunk was just written and sits in the caches).
template <int U>
__global__ __launch_bounds__(kFusedThreads) void allreduce_chunk_gather_kernel(const RankTable t, const Geometry g) {
    const int n = g.n;
    const int c = (int)blockIdx.y;
    long long hi = ar_chunk_lo(c + 1, g) - g.shift;
    hi = hi < g.Vfull ? hi : g.Vfull;
    const TileSpan ts = aligned_tile(ar_chunk_lo(c, g), hi, (long long)blockIdx.x, g.ref, kFusedTile * U);
    if (ts.lo >= ts.hi) return;
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = tile_lane(ts, ts.start + threadIdx.x + u * kFusedTile, ok[u]);
    const long long base = ts.lo * 16;
    const char *p = (const char *)t.dst[c] + base;
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *(const u32x4d *)(p + off[u]);
    for (int r = 0; r < n; ++r) {
        if (r == c) continue;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) __builtin_nontemporal_store(w[u], (u32x4d *)((char *)t.dst[r] + base + off[u]));
    }
}

// Wavefronts per workgroup of the phased reduce-scatter, and the LDS each
// workgroup reserves.  The input line where two tiles meet is fetched once per
// L2 that needs it: with one-wave workgroups neighbouring tiles run on
// different XCDs and every tile boundary cost a second fetch (1.063x the
// algorithmic reads with 2 KB tiles); a workgroup of W wavefronts on W
// consecutive tiles keeps all but its outer boundary inside one L2 (measured
// FETCH_SIZE at n = 8, R - 1 elements: 1.031x with 2, 1.016x with 4).  With 4
// wavefronts per workgroup, fewer resident wavefronts win: 12 per compute unit
// (48 KB per workgroup) up to 4 ranks, 8 (56 KB) beyond.  Measured on MI355X,
// R - 1 elements per slice, 256 MB in per rank (% of peak, one wave -> four):
// bf16 n = 2 73.0 -> 74.9, 3 69.9 -> 75.0, 8 70.7 -> 74.3, 12 70.4 -> 72.9,
// 16 64.0 -> 73.3, 24 41.6 -> 71.3, 72 67.6 -> 76.1; fp32 n = 3 72.1 -> 75.6,
// 8 71.4 -> 72.1, 13-15 level, 17 40.0 -> 69.3, 32 49.1 -> 73.1; fp32 at 16
// ranks ran 64.9 with one wave and 60.3 with four, so 4-byte types keep one
// there.  With the word-aligned loads, 8 wavefronts (the one-wave reservation
// times 8, at most 64 KB) win up to 4 ranks: bf16 n = 2 77.9 -> 79.3, 3
// 73.8 -> 76.9, 4 73.7 -> 78.5; fp32 n = 2 76.9 -> 78.9, 3 74.0 -> 76.8, 4
// 72.2 -> 77.4; while 4 stay ahead at 8 ranks (bf16 76.7 against 74.5, fp32
// 75.5 against 73.7) and 24 (72.1 against 68.7), level at 16.
// AR_PHASED_WAVES=1|2|4|8 overrides the count (the LDS then scales the
// one-wave reservation).
static void phased_rs_shape(int n, int dt, int lds_one_wave, int &waves, int &lds) {
    const char *e = getenv("AR_PHASED_WAVES");
    if (e && (*e == '1' || *e == '2' || *e == '4' || *e == '8')) {
        waves = *e - '0';
        lds = lds_one_wave * waves > 65536 ? 65536 : lds_one_wave * waves;
        return;
    }
    const bool four_byte = dt == F32 || dt == I32;
    if (n == 16 && four_byte) {
        waves = 1;
        lds = lds_one_wave;
        return;
    }
    if (n <= 4) {
        waves = 8;
        lds = lds_one_wave * 8 > 65536 ? 65536 : lds_one_wave * 8;
        return;
    }
    waves = 4;
    lds = 56 * 1024;
}

// Which loads the compile-time-n reduce-scatter takes (the any-n chain always
// takes the word-aligned ones): 0 the aligned pair with the funnel shift, 1
// the word-aligned load on slices whose phase is not a whole number of words
// (only 2-byte types have them) and the pair elsewhere, 2 the word-aligned
// load on every slice.  A misaligned 16-byte load costs more than an aligned
// one, so the word-aligned form pays where it saves the shift.  Measured on
// MI355X, R - 1 elements per slice, % of peak (pair / 1 / 2): bf16 n = 2
// 75.5 / 76.7 / 75.1, n = 4 78.4 / 77.8 / 74.5, fp16 n = 6 68.0 / 71.4 / 75.8,
// bf16 n = 8 70.4 / 73.9 / 76.0 (another box 73.1 / - / 76.3), n = 12
// 69.4 / 71.1 / 72.9, n = 16 71.4 / 72.3 / 72.4; fp32 n = 8 75.7 / 75.8 / 75.5
// (another box 77.3 / - / 75.8), n = 3 77.2 / - / 76.8; past 16 ranks (any n,
// word-aligned against the pair) fp32 n = 17 66.7 -> 68.6, bf16 n = 24
// 70.9 -> 74.1.  AR_PHASED_FORM=funnel|hybrid|words overrides.
static int phased_rs_form(int n, int dt) {
    const char *f = getenv("AR_PHASED_FORM");
    if (f && !strcmp(f, "funnel")) return 0;
    if (f && !strcmp(f, "hybrid")) return 1;
    if (f && !strcmp(f, "words")) return 2;
    return (dt == BF16 || dt == F16) && n >= 5 ? 2 : 1;
}

hipError_t launch_fused_reduce_scatter_phased(int dt, int op, const RankTable &t, const Geometry &g, int lds,
                                              hipStream_t s) {
    if (g.Rv <= 0) return hipSuccess;
    int waves, lds_wg;
    phased_rs_shape(g.n, dt, lds, waves, lds_wg);
    if (getenv("AR_FUSED_LDS_KB") && waves > 1) lds_wg = lds * waves > 65536 ? 65536 : lds * waves;
    Geometry gw = g;
    gw.phased_words = g.phased_words == 2 ? 2 : phased_rs_form(g.n, dt);   // 2 from the caller: mixed phases
    return dispatch(dt, op, [&](auto D, auto O) {
        return by_ranks(g.n, [&](auto R) {
            constexpr int NR = decltype(R)::value;
            const long long tiles = aligned_tiles(g.Rv, (long long)kFusedTile * PhasedTile<NR>::U);
            const dim3 grid((unsigned)((tiles + waves - 1) / waves), (unsigned)g.n);
            return launch(fused_reduce_scatter_phased_kernel<decltype(D)::value, decltype(O)::value, NR>,
                          grid, dim3(kFusedThreads * waves), (size_t)lds_wg, s, narrow<NR>(t), gw);
        });
    });
}

// All-reduce past 16 ranks in ring order as reduce-scatter then all-gather:
// the phased reduce-scatter's layout over the all-reduce's own chunks (each
// finished chunk stored to its owner only), then each chunk copied from its
// owner to the other ranks.  Whole vectors [0, g.Vfull) only; in the shifted
// frame (g.shift = 1) each chunk's vectors stop before the one across its end,
// as in the one-pass kernel, and the element-wise kernel takes the rest.
hipError_t launch_allreduce_halves(int dt, int op, const RankTable &t, const Geometry &g, int lds_rs, int lds_ag,
                                   hipStream_t s) {
    if (g.Vfull <= 0) return hipSuccess;
    Geometry gr = g;
    gr.ar_chunks = 1;
    gr.phased_words = 2;
    gr.Rv = (g.V + g.n - 1) / g.n;                           // the longest chunk, in vectors: sizes the grid
    hipError_t h = launch_fused_reduce_scatter_phased(dt, op, t, gr, lds_rs, s);
    if (h != hipSuccess) return h;
    constexpr int U = 2;
    const dim3 grid((unsigned)aligned_tiles(gr.Rv, (long long)kFusedTile * U), (unsigned)g.n);
    return launch(allreduce_chunk_gather_kernel<U>, grid, dim3(kFusedThreads), (size_t)lds_ag, s, t, g);
}

hipError_t launch_fused_all_gather_phased(const RankTable &t, const Geometry &g, int lds, hipStream_t s) {
    const long long most = g.slice_bytes >> 4;                    // whole output vectors of any piece, at most
    if (most <= 0) return hipSuccess;
    const int U = phased_gather_vectors_per_lane(g.n);
    const dim3 grid((unsigned)aligned_tiles(most, (long long)kFusedTile * U), (unsigned)g.n);
    return by_ranks(g.n, [&](auto R) {
        constexpr int NR = decltype(R)::value;
        if (U == 2)
            return launch(fused_all_gather_phased_kernel<NR, 2>, grid, dim3(kFusedThreads), (size_t)lds, s, narrow<NR>(t), g);
        return launch(fused_all_gather_phased_kernel<NR, 1>, grid, dim3(kFusedThreads), (size_t)lds, s, narrow<NR>(t), g);
    });
}

}  // namespace ar
