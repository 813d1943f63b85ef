// fused_common.hpp -- pieces shared by the fused kernels' translation units
// (fused.hip, fused_rs.hip, fused_phase.hip): the ring hop order, the chain
// that combines the n ranks' vectors in that order, and the compile-time rank
// count dispatch.
#pragma once

#include <type_traits>

#include "ar_device.hpp"
#include "ar_kernels.hpp"

namespace ar {

// Rank holding hop k (k = 0..n-1) of chunk c: c+1+k mod n.
__device__ __forceinline__ int hop_rank(int c, int k, int n) {
    int r = c + 1 + k;
    r = r >= n ? r - n : r;
    return r >= n ? r - n : r;
}

// Combine the n ranks' vectors at bytes ``base + lane_off[u]`` (u < U) in the
// hop order of chunk c (ranks c+1, ..., c) into acc[u].  ``base`` is the
// tile's byte offset (the same for the whole wavefront: it is folded into the
// scalar rank pointer) and ``lane_off`` 32-bit per-lane offsets, so every
// access is a scalar base plus a 32-bit vector offset.  Every lane passes
// valid offsets (lanes past the end of the range re-read its last vector and
// discard the result), so no load sits in a divergent branch and a whole batch
// of loads is in flight at once.  NR > 0: n == NR known at compile time
// (n <= 16), all n*U loads issued before the first combine; NR == 0: any n,
// batches of 16 loads.  KEEP32: bf16 / fp16 partials stay fp32 (rounded in
// ``finish``).  Each acc[u] sees the ranks in the same order whatever U is.
template <int DT, int OP, int NR, bool KEEP32, int U, class TAB>
__device__ __forceinline__ void chain_in(const TAB &t, int n, int c, long long base,
                                         const unsigned (&lane_off)[U], float s, Pack<DT> (&acc)[U]) {
    if constexpr (NR > 0) {
        // the n rank pointers (scalar loads from the kernel arguments at a chunk-dependent index) all issued
        // before the first vector load: placed with the vector loads, each waited for its own pointer in turn
        const void *ptr[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) ptr[k] = t.src[hop_rank(c, k, NR)];
        __builtin_amdgcn_sched_barrier(0);
        u32x4 raw[NR][U];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const char *p = (const char *)ptr[k] + base;
#pragma unroll
            for (int u = 0; u < U; ++u) raw[k][u] = __builtin_nontemporal_load((const u32x4d *)(p + lane_off[u]));
        }
        __builtin_amdgcn_sched_barrier(0);                   // every load issued before the first combine
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[u] = first<DT, OP, KEEP32>(unpack<DT>(raw[0][u]), s);
#pragma unroll
            for (int k = 1; k < NR; ++k) hop<DT, OP, KEEP32>(acc[u], unpack<DT>(raw[k][u]), s);
        }
    } else {
        constexpr int B = 16 / U > 0 ? 16 / U : 1;
        for (int k0 = 0; k0 < n; k0 += B) {
            const void *ptr[B];
#pragma unroll
            for (int kk = 0; kk < B; ++kk) ptr[kk] = t.src[hop_rank(c, k0 + kk < n ? k0 + kk : n - 1, n)];
            __builtin_amdgcn_sched_barrier(0);
            u32x4 raw[B][U];
#pragma unroll
            for (int kk = 0; kk < B; ++kk) {
                const char *p = (const char *)ptr[kk] + base;                // past n: a valid, ignored load
#pragma unroll
                for (int u = 0; u < U; ++u) raw[kk][u] = __builtin_nontemporal_load((const u32x4d *)(p + lane_off[u]));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < B; ++kk) {
                if (k0 + kk >= n) break;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (k0 + kk == 0) acc[u] = first<DT, OP, KEEP32>(unpack<DT>(raw[kk][u]), s);
                    else hop<DT, OP, KEEP32>(acc[u], unpack<DT>(raw[kk][u]), s);
                }
            }
        }
    }
}

// The chain with the partials' precision chosen once per tile (a uniform
// branch; only bf16 / fp16 have two).
template <int DT, int OP, int NR, int U, class TAB>
__device__ __forceinline__ void chain(const TAB &t, int n, int c, long long base, const unsigned (&lane_off)[U],
                                      float s, bool keep32, Pack<DT> (&acc)[U]) {
    if constexpr (DT == BF16 || DT == F16) {
        if (keep32) {
            chain_in<DT, OP, NR, true, U, TAB>(t, n, c, base, lane_off, s, acc);
            return;
        }
    }
    chain_in<DT, OP, NR, false, U, TAB>(t, n, c, base, lane_off, s, acc);
}

// Pick the compile-time rank count: every n up to 16 has its own kernels, so a
// lane issues exactly n loads.  (A generic kernel loading ranks in batches of
// 16 wasted the loads past n: measured on MI355X at 128 MB per rank it ran at
// 3.6 TB/s for n = 3 and 4.9-5.6 TB/s for n = 5-7, against 6.4-6.5 TB/s for
// n = 4 and 8 with their own kernels.)
template <int NR, typename F> hipError_t by_ranks_from(int n, F &&f) {
    if constexpr (NR > 16) {
        return f(std::integral_constant<int, 0>{});
    } else {
        if (n == NR) return f(std::integral_constant<int, NR>{});
        return by_ranks_from<NR + 1>(n, f);
    }
}
template <typename F> hipError_t by_ranks(int n, F &&f) { return by_ranks_from<2>(n, f); }

}  // namespace ar
