// fused_common.hpp -- pieces shared by the fused kernels' translation units
// (fused.hip, fused_phase.hip): the ring hop order and the compile-time rank
// count dispatch.
#pragma once

#include <type_traits>

#include "ar_device.hpp"

namespace ar {

// Rank holding hop k (k = 0..n-1) of chunk c: c+1+k mod n.
__device__ __forceinline__ int hop_rank(int c, int k, int n) {
    int r = c + 1 + k;
    r = r >= n ? r - n : r;
    return r >= n ? r - n : r;
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
