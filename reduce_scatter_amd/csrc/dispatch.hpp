// dispatch.hpp -- turn runtime (dtype, op) codes into template arguments.
#pragma once

#include <type_traits>

#include "ar_device.hpp"

namespace ar {

// Launch ``k`` and return the launch's own status (not the thread's last-error
// state, which earlier unrelated runtime calls may have left set).  The
// runtime reads each argument through its address with the size of the
// kernel's parameter, so every argument must have exactly the parameter's type.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, const A &...args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    static_assert((std::is_same<typename std::decay<P>::type, A>::value && ...), "kernel argument types");
    void *ptrs[] = {(void *)&args...};
    return hipLaunchKernel((const void *)k, grid, block, ptrs, lds, s);
}

template <int DT, typename F> hipError_t dispatch_op(int op, F &&f) {
    switch (op) {
    case SUM: return f(std::integral_constant<int, DT>{}, std::integral_constant<int, SUM>{});
    case PROD: return f(std::integral_constant<int, DT>{}, std::integral_constant<int, PROD>{});
    case MIN: return f(std::integral_constant<int, DT>{}, std::integral_constant<int, MIN>{});
    case MAX: return f(std::integral_constant<int, DT>{}, std::integral_constant<int, MAX>{});
    case AVG: return f(std::integral_constant<int, DT>{}, std::integral_constant<int, AVG>{});
    default: return hipErrorInvalidValue;
    }
}

template <typename F> hipError_t dispatch(int dt, int op, F &&f) {
    switch (dt) {
    case F32: return dispatch_op<F32>(op, f);
    case BF16: return dispatch_op<BF16>(op, f);
    case F16: return dispatch_op<F16>(op, f);
    case I32: return dispatch_op<I32>(op, f);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
