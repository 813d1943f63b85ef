// ar_device.hpp -- device-side building blocks shared by the fused, ring and
// tree kernels: 16-byte vector packs, storage-type rounding, the reduction
// operator and the avg pre-scale / postOp.
//
// Semantics (the "NCCL all-reduce" post, rakshithvasudev.github.io, section
// "What all-reduce promises"; "FSDP collectives 101", the note that bf16
// reductions accumulate in bf16 along the way):
//   * sum / prod / min / max / avg; avg multiplies each floating-point
//     contribution by s = fp32(1/n) as it is read, and divides an int32 sum
//     by n once where the chunk completes (truncating toward zero);
//   * bf16 / fp16 are widened to fp32 for one hop's arithmetic and rounded
//     back (to nearest even) when the value leaves the hop;
//   * int32 sum / prod wrap modulo 2^32;
//   * min(acc, own) keeps acc unless own < acc (max likewise), acc being the
//     incoming partial.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace ar {

enum Dtype : int { F32 = 0, BF16 = 1, F16 = 2, I32 = 3 };
enum Op : int { SUM = 0, PROD = 1, MIN = 2, MAX = 3, AVG = 4 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// The same 16 bytes at an address known only to be 4-byte aligned: a 16-byte
// global load or store on gfx9 needs dword alignment only, so the vector
// kernels that access memory through this type also serve element-aligned
// 4-byte buffers (the instruction is the same global_load/store_dwordx4).
typedef unsigned int u32x4d __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kMaxRanks = 128;

// Elements of each dtype in one 16-byte vector.
template <int DT> struct Lanes { static constexpr int value = (DT == BF16 || DT == F16) ? 8 : 4; };

// One 16-byte vector unpacked to its arithmetic type: fp32 for the float
// dtypes (each value exactly representable in the storage type), 32-bit
// two's complement for int32.
template <int DT> struct Pack {
    static constexpr int K = Lanes<DT>::value;
    typedef typename std::conditional<DT == I32, uint32_t, float>::type T;
    T v[K];
};

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Rounding to the storage type uses gfx950's conversions (v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32: round to nearest even in the default float mode, denormals
// kept, overflow to infinity, NaN stays NaN).  The value to convert first
// passes through an empty asm statement, so the conversion stays a separate
// rounding of an fp32 value: without it the compiler folds an fp32 multiply
// (or add) followed by a float-to-half conversion into one mixed-precision
// FMA that rounds the exact result once, which differs from rounding the fp32
// result when the operands are not already fp16 values (fp32 partials).
__device__ __forceinline__ float fence_value(float f) {
    asm("" : "+v"(f));
    return f;
}

// fp32 -> nearest bf16 (ties to even), returned as the fp32 value.
__device__ __forceinline__ float round_bf16(float f) { return (float)(__bf16)fence_value(f); }

// fp32 -> nearest fp16 (ties to even), returned as the fp32 value.
__device__ __forceinline__ float round_f16(float f) { return (float)(_Float16)fence_value(f); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two values rounded by one packed conversion.
template <int DT> __device__ __forceinline__ void round_pair(float &a, float &b) {
    const f32x2 v = {fence_value(a), fence_value(b)};
    if constexpr (DT == BF16) {
        const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        a = bits_f32(u << 16);
        b = bits_f32(u & 0xffff0000u);
    } else {
        const f16x2 h = __builtin_convertvector(v, f16x2);
        a = (float)h.x;
        b = (float)h.y;
    }
}

template <int DT> __device__ __forceinline__ float round_to(float f) {
    if (DT == BF16) return round_bf16(f);
    if (DT == F16) return round_f16(f);
    return f;
}

// Every element of a pack rounded to the storage type (no-op for fp32 / int32).
template <int DT> __device__ __forceinline__ void round_all(Pack<DT> &p) {
    if constexpr (DT == BF16 || DT == F16) {
#pragma unroll
        for (int i = 0; i < Pack<DT>::K; i += 2) round_pair<DT>(p.v[i], p.v[i + 1]);
    }
}

template <int DT> __device__ __forceinline__ Pack<DT> unpack(u32x4 w) {
    Pack<DT> p;
    if constexpr (DT == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p.v[i] = bits_f32(w[i]);
    } else if constexpr (DT == I32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p.v[i] = w[i];
    } else if constexpr (DT == BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p.v[2 * i] = bits_f32(w[i] << 16);
            p.v[2 * i + 1] = bits_f32(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p.v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            p.v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    }
    return p;
}

// Pack values that are already representable in the storage type.
template <int DT> __device__ __forceinline__ u32x4 pack(const Pack<DT> &p) {
    u32x4 w;
    if constexpr (DT == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = f32_bits(p.v[i]);
    } else if constexpr (DT == I32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = p.v[i];
    } else if constexpr (DT == BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (f32_bits(p.v[2 * i]) >> 16) | (f32_bits(p.v[2 * i + 1]) & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)p.v[2 * i]);
            uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)p.v[2 * i + 1]);
            w[i] = lo | (hi << 16);
        }
    }
    return w;
}

// One element: the contribution as read (float avg pre-scales by s).
template <int DT, int OP> __device__ __forceinline__ typename Pack<DT>::T pre(typename Pack<DT>::T x, float s) {
    if constexpr (DT != I32 && OP == AVG) return x * s;
    else return x;
}

// One element: acc (+) own, in fp32 or in 32-bit two's complement.
template <int DT, int OP>
__device__ __forceinline__ typename Pack<DT>::T combine(typename Pack<DT>::T acc, typename Pack<DT>::T own) {
    if constexpr (DT == I32) {
        if constexpr (OP == SUM || OP == AVG) return acc + own;
        else if constexpr (OP == PROD) return acc * own;
        else if constexpr (OP == MIN) return ((int32_t)own < (int32_t)acc) ? own : acc;
        else return ((int32_t)own > (int32_t)acc) ? own : acc;
    } else {
        if constexpr (OP == SUM || OP == AVG) return acc + own;
        else if constexpr (OP == PROD) return acc * own;
        else if constexpr (OP == MIN) return (own < acc) ? own : acc;
        else return (own > acc) ? own : acc;
    }
}

// Vector forms. ``first`` starts a chain: pre(x), rounded to the storage type
// unless the partials are kept in fp32 (KEEP32: bf16 / fp16 accumulation in
// fp32, rounded once where the reduction completes).
template <int DT, int OP, bool KEEP32 = false> __device__ __forceinline__ Pack<DT> first(const Pack<DT> &x, float s) {
    Pack<DT> r;
#pragma unroll
    for (int i = 0; i < Pack<DT>::K; ++i) r.v[i] = pre<DT, OP>(x.v[i], s);
    if constexpr (!KEEP32) round_all<DT>(r);
    return r;
}

// One hop: acc = round(acc (+) pre(own)) (no rounding with KEEP32).
template <int DT, int OP, bool KEEP32 = false>
__device__ __forceinline__ void hop(Pack<DT> &acc, const Pack<DT> &own, float s) {
#pragma unroll
    for (int i = 0; i < Pack<DT>::K; ++i) acc.v[i] = combine<DT, OP>(acc.v[i], pre<DT, OP>(own.v[i], s));
    if constexpr (!KEEP32) round_all<DT>(acc);
}

// Combine two partials that were both already rounded (tree: parent (+) child).
template <int DT, int OP> __device__ __forceinline__ void merge(Pack<DT> &acc, const Pack<DT> &other) {
#pragma unroll
    for (int i = 0; i < Pack<DT>::K; ++i) acc.v[i] = combine<DT, OP>(acc.v[i], other.v[i]);
    round_all<DT>(acc);
}

// Where a reduction completes (the postOp): int32 avg divides the wrapped sum
// by n once; the split float avg divides the finished sum by g.post_div
// (n / p) in fp32; a result kept in fp32 (g.acc32) or divided is rounded to
// the storage type.  ``G`` is the launch geometry (post_div, acc32).
template <int DT, int OP, typename G> __device__ __forceinline__ void finish(Pack<DT> &acc, int n, const G &g) {
    if constexpr (DT == I32) {
        if constexpr (OP == AVG) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc.v[i] = (uint32_t)((int32_t)acc.v[i] / n);
        }
    } else {
        const bool divide = OP == AVG && g.post_div != 0.0f;
        if (divide) {
#pragma unroll
            for (int i = 0; i < Pack<DT>::K; ++i) acc.v[i] = acc.v[i] / g.post_div;
        }
        if (g.acc32 || divide) round_all<DT>(acc);
    }
}

// ---- scalar (one element) forms, for the element-wise path ----------------
template <int DT> __device__ __forceinline__ typename Pack<DT>::T load1(const void *p, long long i) {
    if constexpr (DT == F32) return ((const float *)p)[i];
    else if constexpr (DT == I32) return ((const uint32_t *)p)[i];
    else if constexpr (DT == BF16) return bits_f32((uint32_t)((const uint16_t *)p)[i] << 16);
    else return (float)((const _Float16 *)p)[i];
}

template <int DT> __device__ __forceinline__ void store1(void *p, long long i, typename Pack<DT>::T v) {
    if constexpr (DT == F32) ((float *)p)[i] = v;
    else if constexpr (DT == I32) ((uint32_t *)p)[i] = v;
    else if constexpr (DT == BF16) ((uint16_t *)p)[i] = (uint16_t)(f32_bits(v) >> 16);
    else ((_Float16 *)p)[i] = (_Float16)v;
}

template <int DT, int OP>
__device__ __forceinline__ typename Pack<DT>::T first1(typename Pack<DT>::T x, float s, bool keep32 = false) {
    if constexpr (DT == I32) return x;
    else return keep32 ? pre<DT, OP>(x, s) : round_to<DT>(pre<DT, OP>(x, s));
}

template <int DT, int OP>
__device__ __forceinline__ typename Pack<DT>::T hop1(typename Pack<DT>::T acc, typename Pack<DT>::T own, float s,
                                                     bool keep32 = false) {
    if constexpr (DT == I32) return combine<DT, OP>(acc, own);
    else {
        const float v = combine<DT, OP>(acc, pre<DT, OP>(own, s));
        return keep32 ? v : round_to<DT>(v);
    }
}

template <int DT, int OP>
__device__ __forceinline__ typename Pack<DT>::T merge1(typename Pack<DT>::T acc, typename Pack<DT>::T other) {
    if constexpr (DT == I32) return combine<DT, OP>(acc, other);
    else return round_to<DT>(combine<DT, OP>(acc, other));
}

template <int DT, int OP, typename G>
__device__ __forceinline__ typename Pack<DT>::T finish1(typename Pack<DT>::T acc, int n, const G &g) {
    if constexpr (DT == I32) {
        if constexpr (OP == AVG) return (uint32_t)((int32_t)acc / n);
        else return acc;
    } else {
        const bool divide = OP == AVG && g.post_div != 0.0f;
        const float v = divide ? acc / g.post_div : acc;
        return (g.acc32 || divide) ? round_to<DT>(v) : v;
    }
}

// Streaming 16-byte loads and stores: every byte is touched once, so they are
// marked non-temporal.
__device__ __forceinline__ u32x4 ld_stream(const void *base, long long vec) {
    return __builtin_nontemporal_load((const u32x4 *)base + vec);
}
__device__ __forceinline__ void st_stream(void *base, long long vec, u32x4 w) {
    __builtin_nontemporal_store(w, (u32x4 *)base + vec);
}

// Bytes [phase, phase + 16) of the 32 bytes a:b (a's bytes first), phase in
// [0, 16): a 16-byte vector read at an address that is not 16-byte aligned,
// assembled from the two aligned vectors around it.  Little-endian: byte 0 of
// a sits in the low bits of a.x.
__device__ __forceinline__ u32x4 funnel16(u32x4 a, u32x4 b, unsigned phase) {
    const uint64_t q0 = (uint64_t)a.x | ((uint64_t)a.y << 32), q1 = (uint64_t)a.z | ((uint64_t)a.w << 32);
    const uint64_t q2 = (uint64_t)b.x | ((uint64_t)b.y << 32), q3 = (uint64_t)b.z | ((uint64_t)b.w << 32);
    const bool hi = phase >= 8;
    const unsigned sh = (phase & 7u) * 8u;
    const uint64_t x0 = hi ? q1 : q0, x1 = hi ? q2 : q1, x2 = hi ? q3 : q2;
    const uint64_t r0 = sh ? (x0 >> sh) | (x1 << (64u - sh)) : x0;
    const uint64_t r1 = sh ? (x1 >> sh) | (x2 << (64u - sh)) : x1;
    u32x4 r;
    r.x = (uint32_t)r0;
    r.y = (uint32_t)(r0 >> 32);
    r.z = (uint32_t)r1;
    r.w = (uint32_t)(r1 >> 32);
    return r;
}

// (a + b) mod n for a, b in [0, n).
__device__ __forceinline__ int add_mod(int a, int b, int n) {
    int r = a + b;
    return r >= n ? r - n : r;
}

}  // namespace ar
