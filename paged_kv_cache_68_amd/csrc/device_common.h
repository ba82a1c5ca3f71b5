// Device-side helpers for the gfx950 kernels: 16-bit storage types, dot2, DPP row
// reductions and the XCD-aware work-group order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp16 storage: v_dot2_f32_f16 for q.k, exact widening, RNE narrowing.
struct F16 {
    static constexpr int kId = KV_DTYPE_F16;
    __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
    }
    __device__ static __forceinline__ float lo(uint32_t u) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
    }
    __device__ static __forceinline__ float hi(uint32_t u) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
    }
    __device__ static __forceinline__ uint16_t narrow(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
};

// bf16 storage: v_dot2_f32_bf16 for q.k; widening is a 16-bit shift.
struct BF16 {
    static constexpr int kId = KV_DTYPE_BF16;
    __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    }
    __device__ static __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
    __device__ static __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
    __device__ static __forceinline__ uint16_t narrow(float x) {
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest, ties to even
        return static_cast<uint16_t>(u >> 16);
    }
};

// DPP lane move inside a row of 16 lanes (every control used here reads an in-row lane).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                              0xf, 0xf, false));
}

constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i inside the row

// Sum over groups of N = 8 or 16 neighbouring lanes; every lane of the group ends with
// the same bits (each step adds a commutative pair).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp_mov<kDppMirror>(x);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-groups are handed to the 8 XCDs round-robin.  Renumber them so that each XCD
// gets one contiguous range of logical work items (and so shares its L2 between
// neighbouring items).  Bijective on [0, n).
__device__ __forceinline__ int xcd_order(int id, int n) {
    constexpr int kXcds = 8;
    const int q = n / kXcds, r = n % kXcds;
    const int x = id % kXcds, loc = id / kXcds;
    return (x < r) ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
}

}  // namespace pkv
