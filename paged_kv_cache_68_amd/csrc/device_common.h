// Device-side helpers for the gfx950 kernels: 16-bit storage types, dot2, DPP row
// reductions and the XCD-aware work-group order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
    // two fp32 -> packed 16-bit (RNE), `lo` in the low half
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        const f16x2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    }
    // D += A(16x32) * B(32x16); each lane passes 8 k-elements of A and of B
    __device__ static __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    // D += A(16x16) * B(16x16); each lane passes 4 k-elements of A and of B
    __device__ static __forceinline__ f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
    // two E4M3 codes (bytes 0-1, or 2-3 with HI) -> packed fp16, exact: every E4M3 value
    // is an fp16 value (v_cvt_scalef32_pk_f16_fp8 with scale 1)
    template <bool HI>
    __device__ static __forceinline__ uint32_t from_fp8x2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
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
    // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
    __device__ static __forceinline__ uint16_t narrow(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                         __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
    }
    // two E4M3 codes -> packed bf16, exact (v_cvt_scalef32_pk_bf16_fp8 with scale 1)
    template <bool HI>
    __device__ static __forceinline__ uint32_t from_fp8x2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }
};

// Two fp32 values as a sum of two packed 16-bit parts of S: x = (RNE(a), RNE(b)) and
// y = the rounded remainders (a - x.a, b - x.b), so that x + y carries about twice the
// significand bits of one 16-bit value (relative error near 2^-18 for bf16, 2^-22 for
// fp16, apart from fp16 underflow below 2^-24).  Used for the softmax weights of the
// value product: x and y each go through the matrix cores, accumulating into one sum.
template <class S>
__device__ __forceinline__ uint2 split_pack2(float a, float b) {
    const uint32_t hi = S::pack2(a, b);
    return make_uint2(hi, S::pack2(a - S::lo(hi), b - S::hi(hi)));
}

// Four E4M3 codes (one dword, code i in byte i) -> four 16-bit values of S, in order.
template <class S>
__device__ __forceinline__ uint2 fp8x4_to(uint32_t w) {
    return make_uint2(S::template from_fp8x2<false>(w), S::template from_fp8x2<true>(w));
}

// Two fp32 values -> two E4M3 codes in the low 16 bits (value a in byte 0): round to
// nearest even (v_cvt_pk_fp8_f32), magnitudes past 448 and infinities saturated to
// +-448, NaN written as S.1111.111 with its sign.
__device__ __forceinline__ uint32_t fp8x2_from(float a, float b) {
    auto sat = [](float x) { return __builtin_isnan(x) ? x : fminf(fmaxf(x, -448.f), 448.f); };
    uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false)) & 0xffffu;
    if (__builtin_isnan(a)) w = (w & 0xff00u) | 0x7fu | ((__float_as_uint(a) >> 24) & 0x80u);
    if (__builtin_isnan(b)) w = (w & 0x00ffu) | ((0x7fu | ((__float_as_uint(b) >> 24) & 0x80u)) << 8);
    return w;
}

// 16-bit halves of two dwords: (x.lo, y.lo) and (x.hi, y.hi), x's half in the low half.
__device__ __forceinline__ uint32_t lo_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// DPP lane move inside a row of 16 lanes (every control used here reads an in-row lane).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xf, 0xf, true));
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

// Lane exchanges across the four 16-lane rows of a wave.
__device__ __forceinline__ float xor16(float x) {      // ds_swizzle, bit mode: lane ^ 16
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float xor32(float x, int addr_xor32) {   // addr = (lane ^ 32) * 4
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr_xor32, __builtin_bit_cast(int, x)));
}

// Buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes return zero and
// touch no memory, which both masks the tail of a partly filled block and lets a wave
// issue a fixed number of loads per iteration.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}
// NT = true sets the non-temporal hint (cache-policy bit 1 on gfx950): the lines are
// fetched for one use and are not kept in the caches, which lets a stream that is read
// once run measurably faster; data that will be re-read soon should not use it.
template <bool NT = false>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}
template <bool NT = false>
__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0));
}
template <bool NT = false>
__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? 2 : 0);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Work-groups are handed to the 8 XCDs round-robin, in launch order.  Renumber them so
// that each XCD walks through chunks of `chunk` consecutive work-groups: work-groups
// that read the same blocks (neighbouring sequences of a shared prefix, the KV heads of
// one block) meet in the same L2, while the chunks still rotate over the XCDs, so long
// and short items stay evenly spread.  Bijective on [0, n); the tail that does not fill
// a whole round of chunks keeps its own number.  chunk <= 0 keeps launch order.
__device__ __forceinline__ int xcd_chunked(int id, int n, int chunk) {
    constexpr int kXcds = 8;
    if (chunk <= 0) return id;
    const int round = kXcds * chunk;
    if (id >= (n / round) * round) return id;
    const int x = id % kXcds;
    const int slot = id / kXcds;
    return (slot / chunk) * round + x * chunk + slot % chunk;
}

}  // namespace pkv
