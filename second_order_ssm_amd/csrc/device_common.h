// Device-side helpers shared by the HIP kernels of the 2Mamba library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twm {

// bf16 stored as its raw 16 bits.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// two fp32 -> two bf16 in one v_cvt_pk_bf16_f32: round to nearest even, the same
// bits as f32_to_bf16 for every non-NaN input
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __bf16 b2v __attribute__((ext_vector_type(2)));
    const f2v f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2v));
}

template <typename T> struct IO;
template <> struct IO<float> {
    static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, size_t i, float x) { p[i] = x; }
    static __device__ __forceinline__ float rnd(float x) { return x; }   // x in this dtype's precision
};
template <> struct IO<bf16> {
    static __device__ __forceinline__ float ld(const bf16* p, size_t i) { return bf16_to_f32(p[i].bits); }
    static __device__ __forceinline__ void st(bf16* p, size_t i, float x) { p[i].bits = f32_to_bf16(x); }
    static __device__ __forceinline__ float rnd(float x) { return bf16_to_f32(f32_to_bf16(x)); }
};

// log decay g = -softplus(z) with softplus(x) = max(x,0) + log1p(exp(-|x|));
// z = -inf gives exactly 0 (no decay).  Softplus A-mask: "2Mamba2Furious", §3-§4.
__device__ __forceinline__ float decay_log(float z) { return -(fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)))); }

// Packed position p -> pair (i, j), i <= j, of the row-major upper triangle of
// a d x d symmetric tensor.  Linear search over rows; used off the hot loops.
__device__ __forceinline__ void pair_of(int p, int d, int& i, int& j) {
    int r = 0;
    int len = d;
    while (p >= len) {
        p -= len;
        ++r;
        --len;
    }
    i = r;
    j = r + p;
}

}  // namespace twm
