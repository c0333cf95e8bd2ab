// The size-2 causal input convolution of one 8-channel group ("2Mamba2Furious",
// §3: kernel size 2 along the sequence, no activation; §4: kept in Mamba-2S;
// App. A: decoding keeps the one previous raw row), shared by the standalone
// pass (conv.hip) and the kernels that apply it while loading their operands,
// so that every site computes bit-identical values:
//     y[c] = fmaf(w1[c], x_t[c], fmaf(w0[c], x_{t-1}[c], b[c]))   in fp32,
// rounded to the input dtype (nearest even for bf16).
#pragma once

#include "device_common.h"

namespace twm {

// Taps and bias of 8 consecutive channels: weight [..][d][2] (tap 0 on x_{t-1},
// tap 1 on x_t) and bias [..][d] (NULL = 0), both at channel offset `ch` of the
// (tensor, head) row; 16-byte aligned.
struct Conv8 {
    float w0[8], w1[8], b[8];
};

__device__ __forceinline__ void conv8_load(Conv8& c, const float* w, const float* b, size_t ch) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 wv = *reinterpret_cast<const float4*>(w + 2 * ch + 4 * i);   // taps of channels 2i, 2i+1
        c.w0[2 * i] = wv.x;
        c.w1[2 * i] = wv.y;
        c.w0[2 * i + 1] = wv.z;
        c.w1[2 * i + 1] = wv.w;
    }
    if (b) {
        const float4 b0 = *reinterpret_cast<const float4*>(b + ch), b1 = *reinterpret_cast<const float4*>(b + ch + 4);
        c.b[0] = b0.x; c.b[1] = b0.y; c.b[2] = b0.z; c.b[3] = b0.w;
        c.b[4] = b1.x; c.b[5] = b1.y; c.b[6] = b1.z; c.b[7] = b1.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c.b[i] = 0.f;
    }
}

// fp32 results of 8 channels from fp32 inputs
__device__ __forceinline__ void conv8_f32(const Conv8& c, const float* x, const float* xp, float* y) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fmaf(c.w1[i], x[i], fmaf(c.w0[i], xp[i], c.b[i]));
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float* o) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16x2_rne(x[2 * i], x[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 8 bf16 channels of row t from the raw rows t and t-1
__device__ __forceinline__ uint4 conv8_bf16(const Conv8& c, const uint4 x, const uint4 xp) {
    float a[8], ap[8], y[8];
    bf16x8_to_f32(x, a);
    bf16x8_to_f32(xp, ap);
    conv8_f32(c, a, ap, y);
    return f32x8_to_bf16(y);
}

}  // namespace twm
