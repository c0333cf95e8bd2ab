// Size-2 causal input convolution in front of the operator ("2Mamba2Furious",
// §3: a convolution of kernel size 2 along the sequence, without activation;
// §4: part of Mamba-2S; App. A: decoding caches the one previous query, key and
// value it needs).  Each channel of q, k and v is convolved separately:
//     y_t = w1 * x_t + w0 * x_{t-1} + b,   x_{-1} = the cached raw row (or 0).
//
// HBM-bound: one thread per (head, token, tensor, 8 channels) loads 2 x 16
// bytes (bf16) of input (the earlier row mostly from L2) and stores 16 bytes;
// the weights of its 8 channels come through the caches.  Index arithmetic is
// 32-bit within a head.
#include "conv_common.h"
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

template <typename In> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void ld(const bf16* p, float* o) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void st(bf16* p, const float* x) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = bf16x2_rne(x[2 * i], x[2 * i + 1]);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    static __device__ __forceinline__ void copy(bf16* d, const bf16* s) {
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void ld(const float* p, float* o) {
        const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    static __device__ __forceinline__ void st(float* p, const float* x) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void copy(float* d, const float* s) {
        *reinterpret_cast<float4*>(d) = *reinterpret_cast<const float4*>(s);
        *reinterpret_cast<float4*>(d + 4) = *reinterpret_cast<const float4*>(s + 4);
    }
};

// grid: x = (head, tile of 256 threads), y = tensor (first + blockIdx.y).  Thread
// (token group of kTok, 8 channels): its weights and bias are loaded once, each
// input row once (the row before the group as well), kTok rows are written.
constexpr int kTok = 4;
template <int D, typename In>
__global__ void __launch_bounds__(256)
conv2_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
             const float* __restrict__ w, const float* __restrict__ b, const In* __restrict__ prev,
             In* __restrict__ qo, In* __restrict__ ko, In* __restrict__ vo, In* __restrict__ prev_out, int H, int T,
             int tiles, int first) {
    constexpr int CG = D / 8;
    const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles, which = first + (int)blockIdx.y;
    const int idx = tile * 256 + threadIdx.x;
    const int ngroups = (T + kTok - 1) / kTok;
    if (idx >= ngroups * CG) return;
    const int tg = idx / CG, cg = idx % CG;
    const int t0 = tg * kTok;
    const int h = bh % H;
    const In* x = which == 0 ? q : which == 1 ? k : v;
    In* y = which == 0 ? qo : which == 1 ? ko : vo;
    const size_t wo = (size_t)(which * H + h) * D + 8 * cg;
    Conv8 cw;
    conv8_load(cw, w, b, wo);
    const size_t row0 = ((size_t)bh * T + t0) * D + 8 * cg;
    float bef[8];
    if (t0 > 0) {
        Vec8<In>::ld(x + row0 - D, bef);
    } else if (prev) {
        Vec8<In>::ld(prev + ((size_t)bh * 3 + which) * D + 8 * cg, bef);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bef[i] = 0.f;
    }
    const int nt = min(kTok, T - t0);
    float cur[kTok][8];
#pragma unroll
    for (int j = 0; j < kTok; ++j)
        if (j < nt) Vec8<In>::ld(x + row0 + (size_t)j * D, cur[j]);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        if (j >= nt) break;
        float o[8];
        conv8_f32(cw, cur[j], j == 0 ? bef : cur[j - 1], o);
        Vec8<In>::st(y + row0 + (size_t)j * D, o);
    }
    if (prev_out && t0 + nt == T)
        Vec8<In>::copy(prev_out + ((size_t)bh * 3 + which) * D + 8 * cg, x + row0 + (size_t)(nt - 1) * D);
}

// T = 0: the cached row passes through (zeros without one)
template <int D, typename In>
__global__ void __launch_bounds__(256)
conv2_pass_kernel(const In* __restrict__ prev, In* __restrict__ prev_out, size_t n) {
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= n) return;
    IO<In>::st(prev_out, id, prev ? IO<In>::ld(prev, id) : 0.f);
}

// The raw rows of token T-1 of q, k and v into the cache [B][H][3][D] (the cached
// rows, or zeros, when T = 0): one thread per element.
template <int D, typename In>
__global__ void __launch_bounds__(256)
conv_tail_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
                 const In* __restrict__ prev, In* __restrict__ prev_out, int T, size_t n) {
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= n) return;
    const int c = (int)(id % D), which = (int)((id / D) % 3);
    const size_t bh = id / (3 * D);
    float x;
    if (T > 0) {
        const In* src = which == 0 ? q : which == 1 ? k : v;
        x = IO<In>::ld(src, (bh * T + (size_t)(T - 1)) * D + c);
    } else {
        x = prev ? IO<In>::ld(prev, id) : 0.f;
    }
    IO<In>::st(prev_out, id, x);
}

template <int D, typename In>
int launch(const ConvArgs& a) {
    hipStream_t st = (hipStream_t)a.stream;
    if (a.T == 0) {
        if (!a.prev_out) return TWOMAMBA_OK;
        const size_t n = (size_t)a.B * a.H * 3 * D;
        hipLaunchKernelGGL((conv2_pass_kernel<D, In>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           (const In*)a.prev, (In*)a.prev_out, n);
    } else {
        const int tiles = ((a.T + kTok - 1) / kTok * (D / 8) + 255) / 256;
        hipLaunchKernelGGL((conv2_kernel<D, In>), dim3((unsigned)(a.B * a.H * tiles), (unsigned)a.count), dim3(256),
                           0, st, (const In*)a.q, (const In*)a.k, (const In*)a.v, a.w, a.b, (const In*)a.prev,
                           (In*)a.qo, (In*)a.ko, (In*)a.vo, (In*)a.prev_out, a.H, a.T, tiles, a.first);
    }
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

template <int D, typename In>
int tail(const ConvArgs& a) {
    const size_t n = (size_t)a.B * a.H * 3 * D;
    hipLaunchKernelGGL((conv_tail_kernel<D, In>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, (const In*)a.v, (const In*)a.prev,
                       (In*)a.prev_out, a.T, n);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

int conv2_launch(const ConvArgs& a) {
    if ((size_t)a.B * a.H == 0 || a.count <= 0) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.d == 64) return bf ? launch<64, bf16>(a) : launch<64, float>(a);
    if (a.d == 16) return bf ? launch<16, bf16>(a) : launch<16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

int conv_tail_launch(const ConvArgs& a) {
    if ((size_t)a.B * a.H == 0 || !a.prev_out) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.d == 64) return bf ? tail<64, bf16>(a) : tail<64, float>(a);
    if (a.d == 16) return bf ? tail<16, bf16>(a) : tail<16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
