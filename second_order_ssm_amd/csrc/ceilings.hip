// Measurement aids: the two ceilings the benchmark reports beside the
// operator's own kernels, so that "fraction of achievable" has a denominator
// measured on the same box with code of the same kind.
//
//  * ceiling_copy: a streaming device-to-device copy.  Each workgroup moves a
//    contiguous 16 KB block per step (256 threads x four 16-byte vectors, all
//    four loads in flight before the first store), non-temporal loads and
//    stores, 4096 workgroups striding over the buffer: the best of a sweep over
//    grid sizes (1K-16K workgroups), vectors per thread (4, 8, 16) and
//    temporal/non-temporal access on MI355X (about 6.0 TB/s at 1 GiB).
//  * ceiling_mfma: a loop of independent 16x16x32 f16 MFMAs on register
//    operands, sixteen accumulator chains per wave with operands of their own,
//    four waves per workgroup; no memory traffic except one store per lane at
//    the end (so the work cannot be removed).  Executed work: waves x iters x
//    16 x 16384 FLOP.  On MI355X the unit's rate needs about 32 independent
//    accumulations in flight per SIMD (8 chains per wave reach about 60 % of it,
//    4 about 30 %).  The
//    first wave of each workgroup also records the shader-clock cycles and the
//    100 MHz real-time ticks its loop took, which give the clock the MFMA
//    units actually ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "../../include/twomamba_ceilings.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) copy_kernel(const u4* __restrict__ src, u4* __restrict__ dst, size_t n16) {
    constexpr int U = 4;
    const size_t per_step = (size_t)U * 256;
    for (size_t base = (size_t)blockIdx.x * per_step; base < n16; base += (size_t)gridDim.x * per_step) {
        u4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * 256 + threadIdx.x;
            if (i < n16) r[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * 256 + threadIdx.x;
            if (i < n16) __builtin_nontemporal_store(r[u], dst + i);
        }
    }
}

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float seed, float* __restrict__ sink,
                                                        unsigned long long* __restrict__ clocks) {
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    // 16 chains, each with operands of its own: dependent MFMAs are 16 apart, and no
    // two chains compute the same values (which a compiler could merge)
    constexpr int kChains = 16;
    const float x = seed + 1e-3f * (float)(threadIdx.x & 63);
    h8 a[kChains], b[kChains];
    f4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[c][e] = (_Float16)(x + 0.01f * e + 0.125f * c);
            b[c][e] = (_Float16)(x - 0.02f * e - 0.0625f * c);
        }
        acc[c] = f4{0.f, 0.f, 0.f, 0.f};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c], b[c], acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (clocks != nullptr && threadIdx.x == 0) {
        const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

int twomamba_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes == 0) return TWOMAMBA_OK;
    if (!src || !dst) return TWOMAMBA_ERR_NULL;
    if ((bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return TWOMAMBA_ERR_UNSUPPORTED;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return TWOMAMBA_ERR_ALIAS;
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const u4*)src, (u4*)dst, n16);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

int twomamba_ceiling_mfma(int workgroups, int iters, float* sink, unsigned long long* clocks, void* stream) {
    if (workgroups <= 0 || iters <= 0) return TWOMAMBA_ERR_SHAPE;
    if (!sink) return TWOMAMBA_ERR_NULL;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, 0.5f, sink,
                       clocks);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // extern "C"
