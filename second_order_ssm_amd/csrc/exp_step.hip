// 2Mamba-E decoding over a key/value cache ("2Mamba2Furious", §6: softmax
// attention with the softplus A-mask; inference keeps every past key and value).
//
// Cache of one head: K, V rows in the caller's dtype and G_s, the fp64 running
// sum of softplus(z) up to token s.  The decay log-bias of key s for the query
// of token t is G_s - G_t; fp64 keeps that difference exact to fp32 whatever
// the sequence length.
//
// A decode step is HBM-bound: every cached key and value is read once.
//  * exp_decode_partial: one workgroup per (head, 512-key split).  Eight lanes
//    share a key (16 bytes of it each), so a wave reads eight consecutive cache
//    rows per load instruction; the dot product is finished with three DPP
//    steps inside the 8-lane group and the online softmax runs per wave.  The
//    partial (max, sum, weighted values) of the split goes to the workspace.
//    The new token's key and value come from the inputs, and split 0 appends
//    them (and G_t) to the caches; no workgroup reads that row.
//  * exp_decode_combine: one wave per head merges the splits.
//  * exp_cache_fill: copies a prompt's keys and values into the caches and
//    writes the running sums G (one workgroup per head, a blocked scan).
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kSplit = 512;         // keys per workgroup
constexpr int kThreadsD = 256;      // 4 waves, 128 keys each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyD = 8.f;       // log2 headroom before the running max moves

__device__ __forceinline__ double softplus64(float zf) {
    const double z = zf;
    return fmax(z, 0.0) + log1p(exp(-fabs(z)));
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float rdl(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// sum over groups of kLpk consecutive lanes (kLpk = 2 or 8)
template <int kLpk>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xb1>(x);                    // quad_perm [1,0,3,2]
    if (kLpk >= 4) x += dpp<0x4e>(x);     // quad_perm [2,3,0,1]
    if (kLpk >= 8) x += dpp<0x141>(x);    // row_half_mirror: the other quad of the 8
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xb1>(x));
    x = fmaxf(x, dpp<0x4e>(x));
    x = fmaxf(x, dpp<0x124>(x));          // row_ror:4
    x = fmaxf(x, dpp<0x128>(x));          // row_ror:8
    return fmaxf(fmaxf(rdl(x, 0), rdl(x, 16)), fmaxf(rdl(x, 32), rdl(x, 48)));
}

// 8 consecutive elements of a row as floats
template <typename In> struct Row8;
template <> struct Row8<bf16> {
    static __device__ __forceinline__ void ld(const bf16* p, float* o) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Row8<float> {
    static __device__ __forceinline__ void ld(const float* p, float* o) {
        const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// G at the new token: G_{pos-1} + softplus(z), G_{-1} = 0
__device__ __forceinline__ double g_now(const double* gc, const float* z, int bh, int max_len, int pos) {
    const double prev = pos > 0 ? gc[(size_t)bh * max_len + pos - 1] : 0.0;
    return prev + softplus64(z[bh]);
}

template <int DK, typename In>
__global__ void __launch_bounds__(kThreadsD)
exp_decode_partial(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
                   const float* __restrict__ z, In* __restrict__ kc, In* __restrict__ vc, double* __restrict__ gc,
                   float* __restrict__ part, int max_len, int pos, int nsplit, float scale) {
    constexpr int kLpk = DK / 8;          // lanes per key
    constexpr int kKpi = 64 / kLpk;       // keys per wave per iteration
    constexpr int kPerWave = kSplit / (kThreadsD / 64);
    constexpr int kIters = kPerWave / kKpi;
    __shared__ float s_m[kThreadsD / 64], s_l[kThreadsD / 64];
    __shared__ float s_o[kThreadsD / 64][kKpi][DK];

    const int bh = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int grp = lane / kLpk, part8 = lane % kLpk;   // key slot and 8-dim chunk of this lane
    const size_t crow = (size_t)bh * max_len;
    const double G = g_now(gc, z, bh, max_len, pos);

    if (split == 0) {   // append the new token
        if (tid < DK) {
            kc[(crow + pos) * DK + tid] = k[(size_t)bh * DK + tid];
            vc[(crow + pos) * DK + tid] = v[(size_t)bh * DK + tid];
        }
        if (tid == 0) gc[crow + pos] = G;
    }

    float qv[8];
    Row8<In>::ld(q + (size_t)bh * DK + 8 * part8, qv);
    const float sl2 = scale * kLog2e;
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] *= sl2;

    float m = -INFINITY, l = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int s_lo = split * kSplit + w * kPerWave;
#pragma unroll 4
    for (int it = 0; it < kIters; ++it) {
        const int s = s_lo + it * kKpi + grp;
        const bool valid = s <= pos;
        // the new token and the slots past it read the (finite) input row: cache
        // row pos is being written by split 0 and later rows hold anything
        const bool from_in = s >= pos;
        const In* kp = from_in ? k + (size_t)bh * DK : kc + (crow + s) * DK;
        const In* vp = from_in ? v + (size_t)bh * DK : vc + (crow + s) * DK;
        float kv[8], vv[8];
        Row8<In>::ld(kp + 8 * part8, kv);
        Row8<In>::ld(vp + 8 * part8, vv);
        const double Gs = from_in ? G : gc[crow + s];
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf(qv[i], kv[i], dot);
        dot = group_sum<kLpk>(dot);
        const float x = valid ? dot + (float)(Gs - G) * kLog2e : -INFINITY;
        const float mx = wave_max(x);
        if (mx > m + kLazyD) {   // wave-uniform
            const float alpha = __builtin_amdgcn_exp2f(m - mx);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] *= alpha;
            m = mx;
        }
        const float p = valid ? __builtin_amdgcn_exp2f(x - m) : 0.f;
        l += p;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(p, vv[i], o[i]);
    }
    // wave partials: each key slot's lanes hold its sum (the same in all of them)
    if (lane == 0) {
        s_m[w] = m;
    }
    float lw = l;
    // sum of l over the key slots: lanes part8 == 0 of every slot
    float lsum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kKpi; ++g2) lsum += rdl(lw, g2 * kLpk);
    if (lane == 0) s_l[w] = lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) s_o[w][grp][8 * part8 + i] = o[i];
    __syncthreads();
    if (tid < DK) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kThreadsD / 64; ++ww) M = fmaxf(M, s_m[ww]);
        float L = 0.f, Ot = 0.f;
#pragma unroll
        for (int ww = 0; ww < kThreadsD / 64; ++ww) {
            const float f = (s_m[ww] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[ww] - M);
            L = fmaf(s_l[ww], f, L);
            float acc = 0.f;
#pragma unroll 8
            for (int g2 = 0; g2 < kKpi; ++g2) acc += s_o[ww][g2][tid];
            Ot = fmaf(acc, f, Ot);
        }
        float* pp = part + ((size_t)bh * nsplit + split) * (DK + 2);
        pp[2 + tid] = Ot;
        if (tid == 0) {
            pp[0] = M;
            pp[1] = L;
        }
    }
}

template <int DK, typename In>
__global__ void __launch_bounds__(64)
exp_decode_combine(const float* __restrict__ part, In* __restrict__ out, int nsplit) {
    const int bh = blockIdx.x, t = threadIdx.x;
    if (t >= DK) return;
    const float* pb = part + (size_t)bh * nsplit * (DK + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, pb[(size_t)sp * (DK + 2)]);
    float L = 0.f, O = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
        const float* pp = pb + (size_t)sp * (DK + 2);
        const float f = (pp[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(pp[0] - M);
        L = fmaf(pp[1], f, L);
        O = fmaf(pp[2 + t], f, O);
    }
    IO<In>::st(out, (size_t)bh * DK + t, O / L);
}

// Prompt -> caches.  One workgroup per head: rows copied with 16-byte moves,
// then G by a blocked scan (per-thread runs, thread totals scanned in order).
template <int DK, typename In>
__global__ void __launch_bounds__(256)
exp_cache_fill_kernel(const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ z,
                      In* __restrict__ kc, In* __restrict__ vc, double* __restrict__ gc, int T, int max_len) {
    __shared__ double s_tot[256];
    const int bh = blockIdx.x, tid = threadIdx.x;
    constexpr int kVec = 16 / sizeof(In);
    const size_t n = (size_t)T * DK;
    const In* ks = k + (size_t)bh * T * DK;
    const In* vs = v + (size_t)bh * T * DK;
    In* kd = kc + (size_t)bh * max_len * DK;
    In* vd = vc + (size_t)bh * max_len * DK;
    for (size_t e = (size_t)tid * kVec; e < n; e += 256 * kVec) {
        *reinterpret_cast<uint4*>(kd + e) = *reinterpret_cast<const uint4*>(ks + e);
        *reinterpret_cast<uint4*>(vd + e) = *reinterpret_cast<const uint4*>(vs + e);
    }
    const int run = (T + 255) / 256;
    const int t0 = tid * run, t1 = min(T, t0 + run);
    const float* zs = z + (size_t)bh * T;
    double acc = 0.0;
    for (int t = t0; t < t1; ++t) acc += softplus64(zs[t]);
    s_tot[tid] = acc;
    __syncthreads();
    if (tid == 0) {
        double r = 0.0;
        for (int i = 0; i < 256; ++i) {
            const double x = s_tot[i];
            s_tot[i] = r;
            r += x;
        }
    }
    __syncthreads();
    double g = s_tot[tid];
    double* gd = gc + (size_t)bh * max_len;
    for (int t = t0; t < t1; ++t) {
        g += softplus64(zs[t]);
        gd[t] = g;
    }
}

template <int DK, typename In>
int launch_step(const ExpCacheArgs& a) {
    const int nbh = a.B * a.H;
    const int nsplit = (a.pos + 1 + kSplit - 1) / kSplit;
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((exp_decode_partial<DK, In>), dim3(nbh * nsplit), dim3(kThreadsD), 0, st, (const In*)a.q,
                       (const In*)a.k, (const In*)a.v, a.z, (In*)a.k_cache, (In*)a.v_cache, a.g_cache, (float*)a.ws,
                       a.max_len, a.pos, nsplit, a.scale);
    hipLaunchKernelGGL((exp_decode_combine<DK, In>), dim3(nbh), dim3(64), 0, st, (const float*)a.ws, (In*)a.out,
                       nsplit);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

template <int DK, typename In>
int launch_fill(const ExpCacheArgs& a) {
    hipLaunchKernelGGL((exp_cache_fill_kernel<DK, In>), dim3(a.B * a.H), dim3(256), 0, (hipStream_t)a.stream,
                       (const In*)a.k, (const In*)a.v, a.z, (In*)a.k_cache, (In*)a.v_cache, a.g_cache, a.pos,
                       a.max_len);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

size_t exp_step_workspace(const ExpCacheArgs& a) {
    const size_t nsplit = ((size_t)a.pos + 1 + kSplit - 1) / kSplit;
    return align256((size_t)a.B * a.H * nsplit * (a.dk + 2) * sizeof(float));
}

int exp_step_launch(const ExpCacheArgs& a) {
    if ((size_t)a.B * a.H == 0) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? launch_step<64, bf16>(a) : launch_step<64, float>(a);
    if (a.dk == 16) return bf ? launch_step<16, bf16>(a) : launch_step<16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

int exp_cache_fill_launch(const ExpCacheArgs& a) {
    if ((size_t)a.B * a.H == 0 || a.pos == 0) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? launch_fill<64, bf16>(a) : launch_fill<64, float>(a);
    if (a.dk == 16) return bf ? launch_fill<16, bf16>(a) : launch_fill<16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
