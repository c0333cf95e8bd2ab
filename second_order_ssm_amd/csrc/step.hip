// Recurrent decode step of 2Mamba ("2Mamba2Furious", §2 constant-size second-order
// hidden state; App. A inference):
//     S <- e^g S + phi(k) v^T,   n <- e^g n + phi(k),   o = phi_q(q).S / phi_q(q).n
//
// Bandwidth-bound: per head the packed fp32 state is D x dv (532 KB at d = 64) and
// is read and written once.  One workgroup per (b, h) streams that head's rows
// front to back; consecutive threads own consecutive 16-byte column slices of a
// row, so every wave reads and writes whole contiguous rows (fully coalesced).
// The state is touched once per step, so the main sweep's loads and stores are
// non-temporal; 512 threads with 6 rows in flight each was the fastest shape
// measured (about 5.9 TB/s at B = 64, H = 32, against 5.1 TB/s for a plain
// device copy).  The short tail sweep uses ordinary loads and stores: making
// it non-temporal as well measured 8 % slower.
// The readout sum over rows is reduced in a fixed order through LDS, so results
// are bit-reproducible.  With an input convolution attached (twomamba_step_conv,
// App. A: one cached previous query, key and value) the three input rows are
// convolved with the cached ones on the way into LDS.
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kStepThreads = 512;
typedef float vf4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_nt(const float4* p) {
    const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_nt(float4* p, float4 y) {
    const vf4 t = {y.x, y.y, y.z, y.w};
    __builtin_nontemporal_store(t, reinterpret_cast<vf4*>(p));
}

// kOrder 2: the packed second-order state and its normaliser; kOrder 1: the
// first-order (Mamba-2S) state S <- e^g S + k v^T, o = scale q.S, D = dk rows,
// no normaliser ("2Mamba2Furious", §2 and §3-§4).
template <int DK, int DV, typename In, int kOrder>
__global__ void __launch_bounds__(kStepThreads)
step_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
            const float* __restrict__ z, float* __restrict__ state, float* __restrict__ norm,
            In* __restrict__ out, float scale, int no_norm, const float* __restrict__ cw,
            const float* __restrict__ cb, In* __restrict__ cst, int H) {
    constexpr int D = kOrder == 2 ? DK * (DK + 1) / 2 : DK;
    constexpr int CG = DV / 4;                 // float4 column groups per row
    constexpr int NR = kStepThreads / CG;      // rows processed per sweep
    constexpr int UNR = 6;                     // rows in flight per thread

    // The feature rows are dead once the sweeps are done; the per-row-group
    // partial sums then reuse their LDS, which keeps a workgroup under 20 KB so
    // that 8 heads run on each CU at once.
    constexpr int kFeat = 2 * D;                                  // floats of s_fk + s_fq
    constexpr int kPart = NR * CG * 4;                            // floats of the partials
    __shared__ __attribute__((aligned(16))) float s_u[kFeat > kPart ? kFeat : kPart];
    __shared__ float s_q[DK], s_k[DK], s_v[DV];
    __shared__ float s_den[kStepThreads / 64];
    float* s_fk = s_u;
    float* s_fq = s_u + D;
    float4 (*s_part)[CG] = reinterpret_cast<float4 (*)[CG]>(s_u);

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t hoff = (size_t)bh;

    // inputs, through the size-2 convolution when one is attached: the cached
    // raw row of the previous token is read and replaced by this token's
    if (tid < 3 * DK) {
        const int which = tid / DK, c = tid % DK;
        const In* src = which == 0 ? q : which == 1 ? k : v;
        float x = IO<In>::ld(src, hoff * DK + c);
        if (cw) {
            const size_t wi = (size_t)(which * H + bh % H) * DK + c;
            In* cs = cst + (hoff * 3 + which) * DK;
            const float before = IO<In>::ld(cs, c);
            IO<In>::st(cs, c, x);
            // as the forward's convolution, which also hands its output over in the input dtype
            x = IO<In>::rnd(fmaf(cw[2 * wi + 1], x, fmaf(cw[2 * wi], before, cb ? cb[wi] : 0.f)));
        }
        if (which == 0) s_q[c] = x * scale;
        else if (which == 1) s_k[c] = x;
        else s_v[c] = x;
    }
    const float a = expf(decay_log(z[hoff]));
    __syncthreads();

    // features of this token, one row i of the upper triangle per thread
    if (tid < DK) {
        const int i = tid;
        if (kOrder == 2) {
            int p = i * DK - (i * (i - 1)) / 2;
            const float ki = s_k[i], qi = s_q[i];
            for (int j = i; j < DK; ++j, ++p) {
                s_fk[p] = ki * s_k[j];
                s_fq[p] = (j == i ? 1.f : 2.f) * qi * s_q[j];
            }
        } else {
            s_fk[i] = s_k[i];
            s_fq[i] = s_q[i];
        }
    }
    __syncthreads();

    const int cg = tid % CG;
    const int rs = tid / CG;
    const float4 v4 = make_float4(s_v[4 * cg], s_v[4 * cg + 1], s_v[4 * cg + 2], s_v[4 * cg + 3]);
    float4* S = reinterpret_cast<float4*>(state + hoff * (size_t)D * DV);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    int p = rs;
    for (; p + (UNR - 1) * NR < D; p += UNR * NR) {
        float4 x[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) x[u] = ld_nt(&S[(size_t)(p + u * NR) * CG + cg]);
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int pr = p + u * NR;
            const float fk = s_fk[pr], fq = s_fq[pr];
            float4 y;
            y.x = fmaf(a, x[u].x, fk * v4.x);
            y.y = fmaf(a, x[u].y, fk * v4.y);
            y.z = fmaf(a, x[u].z, fk * v4.z);
            y.w = fmaf(a, x[u].w, fk * v4.w);
            st_nt(&S[(size_t)pr * CG + cg], y);
            acc.x = fmaf(fq, y.x, acc.x);
            acc.y = fmaf(fq, y.y, acc.y);
            acc.z = fmaf(fq, y.z, acc.z);
            acc.w = fmaf(fq, y.w, acc.w);
        }
    }
    for (; p < D; p += NR) {
        const float4 x = S[(size_t)p * CG + cg];
        const float fk = s_fk[p], fq = s_fq[p];
        float4 y;
        y.x = fmaf(a, x.x, fk * v4.x);
        y.y = fmaf(a, x.y, fk * v4.y);
        y.z = fmaf(a, x.z, fk * v4.z);
        y.w = fmaf(a, x.w, fk * v4.w);
        S[(size_t)p * CG + cg] = y;
        acc.x = fmaf(fq, y.x, acc.x);
        acc.y = fmaf(fq, y.y, acc.y);
        acc.z = fmaf(fq, y.z, acc.z);
        acc.w = fmaf(fq, y.w, acc.w);
    }

    // normaliser rows
    float den = 0.f;
    if (kOrder == 2) {
        float* n = norm + hoff * (size_t)D;
        for (int r = tid; r < D; r += kStepThreads) {
            const float y = fmaf(a, n[r], s_fk[r]);
            n[r] = y;
            den = fmaf(s_fq[r], y, den);
        }
    }
    // fixed-order wave reduction of den
    for (int off = 32; off > 0; off >>= 1) den += __shfl_down(den, off, 64);
    if ((tid & 63) == 0) s_den[tid >> 6] = den;
    __syncthreads();   // every read of s_fk / s_fq is done
    s_part[rs][cg] = acc;
    __syncthreads();

    if (tid < DV) {
        const int c = tid;
        float num = 0.f;
        for (int r = 0; r < NR; ++r) {
            const float4 t4 = s_part[r][c >> 2];
            num += (c & 3) == 0 ? t4.x : (c & 3) == 1 ? t4.y : (c & 3) == 2 ? t4.z : t4.w;
        }
        float dsum = 0.f;
        for (int w = 0; w < kStepThreads / 64; ++w) dsum += s_den[w];
        float o;
        if (no_norm || kOrder == 1) o = num;
        else o = (dsum == 0.f) ? 0.f : num / dsum;
        IO<In>::st(out, hoff * DV + c, o);
    }
}

// First-order step at d = 64: the state is only 64 x 64 fp32 (16 KB) per head, so
// one wave takes a head and four heads share a workgroup.  Lane (rq, cg) owns the
// 16 rows 4i + rq (i = 0..15) of column group cg (4 columns): all 16 row loads are
// in flight at once, every load and store instruction of the wave covers four whole
// consecutive rows (1 KB), and the readout's sum over rows is finished across the
// four lanes of a column group by shuffles in a fixed order (no LDS round trip).
template <typename In>
__global__ void __launch_bounds__(256)
step_first_order64_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
                          const float* __restrict__ z, float* __restrict__ state, In* __restrict__ out,
                          float scale, const float* __restrict__ cw, const float* __restrict__ cb,
                          In* __restrict__ cst, int H, int nbh) {
    constexpr int D = 64;
    __shared__ float s_in[4][3][D];   // per wave: scale q, k, v (convolved when a cache is attached)
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + w;
    const bool live = bh < nbh;   // uniform over the wave
    const int cg = lane & 15, rq = lane >> 4;
    float4* S = reinterpret_cast<float4*>(state + (size_t)bh * D * D);
    // the state's loads go out first: nothing they fetch depends on the inputs
    float4 x[16];
    if (live) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = ld_nt(&S[(4 * i + rq) * 16 + cg]);
    }
    if (live) {
#pragma unroll
        for (int which = 0; which < 3; ++which) {
            const In* src = which == 0 ? q : which == 1 ? k : v;
            float x = IO<In>::ld(src, (size_t)bh * D + lane);
            if (cw) {
                const size_t wi = (size_t)(which * H + bh % H) * D + lane;
                In* cs = cst + ((size_t)bh * 3 + which) * D;
                const float before = IO<In>::ld(cs, lane);
                IO<In>::st(cs, lane, x);
                // as the forward's convolution, which also hands its output over in the input dtype
                x = IO<In>::rnd(fmaf(cw[2 * wi + 1], x, fmaf(cw[2 * wi], before, cb ? cb[wi] : 0.f)));
            }
            s_in[w][which][lane] = which == 0 ? x * scale : x;
        }
    }
    __syncthreads();
    if (!live) return;
    const float a = expf(decay_log(z[bh]));
    const float4 v4 = make_float4(s_in[w][2][4 * cg], s_in[w][2][4 * cg + 1], s_in[w][2][4 * cg + 2],
                                  s_in[w][2][4 * cg + 3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + rq;
        const float fk = s_in[w][1][r], fq = s_in[w][0][r];
        float4 y;
        y.x = fmaf(a, x[i].x, fk * v4.x);
        y.y = fmaf(a, x[i].y, fk * v4.y);
        y.z = fmaf(a, x[i].z, fk * v4.z);
        y.w = fmaf(a, x[i].w, fk * v4.w);
        st_nt(&S[r * 16 + cg], y);
        acc.x = fmaf(fq, y.x, acc.x);
        acc.y = fmaf(fq, y.y, acc.y);
        acc.z = fmaf(fq, y.z, acc.z);
        acc.w = fmaf(fq, y.w, acc.w);
    }
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
    }
    if (rq == 0) {
        IO<In>::st(out, (size_t)bh * D + 4 * cg, acc.x);
        IO<In>::st(out, (size_t)bh * D + 4 * cg + 1, acc.y);
        IO<In>::st(out, (size_t)bh * D + 4 * cg + 2, acc.z);
        IO<In>::st(out, (size_t)bh * D + 4 * cg + 3, acc.w);
    }
}

template <int DK, int DV, typename In>
int launch(const StepArgs& a) {
    const int nbh = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    const bool first = (a.flags & TWOMAMBA_FLAG_FIRST_ORDER) != 0;
    if (first && DK == 64 && DV == 64) {
        hipLaunchKernelGGL(step_first_order64_kernel<In>, dim3((unsigned)((nbh + 3) / 4)), dim3(256), 0, st,
                           (const In*)a.q, (const In*)a.k, (const In*)a.v, a.z, a.state, (In*)a.out, a.scale,
                           a.conv_w, a.conv_b, (In*)a.conv_state, a.H, nbh);
        return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
    }
    auto kern = first ? step_kernel<DK, DV, In, 1> : step_kernel<DK, DV, In, 2>;
    hipLaunchKernelGGL(kern, dim3(nbh), dim3(kStepThreads), 0, st,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.z, a.state, a.norm, (In*)a.out,
                       a.scale, (int)((a.flags & TWOMAMBA_FLAG_NO_NORM) != 0), a.conv_w, a.conv_b,
                       (In*)a.conv_state, a.H);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

int step_launch(const StepArgs& a) {
    if (a.B == 0 || a.H == 0) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? launch<64, 64, bf16>(a) : launch<64, 64, float>(a);
    if (a.dk == 16) return bf ? launch<16, 16, bf16>(a) : launch<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
