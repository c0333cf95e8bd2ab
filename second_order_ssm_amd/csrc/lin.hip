// First-order variant (Mamba-2S) of the operator ("2Mamba2Furious", §2: first
// order linear attention keeps a (dh, dh) state; §3-§4: the Mamba-2S base is
// output-norm linear attention with the softplus A-mask, the norm outside the
// attention kernel):
//     o_t = sum_{s<=t} L_ts (scale q_t.k_s) v_s,   S = sum_s L k_s v_s^T  (dk x dv).
//
// Chunked in three launches, as the SSD duality of Mamba-2 ("Mamba-2 - State
// Space Duality" thread) arranges it:
//   lin_delta: dS_c = sum_{s in c} exp(Gam_c - Gl_s) k_s v_s^T per chunk c, and
//              the chunk's total log decay Gam_c (chunks in parallel);
//   lin_scan:  S_c = exp(Gam_{c-1}) S_{c-1} + dS_{c-1} in place, S_0 = state_in
//              (each state element of a head in parallel, chunks in order);
//   lin_out:   o_t = sum_{s<=t in c} exp(Gl_t - Gl_s)(scale q_t.k_s) v_s
//                    + exp(Gl_t) scale q_t . S_c   (chunks in parallel).
// Gl is the chunk-local inclusive prefix of g = -softplus(z); every exponent is
// a sum of g over a stretch inside one chunk.  The first-order work is small
// (4 dk dv flops per head-token plus the chunk-local part), so the path is bound
// by the traffic of q, k, v, out and the per-chunk states.
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kLinChunk = 64;

struct LinLayout {
    size_t off_S, off_G, total;
};

LinLayout lin_layout(const FwdArgs& a) {
    const size_t nc = (size_t)((a.T + kLinChunk - 1) / kLinChunk);
    const size_t nbh = (size_t)a.B * a.H;
    LinLayout L;
    L.off_S = 0;
    L.off_G = align256(nbh * nc * a.dk * a.dv * sizeof(float));
    L.total = align256(L.off_G + nbh * nc * sizeof(float));
    return L;
}

// one workgroup per (head, chunk); thread (i, column group of 8) owns dS[i][8cg..8cg+7]
template <int DK, int DV, typename In>
__global__ void __launch_bounds__(DK * DV / 8)
lin_delta(const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ z,
          float* __restrict__ wsS, float* __restrict__ wsG, int T, int nc) {
    constexpr int NT = DK * DV / 8;
    __shared__ float s_k[kLinChunk][DK], s_v[kLinChunk][DV], s_w[kLinChunk];
    const int bh = blockIdx.x / nc, c = blockIdx.x % nc;
    const int t0 = c * kLinChunk, Lc = min(kLinChunk, T - t0);
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)bh * T + t0;
    for (int e = tid; e < Lc * DK; e += NT) s_k[e / DK][e % DK] = IO<In>::ld(k, tok0 * DK + e);
    for (int e = tid; e < Lc * DV; e += NT) s_v[e / DV][e % DV] = IO<In>::ld(v, tok0 * DV + e);
    if (tid == 0) {
        float R = 0.f;   // g summed over the chunk's tokens after s
        for (int s = Lc - 1; s >= 0; --s) {
            s_w[s] = expf(R);
            R += decay_log(z[tok0 + s]);
        }
        wsG[(size_t)bh * nc + c] = R;
    }
    __syncthreads();
    const int i = tid / (DV / 8), cg = tid % (DV / 8);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < Lc; ++s) {
        const float f = s_w[s] * s_k[s][i];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(f, s_v[s][8 * cg + u], acc[u]);
    }
    float* dst = wsS + (((size_t)bh * nc + c) * DK + i) * DV + 8 * cg;
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[u] = acc[u];
}

// exclusive scan over chunks, one thread per state element
template <int DK, int DV>
__global__ void __launch_bounds__(256)
lin_scan(float* __restrict__ wsS, const float* __restrict__ wsG, const float* state_in, float* state_out, int nc,
         int etiles) {
    const int bh = blockIdx.x / etiles;
    const int e = (blockIdx.x % etiles) * 256 + threadIdx.x;
    if (e >= DK * DV) return;
    float run = state_in ? state_in[(size_t)bh * DK * DV + e] : 0.f;
    for (int c = 0; c < nc; ++c) {
        float* slot = wsS + ((size_t)bh * nc + c) * DK * DV + e;
        const float x = *slot;
        *slot = run;
        run = fmaf(expf(wsG[(size_t)bh * nc + c]), run, x);
    }
    if (state_out) state_out[(size_t)bh * DK * DV + e] = run;
}

// one workgroup per (head, chunk).  The chunk's masked score matrix
// A[t][s] = exp(Gl_t - Gl_s) (scale q_t.k_s), s <= t, is formed once in LDS
// (each entry by one thread), then thread (token, column group of 8) forms
// o_t = A[t] V + exp(Gl_t) (scale q_t) S_c.
template <int DK, int DV, typename In>
__global__ void __launch_bounds__(kLinChunk * DV / 8)
lin_out(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ z,
        const float* __restrict__ wsS, In* __restrict__ out, int T, int nc, float scale) {
    constexpr int NT = kLinChunk * DV / 8;
    constexpr int KS = DK + 1;   // padded rows: thread (t, s) pairs read distinct banks
    __shared__ float s_q[kLinChunk][KS], s_k[kLinChunk][KS], s_v[kLinChunk][DV], s_S[DK][DV];
    __shared__ float s_A[kLinChunk][kLinChunk + 1], s_gl[kLinChunk];
    const int bh = blockIdx.x / nc, c = blockIdx.x % nc;
    const int t0 = c * kLinChunk, Lc = min(kLinChunk, T - t0);
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)bh * T + t0;
    for (int e = tid; e < Lc * DK; e += NT) {
        s_q[e / DK][e % DK] = IO<In>::ld(q, tok0 * DK + e) * scale;
        s_k[e / DK][e % DK] = IO<In>::ld(k, tok0 * DK + e);
    }
    for (int e = tid; e < Lc * DV; e += NT) s_v[e / DV][e % DV] = IO<In>::ld(v, tok0 * DV + e);
    const float* Sc = wsS + ((size_t)bh * nc + c) * DK * DV;
    for (int e = tid; e < DK * DV; e += NT) s_S[e / DV][e % DV] = Sc[e];
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < Lc; ++t) {
            acc += decay_log(z[tok0 + t]);
            s_gl[t] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kLinChunk * kLinChunk; e += NT) {
        const int t = e / kLinChunk, sk = e % kLinChunk;
        float a = 0.f;
        if (sk <= t && t < Lc) {
#pragma unroll 8
            for (int i = 0; i < DK; ++i) a = fmaf(s_q[t][i], s_k[sk][i], a);
            a *= expf(s_gl[t] - s_gl[sk]);
        }
        s_A[t][sk] = a;
    }
    __syncthreads();
    const int tl = tid / (DV / 8), cg = tid % (DV / 8);
    if (tl >= Lc) return;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sk = 0; sk <= tl; ++sk) {
        const float a = s_A[tl][sk];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = fmaf(a, s_v[sk][8 * cg + u], o[u]);
    }
    float r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < DK; ++i) {
        const float qi = s_q[tl][i];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = fmaf(qi, s_S[i][8 * cg + u], r[u]);
    }
    const float dec = expf(s_gl[tl]);
#pragma unroll
    for (int u = 0; u < 8; ++u) IO<In>::st(out, (tok0 + tl) * DV + 8 * cg + u, fmaf(dec, r[u], o[u]));
}

__global__ void lin_copy_or_zero(const float* src, float* dst, size_t n) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e < n) dst[e] = src ? src[e] : 0.f;
}

template <int DK, int DV, typename In>
int run(const FwdArgs& a) {
    const LinLayout L = lin_layout(a);
    const int nc = (a.T + kLinChunk - 1) / kLinChunk;
    const int nbh = a.B * a.H;
    float* wsS = (float*)((char*)a.ws + L.off_S);
    float* wsG = (float*)((char*)a.ws + L.off_G);
    hipStream_t st = (hipStream_t)a.stream;
    ktimer_begin(a.timer, "lin_delta", a.stream);
    hipLaunchKernelGGL((lin_delta<DK, DV, In>), dim3(nbh * nc), dim3(DK * DV / 8), 0, st, (const In*)a.k,
                       (const In*)a.v, a.z, wsS, wsG, a.T, nc);
    ktimer_end(a.timer, a.stream);
    const int etiles = (DK * DV + 255) / 256;
    ktimer_begin(a.timer, "lin_scan", a.stream);
    hipLaunchKernelGGL((lin_scan<DK, DV>), dim3(nbh * etiles), dim3(256), 0, st, wsS, (const float*)wsG, a.state_in,
                       a.state_out, nc, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "lin_out", a.stream);
    hipLaunchKernelGGL((lin_out<DK, DV, In>), dim3(nbh * nc), dim3(kLinChunk * DV / 8), 0, st, (const In*)a.q,
                       (const In*)a.k, (const In*)a.v, a.z, (const float*)wsS, (In*)a.out, a.T, nc, a.scale);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

size_t lin_workspace(const FwdArgs& a) {
    if ((size_t)a.B * a.H * a.T == 0) return 0;
    return lin_layout(a).total;
}

int lin_fwd(const FwdArgs& a) {
    const size_t nbh = (size_t)a.B * a.H;
    if (nbh == 0) return TWOMAMBA_OK;
    if (a.T == 0) {
        if (a.state_out && a.state_out != a.state_in) {
            const size_t n = nbh * a.dk * a.dv;
            hipLaunchKernelGGL(lin_copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               (hipStream_t)a.stream, a.state_in, a.state_out, n);
        }
        return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
    }
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
