// Reference (plain fp32 VALU) kernels of the 2Mamba chunked forward
// ("2Mamba2Furious", §5: squared QK score, softplus A-mask on the squared score,
// normalised by the sum of weights).  Correct for every supported shape and
// dtype; the MFMA kernels are the fast path for bf16 at d = 64.
//
// Chunked form (chunk C, chunk-local inclusive prefix Gl of g, chunk total Gam):
//   delta:  dS_c = sum_{s in c} exp(Gam_c - Gl_s) phi(k_s) v_s^T     (and dn_c)
//   scan :  S_0 = state_in,  S_{c+1} = exp(Gam_c) S_c + dS_c           (exclusive prefix)
//   out  :  num_t = sum_{s<=t in c} exp(Gl_t-Gl_s)(q_t.k_s)^2 v_s + exp(Gl_t) phi_q(q_t).S_c
//           (den likewise with v -> 1),  o_t = num_t / den_t
// All decay exponents are sums of g over a stretch inside one chunk, so no
// exponent of a positive number is ever taken.
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kMaxRefChunk = 64;

struct RefLayout {
    size_t off_S, off_N, off_G, total;
};

RefLayout ref_layout(const FwdArgs& a) {
    const size_t D = num_pairs(a.dk);
    const size_t nc = (size_t)((a.T + a.chunk - 1) / a.chunk);
    const size_t nbh = (size_t)a.B * a.H;
    RefLayout L;
    L.off_S = 0;
    L.off_N = align256(L.off_S + nbh * nc * D * a.dv * sizeof(float));
    L.off_G = align256(L.off_N + nbh * nc * D * sizeof(float));
    L.total = align256(L.off_G + nbh * nc * sizeof(float));
    return L;
}

// ---------------------------------------------------------------- delta
template <int DK, int DV, typename In>
__global__ void __launch_bounds__(256)
ref_sq_delta(const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ z,
             float* __restrict__ wsS, float* __restrict__ wsN, float* __restrict__ wsG, int T, int C, int nc) {
    constexpr int D = DK * (DK + 1) / 2;
    constexpr int CGN = DV / 8;
    constexpr int PT = 256 / CGN;
    __shared__ float s_k[kMaxRefChunk][DK];
    __shared__ float s_v[kMaxRefChunk][DV];
    __shared__ float s_g[kMaxRefChunk], s_w[kMaxRefChunk];

    const int bh = blockIdx.x / nc;
    const int c = blockIdx.x % nc;
    const int t0 = c * C;
    const int Lc = min(C, T - t0);
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)bh * T + t0;

    for (int e = tid; e < Lc * DK; e += 256) s_k[e / DK][e % DK] = IO<In>::ld(k, tok0 * DK + e);
    for (int e = tid; e < Lc * DV; e += 256) s_v[e / DV][e % DV] = IO<In>::ld(v, tok0 * DV + e);
    for (int e = tid; e < Lc; e += 256) s_g[e] = decay_log(z[tok0 + e]);
    __syncthreads();
    if (tid == 0) {
        float R = 0.f;   // sum of g over tokens after s, up to the chunk end
        for (int s = Lc - 1; s >= 0; --s) {
            s_w[s] = expf(R);
            R += s_g[s];
        }
        if (blockIdx.y == 0) wsG[(size_t)bh * nc + c] = R;
    }
    __syncthreads();

    const int pl = tid / CGN, cg = tid % CGN;
    const int p = blockIdx.y * PT + pl;
    if (p >= D) return;
    int i, j;
    pair_of(p, DK, i, j);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float nacc = 0.f;
    for (int s = 0; s < Lc; ++s) {
        const float f = s_w[s] * s_k[s][i] * s_k[s][j];
        nacc += f;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(f, s_v[s][cg * 8 + u], acc[u]);
    }
    float* dst = wsS + (((size_t)bh * nc + c) * D + p) * DV + cg * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[u] = acc[u];
    if (cg == 0) wsN[((size_t)bh * nc + c) * D + p] = nacc;
}

// ---------------------------------------------------------------- scan
template <int DK, int DV>
__global__ void __launch_bounds__(256)
ref_sq_scan(float* __restrict__ wsS, float* __restrict__ wsN, const float* __restrict__ wsG,
            const float* state_in, const float* norm_in, float* state_out, float* norm_out, int nc, int etiles) {
    constexpr int D = DK * (DK + 1) / 2;
    const int bh = blockIdx.x / etiles;
    const int e = (blockIdx.x % etiles) * 256 + threadIdx.x;
    if (e >= D * DV + D) return;
    const bool is_state = e < D * DV;
    const int eo = is_state ? e : e - D * DV;
    float run = 0.f;
    if (state_in) run = is_state ? state_in[(size_t)bh * D * DV + eo] : norm_in[(size_t)bh * D + eo];
    for (int c = 0; c < nc; ++c) {
        float* slot = is_state ? wsS + (((size_t)bh * nc + c) * D * DV + eo) : wsN + (((size_t)bh * nc + c) * D + eo);
        const float x = *slot;
        *slot = run;
        run = fmaf(expf(wsG[(size_t)bh * nc + c]), run, x);
    }
    if (state_out) {
        if (is_state) state_out[(size_t)bh * D * DV + eo] = run;
        else norm_out[(size_t)bh * D + eo] = run;
    }
}

// ---------------------------------------------------------------- out
template <int DK, int DV, typename In>
__global__ void __launch_bounds__(512)
ref_sq_out(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
           const float* __restrict__ z, const float* __restrict__ wsS, const float* __restrict__ wsN,
           In* __restrict__ out, int T, int C, int nc, float scale, int no_norm, float* __restrict__ row_stat) {
    constexpr int D = DK * (DK + 1) / 2;
    constexpr int CGN = DV / 8;
    constexpr int PTILE = 32;
    __shared__ float s_q[kMaxRefChunk][DK], s_k[kMaxRefChunk][DK], s_v[kMaxRefChunk][DV];
    __shared__ float s_gl[kMaxRefChunk];
    __shared__ float s_St[PTILE][DV], s_nt[PTILE];
    __shared__ uint8_t s_pi[D], s_pj[D];

    const int bh = blockIdx.x / nc;
    const int c = blockIdx.x % nc;
    const int t0 = c * C;
    const int Lc = min(C, T - t0);
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const size_t tok0 = (size_t)bh * T + t0;

    for (int e = tid; e < Lc * DK; e += nthr) {
        s_q[e / DK][e % DK] = IO<In>::ld(q, tok0 * DK + e) * scale;
        s_k[e / DK][e % DK] = IO<In>::ld(k, tok0 * DK + e);
    }
    for (int e = tid; e < Lc * DV; e += nthr) s_v[e / DV][e % DV] = IO<In>::ld(v, tok0 * DV + e);
    if (tid < DK) {
        int p = tid * DK - (tid * (tid - 1)) / 2;
        for (int j = tid; j < DK; ++j, ++p) {
            s_pi[p] = (uint8_t)tid;
            s_pj[p] = (uint8_t)j;
        }
    }
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < Lc; ++t) {
            acc += decay_log(z[tok0 + t]);
            s_gl[t] = acc;
        }
    }
    __syncthreads();

    const int tl = tid / CGN, cg = tid % CGN;
    const bool active = tl < Lc;
    float num[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float den = 0.f;
    if (active) {
        // intra-chunk, causal incl. the diagonal
        for (int s = 0; s <= tl; ++s) {
            float sc = 0.f;
#pragma unroll 8
            for (int i = 0; i < DK; ++i) sc = fmaf(s_q[tl][i], s_k[s][i], sc);
            const float w = expf(s_gl[tl] - s_gl[s]) * sc * sc;
            den += w;
#pragma unroll
            for (int u = 0; u < 8; ++u) num[u] = fmaf(w, s_v[s][cg * 8 + u], num[u]);
        }
    }
    // inter-chunk readout of the carried state S_c
    float inum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float iden = 0.f;
    const float* Sc = wsS + ((size_t)bh * nc + c) * D * DV;
    const float* Nc = wsN + ((size_t)bh * nc + c) * D;
    for (int p0 = 0; p0 < D; p0 += PTILE) {
        const int np = min(PTILE, D - p0);
        __syncthreads();
        for (int e = tid; e < np * DV; e += nthr) s_St[e / DV][e % DV] = Sc[(size_t)p0 * DV + e];
        for (int e = tid; e < np; e += nthr) s_nt[e] = Nc[p0 + e];
        __syncthreads();
        if (active) {
            for (int r = 0; r < np; ++r) {
                const int i = s_pi[p0 + r], j = s_pj[p0 + r];
                const float fq = (i == j ? 1.f : 2.f) * s_q[tl][i] * s_q[tl][j];
                iden = fmaf(fq, s_nt[r], iden);
#pragma unroll
                for (int u = 0; u < 8; ++u) inum[u] = fmaf(fq, s_St[r][cg * 8 + u], inum[u]);
            }
        }
    }
    if (!active) return;
    const float dt = expf(s_gl[tl]);
    den = fmaf(dt, iden, den);
    if (row_stat && cg == 0) row_stat[tok0 + tl] = den;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float nu = fmaf(dt, inum[u], num[u]);
        const float o = no_norm ? nu : (den == 0.f ? 0.f : nu / den);
        IO<In>::st(out, (tok0 + tl) * DV + cg * 8 + u, o);
    }
}

// state_out = state_in (or zero) when there are no tokens
__global__ void copy_or_zero(const float* src, float* dst, size_t n) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e < n) dst[e] = src ? src[e] : 0.f;
}

template <int DK, int DV, typename In>
int run(const FwdArgs& a) {
    constexpr int D = DK * (DK + 1) / 2;
    const RefLayout L = ref_layout(a);
    const int nc = (a.T + a.chunk - 1) / a.chunk;
    const int nbh = a.B * a.H;
    char* ws = (char*)a.ws;
    float* wsS = (float*)(ws + L.off_S);
    float* wsN = (float*)(ws + L.off_N);
    float* wsG = (float*)(ws + L.off_G);
    hipStream_t st = (hipStream_t)a.stream;
    const int ptiles = (D + (256 / (DV / 8)) - 1) / (256 / (DV / 8));
    ktimer_begin(a.timer, "ref_sq_delta", a.stream);
    hipLaunchKernelGGL((ref_sq_delta<DK, DV, In>), dim3(nbh * nc, ptiles), dim3(256), 0, st,
                       (const In*)a.k, (const In*)a.v, a.z, wsS, wsN, wsG, a.T, a.chunk, nc);
    ktimer_end(a.timer, a.stream);
    const int etiles = (D * DV + D + 255) / 256;
    ktimer_begin(a.timer, "ref_sq_scan", a.stream);
    hipLaunchKernelGGL((ref_sq_scan<DK, DV>), dim3(etiles * nbh), dim3(256), 0, st,
                       wsS, wsN, (const float*)wsG, a.state_in, a.norm_in, a.state_out, a.norm_out, nc, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "ref_sq_out", a.stream);
    hipLaunchKernelGGL((ref_sq_out<DK, DV, In>), dim3(nbh * nc), dim3(a.chunk * (DV / 8)), 0, st,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.z, (const float*)wsS, (const float*)wsN,
                       (In*)a.out, a.T, a.chunk, nc, a.scale, (int)((a.flags & TWOMAMBA_FLAG_NO_NORM) != 0),
                       a.row_stat);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

size_t ref_sq_workspace(const FwdArgs& a) {
    if (a.T == 0) return 0;
    return ref_layout(a).total;
}

int ref_sq_fwd(const FwdArgs& a) {
    const size_t nbh = (size_t)a.B * a.H;
    if (nbh == 0) return TWOMAMBA_OK;
    if (a.T == 0) {
        hipStream_t st = (hipStream_t)a.stream;
        if (a.state_out) {
            const size_t D = num_pairs(a.dk);
            const size_t ns = nbh * D * a.dv, nn = nbh * D;
            if (a.state_out != a.state_in)
                hipLaunchKernelGGL(copy_or_zero, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, a.state_in, a.state_out, ns);
            if (a.norm_out != a.norm_in)
                hipLaunchKernelGGL(copy_or_zero, dim3((unsigned)((nn + 255) / 256)), dim3(256), 0, st, a.norm_in, a.norm_out, nn);
        }
        return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
    }
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
