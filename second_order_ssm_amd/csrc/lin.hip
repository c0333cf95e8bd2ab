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
// by the traffic of q, k, v, out and the per-chunk states.  bf16 at d = 64 runs
// 16x16x32 MFMA versions of the delta and output kernels (per-chunk states then
// stored transposed, [dv][dk]); everything else runs the fp32 VALU kernels.
#include "device_common.h"
#include "internal.h"
#include "mfma_tiles.h"

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

// exclusive scan over chunks, one thread per state element.  kT: the
// per-chunk states are stored transposed ([dv][dk], the MFMA kernels' layout),
// while state_in / state_out keep the ABI's [dk][dv].
template <int DK, int DV, bool kT>
__global__ void __launch_bounds__(256)
lin_scan(float* __restrict__ wsS, const float* __restrict__ wsG, const float* state_in, float* state_out, int nc,
         int etiles) {
    const int bh = blockIdx.x / etiles;
    const int e = (blockIdx.x % etiles) * 256 + threadIdx.x;
    if (e >= DK * DV) return;
    const int ea = kT ? (e % DK) * DV + e / DK : e;   // the same element in the ABI layout
    float run = state_in ? state_in[(size_t)bh * DK * DV + ea] : 0.f;
    float* base = wsS + (size_t)bh * nc * DK * DV + e;
    const float* gb = wsG + (size_t)bh * nc;
    // the chain is serial in c: load eight chunks' deltas and decays ahead of it
    constexpr int U = 8;
    int c = 0;
    for (; c + U <= nc; c += U) {
        float x[U], a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x[u] = base[(size_t)(c + u) * DK * DV];
            a[u] = gb[c + u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            base[(size_t)(c + u) * DK * DV] = run;
            run = fmaf(expf(a[u]), run, x[u]);
        }
    }
    for (; c < nc; ++c) {
        const float x = base[(size_t)c * DK * DV];
        base[(size_t)c * DK * DV] = run;
        run = fmaf(expf(gb[c]), run, x);
    }
    if (state_out) state_out[(size_t)bh * DK * DV + ea] = run;
}

// ---------------------------------------------------------------------------
// MFMA kernels for bf16 inputs at d = 64 (one workgroup of 4 waves per chunk)
using namespace tiles;

// dS_c^T[c][d] = sum_t (w V)^T[c][t] K[t][d], w_t = exp(Gam_c - Gl_t): both
// operands come from transposing reads of the row-major tiles; wave w forms the
// value rows 16w .. 16w + 15.
__global__ void __launch_bounds__(kThreads)
lin_delta_mfma(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ z,
               float* __restrict__ wsS, float* __restrict__ wsG, int T, int nc) {
    __shared__ __attribute__((aligned(16))) Tile sK, sV;
    __shared__ float s_w[kTile];
    const int bh = blockIdx.x / nc, c = blockIdx.x % nc;
    const int t0 = c * kTile, Lc = min(kTile, T - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const size_t tok0 = (size_t)bh * T + t0;
    Stage st;
    fetch(st, k + tok0 * kD, Lc, tid);
    store(st, sK, tid);
    if (w == 0) {   // w_t from the chunk-local suffix sums of g (a wave-wide scan)
        const float gv = lane < Lc ? decay_log(z[tok0 + lane]) : 0.f;
        float incl = gv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const float total = __shfl(incl, 63);
        s_w[lane] = expf(total - incl);
        if (lane == 0) wsG[(size_t)bh * nc + c] = total;
    }
    fetch(st, v + tok0 * kD, Lc, tid);
    __syncthreads();
    // V rows scaled by w_t on the way into LDS
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, cc = e & 7;
        const uint32_t x[4] = {st.c[n].x, st.c[n].y, st.c[n].z, st.c[n].w};
        const float ww = s_w[r];
        uint32_t y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            y[i] = pack2(__uint_as_float(x[i] << 16) * ww, __uint_as_float(x[i] & 0xffff0000u) * ww);
        *reinterpret_cast<uint4*>(&sV.X[r][8 * cc]) = make_uint4(y[0], y[1], y[2], y[3]);
    }
    __syncthreads();
    f4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const b8 A = tr_op(sV, w, 2 * h, lane);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(A, tr_op(sK, dt, 2 * h, lane), acc[dt]);
    }
    float* dst = wsS + ((size_t)bh * nc + c) * kD * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * kD + 16 * dt + col] = acc[dt][i];
}

// o_t = sum_{s<=t in c} exp(Gl_t - Gl_s) (scale q_t.k_s) v_s + exp(Gl_t) scale q_t.S_c.
// Wave w owns queries 16w .. 16w + 15, one per lane column: S^T = K Q^T, the
// masked weights P^T as the B operand of O^T = V^T P^T, and the carried state
// as the A operand of O^T += S_c^T Q^T (S_c rounded to bf16 for the product).
__global__ void __launch_bounds__(kThreads)
lin_out_mfma(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
             const float* __restrict__ z, const float* __restrict__ wsS, bf16* __restrict__ out, int T, int nc,
             float scale) {
    __shared__ __attribute__((aligned(16))) Tile sK, sV;
    __shared__ float s_gl[kTile];
    const int bh = blockIdx.x / nc, c = blockIdx.x % nc;
    const int t0 = c * kTile, Lc = min(kTile, T - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const size_t tok0 = (size_t)bh * T + t0;
    const int tl = 16 * w + col;                   // this lane's query within the chunk
    const bool tv = tl < Lc;
    const bf16* qrow = q + (tok0 + (tv ? tl : 0)) * kD;
    const b8 Qb[2] = {own_op(qrow, g, 0), own_op(qrow, g, 1)};
    Stage sk, sv;
    fetch(sk, k + tok0 * kD, Lc, tid);
    fetch(sv, v + tok0 * kD, Lc, tid);
    if (w == 0) {
        const float gv = lane < Lc ? decay_log(z[tok0 + lane]) : 0.f;
        float incl = gv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        s_gl[lane] = incl * kLog2e;
    }
    store(sk, sK, tid);
    store(sv, sV, tid);
    // carried state S_c^T rows as A operands (fp32 -> bf16), loaded while LDS fills
    const float* Sc = wsS + ((size_t)bh * nc + c) * kD * kD;
    b8 SA[4][2];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float* r = Sc + (16 * ct + col) * kD + 8 * g + 32 * kk;
            const float4 a = *reinterpret_cast<const float4*>(r), b = *reinterpret_cast<const float4*>(r + 4);
            SA[ct][kk] = as_b8(make_uint4(pack2(a.x, a.y), pack2(a.z, a.w), pack2(b.x, b.y), pack2(b.z, b.w)));
        }
    __syncthreads();
    const float glt = s_gl[tv ? tl : 0];
    f4 O[4], OI[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        O[ct] = f4{0.f, 0.f, 0.f, 0.f};
        OI[ct] = mfma(SA[ct][1], Qb[1], mfma(SA[ct][0], Qb[0], f4{0.f, 0.f, 0.f, 0.f}));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int st = 2 * h + u, r = 16 * st + col;
            f4 S = mfma(row_op(sK, r, g, 0), Qb[0], f4{0.f, 0.f, 0.f, 0.f});
            S = mfma(row_op(sK, r, g, 1), Qb[1], S);
            const float4 g4 = *reinterpret_cast<const float4*>(&s_gl[16 * st + 4 * g]);
            const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 16 * st + 4 * g + i;
                p[4 * u + i] = sl <= tl ? scale * fexp2(glt - gs[i]) * S[i] : 0.f;
            }
        }
        const b8 B = to_b(p);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) O[ct] = mfma(tr_op(sV, ct, 2 * h, lane), B, O[ct]);
    }
    if (!tv) return;
    const float dec = scale * fexp2(glt);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        uint2 o;
        o.x = pack2(fmaf(dec, OI[ct][0], O[ct][0]), fmaf(dec, OI[ct][1], O[ct][1]));
        o.y = pack2(fmaf(dec, OI[ct][2], O[ct][2]), fmaf(dec, OI[ct][3], O[ct][3]));
        *reinterpret_cast<uint2*>(out + (tok0 + tl) * kD + 16 * ct + 4 * g) = o;
    }
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
    hipLaunchKernelGGL((lin_scan<DK, DV, false>), dim3(nbh * etiles), dim3(256), 0, st, wsS, (const float*)wsG,
                       a.state_in, a.state_out, nc, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "lin_out", a.stream);
    hipLaunchKernelGGL((lin_out<DK, DV, In>), dim3(nbh * nc), dim3(kLinChunk * DV / 8), 0, st, (const In*)a.q,
                       (const In*)a.k, (const In*)a.v, a.z, (const float*)wsS, (In*)a.out, a.T, nc, a.scale);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

int run_mfma(const FwdArgs& a) {
    const LinLayout L = lin_layout(a);
    const int nc = (a.T + kTile - 1) / kTile;
    const int nbh = a.B * a.H;
    float* wsS = (float*)((char*)a.ws + L.off_S);
    float* wsG = (float*)((char*)a.ws + L.off_G);
    hipStream_t st = (hipStream_t)a.stream;
    ktimer_begin(a.timer, "lin_delta", a.stream);
    hipLaunchKernelGGL(lin_delta_mfma, dim3(nbh * nc), dim3(kThreads), 0, st, (const bf16*)a.k, (const bf16*)a.v,
                       a.z, wsS, wsG, a.T, nc);
    ktimer_end(a.timer, a.stream);
    const int etiles = (kD * kD + 255) / 256;
    ktimer_begin(a.timer, "lin_scan", a.stream);
    hipLaunchKernelGGL((lin_scan<kD, kD, true>), dim3(nbh * etiles), dim3(256), 0, st, wsS, (const float*)wsG,
                       a.state_in, a.state_out, nc, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "lin_out", a.stream);
    hipLaunchKernelGGL(lin_out_mfma, dim3(nbh * nc), dim3(kThreads), 0, st, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, a.z, (const float*)wsS, (bf16*)a.out, a.T, nc, a.scale);
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
    if (bf && a.dk == 64 && !(a.flags & TWOMAMBA_FLAG_REFERENCE_KERNELS)) return run_mfma(a);
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
