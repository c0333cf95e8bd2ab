// Reference (plain fp32 VALU) kernels of the 2Mamba / 2Mamba-E backward pass
// ("2Mamba2Furious", App. C: gradients of the attention kernels with Q, K, V as
// inputs and the post-attention outputs as outputs; C.1: the A-mask gradient
// sums the masked matrix along the key axis and along the query axis).
//
// Per head, with G_t = softplus(z_0) + ... + softplus(z_t) (fp64), the log-mask
// of a pair s <= t is lambda_ts = G_s - G_t.  For a pair, x = scale q_t.k_s and
// dP = dout_t.v_s; with the row statistics of the query (1/den_t or the
// log-sum-exp) and D_t = dout_t.o_t:
//   2Mamba:   w = e^lambda x^2, P = w / den_t, dw = (dP - D_t) / den_t,
//             dS = 2 e^lambda x dw (the derivative by q_t.k_s / scale), M = dw w
//             (without normalisation: 1/den_t = 1 and D_t = 0);
//   2Mamba-E: P = exp(x + lambda - lse_t), dS = P (dP - D_t), M = dS;
//   first order: P = e^lambda x, dS = e^lambda dP, M = dP P (no row statistic).
// Then dv_s = sum_t P dout_t, dq_t = scale sum_s dS k_s, dk_s = scale sum_t dS q_t,
// and M (the gradient by lambda_ts) reaches g_r for s < r <= t:
//   dg_r = sum_{t >= r, s < r} M_ts = sum_{r' < r} (colsum_r' - rowsum_r'),
// rowsum_t = sum_{s<t} M_ts, colsum_s = sum_{t>s} M_ts; dz = -sigmoid(z) dg.
//
//  * bwd_prep_kernel: G and D_t (one workgroup per head; the MFMA path takes
//    only G from it and forms D_t in its query-major kernel).
//  * bwd_ref_q_kernel: one thread per query; a pass over the keys for the row
//    statistic, a second one for dq and rowsum.
//  * bwd_ref_kv_kernel: two threads per key (half of the dims each); a pass
//    over the queries t >= s for dk, dv and colsum.
//  * bwd_dz_kernel: the scan of colsum - rowsum and dz (one workgroup per 2048
//    tokens of a head).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kTile = 64;
enum { kSq = 0, kExpV = 1, kLin = 2 };   // second order, exponentiated, first order

__device__ __forceinline__ double softplus_d(float zf) {
    const double z = zf;
    return fmax(z, 0.0) + log1p(exp(-fabs(z)));
}

__device__ __forceinline__ float sigmoid_f(float x) {
    const float e = expf(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// G (running fp64 softplus sums) and, when use_d, D_t = dout_t . out_t
// (0 without normalisation).  One workgroup of kPrep threads per head.
constexpr int kPrep = 1024;
template <int DV, typename In>
__global__ void __launch_bounds__(kPrep)
bwd_prep_kernel(const float* __restrict__ z, const In* __restrict__ out, const In* __restrict__ dout,
                double* __restrict__ G, float* __restrict__ Dt, int T, int use_d, int write_d) {
    __shared__ double s_tot[kPrep];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const size_t base = (size_t)bh * T;
    const int run = (T + kPrep - 1) / kPrep;
    const int t0 = min(T, tid * run), t1 = min(T, t0 + run);
    double acc = 0.0;
    for (int t = t0; t < t1; ++t) acc += softplus_d(z[base + t]);
    s_tot[tid] = acc;
    __syncthreads();
    // exclusive scan of the kPrep run totals: within each wave by its first
    // lane, then over the wave totals
    __shared__ double s_wave[kPrep / 64];
    if ((tid & 63) == 0) {
        double r = 0.0;
        for (int i = tid; i < tid + 64; ++i) {
            const double x = s_tot[i];
            s_tot[i] = r;
            r += x;
        }
        s_wave[tid >> 6] = r;
    }
    __syncthreads();
    if (tid == 0) {
        double r = 0.0;
        for (int i = 0; i < kPrep / 64; ++i) {
            const double x = s_wave[i];
            s_wave[i] = r;
            r += x;
        }
    }
    __syncthreads();
    double g = s_tot[tid] + s_wave[tid >> 6];
    for (int t = t0; t < t1; ++t) {
        g += softplus_d(z[base + t]);
        G[base + t] = g;
    }
    if (write_d)
        for (int t = tid; t < T; t += kPrep) {
            float d = 0.f;
            if (use_d)
                for (int c = 0; c < DV; ++c)
                    d = fmaf(IO<In>::ld(dout, (base + t) * DV + c), IO<In>::ld(out, (base + t) * DV + c), d);
            Dt[base + t] = d;
        }
}

// one thread per query row
template <int D, typename In, int kVar>
__global__ void __launch_bounds__(kTile)
bwd_ref_q_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
                 const In* __restrict__ dout, const double* __restrict__ G, const float* __restrict__ Dt,
                 const float* __restrict__ fstat, float* __restrict__ stat, float* __restrict__ rowsum,
                 In* __restrict__ dq, int T, int nqt, float scale, int norm) {
    __shared__ float s_k[kTile][D], s_v[kTile][D];
    __shared__ double s_g[kTile];
    const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
    const int tid = threadIdx.x;
    const size_t base = (size_t)bh * T;
    const int t = qt * kTile + tid;
    const bool active = t < T;
    float qv[D], dov[D], dqv[D];
    double Gt = 0.0;
    float Dq = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        qv[i] = active ? IO<In>::ld(q, (base + t) * D + i) : 0.f;
        dov[i] = active ? IO<In>::ld(dout, (base + t) * D + i) : 0.f;
        dqv[i] = 0.f;
    }
    if (active) {
        Gt = G[base + t];
        Dq = Dt[base + t];
    }

    auto stage = [&](int kt) {
        const int s0 = kt * kTile, Lk = min(kTile, T - s0);
        __syncthreads();
        for (int e = tid; e < Lk * D; e += kTile) {
            s_k[e / D][e % D] = IO<In>::ld(k, (base + s0) * D + e);
            s_v[e / D][e % D] = IO<In>::ld(v, (base + s0) * D + e);
        }
        if (tid < Lk) s_g[tid] = G[base + s0 + tid];
        __syncthreads();
        return Lk;
    };

    // pass 1: row statistic (none for the first order; not needed without
    // normalisation or when the forward handed it over)
    float den = 0.f, m = -INFINITY, l = 0.f;
    const bool sweep = kVar != kLin && !fstat && !(kVar == kSq && !norm);
    for (int kt = 0; kt <= (sweep ? qt : -1); ++kt) {
        const int Lk = stage(kt);
        const int s0 = kt * kTile;
        if (!active) continue;
        for (int sl = 0; sl < Lk && s0 + sl <= t; ++sl) {
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) x = fmaf(qv[i], s_k[sl][i], x);
            x *= scale;
            const float lam = (float)(s_g[sl] - Gt);
            if (kVar == kExpV) {
                const float y = x + lam;
                const float mn = fmaxf(m, y);
                l = l * expf(m - mn) + expf(y - mn);
                m = mn;
            } else if (kVar == kSq) {
                den = fmaf(expf(lam) * x, x, den);
            }
        }
    }
    const float given = fstat && active ? fstat[base + t] : 0.f;   // lse_t or den_t from the forward
    float st;
    if (kVar == kExpV) {
        st = fstat ? given : m + logf(l);
    } else if (kVar == kSq) {
        if (fstat) den = given;
        st = norm ? (den > 0.f ? 1.f / den : 0.f) : 1.f;
    } else {
        st = 1.f;
    }

    // pass 2: dq and rowsum
    float rs = 0.f;
    for (int kt = 0; kt <= qt; ++kt) {
        const int Lk = stage(kt);
        const int s0 = kt * kTile;
        if (!active) continue;
        for (int sl = 0; sl < Lk && s0 + sl <= t; ++sl) {
            float x = 0.f, dp = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                x = fmaf(qv[i], s_k[sl][i], x);
                dp = fmaf(dov[i], s_v[sl][i], dp);
            }
            x *= scale;
            const float lam = (float)(s_g[sl] - Gt);
            float ds, Mv;
            if (kVar == kExpV) {
                const float p = expf(x + lam - st);
                ds = p * (dp - Dq);
                Mv = ds;
            } else if (kVar == kSq) {
                const float L = expf(lam);
                const float dw = (dp - Dq) * st;
                ds = 2.f * L * x * dw;
                Mv = dw * L * x * x;
            } else {
                const float L = expf(lam);
                ds = L * dp;
                Mv = dp * L * x;
            }
            if (s0 + sl < t) rs += Mv;
            const float c = scale * ds;
#pragma unroll
            for (int i = 0; i < D; ++i) dqv[i] = fmaf(c, s_k[sl][i], dqv[i]);
        }
    }
    if (active) {
#pragma unroll
        for (int i = 0; i < D; ++i) IO<In>::st(dq, (base + t) * D + i, dqv[i]);
        stat[base + t] = st;
        rowsum[base + t] = rs;
    }
}

// two threads per key: thread 2j+h holds dims [h D/2, (h+1) D/2) of key j
template <int D, typename In, int kVar>
__global__ void __launch_bounds__(2 * kTile)
bwd_ref_kv_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
                  const In* __restrict__ dout, const double* __restrict__ G, const float* __restrict__ Dt,
                  const float* __restrict__ stat, float* __restrict__ colsum, In* __restrict__ dk,
                  In* __restrict__ dv, int T, int nkt, float scale) {
    constexpr int DH = D / 2;
    __shared__ float s_q[kTile][D], s_do[kTile][D];
    __shared__ float s_st[kTile], s_D[kTile];
    __shared__ double s_g[kTile];
    const int bh = blockIdx.x / nkt, kt = blockIdx.x % nkt;
    const int tid = threadIdx.x, j = tid >> 1, h = tid & 1;
    const size_t base = (size_t)bh * T;
    const int s = kt * kTile + j;
    const bool active = s < T;
    float kv[DH], vv[DH], dkv[DH], dvv[DH];
#pragma unroll
    for (int i = 0; i < DH; ++i) {
        kv[i] = active ? IO<In>::ld(k, (base + s) * D + h * DH + i) : 0.f;
        vv[i] = active ? IO<In>::ld(v, (base + s) * D + h * DH + i) : 0.f;
        dkv[i] = dvv[i] = 0.f;
    }
    const double Gs = active ? G[base + s] : 0.0;
    float cs = 0.f;
    const int nqt = (T + kTile - 1) / kTile;
    for (int qt = kt; qt < nqt; ++qt) {
        const int t0 = qt * kTile, Lq = min(kTile, T - t0);
        __syncthreads();
        for (int e = tid; e < Lq * D; e += 2 * kTile) {
            s_q[e / D][e % D] = IO<In>::ld(q, (base + t0) * D + e);
            s_do[e / D][e % D] = IO<In>::ld(dout, (base + t0) * D + e);
        }
        if (tid < Lq) {
            s_st[tid] = stat[base + t0 + tid];
            s_D[tid] = Dt[base + t0 + tid];
            s_g[tid] = G[base + t0 + tid];
        }
        __syncthreads();
        if (!active) continue;
        for (int tl = 0; tl < Lq; ++tl) {
            if (t0 + tl < s) continue;   // the same for both threads of a key
            float xh = 0.f, dph = 0.f;
#pragma unroll
            for (int i = 0; i < DH; ++i) {
                xh = fmaf(s_q[tl][h * DH + i], kv[i], xh);
                dph = fmaf(s_do[tl][h * DH + i], vv[i], dph);
            }
            const float x = scale * (xh + __shfl_xor(xh, 1));
            const float dp = dph + __shfl_xor(dph, 1);
            const float lam = (float)(Gs - s_g[tl]);
            float p, ds, Mv;
            if (kVar == kExpV) {
                p = expf(x + lam - s_st[tl]);
                ds = p * (dp - s_D[tl]);
                Mv = ds;
            } else if (kVar == kSq) {
                const float L = expf(lam);
                const float w = L * x * x;
                p = w * s_st[tl];
                const float dw = (dp - s_D[tl]) * s_st[tl];
                ds = 2.f * L * x * dw;
                Mv = dw * w;
            } else {
                const float L = expf(lam);
                p = L * x;
                ds = L * dp;
                Mv = dp * p;
            }
            if (t0 + tl > s) cs += Mv;
            const float c = scale * ds;
#pragma unroll
            for (int i = 0; i < DH; ++i) {
                dvv[i] = fmaf(p, s_do[tl][h * DH + i], dvv[i]);
                dkv[i] = fmaf(c, s_q[tl][h * DH + i], dkv[i]);
            }
        }
    }
    if (active) {
#pragma unroll
        for (int i = 0; i < DH; ++i) {
            IO<In>::st(dk, (base + s) * D + h * DH + i, dkv[i]);
            IO<In>::st(dv, (base + s) * D + h * DH + i, dvv[i]);
        }
        if (h == 0) colsum[base + s] = cs;
    }
}

}  // namespace

// dz from the row and column sums: exclusive fp64 prefix of colsum - rowsum.
// A workgroup takes 2048 consecutive tokens of a head (8 per thread): it sums every
// earlier token of the head itself (coalesced reads, which the workgroups of a head
// share through L2), scans its own block, and writes dz.  No workgroup waits on
// another, and every sum is taken in a fixed order, so the result is deterministic.
constexpr int kDzThreads = 256, kDzPer = 8, kDzBlock = kDzThreads * kDzPer;

__global__ void __launch_bounds__(kDzThreads)
bwd_dz_kernel(const float* __restrict__ z, const float* __restrict__ rowsum, const float* __restrict__ colsum,
              float* __restrict__ dz, int T, int nblk) {
    __shared__ double s_pre[kDzThreads], s_run[kDzThreads];
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk, tid = threadIdx.x;
    const size_t base = (size_t)bh * T;
    const int b0 = blk * kDzBlock;
    double pre = 0.0;   // this thread's share of the tokens before the block
#pragma unroll 4
    for (int t = tid; t < b0; t += kDzThreads) pre += (double)colsum[base + t] - (double)rowsum[base + t];
    const int t0 = b0 + kDzPer * tid;
    double x[kDzPer], run = 0.0;
#pragma unroll
    for (int i = 0; i < kDzPer; ++i) {
        const int t = t0 + i;
        x[i] = t < T ? (double)colsum[base + t] - (double)rowsum[base + t] : 0.0;
        run += x[i];
    }
    s_pre[tid] = pre;
    s_run[tid] = run;
    __syncthreads();
    // total of the earlier tokens (tree, fixed order) and the inclusive scan of the
    // threads' runs (Hillis-Steele)
    for (int off = kDzThreads / 2; off > 0; off >>= 1) {
        if (tid < off) s_pre[tid] += s_pre[tid + off];
        __syncthreads();
    }
    for (int off = 1; off < kDzThreads; off <<= 1) {
        const double y = tid >= off ? s_run[tid - off] : 0.0;
        __syncthreads();
        s_run[tid] += y;
        __syncthreads();
    }
    double c = s_pre[0] + (s_run[tid] - run);   // sum over every token before t0
#pragma unroll
    for (int i = 0; i < kDzPer; ++i) {
        const int t = t0 + i;
        if (t < T) dz[base + t] = -sigmoid_f(z[base + t]) * (float)c;
        c += x[i];
    }
}

size_t bwd_workspace(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T;
    return align256(n * sizeof(double)) + 4 * align256(n * sizeof(float));
}

BwdScratch bwd_scratch(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T;
    char* p = (char*)a.ws;
    BwdScratch s;
    s.G = (double*)p;
    p += align256(n * sizeof(double));
    s.stat = (float*)p;
    p += align256(n * sizeof(float));
    s.Dt = (float*)p;
    p += align256(n * sizeof(float));
    s.rowsum = (float*)p;
    p += align256(n * sizeof(float));
    s.colsum = (float*)p;
    return s;
}

template <int D, typename In>
static int launch_prep(const BwdArgs& a, const BwdScratch& s, bool with_d) {
    hipStream_t st = (hipStream_t)a.stream;
    const int use_d = (a.variant == TWOMAMBA_EXP) ||
                      (a.variant == TWOMAMBA_SQ && !(a.flags & TWOMAMBA_FLAG_NO_NORM));
    ktimer_begin(a.timer, "bwd_prep", a.stream);
    hipLaunchKernelGGL((bwd_prep_kernel<D, In>), dim3(a.B * a.H), dim3(kPrep), 0, st, a.z, (const In*)a.out,
                       (const In*)a.dout, s.G, s.Dt, a.T, use_d, (int)with_d);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

int bwd_prep_launch(const BwdArgs& a, const BwdScratch& s, bool with_d) {
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dv == 64) return bf ? launch_prep<64, bf16>(a, s, with_d) : launch_prep<64, float>(a, s, with_d);
    return bf ? launch_prep<16, bf16>(a, s, with_d) : launch_prep<16, float>(a, s, with_d);
}

int bwd_dz_launch(const BwdArgs& a, const BwdScratch& s) {
    ktimer_begin(a.timer, "bwd_dz", a.stream);
    const int nblk = (a.T + kDzBlock - 1) / kDzBlock;
    if ((size_t)a.B * a.H * nblk == 0) {
        ktimer_end(a.timer, a.stream);
        return TWOMAMBA_OK;
    }
    hipLaunchKernelGGL(bwd_dz_kernel, dim3((unsigned)(a.B * a.H * nblk)), dim3(kDzThreads), 0, (hipStream_t)a.stream,
                       a.z, s.rowsum, s.colsum, a.gz, a.T, nblk);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

template <int D, typename In, int kVar>
static int launch_ref(const BwdArgs& a, const BwdScratch& s) {
    hipStream_t st = (hipStream_t)a.stream;
    const int nt = (a.T + kTile - 1) / kTile;
    const int norm = !(a.flags & TWOMAMBA_FLAG_NO_NORM);
    ktimer_begin(a.timer, "ref_bwd_q", a.stream);
    hipLaunchKernelGGL((bwd_ref_q_kernel<D, In, kVar>), dim3(a.B * a.H * nt), dim3(kTile), 0, st, (const In*)a.q,
                       (const In*)a.k, (const In*)a.v, (const In*)a.dout, s.G, s.Dt, a.row_stat, s.stat, s.rowsum,
                       (In*)a.gq, a.T, nt, a.scale, norm);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "ref_bwd_kv", a.stream);
    hipLaunchKernelGGL((bwd_ref_kv_kernel<D, In, kVar>), dim3(a.B * a.H * nt), dim3(2 * kTile), 0, st,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, (const In*)a.dout, s.G, s.Dt, s.stat,
                       s.colsum, (In*)a.gk, (In*)a.gv, a.T, nt, a.scale);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

int ref_bwd(const BwdArgs& a) {
    if ((size_t)a.B * a.H * a.T == 0) return TWOMAMBA_OK;
    const BwdScratch s = bwd_scratch(a);
    int r = bwd_prep_launch(a, s, true);
    if (r != TWOMAMBA_OK) return r;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    const int var = a.variant == TWOMAMBA_EXP ? kExpV : a.variant == TWOMAMBA_LIN ? kLin : kSq;
    auto pick = [&](auto d_tag, auto in_tag) {
        constexpr int DD = decltype(d_tag)::value;
        using In = decltype(in_tag);
        return var == kExpV ? launch_ref<DD, In, kExpV>(a, s)
                            : var == kLin ? launch_ref<DD, In, kLin>(a, s) : launch_ref<DD, In, kSq>(a, s);
    };
    if (a.dk == 64) r = bf ? pick(std::integral_constant<int, 64>{}, bf16{}) : pick(std::integral_constant<int, 64>{}, 0.f);
    else r = bf ? pick(std::integral_constant<int, 16>{}, bf16{}) : pick(std::integral_constant<int, 16>{}, 0.f);
    if (r != TWOMAMBA_OK) return r;
    return bwd_dz_launch(a, s);
}

}  // namespace twm
