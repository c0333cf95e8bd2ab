// Reference (plain fp32 VALU) kernel of the 2Mamba-E forward ("2Mamba2Furious",
// §6: the QK product exponentiated, i.e. softmax attention whose logits carry
// the softplus A-mask as an additive log-bias).
//
// One workgroup per (b, h, 64-query tile); each thread keeps an online softmax
// (running max, sum, weighted values) for one query row and 8 value columns.
// Key tiles are visited from the diagonal backwards so that the log-decay
// between a key s and a query t,
//     lambda_ts = B_s + M + A_t,
// is assembled from stretch sums that never span more than what separates the
// two tiles: A_t sums g over the query tile up to t, B_s over the key tile after
// s, and M over the whole tiles in between (accumulated tile by tile).
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

constexpr int kQT = 64;   // query rows per workgroup
constexpr int kKT = 64;   // keys per LDS tile

template <int DK, int DV, typename In>
__global__ void __launch_bounds__(512)
ref_exp_kernel(const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
               const float* __restrict__ z, In* __restrict__ out, int T, int nqt, float scale,
               float* __restrict__ row_stat) {
    constexpr int CGN = DV / 8;
    __shared__ float s_q[kQT][DK];
    __shared__ float s_k[kKT][DK], s_v[kKT][DV];
    __shared__ float s_A[kQT], s_B[kKT];
    __shared__ float s_tot;

    const int bh = blockIdx.x / nqt;
    const int qt = blockIdx.x % nqt;
    const int t0 = qt * kQT;
    const int Lq = min(kQT, T - t0);
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const size_t base = (size_t)bh * T;

    for (int e = tid; e < Lq * DK; e += nthr) s_q[e / DK][e % DK] = IO<In>::ld(q, (base + t0) * DK + e) * scale;
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < Lq; ++t) {
            acc += decay_log(z[base + t0 + t]);
            s_A[t] = acc;
        }
    }

    const int tl = tid / CGN, cg = tid % CGN;
    const bool active = tl < Lq;
    float m = -INFINITY, l = 0.f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float M = 0.f;

    for (int kt = qt; kt >= 0; --kt) {
        const int s0 = kt * kKT;
        const int Lk = min(kKT, T - s0);
        __syncthreads();
        for (int e = tid; e < Lk * DK; e += nthr) s_k[e / DK][e % DK] = IO<In>::ld(k, (base + s0) * DK + e);
        for (int e = tid; e < Lk * DV; e += nthr) s_v[e / DV][e % DV] = IO<In>::ld(v, (base + s0) * DV + e);
        if (tid == 0 && kt != qt) {
            float R = 0.f;   // g summed over key-tile tokens after s
            for (int s = Lk - 1; s >= 0; --s) {
                s_B[s] = R;
                R += decay_log(z[base + s0 + s]);
            }
            s_tot = R;
        }
        __syncthreads();
        if (active) {
            const int send = (kt == qt) ? tl + 1 : Lk;
            for (int s = 0; s < send; ++s) {
                float x = 0.f;
#pragma unroll 8
                for (int i = 0; i < DK; ++i) x = fmaf(s_q[tl][i], s_k[s][i], x);
                x += (kt == qt) ? (s_A[tl] - s_A[s]) : (s_B[s] + M + s_A[tl]);
                if (x == -INFINITY) continue;
                const float mn = fmaxf(m, x);
                const float alpha = expf(m - mn);
                const float p = expf(x - mn);
                l = fmaf(l, alpha, p);
#pragma unroll
                for (int u = 0; u < 8; ++u) acc[u] = fmaf(acc[u], alpha, p * s_v[s][cg * 8 + u]);
                m = mn;
            }
        }
        if (kt != qt) M += s_tot;
    }
    if (!active) return;
    if (row_stat && cg == 0) row_stat[base + t0 + tl] = m + logf(l);   // logits carry their true bias
    const float inv = 1.f / l;
#pragma unroll
    for (int u = 0; u < 8; ++u) IO<In>::st(out, (base + t0 + tl) * DV + cg * 8 + u, acc[u] * inv);
}

template <int DK, int DV, typename In>
int run(const FwdArgs& a) {
    const int nqt = (a.T + kQT - 1) / kQT;
    const int nbh = a.B * a.H;
    ktimer_begin(a.timer, "ref_exp", a.stream);
    hipLaunchKernelGGL((ref_exp_kernel<DK, DV, In>), dim3(nbh * nqt), dim3(kQT * (DV / 8)), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, (const In*)a.v, a.z, (In*)a.out,
                       a.T, nqt, a.scale, a.row_stat);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

int ref_exp_fwd(const FwdArgs& a) {
    if ((size_t)a.B * a.H == 0 || a.T == 0) return TWOMAMBA_OK;
    const bool bf = a.dtype == TWOMAMBA_BF16;
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
