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
// by the traffic of q, k, v, out and the per-chunk states.  That three-pass form
// serves fp32 and d = 16; bf16 at d = 64 runs a segmented single pass on
// 16x16x32 MFMAs instead (see below), which reads k and v twice and q once and
// keeps the states of whole segments, not of chunks.
#include <algorithm>

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

// ---------------------------------------------------------------------------
// MFMA kernels for bf16 inputs at d = 64
using namespace tiles;

// ---------------------------------------------------------------------------
// Segmented single pass (bf16, d = 64): the sequence of a head is cut into
// segments of whole chunks.  lin_seg_mfma forms every segment's own end state
// (weights relative to the segment end), lin_scan over segments turns them into
// the carry entering each segment (and the final state), and lin_main_mfma walks
// a segment's chunks with the state in MFMA accumulators: per chunk the
// intra-chunk scores, the readout of the carried state and the state update.
// HBM traffic is then q, k, v, out plus one k, v read and small per-segment states.

// B operand of Q for the K-slot order of tr_op: dims {16 dtt + 4g .. +3, 16 dtt + 16 + 4g .. +3} of row t
__device__ __forceinline__ b8 q_tr_order(const Tile& t, int row, int dtt, int g) {
    const uint2 a = *reinterpret_cast<const uint2*>(&t.X[row][16 * dtt + 4 * g]);
    const uint2 b = *reinterpret_cast<const uint2*>(&t.X[row][16 * dtt + 16 + 4 * g]);
    return as_b8(make_uint4(a.x, a.y, b.x, b.y));
}

// chunk-local inclusive prefix of g (log2 units) over the 64 lanes of one wave
__device__ __forceinline__ float chunk_prefix(const float* z, int lane, int Lc) {
    float incl = lane < Lc ? decay_log(z[lane]) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    return incl * kLog2e;
}

// V rows scaled by w_t = 2^(s_w[t]) into a tile
__device__ __forceinline__ void store_scaled(const Stage& st, Tile& t, const float* s_w, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, cc = e & 7;
        const uint32_t x[4] = {st.c[n].x, st.c[n].y, st.c[n].z, st.c[n].w};
        const float ww = fexp2(s_w[r]);
        uint32_t y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            y[i] = pack2(__uint_as_float(x[i] << 16) * ww, __uint_as_float(x[i] & 0xffff0000u) * ww);
        *reinterpret_cast<uint4*>(&t.X[r][8 * cc]) = make_uint4(y[0], y[1], y[2], y[3]);
    }
}

// segment end states S_g^T[c][d] (transposed), weights relative to the segment end
__global__ void __launch_bounds__(kThreads)
lin_seg_mfma(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ z,
             float* __restrict__ wsS, float* __restrict__ wsG, int T, int nseg, int seg_chunks) {
    __shared__ __attribute__((aligned(16))) Tile sK, sV;
    __shared__ float s_w[kTile];
    const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const int nc = (T + kTile - 1) / kTile;
    const int c0 = seg * seg_chunks, c1 = min(nc, c0 + seg_chunks);
    const size_t base = (size_t)bh * T;
    f4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float later = 0.f;   // log2 decay from the end of the current chunk to the segment end
    Stage sk, sv;
    {
        const int t0 = (c1 - 1) * kTile;
        fetch(sk, k + (base + t0) * kD, min(kTile, T - t0), tid);
        fetch(sv, v + (base + t0) * kD, min(kTile, T - t0), tid);
    }
    for (int c = c1 - 1; c >= c0; --c) {   // from the segment end backwards
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        if (w == 0) {
            const float incl = chunk_prefix(z + base + t0, lane, Lc);
            const float total = __shfl(incl, 63);
            s_w[lane] = total - incl + later;      // log2 w_t relative to the segment end
            later += total;   // kept by wave 0, which also writes the segment's decay
        }
        __syncthreads();
        store(sk, sK, tid);
        store_scaled(sv, sV, s_w, tid);
        __syncthreads();
        if (c > c0) {
            const int tn = t0 - kTile;
            fetch(sk, k + (base + tn) * kD, kTile, tid);
            fetch(sv, v + (base + tn) * kD, kTile, tid);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const b8 A = tr_op(sV, w, 2 * h, lane);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(A, tr_op(sK, dt, 2 * h, lane), acc[dt]);
        }
        __syncthreads();
    }
    float* dst = wsS + ((size_t)bh * nseg + seg) * kD * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * kD + 16 * dt + col] = acc[dt][i];
    if (tid == 0) wsG[(size_t)bh * nseg + seg] = later / kLog2e;
}

// one segment of one head: carried state in accumulators (wave w: value rows
// 16w..16w+15 of S^T), per chunk intra-chunk scores + readout + update
__global__ void __launch_bounds__(kThreads)
lin_main_mfma(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
              const float* __restrict__ z, const float* __restrict__ carry, bf16* __restrict__ out, int T, int nseg,
              int seg_chunks, float scale) {
    __shared__ __attribute__((aligned(16))) Tile sQ, sK, sV, sW, sS;
    __shared__ float s_gl[kTile], s_w[kTile];
    const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const int nc = (T + kTile - 1) / kTile;
    const int c0 = seg * seg_chunks, c1 = min(nc, c0 + seg_chunks);
    const size_t base = (size_t)bh * T;
    // carry S^T[c][d] into the accumulator layout: rows 16w + 4g + i, column 16 dt + col
    f4 S[4];
    {
        const float* src = carry + ((size_t)bh * nseg + seg) * kD * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[dt][i] = src[(16 * w + 4 * g + i) * kD + 16 * dt + col];
    }
    Stage sq, sk, sv;
    {
        const int t0 = c0 * kTile, Lc = min(kTile, T - t0);
        fetch(sq, q + (base + t0) * kD, Lc, tid);
        fetch(sk, k + (base + t0) * kD, Lc, tid);
        fetch(sv, v + (base + t0) * kD, Lc, tid);
    }
    for (int c = c0; c < c1; ++c) {
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        if (w == 0) {
            const float incl = chunk_prefix(z + base + t0, lane, Lc);
            const float total = __shfl(incl, 63);
            s_gl[lane] = incl;
            s_w[lane] = total - incl;              // log2 of w_t = exp(Gam - Gl_t)
        }
        // the state before this chunk, bf16, as S[d][c] rows (4 consecutive c per lane)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            uint2 o;
            o.x = pack2(S[dt][0], S[dt][1]);
            o.y = pack2(S[dt][2], S[dt][3]);
            *reinterpret_cast<uint2*>(&sS.X[16 * dt + col][16 * w + 4 * g]) = o;
        }
        store(sq, sQ, tid);
        store(sk, sK, tid);
        __syncthreads();
        store_scaled(sv, sW, s_w, tid);
        store(sv, sV, tid);
        __syncthreads();
        if (c + 1 < c1) {
            const int tn = t0 + kTile, Ln = min(kTile, T - tn);
            fetch(sq, q + (base + tn) * kD, Ln, tid);
            fetch(sk, k + (base + tn) * kD, Ln, tid);
            fetch(sv, v + (base + tn) * kD, Ln, tid);
        }
        // this wave's queries 16w .. 16w + 15, one per lane column
        const int tl = 16 * w + col;
        const float glt = s_gl[tl];
        const b8 Qb[2] = {row_op(sQ, tl, g, 0), row_op(sQ, tl, g, 1)};
        f4 O[4], OI[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            O[ct] = f4{0.f, 0.f, 0.f, 0.f};
            OI[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dtt = 0; dtt < 2; ++dtt)
                OI[ct] = mfma(tr_op(sS, ct, 2 * dtt, lane), q_tr_order(sQ, tl, 2 * dtt, g), OI[ct]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float p[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int st = 2 * h + u, r = 16 * st + col;
                f4 X = mfma(row_op(sK, r, g, 0), Qb[0], f4{0.f, 0.f, 0.f, 0.f});
                X = mfma(row_op(sK, r, g, 1), Qb[1], X);
                const float4 g4 = *reinterpret_cast<const float4*>(&s_gl[16 * st + 4 * g]);
                const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sl = 16 * st + 4 * g + i;
                    p[4 * u + i] = sl <= tl ? scale * fexp2(glt - gs[i]) * X[i] : 0.f;
                }
            }
            const b8 B = to_b(p);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) O[ct] = mfma(tr_op(sV, ct, 2 * h, lane), B, O[ct]);
        }
        if (tl < Lc) {
            const float dec = scale * fexp2(glt);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                uint2 o;
                o.x = pack2(fmaf(dec, OI[ct][0], O[ct][0]), fmaf(dec, OI[ct][1], O[ct][1]));
                o.y = pack2(fmaf(dec, OI[ct][2], O[ct][2]), fmaf(dec, OI[ct][3], O[ct][3]));
                *reinterpret_cast<uint2*>(out + (base + t0 + tl) * kD + 16 * ct + 4 * g) = o;
            }
        }
        // update: S^T = exp(Gam) S^T + (w V)^T K
        const float eg = fexp2(s_gl[63]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) S[dt] *= eg;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const b8 A = tr_op(sW, w, 2 * h, lane);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) S[dt] = mfma(A, tr_op(sK, dt, 2 * h, lane), S[dt]);
        }
        __syncthreads();
    }
}

int run_fused(const FwdArgs& a) {
    const int nc = (a.T + kTile - 1) / kTile;
    const int nbh = a.B * a.H;
    // segments: about two workgroups per CU, at least two chunks each
    int want = std::max(1, (512 + nbh - 1) / nbh);
    want = std::min(want, std::max(1, nc / 2));
    const int sc = (nc + want - 1) / want;
    const int nseg = (nc + sc - 1) / sc;
    const LinLayout L = lin_layout(a);   // per-chunk slots; nseg <= nc of them are used
    float* wsS = (float*)((char*)a.ws + L.off_S);
    float* wsG = (float*)((char*)a.ws + L.off_G);
    hipStream_t st = (hipStream_t)a.stream;
    ktimer_begin(a.timer, "lin_seg", a.stream);
    hipLaunchKernelGGL(lin_seg_mfma, dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.k, (const bf16*)a.v, a.z,
                       wsS, wsG, a.T, nseg, sc);
    ktimer_end(a.timer, a.stream);
    const int etiles = (kD * kD + 255) / 256;
    ktimer_begin(a.timer, "lin_scan", a.stream);
    hipLaunchKernelGGL((lin_scan<kD, kD, true>), dim3(nbh * etiles), dim3(256), 0, st, wsS, (const float*)wsG,
                       a.state_in, a.state_out, nseg, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "lin_main", a.stream);
    hipLaunchKernelGGL(lin_main_mfma, dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, a.z, (const float*)wsS, (bf16*)a.out, a.T, nseg, sc, a.scale);
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
    if (bf && a.dk == 64 && !(a.flags & TWOMAMBA_FLAG_REFERENCE_KERNELS)) return run_fused(a);
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
