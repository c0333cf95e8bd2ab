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
#include <string.h>

#include <algorithm>

#include "conv_common.h"
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
    // the chain is serial in c: load sixteen chunks' (segments') deltas and decays ahead of it
    constexpr int U = 16;
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

// Reverse-time mode (the first-order backward): the kernels walk the sequence
// back to front.  Logical position tau is the stored row T-1-tau, and the decay
// between logical positions takes the logit of the token one step later in
// stored order, so that a logical prefix sum over (s, t] equals the stored sum
// over [T-1-t, T-1-s): logical tau takes z_{T-tau}, and tau = 0 no decay at all.
__device__ __forceinline__ int stored_row(int tau, int T, bool rev) { return rev ? T - 1 - tau : tau; }


// Per-head buffer resources: an access past `bytes` (or at a negative offset, which
// wraps past it) loads zeros or stores nothing, so that ragged chunks need no branch
// around a memory instruction.  Without such branches the compiler knows how many
// loads and stores are in flight at every wait and waits for exactly the ones it
// needs, instead of for all of them (the previous chunk's output stores included).
// A head's rows are addressable this way while T * 128 bytes < 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 x) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, x), r,
                                          off, 0, 0);
}
__device__ __forceinline__ void buf_st4f(__amdgpu_buffer_rsrc_t r, uint32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, off, 0, 0);
}
// an offset past every resource (they hold < 2^31 bytes), also after the few hundred
// bytes a caller may add to it
constexpr uint32_t kNoAccess = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rows(const bf16* head, int T) {
    return buf_rsrc(head, (uint32_t)T * kD * 2);
}

// rows t0 .. t0 + 63 (logical) of a head's tensor in the Stage layout (zeros past T).
// Not `live`: the same loads at an offset past the buffer (zeros, no memory access), so
// that every path through a chunk loop issues the same loads and the compiler can size
// its waits for the one buffer a chunk consumes.
__device__ __forceinline__ void fetch_rows(Stage& s, __amdgpu_buffer_rsrc_t head, int t0, int T, bool rev, int tid,
                                           bool live) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, c = e & 7;
        s.c[n] = buf_ld16(head, live ? (uint32_t)(stored_row(t0 + r, T, rev) * kD + 8 * c) * 2 : kNoAccess);
    }
}

// The logit z behind g of logical token t0 + lane, loaded a chunk ahead (0 where the
// token has no decay: past the chunk's last token, and logical 0 in reverse mode);
// softplus is applied only when the chunk is processed, so that the load stays in
// flight meanwhile.
__device__ __forceinline__ bool lane_has_decay(int t0, int rev, int lane, int Lc) {
    return lane < Lc && !(rev && t0 + lane == 0);
}
__device__ __forceinline__ float lane_z(__amdgpu_buffer_rsrc_t zhead, int t0, int T, bool rev, int lane, int Lc) {
    const int i = rev ? T - (t0 + lane) : t0 + lane;
    return buf_ld4f(zhead, lane_has_decay(t0, rev, lane, Lc) ? (uint32_t)i * 4 : kNoAccess);
}
__device__ __forceinline__ float lane_decay(float zraw, int t0, bool rev, int lane, int Lc) {
    return lane_has_decay(t0, rev, lane, Lc) ? decay_log(zraw) : 0.f;
}

// chunk-local inclusive prefix of g (log2 units) over the 64 lanes of one wave,
// from each lane's own g
__device__ __forceinline__ float chunk_prefix_of(float incl) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(incl, o);
        if ((int)(threadIdx.x & 63) >= o) incl += y;
    }
    return incl * kLog2e;
}

// Input convolution on the staged rows (twomamba_fwd_conv): the raw rows of a
// chunk and the raw rows one token earlier (the cached row, or zeros, before
// t = 0), convolved just before the tile is written to LDS, with the same
// arithmetic as the standalone pass.  Weights and bias of the three tensors sit
// in LDS as ConvLds: [tensor][w0 | w1 | b][channel].
struct ConvLds {
    float x[3][3][kD];
};

__device__ __forceinline__ void conv_lds_fill(ConvLds& c, const float* w, const float* b, int h, int H, int tid) {
    for (int e = tid; e < 3 * kD; e += kThreads) {
        const int tensor = e / kD, ch = e % kD;
        const size_t o = (size_t)(tensor * H + h) * kD + ch;
        c.x[tensor][0][ch] = w[2 * o];
        c.x[tensor][1][ch] = w[2 * o + 1];
        c.x[tensor][2][ch] = b ? b[o] : 0.f;
    }
}

__device__ __forceinline__ Conv8 conv_lds_get(const ConvLds& c, int tensor, int ch0) {
    Conv8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        r.w0[i] = c.x[tensor][0][ch0 + i];
        r.w1[i] = c.x[tensor][1][ch0 + i];
        r.b[i] = c.x[tensor][2][ch0 + i];
    }
    return r;
}

// The raw row before each staged row (rows t0 - 1 .. t0 + 62), for the convolution.
// Lane l of a wave stages row 8w' + (l >> 3) (w' = the wave's row group), so the row
// before it sits in lane l - 8 of the same wave for all but the first 8 lanes: only
// those load one here, from the head (row t0 + r - 1), or, for the first rows of the
// sequence, from `prev`, the cached raw row of token -1 (an empty resource = zeros);
// conv_stage takes the others from their neighbours.
__device__ __forceinline__ void fetch_before(Stage& s, __amdgpu_buffer_rsrc_t head, __amdgpu_buffer_rsrc_t prev,
                                             int t0, int tid, bool live) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool edge = ((tid & 63) >> 3) == 0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, c = e & 7;
        const bool from_prev = t0 == 0 && n == 0 && w == 0;   // row -1 (uniform per wave)
        const uint32_t off = (!edge || !live) ? kNoAccess
                             : from_prev        ? (uint32_t)(8 * c) * 2
                                                : (uint32_t)((t0 + r - 1) * kD + 8 * c) * 2;
        s.c[n] = buf_ld16(from_prev ? prev : head, off);
    }
}

// rows past the chunk's last token stay zero (a bias would otherwise make them count)
__device__ __forceinline__ void conv_stage(Stage& s, const Stage& before, const ConvLds& c, int tensor, int rows,
                                           int tid) {
    const Conv8 w = conv_lds_get(c, tensor, 8 * (tid & 7));   // a thread's channel group is the same for n = 0, 1
    const int lane = tid & 63, src = (lane - 8) & 63;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = (tid + n * kThreads) >> 3;
        uint4 b;   // the raw row r - 1: the neighbour's staged row, or the one fetched for the first 8 lanes
        b.x = __shfl(s.c[n].x, src);
        b.y = __shfl(s.c[n].y, src);
        b.z = __shfl(s.c[n].z, src);
        b.w = __shfl(s.c[n].w, src);
        if (lane < 8) b = before.c[n];
        s.c[n] = r < rows ? conv8_bf16(w, s.c[n], b) : make_uint4(0u, 0u, 0u, 0u);
    }
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
template <bool kConv, bool kRev>
__global__ void __launch_bounds__(kThreads)
lin_seg_mfma(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ z,
             float* __restrict__ wsS, float* __restrict__ wsG, int T, int nseg, int seg_chunks,
             const float* __restrict__ cw, const float* __restrict__ cb, const bf16* __restrict__ cprev, int H) {
    __shared__ __attribute__((aligned(16))) Tile sK, sV;
    __shared__ float s_w[kTile];
    __shared__ ConvLds s_conv;
    const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, col = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = (T + kTile - 1) / kTile;
    const int c0 = seg * seg_chunks, c1 = min(nc, c0 + seg_chunks);
    const size_t base = (size_t)bh * T;
    constexpr bool conv = kConv;
    const __amdgpu_buffer_rsrc_t rk = head_rows(k + base * kD, T), rv = head_rows(v + base * kD, T),
                                 rz = buf_rsrc(z + base, (uint32_t)T * 4);
    const __amdgpu_buffer_rsrc_t rkp = buf_rsrc(cprev ? cprev + ((size_t)bh * 3 + 1) * kD : nullptr, cprev ? kD * 2 : 0),
                                 rvp = buf_rsrc(cprev ? cprev + ((size_t)bh * 3 + 2) * kD : nullptr, cprev ? kD * 2 : 0);
    if (conv) conv_lds_fill(s_conv, cw, cb, bh % H, H, tid);
    f4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float later = 0.f;   // log2 decay from the end of the current chunk to the segment end
    // the next kDepth chunks' rows in flight to registers while this one is computed, one
    // buffer per chunk (the chunk loop is unrolled so that each is named statically)
    constexpr int kDepth = 2;
    struct Ahead {
        Stage k, v, bk, bv;
        float gz;   // wave 0: this lane's z
    };
    auto fetch_chunk = [&](Ahead& f, int c, bool live) {
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        f.gz = lane_z(rz, t0, T, kRev, lane, (live && w == 0) ? Lc : 0);
        fetch_rows(f.k, rk, t0, T, kRev, tid, live);
        fetch_rows(f.v, rv, t0, T, kRev, tid, live);
        if (conv) {
            fetch_before(f.bk, rk, rkp, t0, tid, live);
            fetch_before(f.bv, rv, rvp, t0, tid, live);
        }
    };
    // one chunk from buffer f, which is refilled with chunk c - kDepth once staged
    auto chunk = [&](int c, Ahead& f) {
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        if (w == 0) {
            const float incl = chunk_prefix_of(lane_decay(f.gz, t0, kRev, lane, Lc));
            const float total = __shfl(incl, 63);
            s_w[lane] = total - incl + later;      // log2 w_t relative to the segment end
            later += total;   // kept by wave 0, which also writes the segment's decay
        }
        __syncthreads();
        if (conv) {
            conv_stage(f.k, f.bk, s_conv, 1, Lc, tid);
            conv_stage(f.v, f.bv, s_conv, 2, Lc, tid);
        }
        store(f.k, sK, tid);
        store_scaled(f.v, sV, s_w, tid);
        __syncthreads();
        fetch_chunk(f, c - kDepth, c - kDepth >= c0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const b8 A = tr_op(sV, w, 2 * h, lane);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(A, tr_op(sK, dt, 2 * h, lane), acc[dt]);
        }
        __syncthreads();
    };
    Ahead f[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) fetch_chunk(f[i], c1 - 1 - i, c1 - 1 - i >= c0);   // from the segment end backwards
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): nothing issued before the loop left in flight at its top
    int c = c1 - 1;
    for (; c - (kDepth - 1) >= c0; c -= kDepth) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) chunk(c - i, f[i]);
    }
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i)
        if (c - i >= c0) chunk(c - i, f[i]);
    float* dst = wsS + ((size_t)bh * nseg + seg) * kD * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * kD + 16 * dt + col] = acc[dt][i];
    if (tid == 0) wsG[(size_t)bh * nseg + seg] = later / kLog2e;
}

// one segment of one head: carried state in accumulators (wave w: value rows
// 16w..16w+15 of S^T), per chunk intra-chunk scores + readout + update.  kStrict
// (the backward's passes): the sums run over strictly earlier tokens, the optional
// dot with xdot is taken over that strict output, and the diagonal term
// scale (q_t.k_t) v_t is added to the stored output only afterwards.
// Bounded to two workgroups per CU (256 registers): the grid never holds more than
// about two per CU, but under that register target the compiler schedules the chunk
// loop into 170-180 registers and it runs 3-6 % faster than the 200+ it takes otherwise.
template <bool kConv, bool kRev, bool kStrict>
__global__ void __launch_bounds__(kThreads, 2)
lin_main_mfma(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
              const float* __restrict__ z, const float* __restrict__ carry, bf16* __restrict__ out, int T, int nseg,
              int seg_chunks, float scale, const float* __restrict__ cw, const float* __restrict__ cb,
              const bf16* __restrict__ cprev, int H, const bf16* __restrict__ xdot, float* __restrict__ dot_out) {
    __shared__ __attribute__((aligned(16))) Tile sQ, sK, sV, sW, sS, sSlo;
    __shared__ float s_gl[kTile], s_w[kTile];
    __shared__ ConvLds s_conv;
    const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, col = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = (T + kTile - 1) / kTile;
    const int c0 = seg * seg_chunks, c1 = min(nc, c0 + seg_chunks);
    const size_t base = (size_t)bh * T;
    constexpr bool conv = kConv;
    const __amdgpu_buffer_rsrc_t rq = head_rows(q + base * kD, T), rk = head_rows(k + base * kD, T),
                                 rv = head_rows(v + base * kD, T), rz = buf_rsrc(z + base, (uint32_t)T * 4),
                                 ro = head_rows(out + base * kD, T);
    auto prev_rows = [&](int which) {
        return buf_rsrc(cprev ? cprev + ((size_t)bh * 3 + which) * kD : nullptr, cprev ? kD * 2 : 0);
    };
    const __amdgpu_buffer_rsrc_t rqp = prev_rows(0), rkp = prev_rows(1), rvp = prev_rows(2);
    if (conv) {
        conv_lds_fill(s_conv, cw, cb, bh % H, H, tid);
        __syncthreads();
    }
    // carry S^T[c][d] into the accumulator layout: rows 16w + 4g + i, column 16 dt + col
    f4 S[4];
    {
        const float* src = carry + ((size_t)bh * nseg + seg) * kD * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[dt][i] = src[(16 * w + 4 * g + i) * kD + 16 * dt + col];
    }
    // the next chunk's rows in flight to registers while this one is computed (a second
    // buffer, two chunks ahead, measured no faster here and costs 64 registers)
    const bool dots = kStrict && xdot != nullptr;
    const __amdgpu_buffer_rsrc_t rx = head_rows(dots ? xdot + base * kD : out, T);
    const int tl = 16 * w + col;   // this lane's query in the chunk (with its lane group g)
    struct Ahead {
        Stage q, k, v, bq, bk, bv;
        uint2 x[4];   // the backward's dot operand at this lane's output positions
        float gz;     // wave 0: this lane's z
    };
    auto fetch_chunk = [&](Ahead& f, int c, bool live) {
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        f.gz = lane_z(rz, t0, T, kRev, lane, (live && w == 0) ? Lc : 0);
        fetch_rows(f.q, rq, t0, T, kRev, tid, live);
        fetch_rows(f.k, rk, t0, T, kRev, tid, live);
        fetch_rows(f.v, rv, t0, T, kRev, tid, live);
        if (conv) {
            fetch_before(f.bq, rq, rqp, t0, tid, live);
            fetch_before(f.bk, rk, rkp, t0, tid, live);
            fetch_before(f.bv, rv, rvp, t0, tid, live);
        }
        if (dots) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                f.x[ct] = buf_ld8(rx, live ? (uint32_t)(stored_row(t0 + tl, T, kRev) * kD + 16 * ct + 4 * g) * 2
                                           : kNoAccess);
        }
    };
    // This chunk's output is stored one chunk later, right after the next prefetch is
    // issued: stores issued at the end of a chunk would still be in flight at the next
    // chunk's first wait for its rows.  An offset past the buffer = nothing pending.
    uint2 po[4];
    uint32_t poff = kNoAccess;
    auto store_out = [&]() {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) buf_st8(ro, poff + 32 * ct, po[ct]);
    };
    // one chunk from buffer f, which is refilled with chunk c + 1 once staged
    auto chunk = [&](int c, Ahead& f) {
        const int t0 = c * kTile, Lc = min(kTile, T - t0);
        if (w == 0) {
            const float incl = chunk_prefix_of(lane_decay(f.gz, t0, kRev, lane, Lc));
            const float total = __shfl(incl, 63);
            s_gl[lane] = incl;
            s_w[lane] = total - incl;              // log2 of w_t = exp(Gam - Gl_t)
        }
        // the state before this chunk as S[d][c] rows (4 consecutive c per lane), split into
        // a bf16 high part and the bf16 rounding of what it leaves: 16 significant bits.  A
        // state with a large common component (inputs with a bias, slow decay) read through
        // one bf16 copy loses the small differences the output is made of.
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            uint2 o, r;
            o.x = pack2(S[dt][0], S[dt][1]);
            o.y = pack2(S[dt][2], S[dt][3]);
            r.x = pack2(S[dt][0] - __uint_as_float(o.x << 16), S[dt][1] - __uint_as_float(o.x & 0xffff0000u));
            r.y = pack2(S[dt][2] - __uint_as_float(o.y << 16), S[dt][3] - __uint_as_float(o.y & 0xffff0000u));
            *reinterpret_cast<uint2*>(&sS.X[16 * dt + col][16 * w + 4 * g]) = o;
            *reinterpret_cast<uint2*>(&sSlo.X[16 * dt + col][16 * w + 4 * g]) = r;
        }
        if (conv) {
            conv_stage(f.q, f.bq, s_conv, 0, Lc, tid);
            conv_stage(f.k, f.bk, s_conv, 1, Lc, tid);
            conv_stage(f.v, f.bv, s_conv, 2, Lc, tid);
        }
        uint2 xc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) xc[ct] = f.x[ct];
        store(f.q, sQ, tid);
        store(f.k, sK, tid);
        __syncthreads();
        store_scaled(f.v, sW, s_w, tid);
        store(f.v, sV, tid);
        __syncthreads();
        fetch_chunk(f, c + 1, c + 1 < c1);
        store_out();   // the previous chunk's
        // this wave's queries 16w .. 16w + 15, one per lane column
        const float glt = s_gl[tl];
        const b8 Qb[2] = {row_op(sQ, tl, g, 0), row_op(sQ, tl, g, 1)};
        f4 O[4], OI[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            O[ct] = f4{0.f, 0.f, 0.f, 0.f};
            OI[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dtt = 0; dtt < 2; ++dtt) {
                const b8 qb = q_tr_order(sQ, tl, 2 * dtt, g);
                OI[ct] = mfma(tr_op(sSlo, ct, 2 * dtt, lane), qb, OI[ct]);
                OI[ct] = mfma(tr_op(sS, ct, 2 * dtt, lane), qb, OI[ct]);
            }
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
                    p[4 * u + i] = (kStrict ? sl < tl : sl <= tl) ? scale * fexp2(glt - gs[i]) * X[i] : 0.f;
                }
            }
            const b8 B = to_b(p);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) O[ct] = mfma(tr_op(sV, ct, 2 * h, lane), B, O[ct]);
        }
        {
            // optional fp32 epilogue: dot_out_t = xdot_t . o_t over the 64 columns, before the
            // output is rounded (the backward's strict row and column sums of dL/dlambda)
            const float dec = scale * fexp2(glt);
            // the token's row in the head; rows past the chunk's last token fall outside the
            // buffers (negative ones wrap past them), so their stores are dropped
            const int hrow = stored_row(t0 + tl, T, kRev);
            poff = (uint32_t)(hrow * kD + 4 * g) * 2;
            // strict passes: the diagonal term scale (q_t.k_t) v_t joins the output after the
            // dot has been taken (q.k over the token's 64 dims: 16 per lane group)
            float diag = 0.f;
            if (kStrict) {
                float fq[16], fk[16];
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(&sQ.X[tl][16 * g]), fq);
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(&sQ.X[tl][16 * g + 8]), fq + 8);
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(&sK.X[tl][16 * g]), fk);
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(&sK.X[tl][16 * g + 8]), fk + 8);
#pragma unroll
                for (int i = 0; i < 16; ++i) diag = fmaf(fq[i], fk[i], diag);
                diag += __shfl_xor(diag, 16);
                diag += __shfl_xor(diag, 32);
                diag *= scale;
            }
            float dot = 0.f;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = fmaf(dec, OI[ct][i], O[ct][i]);
                if (kStrict) {
                    const uint2 vv = *reinterpret_cast<const uint2*>(&sV.X[tl][16 * ct + 4 * g]);
                    const float fv[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                                         __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
                    po[ct] = make_uint2(pack2(fmaf(diag, fv[0], y[0]), fmaf(diag, fv[1], y[1])),
                                        pack2(fmaf(diag, fv[2], y[2]), fmaf(diag, fv[3], y[3])));
                } else {
                    po[ct] = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
                }
                if (dots) {
                    const uint2 xv = xc[ct];
                    dot = fmaf(__uint_as_float(xv.x << 16), y[0], dot);
                    dot = fmaf(__uint_as_float(xv.x & 0xffff0000u), y[1], dot);
                    dot = fmaf(__uint_as_float(xv.y << 16), y[2], dot);
                    dot = fmaf(__uint_as_float(xv.y & 0xffff0000u), y[3], dot);
                }
            }
            if (dots) {
                // the four lanes of a token (lane groups g = 0..3, 16 apart) hold its 64 columns
                dot += __shfl_xor(dot, 16);
                dot += __shfl_xor(dot, 32);
                buf_st4f(buf_rsrc(dot_out + base, (uint32_t)T * 4), g == 0 ? (uint32_t)hrow * 4 : kNoAccess, dot);
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
    };
    Ahead f;
    fetch_chunk(f, c0, true);
    // Retire the loads above (the carry and the first chunk) before the loop: the waits
    // inside it are sized for the loop's own order of loads and stores, which only holds
    // when nothing issued before the loop is still in flight at its top.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int c = c0; c < c1; ++c) chunk(c, f);
    store_out();   // the last chunk's
}

// the segmented kernels address a head's rows through 32-bit buffer offsets
static bool lin_rows_addressable(int T) { return (size_t)T * kD * 2 < ((size_t)1 << 31); }

template <bool kRev, bool kStrict = kRev>
int run_fused(const FwdArgs& a, const bf16* xdot = nullptr, float* dot_out = nullptr) {
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
    const bf16* cprev = (const bf16*)a.conv_prev;
    if (!kRev && a.conv_w)
        hipLaunchKernelGGL((lin_seg_mfma<true, false>), dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.k,
                           (const bf16*)a.v, a.z, wsS, wsG, a.T, nseg, sc, a.conv_w, a.conv_b, cprev, a.H);
    else
        hipLaunchKernelGGL((lin_seg_mfma<false, kRev>), dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.k,
                           (const bf16*)a.v, a.z, wsS, wsG, a.T, nseg, sc, nullptr, nullptr, nullptr, a.H);
    ktimer_end(a.timer, a.stream);
    const int etiles = (kD * kD + 255) / 256;
    ktimer_begin(a.timer, "lin_scan", a.stream);
    hipLaunchKernelGGL((lin_scan<kD, kD, true>), dim3(nbh * etiles), dim3(256), 0, st, wsS, (const float*)wsG,
                       a.state_in, a.state_out, nseg, etiles);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "lin_main", a.stream);
    if (!kRev && a.conv_w)
        hipLaunchKernelGGL((lin_main_mfma<true, false, false>), dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.q,
                           (const bf16*)a.k, (const bf16*)a.v, a.z, (const float*)wsS, (bf16*)a.out, a.T, nseg, sc,
                           a.scale, a.conv_w, a.conv_b, cprev, a.H, nullptr, nullptr);
    else
        hipLaunchKernelGGL((lin_main_mfma<false, kRev, kStrict>), dim3(nbh * nseg), dim3(kThreads), 0, st, (const bf16*)a.q,
                           (const bf16*)a.k, (const bf16*)a.v, a.z, (const float*)wsS, (bf16*)a.out, a.T, nseg, sc,
                           a.scale, nullptr, nullptr, nullptr, a.H, xdot, dot_out);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

FwdArgs lin_bwd_fwd_args(const BwdArgs& a) {
    FwdArgs f;
    memset(&f, 0, sizeof(f));
    f.B = a.B; f.H = a.H; f.T = a.T; f.dk = a.dk; f.dv = a.dv; f.chunk = kLinChunk;
    f.scale = a.scale; f.variant = TWOMAMBA_LIN; f.dtype = a.dtype;
    f.z = a.z; f.ws = a.ws; f.ws_bytes = a.ws_bytes; f.stream = a.stream; f.timer = a.timer;
    return f;
}

}  // namespace

// ---------------------------------------------------------------------------
// First-order backward in O(T) (bf16, d = 64).  With w_ts = L_ts scale q_t.k_s and
// no normaliser, the gradients are three first-order forwards of the same decay:
//     dq_t = sum_{s<=t} L_ts scale (dout_t.v_s) k_s      queries dout, keys v, values k
//     dk_s = sum_{t>=s} L_ts scale (v_s.dout_t) q_t      the same in reverse time: queries v,
//     dv_s = sum_{t>=s} L_ts scale (k_s.q_t) dout_t      keys dout, values q / queries k, keys q,
//                                                       values dout
// run by the segmented chunk kernels of the forward (the last two back to front).
// dL/dg comes from the strict row and column sums of dL/dlambda (2Mamba2Furious,
// App. C, C.1): rowsum_t = q_t . dq^S_t = sum_{s<t} dL/dlambda_ts and colsum_s =
// k_s . dk^S_s = sum_{t>s} dL/dlambda_ts, with dq^S, dk^S the strictly causal parts.
// The passes therefore run with the strict mask, take these dots in fp32 before
// anything is rounded (dz is their running difference over the whole sequence),
// and only then add the diagonal term, scale (q.k) v of their own operands:
// a_t k_t to dq, a_t q_t to dk, c_t dout_t to dv (a_t = scale dout_t.v_t,
// c_t = scale q_t.k_t).
bool lin_bwd_chunked_supported(const BwdArgs& a) {
    return a.variant == TWOMAMBA_LIN && a.dtype == TWOMAMBA_BF16 && a.dk == 64 && a.dv == 64 &&
           lin_rows_addressable(a.T) &&
           !(a.flags & (TWOMAMBA_FLAG_REFERENCE_KERNELS | TWOMAMBA_FLAG_ATTENTION_FORM));
}

size_t lin_bwd_chunked_workspace(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T;
    if (n == 0) return 0;
    return align256(lin_layout(lin_bwd_fwd_args(a)).total) + 2 * align256(n * sizeof(float));
}

int lin_bwd_chunked(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T;
    if (n == 0) return TWOMAMBA_OK;
    FwdArgs f = lin_bwd_fwd_args(a);
    int r;
    BwdScratch sc;
    memset(&sc, 0, sizeof(sc));
    char* p = (char*)a.ws + align256(lin_layout(f).total);
    sc.rowsum = (float*)p;
    sc.colsum = (float*)(p + align256(n * sizeof(float)));
    // rowsum_t = q_t . dq^S_t and colsum_s = k_s . dk^S_s are taken in fp32 by the passes
    f.q = a.dout; f.k = a.v; f.v = a.k; f.out = a.gq;
    if ((r = run_fused<false, true>(f, (const bf16*)a.q, sc.rowsum)) != TWOMAMBA_OK) return r;
    f.q = a.v; f.k = a.dout; f.v = a.q; f.out = a.gk;
    if ((r = run_fused<true, true>(f, (const bf16*)a.k, sc.colsum)) != TWOMAMBA_OK) return r;
    f.q = a.k; f.k = a.q; f.v = a.dout; f.out = a.gv;
    if ((r = run_fused<true, true>(f)) != TWOMAMBA_OK) return r;
    return bwd_dz_launch(a, sc);
}

bool lin_conv_fused(const FwdArgs& a) {
    return a.dtype == TWOMAMBA_BF16 && a.dk == 64 && a.dv == 64 && lin_rows_addressable(a.T) &&
           !(a.flags & TWOMAMBA_FLAG_REFERENCE_KERNELS);
}

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
    if (bf && a.dk == 64 && lin_rows_addressable(a.T) && !(a.flags & TWOMAMBA_FLAG_REFERENCE_KERNELS))
        return run_fused<false, false>(a);
    if (a.dk == 64) return bf ? run<64, 64, bf16>(a) : run<64, 64, float>(a);
    if (a.dk == 16) return bf ? run<16, 16, bf16>(a) : run<16, 16, float>(a);
    return TWOMAMBA_ERR_UNSUPPORTED;
}

}  // namespace twm
