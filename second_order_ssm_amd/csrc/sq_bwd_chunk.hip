// 2Mamba backward in O(T) for bf16 inputs and d_k = d_v = 64 ("2Mamba2Furious",
// App. C: the gradients of the attention kernel with Q, K, V as inputs; C.1: the
// A-mask gradient from sums of the masked matrix along the key and query axes).
//
// With x_ts = q_t.k_s, lambda_ts = exp(G_t - G_s) (G the running sum of
// g = -softplus(z)), P_ts = lambda_ts scale^2 x_ts^2, den_t = sum_{s<=t} P_ts,
// w_t = dout_t / den_t and mu_t = (dout_t.o_t) / den_t (without normalisation
// w_t = dout_t, mu_t = 0), the gradient of the loss through P_ts is
// dP_ts = v_s.w_t - mu_t, and
//     dq_t = 2 scale^2 sum_{s<=t} lambda_ts x_ts (w_t.v_s - mu_t) k_s
//     dk_s = 2 scale^2 sum_{t>=s} lambda_ts x_ts (v_s.w_t - mu_t) q_t
//     dv_s = sum_{t>=s} P_ts w_t.
// dv is the unnormalised 2Mamba forward in reversed time (queries k, keys q,
// values w).  dq and dk are the same "mixed" sum
//     A_t = sum_{s<=t} lambda_ts (a_t.b_s) (c_t.e_s + c65_t e65_s) f_s b_s
// (dq: a = q, b = k, c = dout, e = v, c65 = -D, e65 = 1, f = 1, and dq_t takes
// 1/den_t at the end; dk in reversed time: a = k, b = q, c = v, e = dout,
// c65 = -1, e65 = D, f = 1/den).  Keeping dout unscaled in the dot products
// matters where dout_t.v_s and D_t nearly cancel (a row whose output is mostly
// one value, e.g. the first token, has a small den_t and a large w_t, and a
// bf16 copy of w_t would leave its rounding in that difference).  Its state after the keys up
// to u is S[i, c, j] = sum_{s<=u} lambda_us b_s[i] e_s[c] b_s[j] (64 x 65 x 64,
// the forward's state with both pair orders kept), read out by
// A_t[j] = sum_{i,c} a_t[i] c_t[c] S[i, c, j]: a contraction with K = (i, c).
// The strict row and column sums of dL/dlambda (C.1) need no pass of their own:
// P_ts is homogeneous of degree 2 in q_t and in k_s, so the keys two or more chunks
// back give q_t.dq^far_t / 2 (and the queries two or more chunks ahead
// k_s.dk^far_s / 2), while the pairs within a query's own chunk and the chunk before
// it are summed in fp32 by the kernel that forms their weights.  dz is a running sum
// of column minus row sums over the whole sequence; leaving the nearest chunk out of
// the bf16 state readout keeps the large near terms exact (with the previous chunk in
// the readout, that rounding accumulated to 5e-2 of dz at 2x16x8192).
//
// sqc_walk_kernel: one workgroup of 8 waves per (head, segment, quarter of the
// value columns c), the quarter's S (64 i x 16 c x 64 j, fp32) held in MFMA
// accumulators: 16x16 tiles (i, jt) with rows c and columns j, wave w owning
// i = 8w .. 8w+7.  The first quarter also carries the 65th column
// N[i, j] = sum lambda e65_s b_s[i] b_s[j].  Per chunk of 64 tokens:
//   intra:   W^T[s, t] = exp(Gl_t - Gl_s) (b_s.a_t) (e_s.c_t + e65_s c65_t) for
//            s <= t in the chunk, then A += W b (16x16x32 and 16x16x16 MFMAs);
//   readout: A_t += sum_{i,c} (exp(G_t - G_anchor) a_t[i] c_t[c]) S[i, c, j] from the
//            state of the keys before the previous chunk (anchored at its start), with K = 32
//            slots = two i by four c per lane group, the state tiles of i and
//            i + 1 stacked as the B operand (the rows 4g..4g+3 a lane holds are
//            its K-slots);
//   update:  S <- e^Gamma S + sum_s (exp(Gamma - Gl_s) e_s[c] b_s[i]) b_s[j];
//   the eight waves' partial A are summed through LDS and stored in fp32 per
//   quarter; sqc_combine adds the quarters.
// Segments: a pre-pass (kPre) walks every segment but the last with the update
// alone and stores its end state and total log decay; segment g starts from the
// decayed sum of the end states before it.
#include <string.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "mfma_tiles.h"

namespace twm {
namespace {

using namespace tiles;

constexpr int kCk = 64;           // tokens per chunk
constexpr int kQc = 16;           // value columns per workgroup
constexpr int kWv = 8;            // waves per workgroup
constexpr int kTh = 64 * kWv;
constexpr int kR4 = 34;           // carried float4 per lane: S (32) and N (2)
constexpr int kMaxSeg = 8;
constexpr int kMaxPieces = 4;     // pre-pass pieces per segment

typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4 mfma16(uint2 a, uint2 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, a), __builtin_bit_cast(s4v, b), c, 0,
                                                     0, 0);
}
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ uint32_t pk(float a, float b) { return pack2(a, b); }
__device__ __forceinline__ float lo16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// One chunk's keys as the update reads them.  The main pass adds a chunk's keys one
// chunk after staging them (its readout of chunk c leaves out the keys of chunk c - 1,
// which the chunk-local kernel takes), so it holds two.
struct KeySide {
    float b32t[kD][68];      // b_s[i] as [i][s]: products of the update operand
    float el[kQc][68];       // exp(Gamma - Gl_s) e_s[c] / frame as [c][s]
    uint16_t bt16[kD][72];   // b_s[j] as [j][s], bf16 (update B operand)
    float el65[kCk];         // the 65th column's weights
};
struct Lds {
    KeySide kb[2];
    float ag[kCk][68];       // (frame) exp(G_t - G_anchor) a_t[i] as [t][i]: readout products
    float cq[kCk][20];       // c_t[c] as [t][c]
    float c65[kCk];
    float red[kWv][2 * 16 * 64];   // the waves' partial A over two query tiles
};

struct Fetch {
    uint4 a, b;   // 8 dims of one token's a and b
    uint2 ce;     // 4 columns of one token's c (threads < 256) or e (the others)
    float z, x65, ks;   // the lane's token (every wave): decay logit, 65th-column value, key scale
};

// A head's rows (or per-token scalars) as a buffer resource: loads past the end
// return zero, so ragged chunks need no branch around a memory instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
struct Src {
    __amdgpu_buffer_rsrc_t a, b, c, e, z, x65, ks;
};

// Loads one chunk (tokens c0 .. c0 + 63); rows past T read as zero.
template <bool kPre>
__device__ __forceinline__ void fetch(Fetch& f, const Src& r, int c0, int q, int tid) {
    const int lane = tid & 63;
    const int so = c0 * kD * 2;
    {
        const int off = (tid >> 3) * kD * 2 + 16 * (tid & 7);
        f.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.b, off, so, 0));
        if (!kPre) f.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.a, off, so, 0));
    }
    {
        const int u = tid & 255;
        const int off = (u >> 2) * kD * 2 + 2 * (kQc * q + 4 * (u & 3));
        if (kPre) {
            if (tid >= 256) f.ce = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r.e, off, so, 0));
        } else {
            f.ce = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(tid < 256 ? r.c : r.e, off, so, 0));
        }
    }
    f.z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r.z, lane * 4, c0 * 4, 0));
    f.x65 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r.x65, lane * 4, c0 * 4, 0));
    f.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r.ks, lane * 4, c0 * 4, 0));
}

__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// Stages one chunk's keys (b, e, the 65th column) into K, with the update weights
// exp(Gamma - Gl_s) f_s / frame.  Gl (of the lane's token) and Gamma are per wave.
__device__ __forceinline__ void stage_keys(KeySide& K, const Fetch& f, float Gl, float Gam, float rfn, int tid,
                                           bool has65, bool x65_on_key, bool has_ks) {
    const int lane = tid & 63;
    {   // b: token tid / 8, dims 8 (tid mod 8) .. + 7
        const int t = tid >> 3, d = 8 * (tid & 7);
        const uint32_t bw[4] = {f.b.x, f.b.y, f.b.z, f.b.w};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t u = bw[m >> 1];
            K.b32t[d + m][t] = (m & 1) ? hi16(u) : lo16(u);
            K.bt16[d + m][t] = (uint16_t)(u >> (16 * (m & 1)));
        }
    }
    if (tid >= 256) {   // e: token u / 4, columns 4 (u mod 4) .. + 3
        const int u = tid & 255, t = u >> 2, col = 4 * (u & 3);
        const uint2 x = f.ce;
        const float l = rfn * fexp(Gam - __shfl(Gl, t)) * (has_ks ? __shfl(f.ks, t) : 1.f);
        K.el[col + 0][t] = l * lo16(x.x);
        K.el[col + 1][t] = l * hi16(x.x);
        K.el[col + 2][t] = l * lo16(x.y);
        K.el[col + 3][t] = l * hi16(x.y);
    }
    if (has65 && tid < 64) {   // e65_s: x_s (key side) or 1
        const float ev = x65_on_key ? f.x65 : 1.f;
        K.el65[lane] = rfn * fexp(Gam - Gl) * (has_ks ? f.ks : 1.f) * ev;
    }
}

// Stages one chunk's queries (a with the factor frq exp(Gl_t), c, the 65th column).
__device__ __forceinline__ void stage_queries(Lds& L, const Fetch& f, float Gl, float frq, int tid, bool has65,
                                              bool x65_on_key) {
    const int lane = tid & 63;
    {   // a: token tid / 8, dims 8 (tid mod 8) .. + 7
        const int t = tid >> 3, d = 8 * (tid & 7);
        const float eg = frq * fexp(__shfl(Gl, t));
        const uint4 u = f.a;
        *reinterpret_cast<float4*>(&L.ag[t][d]) =
            make_float4(eg * lo16(u.x), eg * hi16(u.x), eg * lo16(u.y), eg * hi16(u.y));
        *reinterpret_cast<float4*>(&L.ag[t][d + 4]) =
            make_float4(eg * lo16(u.z), eg * hi16(u.z), eg * lo16(u.w), eg * hi16(u.w));
    }
    if (tid < 256) {   // c: token u / 4, columns 4 (u mod 4) .. + 3
        const int u = tid, t = u >> 2, col = 4 * (u & 3);
        const uint2 x = f.ce;
        *reinterpret_cast<float4*>(&L.cq[t][col]) = make_float4(lo16(x.x), hi16(x.x), lo16(x.y), hi16(x.y));
    }
    if (has65 && tid < 64) L.c65[lane] = x65_on_key ? -1.f : -f.x65;   // c65_t: -1 or -x_t (query side)
}

// The 65th column's readout into the accumulators of key tile JT, for the query tiles
// 2 pass, 2 pass + 1: A[t][j] += sum_i (c65_t exp(Gl_t) a_t[i]) N[i][j] over the two
// row tiles of N this wave holds (i = 32 (w >> 2) + 0 .. 31).
template <int JT>
__device__ __forceinline__ void n_readout(f4 (&O)[2][4], const f4 (&N)[2], const Lds& L, int w, int g, int m16,
                                          int pass) {
    const int ib = 32 * (w >> 2);
    const float xs[8] = {N[0][0], N[0][1], N[0][2], N[0][3], N[1][0], N[1][1], N[1][2], N[1][3]};
    const b8 BN = to_b(xs);
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
        const int t = 16 * (2 * pass + tl) + m16;
        const float cf = L.c65[t];
        const float4 u0 = *reinterpret_cast<const float4*>(&L.ag[t][ib + 4 * g]);
        const float4 u1 = *reinterpret_cast<const float4*>(&L.ag[t][ib + 16 + 4 * g]);
        const b8 X = as_b8(make_uint4(pk(cf * u0.x, cf * u0.y), pk(cf * u0.z, cf * u0.w), pk(cf * u1.x, cf * u1.y),
                                      pk(cf * u1.z, cf * u1.w)));
        O[tl][JT] = mfma(X, BN, O[tl][JT]);
    }
}

// S <- e^Gamma S + sum_s (exp(Gamma - Gl_s) e_s[c] b_s[i]) b_s[j] in the frame (el
// carries the new frame's reciprocal); resc: the stored state first takes the
// factor fn0 (the frame was reset to 1).  K = the chunk's tokens, 32 per MFMA.
__device__ __forceinline__ void state_update(f4 (&S)[8][4], f4 (&N)[2], const KeySide& L, bool resc, float fn0,
                                             bool n_here, int w, int g, int m16) {
    if (resc) {
#pragma unroll
        for (int il = 0; il < 8; ++il)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) S[il][jt] *= fn0;
#pragma unroll
        for (int n = 0; n < 2; ++n) N[n] *= fn0;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int s0 = 32 * kk + 8 * g;
        const float4 e0 = *reinterpret_cast<const float4*>(&L.el[m16][s0]);
        const float4 e1 = *reinterpret_cast<const float4*>(&L.el[m16][s0 + 4]);
        b8 Bu[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) Bu[jt] = as_b8(*reinterpret_cast<const uint4*>(&L.bt16[16 * jt + m16][s0]));
#pragma unroll
        for (int il = 0; il < 8; ++il) {
            const float4 b0 = *reinterpret_cast<const float4*>(&L.b32t[8 * w + il][s0]);
            const float4 b1 = *reinterpret_cast<const float4*>(&L.b32t[8 * w + il][s0 + 4]);
            const b8 A = as_b8(make_uint4(pk(e0.x * b0.x, e0.y * b0.y), pk(e0.z * b0.z, e0.w * b0.w),
                                          pk(e1.x * b1.x, e1.y * b1.y), pk(e1.z * b1.z, e1.w * b1.w)));
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) S[il][jt] = mfma(A, Bu[jt], S[il][jt]);
            __builtin_amdgcn_sched_barrier(0);   // keep the next row's loads from piling up early
        }
        if (n_here) {   // N <- ... + sum_s (exp(Gamma - Gl_s) e65_s b_s[i]) b_s[j]
            const b8 Bn = as_b8(*reinterpret_cast<const uint4*>(&L.bt16[16 * (w & 3) + m16][s0]));
            const float4 l0 = *reinterpret_cast<const float4*>(&L.el65[s0]);
            const float4 l1 = *reinterpret_cast<const float4*>(&L.el65[s0 + 4]);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int i = 16 * (2 * (w >> 2) + n) + m16;
                const float4 b0 = *reinterpret_cast<const float4*>(&L.b32t[i][s0]);
                const float4 b1 = *reinterpret_cast<const float4*>(&L.b32t[i][s0 + 4]);
                const b8 A = as_b8(make_uint4(pk(l0.x * b0.x, l0.y * b0.y), pk(l0.z * b0.z, l0.w * b0.w),
                                              pk(l1.x * b1.x, l1.y * b1.y), pk(l1.z * b1.z, l1.w * b1.w)));
                N[n] = mfma(A, Bn, N[n]);
            }
        }
    }
}

// One launch: kPre = update only over the pieces of segments 0 .. nseg-2 (m per
// segment, pc chunks each; end states out); otherwise every segment, from the
// decayed sum of the end states of the pieces before it, with A out.
template <bool kPre>
__global__ void __launch_bounds__(kTh)
sqc_walk_kernel(const bf16* __restrict__ ga, const bf16* __restrict__ gb, const bf16* __restrict__ gc,
                const bf16* __restrict__ ge, const float* __restrict__ gz, const float* __restrict__ gx65,
                int x65_on_key, const float* __restrict__ gks, int T, int nbh, int nseg, int sc, int m, int pc,
                float* __restrict__ E, float* __restrict__ Lam,
                float* __restrict__ Aout) {
    __shared__ __attribute__((aligned(16))) Lds L;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m16 = lane & 15;
    // the wave index as a wave-uniform value: branches on it are then scalar, so no MFMA of
    // another wave's case runs under an empty exec mask (MFMAs ignore exec)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the four quarters of one (head, segment) on one XCD: block i runs on XCD i mod 8
    const int segs = kPre ? (nseg - 1) * m : nseg;   // pieces (pre-pass) or segments
    const int x = blockIdx.x % kXcd, jx = blockIdx.x / kXcd;
    const int q = jx & 3, unit = (jx >> 2) * kXcd + x;
    if (unit >= nbh * segs) return;
    const int bh = unit / segs, seg = unit % segs;
    const bool has65 = gx65 != nullptr, has_ks = gks != nullptr;
    const bool n_here = has65 && q == 0;
    const size_t hoff = (size_t)bh * T;
    Src src;
    {
        const size_t rb = (size_t)T * kD * 2;
        src.a = rsrc(ga + hoff * kD, rb);
        src.b = rsrc(gb + hoff * kD, rb);
        src.c = rsrc(gc + hoff * kD, rb);
        src.e = rsrc(ge + hoff * kD, rb);
        src.z = rsrc(gz + hoff, (size_t)T * 4);
        src.x65 = has65 ? rsrc(gx65 + hoff, (size_t)T * 4) : rsrc(gz, 0);
        src.ks = has_ks ? rsrc(gks + hoff, (size_t)T * 4) : rsrc(gz, 0);
    }
    const int nc = (T + kCk - 1) / kCk;
    const int npieces = (nseg - 1) * m;
    int ch0, ch1;
    if (kPre) {   // piece seg = segment seg / m, part seg mod m, over the keys the main pass does
                  // not add itself: segment sg's keys are chunks sg sc - 1 .. (sg + 1) sc - 2
        const int sg = seg / m, r = seg - sg * m;
        const int k0 = max(0, sg * sc - 1), k1 = min(nc, (sg + 1) * sc - 1);
        ch0 = min(k1, k0 + r * pc);
        ch1 = min(k1, ch0 + pc);
    } else {
        ch0 = seg * sc;
        ch1 = min(nc, ch0 + sc);
    }

    f4 S[8][4];    // S[i = 8w + il][c = 4g + r][j = 16 jt + m16]
    f4 N[2];       // N[i = 16 (2 (w >> 2) + n) + 4g + r][j = 16 (w & 3) + m16]
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int il = 0; il < 8; ++il)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) S[il][jt] = zero4;
#pragma unroll
    for (int n = 0; n < 2; ++n) N[n] = zero4;
    const size_t slot = (size_t)kWv * kR4 * 64 * 4;   // floats of one (segment, quarter) end state
    if (!kPre && seg > 0) {
        // carry: the pieces before the segment, sum_{p < seg m} exp(Lam_{p+1} + ...) E_p
        float lsum = 0.f;
        for (int gp = seg * m - 1; gp >= 0; --gp) {
            const float f = fexp(lsum);
            const float4* src = reinterpret_cast<const float4*>(E + ((size_t)(bh * npieces + gp) * 4 + q) * slot) +
                                (size_t)w * kR4 * 64 + lane;
#pragma unroll
            for (int il = 0; il < 8; ++il)
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const float4 v = src[(il * 4 + jt) * 64];
                    S[il][jt][0] += f * v.x; S[il][jt][1] += f * v.y;
                    S[il][jt][2] += f * v.z; S[il][jt][3] += f * v.w;
                }
            if (n_here) {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const float4 v = src[(32 + n) * 64];
                    N[n][0] += f * v.x; N[n][1] += f * v.y; N[n][2] += f * v.z; N[n][3] += f * v.w;
                }
            }
            lsum += Lam[bh * npieces + gp];
        }
    }

    // The state is kept in a frame: true S = fr * stored S, so that the chunk decay
    // multiplies one scalar instead of every accumulator; the stored state is rescaled
    // only when the frame would drop below 2^-64 (or underflow).  Every wave forms the
    // same frame and decay totals, so branches on them are uniform.
    float fr = 1.f;
    float lam_tot = 0.f;
    // The main pass reads chunk c's queries out of the state of the keys before chunk
    // c - 1 (the chunk-local kernel takes chunk c - 1's keys), then adds chunk c - 1's
    // keys: "pend" is that chunk, staged one iteration earlier, with its decay total and
    // the frame its weights were staged in.
    bool pend = false, pend_resc = false;
    float pend_gam = 0.f, pend_fn0 = 1.f, pend_fnew = 1.f;
    Fetch f;
    if (!kPre && seg > 0) {   // the previous segment's last chunk: staged now, added after the first readout
        fetch<true>(f, src, (ch0 - 1) * kCk, q, tid);
        const float glp = wave_incl_scan(decay_log(f.z), lane);
        const float gp = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __shfl(glp, 63))));
        pend_fn0 = fr * fexp(gp);
        pend_resc = pend_fn0 < 0x1p-64f;
        pend_fnew = pend_resc ? 1.f : pend_fn0;
        pend_gam = gp;
        pend = true;
        stage_keys(L.kb[(ch0 - 1) & 1], f, glp, gp, 1.f / pend_fnew, tid, has65, x65_on_key != 0, has_ks);
    }
    fetch<kPre>(f, src, ch0 * kCk, q, tid);
    for (int ch = ch0; ch < ch1; ++ch) {
        const int c0 = ch * kCk;
        // chunk-local cumulative log decay of the lane's token, and the chunk total
        const float gl = wave_incl_scan(c0 + lane < T ? decay_log(f.z) : 0.f, lane);
        // the chunk total as a wave-uniform value: the frame bookkeeping below stays scalar
        const float Gam = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __shfl(gl, 63))));
        lam_tot += Gam;
        // the frame of this chunk's keys: after the pending update, times e^Gamma
        const float fr_after = pend ? pend_fnew : fr;
        const float fn0 = fr_after * fexp(Gam);
        const bool resc = fn0 < 0x1p-64f;
        const float fnew = resc ? 1.f : fn0;
        KeySide& K = L.kb[kPre ? 0 : (ch & 1)];
        stage_keys(K, f, gl, Gam, 1.f / fnew, tid, has65, x65_on_key != 0, has_ks);
        // the queries see the stored state (frame fr) anchored before the pending chunk
        if (!kPre) stage_queries(L, f, gl, fr * (pend ? fexp(pend_gam) : 1.f), tid, has65, x65_on_key != 0);
        __syncthreads();
        fetch<kPre>(f, src, c0 + kCk, q, tid);   // past the segment: loads nothing used

        if (kPre) {
            state_update(S, N, K, resc, fn0, n_here, w, g, m16);
            fr = fnew;
            __syncthreads();   // the update's reads done before the next chunk is staged
            continue;
        }
        // ---- readout from the stored state, in two passes of two query tiles
        float* dst = Aout + ((size_t)q * nbh * T + hoff) * kD;
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            f4 O[2][4];   // partial A[t = 16 (2 pass + tl) + 4g + r][j = 16 jt + m16] of this wave
            const int ag0 = (32 * pass + m16) * 68, cq0 = (32 * pass + m16) * 20 + 4 * g;   // 32-bit LDS offsets
#pragma unroll
            for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) O[tl][jt] = zero4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                b8 B[4];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const float xs[8] = {S[2 * p][jt][0],     S[2 * p][jt][1],     S[2 * p][jt][2],
                                         S[2 * p][jt][3],     S[2 * p + 1][jt][0], S[2 * p + 1][jt][1],
                                         S[2 * p + 1][jt][2], S[2 * p + 1][jt][3]};
                    B[jt] = to_b(xs);
                }
                const int i0 = 8 * w + 2 * p;
#pragma unroll
                for (int tl = 0; tl < 2; ++tl) {
                    // row 32 pass + 16 tl + m16 of ag and cq, from the pass's base offsets
                    const float2 av = *reinterpret_cast<const float2*>(&L.ag[0][0] + ag0 + tl * 16 * 68 + i0);
                    const float4 cv = *reinterpret_cast<const float4*>(&L.cq[0][0] + cq0 + tl * 16 * 20);
                    const b8 X = as_b8(make_uint4(pk(av.x * cv.x, av.x * cv.y), pk(av.x * cv.z, av.x * cv.w),
                                                  pk(av.y * cv.x, av.y * cv.y), pk(av.y * cv.z, av.y * cv.w)));
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) O[tl][jt] = mfma(X, B[jt], O[tl][jt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (n_here) {   // the 65th column: K = i over the two row tiles this wave holds
                switch (w & 3) {
                    case 0: n_readout<0>(O, N, L, w, g, m16, pass); break;
                    case 1: n_readout<1>(O, N, L, w, g, m16, pass); break;
                    case 2: n_readout<2>(O, N, L, w, g, m16, pass); break;
                    default: n_readout<3>(O, N, L, w, g, m16, pass); break;
                }
            }
#pragma unroll
            for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) L.red[w][((tl * 4 + jt) * 4 + r) * 64 + lane] = O[tl][jt][r];
            if (pass == 1 && pend) {   // the pending chunk's keys, after this chunk's readout
                state_update(S, N, L.kb[(ch - 1) & 1], pend_resc, pend_fn0, n_here, w, g, m16);
                fr = pend_fnew;
            }
            __syncthreads();   // every wave's partial in LDS (and, after the second pass, the update's reads done)
            // the eight partials summed and stored: fp32, this quarter's share
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int ei = tid + kTh * n, rho = ei >> 6, l = ei & 63;
                const int tl = rho >> 4, jt = (rho >> 2) & 3, r = rho & 3;
                const int t = c0 + 16 * (2 * pass + tl) + 4 * (l >> 4) + r, j = 16 * jt + (l & 15);
                float v = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWv; ++ww) v += L.red[ww][ei];
                if (t < T) dst[(size_t)t * kD + j] = v;
            }
            if (pass == 0) __syncthreads();   // the sums read before the second pass writes
        }
        pend = true;
        pend_gam = Gam;
        pend_fn0 = fn0;
        pend_resc = resc;
        pend_fnew = fnew;
    }

    if (kPre) {
        float4* dst = reinterpret_cast<float4*>(E + ((size_t)(bh * npieces + seg) * 4 + q) * slot) +
                      (size_t)w * kR4 * 64 + lane;
#pragma unroll
        for (int il = 0; il < 8; ++il)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                dst[(il * 4 + jt) * 64] =
                    make_float4(fr * S[il][jt][0], fr * S[il][jt][1], fr * S[il][jt][2], fr * S[il][jt][3]);
#pragma unroll
        for (int n = 0; n < 2; ++n)
            dst[(32 + n) * 64] = make_float4(fr * N[n][0], fr * N[n][1], fr * N[n][2], fr * N[n][3]);
        if (q == 0 && tid == 0) Lam[bh * npieces + seg] = lam_tot;
    }
}

// The keys of the query's own chunk and of the chunk before it (which the main pass
// leaves out of its readout): A_t += sum_{s in [c0 - 64, t]} exp(G_t - G_s) (b_s.a_t)
// (e_s.c_t + e65_s c65_t) f_s b_s over all 64 value columns (the dot products in fp32
// from the bf16 rows, before any rounding), into the fifth slot of A; and rsum_t =
// the same keys' sum with s < t of that weight times b_s.a_t, which is their share of
// the strict row sum of dL/dlambda (up to scale^2 and the row's 1/den_t), summed in
// fp32.  One workgroup of four waves per (head, chunk); wave w takes query tile w.
// Scores transposed (S^T = B A^T and U^T = E C^T on 16x16x32 MFMAs, so a lane column is
// one query), then A = W B with W^T's accumulators as the A operand and B read through
// the transposing LDS read.
__global__ void __launch_bounds__(256)
sqc_intra_kernel(const bf16* __restrict__ ga, const bf16* __restrict__ gb, const bf16* __restrict__ gc,
                 const bf16* __restrict__ ge, const float* __restrict__ gz, const float* __restrict__ gx65,
                 int x65_on_key, const float* __restrict__ gks, int T, int nc, float* __restrict__ Aout,
                 float* __restrict__ rsum) {
    __shared__ Tile tA, tC, tB[2], tE[2];   // queries of the chunk; keys of the chunk before it [0] and of it [1]
    __shared__ float sGl[2 * kCk], sE65[2 * kCk], sKs[2 * kCk], sC65[kCk];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / nc, ch = blockIdx.x % nc, c0 = ch * kCk;
    const bool has_prev = ch > 0;
    const size_t hoff = (size_t)bh * T;
    const bool has65 = gx65 != nullptr, has_ks = gks != nullptr;
    {
        const size_t rb = (size_t)T * kD * 2;
        const __amdgpu_buffer_rsrc_t ra = rsrc(ga + hoff * kD, rb), rbb = rsrc(gb + hoff * kD, rb),
                                     rc = rsrc(gc + hoff * kD, rb), re = rsrc(ge + hoff * kD, rb);
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int e = tid + 256 * n, r = e >> 3, d = 8 * (e & 7);
            const int off = r * kD * 2 + 2 * d;
            *reinterpret_cast<uint4*>(&tA.X[r][d]) = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, c0 * kD * 2, 0));
            *reinterpret_cast<uint4*>(&tC.X[r][d]) = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, off, c0 * kD * 2, 0));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = h == 1 || has_prev;
                const int so = (c0 + (h - 1) * kCk) * kD * 2;
                *reinterpret_cast<uint4*>(&tB[h].X[r][d]) =
                    ok ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rbb, off, ok ? so : 0, 0)) : z4;
                *reinterpret_cast<uint4*>(&tE[h].X[r][d]) =
                    ok ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(re, off, ok ? so : 0, 0)) : z4;
            }
        }
        if (w < 2) {   // wave 0: the chunk before (zeros for the first chunk), wave 1: the chunk
            const int h = w, t = c0 + (h - 1) * kCk + lane;
            const bool ok = h == 1 || has_prev;
            const int so = ok ? (c0 + (h - 1) * kCk) * 4 : 0;
            const float zz = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(gz + hoff, (size_t)T * 4), lane * 4, so, 0));
            const float gv = (ok && t < T) ? decay_log(zz) : 0.f;
            sGl[h * kCk + lane] = wave_incl_scan(gv, lane);
            const float m = has65 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        rsrc(gx65 + hoff, (size_t)T * 4), lane * 4, so, 0))
                                  : 0.f;
            const float ksv = has_ks ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rsrc(gks + hoff, (size_t)T * 4), lane * 4, so, 0))
                                     : 1.f;
            sE65[h * kCk + lane] = (has65 && ok) ? (x65_on_key ? m : 1.f) : 0.f;
            sKs[h * kCk + lane] = ksv;
            if (h == 1) sC65[lane] = has65 ? (x65_on_key ? -1.f : -m) : 0.f;
        }
    }
    __syncthreads();
    // the window's running log decay: the chunk's own offset by the chunk before's total
    if (tid < kCk) sGl[kCk + tid] += sGl[kCk - 1];
    __syncthreads();
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int tt = w, t = 16 * tt + m16;
    const float glt = sGl[kCk + t], c65t = sC65[t];
    f4 Oi[4] = {zero4, zero4, zero4, zero4};
    float rs = 0.f;   // sum over the window's earlier keys of W_ts (b_s.a_t), in fp32
    // key pairs of tiles: the chunk before (two pairs, every key earlier), then the chunk's
    // own tiles up to the query tile
    for (int kp = 0; kp < 2 + (tt >> 1) + 1; ++kp) {
        const int h = kp < 2 ? 0 : 1, sp = kp < 2 ? kp : kp - 2;
        const Tile& KB = tB[h];
        const Tile& KE = tE[h];
        float wv[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int st = 2 * sp + hh;
            const bool live = h == 0 || st <= tt;
            f4 sab = zero4, uce = zero4;
            if (live) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    sab = mfma(row_op(KB, 16 * st + m16, g, kk), row_op(tA, t, g, kk), sab);
                    uce = mfma(row_op(KE, 16 * st + m16, g, kk), row_op(tC, t, g, kk), uce);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * st + 4 * g + r, sw = h * kCk + s;
                const bool before = h == 0 || s < t;
                const float v = fexp(glt - sGl[sw]) * sab[r] * (uce[r] + sE65[sw] * c65t) * sKs[sw];
                wv[4 * hh + r] = (live && (before || s == t)) ? v : 0.f;
                rs += (live && before) ? v * sab[r] : 0.f;
            }
        }
        const b8 wa = to_b(wv);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) Oi[jt] = mfma(wa, tr_op(KB, jt, 2 * sp, lane), Oi[jt]);
    }
    // the strict row sum: the lane groups' shares of the keys, then one lane per query
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    if (rsum && g == 0 && c0 + t < T) rsum[hoff + c0 + t] = rs;
    float* dst = Aout + hoff * kD;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = c0 + 16 * tt + 4 * g + r;
            if (tok < T) dst[(size_t)tok * kD + 16 * jt + m16] = Oi[jt][r];
        }
}

// ---------------------------------------------------------------------------
// Per token: D_t = dout_t.out_t, inv_t = 1/den_t (0 for a row whose weight sum is
// 0; without normalisation D = 0, inv = 1, and the arrays below that hold them
// are not used), and the reversed copies for the reversed-time passes:
// x^R[T-1-t] = x[t] for k, q, v, dout, w = dout/den (bf16, the values of the dv
// forward), D and inv; z^R[u] = z[T-u] (u >= 1), so that the decay between
// reversed positions sigma < tau is exp(G_t - G_s) for s = T-1-tau and
// t = T-1-sigma; z^R[0] = -30 gives a decay logit within 1e-13 of 0 there, where
// it multiplies nothing.  Eight threads per token.
struct PrepOut {
    float *D, *inv, *Dr, *invr, *zr;
    bf16 *kr, *qr, *vr, *dor, *wr;
};
__global__ void __launch_bounds__(256)
sqc_prep_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const float* __restrict__ z, const bf16* __restrict__ out, const bf16* __restrict__ dout,
                const float* __restrict__ den, int no_norm, int T, size_t n, PrepOut o) {
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t tok = gid >> 3;
    const int part = (int)(gid & 7);
    const bool ok = tok < n;
    const size_t tk = ok ? tok : 0;
    const size_t bh = tk / T;
    const int t = (int)(tk - bh * T);
    const size_t rt = bh * T + (T - 1 - t);
    const int d = 8 * part;
    uint4 du = make_uint4(0u, 0u, 0u, 0u), ou = du;
    if (ok) {
        du = *reinterpret_cast<const uint4*>(dout + tk * kD + d);
        ou = *reinterpret_cast<const uint4*>(out + tk * kD + d);
    }
    const uint32_t dw[4] = {du.x, du.y, du.z, du.w}, ow[4] = {ou.x, ou.y, ou.z, ou.w};
    float D = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) D += lo16(dw[m]) * lo16(ow[m]) + hi16(dw[m]) * hi16(ow[m]);
    D += __shfl_xor(D, 1);
    D += __shfl_xor(D, 2);
    D += __shfl_xor(D, 4);
    if (!ok) return;
    float inv = 1.f;
    if (!no_norm) {
        const float dn = den[tk];
        inv = dn > 0.f ? 1.f / dn : 0.f;
    }
    uint32_t ww[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) ww[m] = bf16x2_rne(lo16(dw[m]) * inv, hi16(dw[m]) * inv);
    *reinterpret_cast<uint4*>(o.wr + rt * kD + d) = make_uint4(ww[0], ww[1], ww[2], ww[3]);
    *reinterpret_cast<uint4*>(o.dor + rt * kD + d) = du;
    *reinterpret_cast<uint4*>(o.kr + rt * kD + d) = *reinterpret_cast<const uint4*>(k + tk * kD + d);
    *reinterpret_cast<uint4*>(o.qr + rt * kD + d) = *reinterpret_cast<const uint4*>(q + tk * kD + d);
    *reinterpret_cast<uint4*>(o.vr + rt * kD + d) = *reinterpret_cast<const uint4*>(v + tk * kD + d);
    if (part == 0) {
        const float Dn = no_norm ? 0.f : D;
        o.D[tk] = Dn;
        o.inv[tk] = inv;
        o.Dr[rt] = Dn;
        o.invr[rt] = inv;
        o.zr[bh * T + (t == 0 ? 0 : T - t)] = t == 0 ? -30.f : z[tk];
    }
}

// Sums the five parts of A (four quarters of the carried state and the chunk's
// own keys) for the gradient of one walk, scales it by 2 scale^2 (and by the
// token's factor tf, when given), stores it (bf16) and the strict sum of
// dL/dlambda over the walk's keys (fp32,
// before rounding).  rev: the walk ran in reversed time (dk); then dv is also
// copied back from its reversed-time forward.  Sixteen threads per token.
__global__ void __launch_bounds__(256)
sqc_combine_kernel(const float* __restrict__ A, const float* __restrict__ rsum, const bf16* __restrict__ x,
                   const float* __restrict__ tf, float scale2, int T, size_t n, int rev, bf16* __restrict__ grad,
                   float* __restrict__ dot, const bf16* __restrict__ dvr, bf16* __restrict__ dv) {
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t tok = gid >> 4;
    const int part = (int)(gid & 15);
    const bool ok = tok < n;
    const size_t tk = ok ? tok : 0;
    const size_t bh = tk / T;
    const int t = (int)(tk - bh * T);
    const size_t src = rev ? bh * T + (T - 1 - t) : tk;
    const int d = 4 * part;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);   // the carried state's part (quarters 0..3)
    float4 in = s;                                  // the chunk's own keys
    float dd = 0.f;
    if (ok) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float4 v = *reinterpret_cast<const float4*>(A + ((size_t)qq * n + src) * kD + d);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        in = *reinterpret_cast<const float4*>(A + ((size_t)4 * n + src) * kD + d);
        const uint2 xu = *reinterpret_cast<const uint2*>(x + tk * kD + d);
        dd = lo16(xu.x) * s.x + hi16(xu.x) * s.y + lo16(xu.y) * s.z + hi16(xu.y) * s.w;
    }
    const float tfv = (tf && ok) ? tf[tk] : 1.f;
    const float f = 2.f * scale2 * tfv;
    s.x = f * (s.x + in.x); s.y = f * (s.y + in.y); s.z = f * (s.z + in.z); s.w = f * (s.w + in.w);
    dd += __shfl_xor(dd, 1);
    dd += __shfl_xor(dd, 2);
    dd += __shfl_xor(dd, 4);
    dd += __shfl_xor(dd, 8);
    if (!ok) return;
    *reinterpret_cast<uint2*>(grad + tk * kD + d) = make_uint2(bf16x2_rne(s.x, s.y), bf16x2_rne(s.z, s.w));
    // the strict sum of dL/dlambda: x_t.grad^inter_t / 2 (by homogeneity; the carried
    // keys never include the diagonal) plus the chunk's own share, summed in fp32
    if (dot && part == 0) dot[tk] = scale2 * tfv * (dd + rsum[src]);
    if (rev) *reinterpret_cast<uint2*>(dv + tk * kD + d) = *reinterpret_cast<const uint2*>(dvr + src * kD + d);
}

struct Plan {
    int nseg, sc;   // segments of the main walk, chunks per segment
    int m, pc;      // pre-pass pieces per segment, chunks per piece
};
Plan plan_for(const BwdArgs& a) {
    const int nc = (a.T + kCk - 1) / kCk;
    const int nbh = a.B * a.H;
    int want = std::max(1, (256 + 4 * nbh - 1) / (4 * nbh));
    want = std::min(std::min(want, kMaxSeg), nc);
    Plan p;
    p.sc = (nc + want - 1) / want;
    p.nseg = (nc + p.sc - 1) / p.sc;
    // pre-pass pieces: the fewest per segment that minimise rounds x chunks per piece
    // over the CUs (256, one workgroup each)
    p.m = 1;
    p.pc = p.sc;
    if (p.nseg > 1) {
        long best = -1;
        for (int m = 1; m <= kMaxPieces; ++m) {
            const int pc = (p.sc + m - 1) / m;
            const long wgs = (long)nbh * 4 * (p.nseg - 1) * m;
            const long cost = (wgs + 255) / 256 * pc;
            if (best < 0 || cost < best) {
                best = cost;
                p.m = m;
                p.pc = pc;
            }
        }
    }
    return p;
}

FwdArgs fwd_args_for(const BwdArgs& a) {
    FwdArgs f;
    memset(&f, 0, sizeof(f));
    f.B = a.B; f.H = a.H; f.T = a.T; f.dk = 64; f.dv = 64; f.chunk = 64;
    f.scale = a.scale; f.variant = TWOMAMBA_SQ; f.dtype = TWOMAMBA_BF16;
    f.stream = a.stream; f.timer = a.timer;
    return f;
}

struct Layout {
    size_t fws, dor, kr, qr, vr, wr, dvr, D, inv, Dr, invr, zr, den, rows, cols, rsum, A, E, Lam, total;
};
Layout layout_for(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T, nbh = (size_t)a.B * a.H;
    const size_t rows = align256(n * kD * 2), toks = align256(n * 4);
    Layout L;
    size_t o = 0;
    {
        FwdArgs f = fwd_args_for(a);
        const size_t w0 = mfma_sq_workspace(f);
        f.flags = TWOMAMBA_FLAG_NO_NORM;
        L.fws = o; o += align256(std::max(w0, mfma_sq_workspace(f)));
    }
    L.dor = o; o += rows;
    L.kr = o; o += rows;
    L.qr = o; o += rows;
    L.vr = o; o += rows;
    L.wr = o; o += rows;
    L.dvr = o; o += rows;
    L.D = o; o += toks;
    L.inv = o; o += toks;
    L.Dr = o; o += toks;
    L.invr = o; o += toks;
    L.zr = o; o += toks;
    L.den = o; o += toks;
    L.rows = o; o += toks;
    L.cols = o; o += toks;
    L.rsum = o; o += toks;
    L.A = o; o += align256(5 * n * kD * 4);
    const Plan pl = plan_for(a);
    const size_t npieces = (size_t)std::max(1, (pl.nseg - 1) * pl.m);
    L.E = o; o += align256(nbh * npieces * 4 * (size_t)kWv * kR4 * 64 * 16);
    L.Lam = o; o += align256(nbh * npieces * 4);
    L.total = o;
    return L;
}

int walk(const BwdArgs& a, const Layout& Ly, const Plan& p, const void* A_, const void* B_, const void* C_,
         const void* E_, const float* z, const float* x65, bool x65_on_key, const float* ks, float* rsum,
         const char* pre_name,
         const char* main_name) {
    char* ws = (char*)a.ws;
    const int nbh = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    float* E = (float*)(ws + Ly.E);
    float* Lam = (float*)(ws + Ly.Lam);
    float* Aout = (float*)(ws + Ly.A);
    if (p.nseg > 1) {
        const int units = nbh * (p.nseg - 1) * p.m;
        const int grid = ((units + kXcd - 1) / kXcd) * kXcd * 4;
        ktimer_begin(a.timer, pre_name, a.stream);
        hipLaunchKernelGGL(sqc_walk_kernel<true>, dim3(grid), dim3(kTh), 0, st, (const bf16*)A_, (const bf16*)B_,
                           (const bf16*)C_, (const bf16*)E_, z, x65, (int)x65_on_key, ks, a.T, nbh, p.nseg, p.sc, p.m, p.pc, E, Lam,
                           Aout);
        ktimer_end(a.timer, a.stream);
    }
    const int units = nbh * p.nseg;
    const int grid = ((units + kXcd - 1) / kXcd) * kXcd * 4;
    ktimer_begin(a.timer, main_name, a.stream);
    hipLaunchKernelGGL(sqc_walk_kernel<false>, dim3(grid), dim3(kTh), 0, st, (const bf16*)A_, (const bf16*)B_,
                       (const bf16*)C_, (const bf16*)E_, z, x65, (int)x65_on_key, ks, a.T, nbh, p.nseg, p.sc, p.m, p.pc, E, Lam, Aout);
    ktimer_end(a.timer, a.stream);
    const int nc = (a.T + kCk - 1) / kCk;
    ktimer_begin(a.timer, "sqc_intra", a.stream);
    hipLaunchKernelGGL(sqc_intra_kernel, dim3((unsigned)(nbh * nc)), dim3(256), 0, st, (const bf16*)A_,
                       (const bf16*)B_, (const bf16*)C_, (const bf16*)E_, z, x65, (int)x65_on_key, ks, a.T, nc,
                       Aout + (size_t)4 * nbh * a.T * kD, rsum);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

// The chunked form takes 2Mamba at bf16, d = 64, heads under 2^24 tokens, when
// TWOMAMBA_FLAG_CHUNKED_FORM asks for it, and by default from kSqChunkedMinT tokens
// per head on (TWOMAMBA_FLAG_ATTENTION_FORM keeps the attention form).
bool sq_bwd_chunked_supported(const BwdArgs& a) {
    if (a.variant != TWOMAMBA_SQ || a.dtype != TWOMAMBA_BF16 || a.dk != 64 || a.dv != 64 || a.T <= 0) return false;
    if (a.T >= (1 << 24)) return false;   // rows through 32-bit buffer offsets
    if (a.flags & (TWOMAMBA_FLAG_REFERENCE_KERNELS | TWOMAMBA_FLAG_ATTENTION_FORM)) return false;
    return (a.flags & TWOMAMBA_FLAG_CHUNKED_FORM) != 0 || a.T >= kSqChunkedMinT;
}

size_t sq_bwd_chunked_workspace(const BwdArgs& a) {
    if ((size_t)a.B * a.H * a.T == 0) return 0;
    return layout_for(a).total;
}

int sq_bwd_chunked(const BwdArgs& a) {
    const size_t n = (size_t)a.B * a.H * a.T;
    if (n == 0) return TWOMAMBA_OK;
    const Layout Ly = layout_for(a);
    const Plan p = plan_for(a);
    char* ws = (char*)a.ws;
    hipStream_t st = (hipStream_t)a.stream;
    const bool no_norm = (a.flags & TWOMAMBA_FLAG_NO_NORM) != 0;
    PrepOut po;
    po.D = (float*)(ws + Ly.D); po.inv = (float*)(ws + Ly.inv);
    po.Dr = (float*)(ws + Ly.Dr); po.invr = (float*)(ws + Ly.invr); po.zr = (float*)(ws + Ly.zr);
    po.kr = (bf16*)(ws + Ly.kr); po.qr = (bf16*)(ws + Ly.qr); po.vr = (bf16*)(ws + Ly.vr);
    po.dor = (bf16*)(ws + Ly.dor); po.wr = (bf16*)(ws + Ly.wr);
    bf16* dvr = (bf16*)(ws + Ly.dvr);
    float* rows = (float*)(ws + Ly.rows);
    float* cols = (float*)(ws + Ly.cols);
    int r;
    // the weight sums: the caller's row statistics, or one forward that writes them
    const float* den = a.row_stat;
    if (!no_norm && !den) {
        FwdArgs f = fwd_args_for(a);
        f.q = a.q; f.k = a.k; f.v = a.v; f.z = a.z;
        f.out = dvr;   // scratch: overwritten by the dv pass below
        f.row_stat = (float*)(ws + Ly.den);
        f.ws = ws + Ly.fws; f.ws_bytes = Ly.dor - Ly.fws;
        if ((r = mfma_sq_fwd(f)) != TWOMAMBA_OK) return r;
        den = f.row_stat;
    }
    ktimer_begin(a.timer, "sqc_prep", a.stream);
    {
        const size_t threads = n * 8;
        hipLaunchKernelGGL(sqc_prep_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, (const bf16*)a.q,
                           (const bf16*)a.k, (const bf16*)a.v, a.z, (const bf16*)a.out, (const bf16*)a.dout, den,
                           (int)no_norm, a.T, n, po);
    }
    ktimer_end(a.timer, a.stream);
    const float s2 = a.scale * a.scale;
    const unsigned cgrid = (unsigned)((n * 16 + 255) / 256);
    // dq: forward time, a = q, b = k, c = dout, e = v, 65th column -D_t (query side);
    // the row's 1/den_t taken by the combine
    float* rsum = (float*)(ws + Ly.rsum);
    if ((r = walk(a, Ly, p, a.q, a.k, a.dout, a.v, a.z, no_norm ? nullptr : po.D, false, nullptr, rsum, "sqc_pre_q",
                  "sqc_walk_q")) != TWOMAMBA_OK)
        return r;
    ktimer_begin(a.timer, "sqc_combine_q", a.stream);
    hipLaunchKernelGGL(sqc_combine_kernel, dim3(cgrid), dim3(256), 0, st, (const float*)(ws + Ly.A), (const float*)rsum,
                       (const bf16*)a.q, no_norm ? (const float*)nullptr : (const float*)po.inv, s2, a.T, n, 0, (bf16*)a.gq,
                       rows,
                       (const bf16*)nullptr, (bf16*)nullptr);
    ktimer_end(a.timer, a.stream);
    // dv: the unnormalised forward in reversed time (queries k, keys q, values w)
    {
        FwdArgs f = fwd_args_for(a);
        f.flags = TWOMAMBA_FLAG_NO_NORM;
        f.q = po.kr; f.k = po.qr; f.v = po.wr; f.z = po.zr; f.out = dvr;
        f.ws = ws + Ly.fws; f.ws_bytes = Ly.dor - Ly.fws;
        if ((r = mfma_sq_fwd(f)) != TWOMAMBA_OK) return r;
    }
    // dk: reversed time, a = k, b = q, c = v, e = dout, 65th column -D_t and the key
    // factor 1/den_t (key side)
    if ((r = walk(a, Ly, p, po.kr, po.qr, po.vr, po.dor, po.zr, no_norm ? nullptr : po.Dr, true,
                  no_norm ? nullptr : po.invr, rsum, "sqc_pre_k", "sqc_walk_k")) != TWOMAMBA_OK)
        return r;
    ktimer_begin(a.timer, "sqc_combine_k", a.stream);
    hipLaunchKernelGGL(sqc_combine_kernel, dim3(cgrid), dim3(256), 0, st, (const float*)(ws + Ly.A), (const float*)rsum,
                       (const bf16*)a.k, (const float*)nullptr, s2, a.T, n, 1, (bf16*)a.gk, cols, (const bf16*)dvr, (bf16*)a.gv);
    ktimer_end(a.timer, a.stream);
    if (hipGetLastError() != hipSuccess) return TWOMAMBA_ERR_DEVICE;
    BwdScratch sc;
    memset(&sc, 0, sizeof(sc));
    sc.rowsum = rows;
    sc.colsum = cols;
    return bwd_dz_launch(a, sc);
}

}  // namespace twm
