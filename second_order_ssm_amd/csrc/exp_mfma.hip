// MFMA kernel of the 2Mamba-E forward for d_k = d_v = 64 and bf16 inputs
// ("2Mamba2Furious", §6: the query-key product is exponentiated, i.e. causal
// softmax attention whose logits carry the softplus A-mask as an additive
// log-decay, lambda_ts = sum over r = s+1..t of g_r, g = -softplus(z)).
//
// Design (one workgroup = 4 waves = 256 queries of one head; one wave = 64
// queries as two 32-query column blocks):
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs: a
//    lane then holds one query and 16 keys, so the per-query max and sum need
//    one exchange between the two lane halves only.  The probabilities P^T
//    leave the accumulators as the B operand of O^T = V^T P^T directly (the key
//    order a lane holds is matched by the order in which V^T is staged), and the
//    per-query rescale of O^T is one multiplier per lane.
//  * Decay bias.  For the queries of a wave with last token E, the bias of key
//    s is -c_s with c_s = sum over r = s+1..E of softplus(z_r); the true bias
//    -sum_{r=s+1..t} differs from it by c_t, a per-query constant that the
//    softmax cancels, and c_t spans at most 64 tokens so no precision is lost.
//    The bias enters as the accumulator's initial value (in units of the score
//    before scaling), so the softmax needs one fma and one exp2 per score.
//  * Key tiles of 64 travel by buffer-to-LDS transfers into a ring of three
//    slots, two tiles ahead of their use; K and V stay row-major (swizzled) and
//    the V^T operand comes from transposing LDS reads.  Tiles are visited from
//    the diagonal backwards, so the running max is set by the most recent keys
//    and is moved (rescaling O) only when a score exceeds it by more than 2^8.
//  * Query tiles are dispatched longest first for load balance.
#include <algorithm>

#include "conv_common.h"
#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kD = 64;               // head dim (keys and values)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 64;              // queries per wave
constexpr int kQT = kWaves * kQW;    // queries per workgroup
constexpr int kKT = 64;              // keys per LDS tile
constexpr int kLS = 72;              // LDS row stride in bf16 (144 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;         // log2 headroom before the running max moves

__device__ __forceinline__ f16v mfma(b8 a, b8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// Lanes l and l + 32 hold the same query.  v_permlane32_swap with both operands
// x leaves the lower-half values of x in the first result and the upper-half
// values in the second, in every lane, so both halves combine them in the same
// order.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_m(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xf, true));
}
// inclusive prefix sum over the 64 lanes (row shifts 1, 2, 4, 8, then the row
// totals are broadcast into the following rows)
__device__ __forceinline__ float wave_scan(float s) {
    s += dpp_m<0x111, 0xf>(s);
    s += dpp_m<0x112, 0xf>(s);
    s += dpp_m<0x114, 0xf>(s);
    s += dpp_m<0x118, 0xf>(s);
    s += dpp_m<0x142, 0xa>(s);
    s += dpp_m<0x143, 0xc>(s);
    return s;
}
// softplus(z) from the hardware exp2/log2 (log1p term dropped below 2^-24)
__device__ __forceinline__ float softplus_fast(float z) {
    const float y = fexp2(-fabsf(z) * kLog2e);
    return fmaxf(z, 0.f) + flog2(1.f + y) * 0.6931471805599453f;
}

__device__ __forceinline__ b8 as_b8(uint4 u) { return __builtin_bit_cast(b8, u); }
// sum of the two bf16 halves of w added to c (exact products, fp32 sum)
__device__ __forceinline__ float dot2_ones(uint32_t w, float c) {
    const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), one, c, false);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2));
}

constexpr int kNST = 3;             // key tiles in flight (LDS ring)

// K and V tiles are stored row-major, 128 bytes per key row, with the 16-byte
// chunks of each row XOR-swizzled (see k_off, v_off) against bank conflicts.
// The tiles are written by buffer-to-LDS transfers two tiles ahead of use.
struct __attribute__((aligned(16))) Slot {
    uint16_t K[kKT * kD];
    uint16_t V[kKT * kD];
    float Z[kWaves][kKT];         // decay logits of the tile, one copy per wave
    float B[kWaves][kKT];         // per wave: -c_s / scale, computed from Z
};

// K: chunk c of key row r sits at position c ^ fk(r), fk using only r mod 32,
// so that the two 32-row halves share per-lane offsets; eight consecutive rows
// (and the same-parity rows of sixteen) fall on distinct positions.
__device__ __forceinline__ int fk(int row) { return ((row & 31) ^ ((row & 31) >> 3)) & 7; }
__device__ __forceinline__ int k_off(int row, int c) { return row * 128 + ((c ^ fk(row)) << 4); }
// V: only the two low chunk bits are swizzled, by r mod 4, which keeps the
// transposing reads' addresses a per-lane constant plus immediates.
__device__ __forceinline__ int v_pos(int row, int c) { return (c & 4) | ((c & 3) ^ (row & 3)); }
__device__ __forceinline__ int v_off(int row, int c) { return row * 128 + (v_pos(row, c) << 4); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// Per-head buffer resource: loads past `bytes` return zero, which pads the
// ragged last tile without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Start the transfers of key tile s0 into ring slot st: wave w fills key rows
// 16w..16w+15 of K and V (two 1 KB transfers each; lane l of a transfer lands
// at byte 16 l, so it fetches the chunk the swizzle places there) and its own
// copy of the 64 decay logits.  Five transfers per lane per tile.
__device__ __forceinline__ void issue_tile(Slot& sl, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           __amdgpu_buffer_rsrc_t rz, int s0, int w, int lane) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = 16 * w + 8 * n + (lane >> 3);
        const int p = lane & 7;                       // position this lane fills
        const int ck = p ^ fk(r);                     // logical chunk stored there (the maps are involutions)
        const int cv = v_pos(r, p);
        char* kd = reinterpret_cast<char*>(sl.K) + (16 * w + 8 * n) * 128;
        char* vd = reinterpret_cast<char*>(sl.V) + (16 * w + 8 * n) * 128;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)kd, 16, (uint32_t)((s0 + r) * kD + 8 * ck) * 2, 0, 0,
                                                 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)vd, 16, (uint32_t)((s0 + r) * kD + 8 * cv) * 2, 0, 0,
                                                 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)sl.Z[w], 4, (uint32_t)(s0 + lane) * 4, 0, 0, 0);
}

// A operand of S^T = K Q^T: key row 32 kb + lo, dims 16 ks + 8 g .. + 7
__device__ __forceinline__ b8 k_operand(const Slot& sl, int kb, int ks, int lo, int g) {
    const char* t = reinterpret_cast<const char*>(sl.K);
    return as_b8(*reinterpret_cast<const uint4*>(t + k_off(32 * kb + lo, 2 * ks + g)));
}

// A operand of O^T = V^T P^T for value columns 32 mb .. + 31 and the key
// group 32 kb + 16 u: lane (c, g) needs V[key][c] for keys 4g..4g+3 and
// 8+4g..8+4g+3 of the group.  Two transposing reads: inside a 16-lane group,
// lane 4j + r addresses 4 columns c0 + 4r .. + 3 of key row base + j, and lane
// l then receives column c0 + l of the four rows base .. base + 3.
__device__ __forceinline__ b8 vt_operand(const Slot& sl, int kb, int mb, int u, int lane) {
    const int G = lane >> 4, m16 = lane & 15, j = m16 >> 2, r = m16 & 3;
    const int g = G >> 1, half = G & 1;
    const int col = 32 * mb + 16 * half + 4 * r;
    const int row = 32 * kb + 16 * u + 4 * g + j;
    const char* t = reinterpret_cast<const char*>(sl.V);
    const int sub = (col & 7) * 2;
    const s4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(t + v_off(row, col >> 3) + sub));
    const s4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(t + v_off(row + 8, col >> 3) + sub));
    const uint2 a = __builtin_bit_cast(uint2, x0), b = __builtin_bit_cast(uint2, x1);
    return as_b8(make_uint4(a.x, a.y, b.x, b.y));
}

// The wave's decay bias for the tile: with a_s = softplus(z_s) for keys up to
// E (0 after it), bias_s = -(sum of a over s+1 .. tile end + M) / scale, where
// M is the sum over the later tiles already visited.
__device__ __forceinline__ void tile_bias(Slot& sl, int w, int lane, int s0, int E, float& M,
                                          float inv_scale) {
    const float a = (s0 + lane <= E) ? softplus_fast(sl.Z[w][lane]) : 0.f;
    const float incl = wave_scan(a);
    const float total = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
    sl.B[w][lane] = -((total - incl) + M) * inv_scale;
    M += total;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the row is written before the wave reads it back
}

__device__ __forceinline__ f16v bias_init(const Slot& sl, int w, int kb, int g) {
    f16v C;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const float4 c4 = *reinterpret_cast<const float4*>(&sl.B[w][32 * kb + 8 * a + 4 * g]);
        C[4 * a] = c4.x;
        C[4 * a + 1] = c4.y;
        C[4 * a + 2] = c4.z;
        C[4 * a + 3] = c4.w;
    }
    return C;
}

// Probabilities of one 32-key x 32-query score block as two bf16 B operands;
// the row sum is taken over the rounded values the PV product uses.
__device__ __forceinline__ void probs(const f16v& S, float nm, float scl, float& l, b8 (&P)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = fexp2(fmaf(S[8 * u + 2 * e], scl, nm));
            const float p1 = fexp2(fmaf(S[8 * u + 2 * e + 1], scl, nm));
            wd[e] = pack2(p0, p1);
            l = dot2_ones(wd[e], l);
        }
        P[u] = as_b8(make_uint4(wd[0], wd[1], wd[2], wd[3]));
    }
}

__device__ __forceinline__ void rescale(float mx, float& m, float& l, f16v (&O)[2], float scl) {
    const float mn = fmaxf(m, mx);
    const float alpha = fexp2((m - mn) * scl);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        O[0][i] *= alpha;
        O[1][i] *= alpha;
    }
    m = mn;
}

// One 32-key block of scores for one 32-query block (diagonal tiles): softmax
// statistics update (running max m, partial sum l over this lane half's keys,
// rescale of O) and the probabilities as two bf16 B operands.
__device__ __forceinline__ void softmax_block(f16v S, float& m, float& l, f16v (&O)[2], b8 (&P)[2], float scl,
                                              float lazy) {
    float mx = S[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[i]);
    mx = half_max(mx);
    if (__any(mx > m + lazy)) rescale(mx, m, l, O, scl);
    probs(S, -m * scl, scl, l, P);
}

// A 64-key tile wholly before this wave's queries, in two 32-key halves (the
// later keys first): per half, the two query blocks' score MFMAs, one
// max / rescale decision, then probabilities and the PV products.
__device__ __forceinline__ void tile_full(const Slot& sl, int w, int lane, const b8 (&Qop)[2][4],
                                          f16v (&O)[2][2], float (&m)[2], float (&l)[2], float scl, float lazy) {
    const int lo = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kb = 1; kb >= 0; --kb) {
        f16v S[2];
        {
            b8 Kop[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) Kop[ks] = k_operand(sl, kb, ks, lo, g);
            const f16v C = bias_init(sl, w, kb, g);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                S[qb] = mfma(Kop[0], Qop[qb][0], C);
#pragma unroll
                for (int ks = 1; ks < 4; ++ks) S[qb] = mfma(Kop[ks], Qop[qb][ks], S[qb]);
            }
        }
        float mx[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float x = S[qb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) x = fmaxf(x, S[qb][i]);
            mx[qb] = half_max(x);
        }
        if (__any(mx[0] > m[0] + lazy || mx[1] > m[1] + lazy)) {
            rescale(mx[0], m[0], l[0], O[0], scl);
            rescale(mx[1], m[1], l[1], O[1], scl);
        }
        b8 P[2][2];
        // The exponentials at a raised issue priority: the two waves of a SIMD then
        // drift out of phase, one in its exp/fma stream while the other issues MFMAs
        // (measured: -11 % for the kernel at 2x16x8192).
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) probs(S[qb], -m[qb] * scl, scl, l[qb], P[qb]);
        __builtin_amdgcn_s_setprio(0);
        b8 Vop[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int u = 0; u < 2; ++u) Vop[mb][u] = vt_operand(sl, kb, mb, u, lane);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int u = 0; u < 2; ++u) O[qb][mb] = mfma(Vop[mb][u], P[qb][u], O[qb][mb]);
    }
}

// The diagonal tile of a wave: per 32-key block, causal mask inside the
// blocks on the diagonal, blocks above it skipped.
__device__ __forceinline__ void tile_diag(const Slot& sl, int w, int lane, const b8 (&Qop)[2][4],
                                          f16v (&O)[2][2], float (&m)[2], float (&l)[2], float scl, float lazy) {
    const int lo = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kb = 1; kb >= 0; --kb) {
        b8 Kop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Kop[ks] = k_operand(sl, kb, ks, lo, g);
        const f16v C = bias_init(sl, w, kb, g);
        b8 P[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            if (kb > qb) continue;
            f16v S = C;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) S = mfma(Kop[ks], Qop[qb][ks], S);
            if (kb == qb) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        if (8 * a + 4 * g + b > lo) S[4 * a + b] = -INFINITY;
            }
            softmax_block(S, m[qb], l[qb], O[qb], P[qb], scl, lazy);
        }
        b8 Vop[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int u = 0; u < 2; ++u) Vop[mb][u] = vt_operand(sl, kb, mb, u, lane);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            if (kb > qb) continue;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int u = 0; u < 2; ++u) O[qb][mb] = mfma(Vop[mb][u], P[qb][u], O[qb][mb]);
        }
    }
}

struct WaveState {
    f16v O[2][2];
    float m[2], l[2], M;
};

// One key tile j from slot `cur` while the transfers of tile j - 2 go into
// slot `nxt` (the slot tile j + 1 used).  The slots are distinct shared
// arrays, so the compiler can tell the reads of `cur` from the transfers in
// flight into the other two and needs no wait for them.
__device__ __forceinline__ void tile_step(Slot* __restrict__ curp, Slot* __restrict__ nxtp, int j, int w, int lane, int jdiag, int Ew,
                                          bool wact, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          __amdgpu_buffer_rsrc_t rz, const b8 (&Qop)[2][4], WaveState& ws, float scl,
                                          float lazy, float inv_scale) {
    Slot& cur = *curp;
    Slot& nxt = *nxtp;
    // this wave's transfers of tile j have landed (those of tile j - 1 may not)
    if (j >= 1) __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
    else __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
    // every wave's transfers of tile j are visible and every wave is done with
    // tile j + 1, whose slot is refilled next
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The tile's bias row before the next transfers are issued: where the compiler has
    // lost track of which slot a transfer in flight targets (at the top of the loop), the
    // first LDS access after it waits for every transfer, and this way those are at least
    // a tile old.
    const bool act = wact && j <= jdiag;
    if (act) tile_bias(cur, w, lane, j * kKT, Ew, ws.M, inv_scale);
    if (j >= 2) issue_tile(nxt, rk, rv, rz, (j - 2) * kKT, w, lane);
    if (act) {
        if (j < jdiag) tile_full(cur, w, lane, Qop, ws.O, ws.m, ws.l, scl, lazy);
        else tile_diag(cur, w, lane, Qop, ws.O, ws.m, ws.l, scl, lazy);
    }
}

__global__ void __launch_bounds__(kThreads, 2)
exp_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                const float* __restrict__ z, uint16_t* __restrict__ out, int T, int nqt, int nbh, float scale,
                float* __restrict__ row_stat, const float* __restrict__ cw, const float* __restrict__ cb,
                const uint16_t* __restrict__ cprev, int H) {
    __shared__ Slot slot0, slot1, slot2;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lo = lane & 31, g = lane >> 5;
    const int qt = nqt - 1 - (int)(blockIdx.x / nbh);   // longest query tiles first
    const int bh = blockIdx.x % nbh;
    const size_t base = (size_t)bh * T;
    const int t0 = qt * kQT;
    const int E = min(T, t0 + kQT) - 1;
    const int jE = E / kKT;
    const int tw = t0 + w * kQW;                       // first query of this wave
    const bool wact = tw < T;
    const int Ew = min(T - 1, tw + kQW - 1);
    const int jdiag = tw / kKT;
    const uint32_t hb = (uint32_t)T * kD * 2;
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(q + base * kD, hb), rk = head_rsrc(k + base * kD, hb),
                                 rv = head_rsrc(v + base * kD, hb), rz = head_rsrc(z + base, (uint32_t)T * 4);
    const float scl = scale * kLog2e;
    const float inv_scale = 1.f / scale;
    const float lazy = kLazy / scl;

    // queries as B operands: lane (lo, g) holds query tw + 32 qb + lo, dims 16 ks + 8 g .. + 7
    b8 Qop[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int t = tw + 32 * qb + lo;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Qop[qb][ks] = as_b8(ld16(rq, (uint32_t)(t * kD + 16 * ks + 8 * g) * 2));
        }
    }
    if (cw != nullptr) {
        // input convolution of the queries (twomamba_fwd_conv): each row with the raw row
        // before it (the cached one, or zeros, before token 0); rows past T stay zero
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Conv8 c8;
            conv8_load(c8, cw, cb, (size_t)(bh % H) * kD + 16 * ks + 8 * g);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int t = tw + 32 * qb + lo;
                uint4 xp = make_uint4(0u, 0u, 0u, 0u);
                if (t > 0) xp = ld16(rq, (uint32_t)((t - 1) * kD + 16 * ks + 8 * g) * 2);
                else if (cprev) xp = *reinterpret_cast<const uint4*>(cprev + (size_t)bh * 3 * kD + 16 * ks + 8 * g);
                const uint4 x = __builtin_bit_cast(uint4, Qop[qb][ks]);
                Qop[qb][ks] = as_b8(t < T ? conv8_bf16(c8, x, xp) : make_uint4(0u, 0u, 0u, 0u));
            }
        }
    }

    WaveState ws;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ws.O[qb][0][i] = ws.O[qb][1][i] = 0.f;
        ws.m[qb] = -INFINITY;
        ws.l[qb] = 0.f;
    }
    ws.M = 0.f;

    // Ring of three key-tile slots, two tiles in flight ahead of the one in
    // use: tile j lives in slot (jE - j) mod 3.
    issue_tile(slot0, rk, rv, rz, jE * kKT, w, lane);
    if (jE >= 1) {
        issue_tile(slot1, rk, rv, rz, (jE - 1) * kKT, w, lane);
        __builtin_amdgcn_s_waitcnt(0x0F7A);   // vmcnt(10): the query operands have landed
    } else {
        __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
    }
    for (int j = jE; j >= 0; j -= 3) {
        tile_step(&slot0, &slot2, j, w, lane, jdiag, Ew, wact, rk, rv, rz, Qop, ws, scl, lazy, inv_scale);
        if (j - 1 < 0) break;
        tile_step(&slot1, &slot0, j - 1, w, lane, jdiag, Ew, wact, rk, rv, rz, Qop, ws, scl, lazy, inv_scale);
        if (j - 2 < 0) break;
        tile_step(&slot2, &slot1, j - 2, w, lane, jdiag, Ew, wact, rk, rv, rz, Qop, ws, scl, lazy, inv_scale);
    }

    if (!wact) return;
    // log-sum-exp of the true logits: the accumulator held scale^-1 (scale q.k - c_s)
    // with c_s the softplus sum from s+1 to the wave end Ew, so add back c_t
    float csuf = 0.f;
    if (row_stat) {
        const float sp = (tw + lane <= Ew) ? softplus_fast(z[base + tw + lane]) : 0.f;
        const float incl = wave_scan(sp);
        csuf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63)) - incl;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int t = tw + 32 * qb + lo;
        const float lt = half_sum(ws.l[qb]);
        const float inv = 1.f / lt;
        const float ct = __shfl(csuf, 32 * qb + lo);
        if (t >= T) continue;
        if (row_stat && g == 0)   // log2 of the sum, converted to the natural log
            row_stat[base + t] = scale * ws.m[qb] + __builtin_amdgcn_logf(lt) * 0.6931471805599453f + ct;
        uint16_t* o = out + (base + t) * kD;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int c = 32 * mb + 8 * a + 4 * g;
                const uint2 wv = make_uint2(pack2(ws.O[qb][mb][4 * a] * inv, ws.O[qb][mb][4 * a + 1] * inv),
                                            pack2(ws.O[qb][mb][4 * a + 2] * inv, ws.O[qb][mb][4 * a + 3] * inv));
                *reinterpret_cast<uint2*>(o + c) = wv;
            }
    }
}

}  // namespace

bool mfma_exp_supported(const FwdArgs& a) {
    // The bias enters the accumulator divided by the scale: positive, not tiny.  A
    // head's rows are addressed through a buffer resource with 32-bit byte offsets
    // formed in int arithmetic (row * 64 * 2 bytes): heads of 2^24 tokens or more run
    // on the reference kernel instead.
    return a.dtype == TWOMAMBA_BF16 && a.dk == kD && a.dv == kD && a.scale > 1e-20f && a.T > 0 &&
           (size_t)a.T * kD * 2 < ((size_t)1 << 31) && (size_t)a.B * a.H > 0;
}

int mfma_exp_fwd(const FwdArgs& a) {
    const int nbh = a.B * a.H;
    const int nqt = (a.T + kQT - 1) / kQT;
    ktimer_begin(a.timer, "exp_mfma", a.stream);
    hipLaunchKernelGGL(exp_mfma_kernel, dim3((unsigned)nbh * nqt), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.z, (uint16_t*)a.out, a.T,
                       nqt, nbh, a.scale, a.row_stat, a.conv_w, a.conv_b, (const uint16_t*)a.conv_prev, a.H);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace twm
