// MFMA kernels of the 2Mamba chunked forward for d_k = d_v = 64 and bf16 inputs,
// "2Mamba2Furious", §5 (squared score, A-mask on the squared score, normalised
// by the sum of weights) with the second-order state of §2.
//
// Design (one head = (b, h)):
//  * The packed second-order state (2080 x 64 fp32) stays in MFMA accumulator
//    registers while a workgroup walks a segment of the sequence.  It does not
//    fit one CU (532 KB > 512 KB of VGPRs), so each head is split over two
//    workgroups by value column (32 columns each).
//  * Pair space.  The symmetric dim-pair matrix is cut into 4x4 blocks
//    (ib <= jb): 120 off-diagonal blocks and 16 diagonal ones, 136 "tiles" of
//    16 slots; slot r of tile (ib, jb) is the pair (4ib + r/4, 4jb + r%4).
//    Wave w owns the block rows ib = w and ib = 15 - w (17 tiles) x 2 column
//    tiles of 16x16 fp32 accumulators.  Diagonal tiles hold c * S (c = 2 above,
//    1 on, 0 below the dim diagonal) so the query side needs no per-slot weight;
//    off-diagonal tiles hold S and the query side reads 2 q_i.
//  * Per 64-token chunk c (S_c = state before the chunk):
//      readout  O = phi_q(Q) . S_c           MFMA, K = pair slots, computed as
//               O^T = S_c^T phi_q(Q)^T: the state accumulators are themselves
//               the A operand (a lane's rows 4g..4g+3 of two tiles are exactly
//               the K-slots it supplies)
//      intra    A = (Q K^T)^2 * exp(Gl_t - Gl_s), s <= t; A . [V | 1]  (MFMA)
//      den      q^T N q with the d x d normaliser N in accumulators  (MFMA)
//      update   S_{c+1} = e^Gam S_c + phi(K)^T diag(w) V   MFMA, K = tokens
//  * Operands are fp16: per chunk q and k are scaled by powers of two to
//    |x| < 1 (exact for bf16 inputs).  The intra weights and [V | 1] are bf16
//    instead: a row whose weights are all tiny (its first token, or very strong
//    decay with q nearly orthogonal to k) would underflow fp16 and lose its
//    denominator, while bf16 keeps fp32's exponent range; the weights' rounding
//    enters numerator and denominator alike.  The accumulators carry a "frame"
//    (true value = acc * 2^lf) kept so that a running bound on |acc| stays at
//    or below 2^14, which makes the readout's fp16 conversion a bare convert.
//    The chunk decay is absorbed into the frame whenever the bound allows;
//    otherwise the accumulators are rescaled, or restarted from zero when the
//    decayed carry is below 2^-40 of the bound (it cannot change an fp32 sum).
//  * Long sequences are split into segments.  A first kernel computes the end
//    states of the stretches before the last segment as backward passes (a
//    plain accumulation with weights relative to the stretch's end), cutting
//    them into as many pieces as fill the CUs; a piece that crosses a segment
//    boundary ends one end state there and starts the next.  Each end state is
//    stored as fp16 with one power-of-two scale per slot and value half (2^-11
//    relative rounding, below that of the bf16 inputs).  The main kernel starts
//    segment g from the decayed sum of the end states before it, or, for heads
//    with many of them, from one slot that a scan kernel has turned into the
//    whole carry.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace twm {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bh8 __attribute__((ext_vector_type(8)));
typedef __bf16 bh4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;          // head dim (keys and values)
constexpr int kDV = 32;         // value columns per workgroup
constexpr int kC = 64;          // chunk length
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTiles = 17;      // pair tiles per wave
constexpr int kPairs = kD * (kD + 1) / 2;
constexpr int kLS = 72;         // LDS row stride in halves (144 B)
constexpr int kRow = 2 * kLS;   // ... in bytes
constexpr int kStateLane = kTiles * 2 * 4;            // fp32 state values per lane
constexpr int kStateHalf = kWaves * 64 * kStateLane;  // per workgroup (one value half)
static_assert(kStateHalf % 4 == 0, "fp16 slots are addressed in groups of four");
constexpr int kNormWG = kD * kD;                      // full d x d normaliser
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTarget = 14.f;                       // log2 of the accumulator bound

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4 mfma(bh8 a, bh8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }   // no denormal fix-up
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int pidx(int i, int j) { return i * kD - (i * (i - 1)) / 2 + (j - i); }

// Wave w owns block rows ib = w and ib = 15 - w.  Tile u: u = 0 and u = 16 are
// the diagonal blocks (w, w) and (15-w, 15-w); 1 <= u <= 15 - w is (w, w + u);
// otherwise (15 - w, u).
__device__ __forceinline__ void tile_block(int w, int u, int& ib, int& jb) {
    if (u == 0) {
        ib = jb = w;
    } else if (u == 16) {
        ib = jb = 15 - w;
    } else if (u <= 15 - w) {
        ib = w;
        jb = w + u;
    } else {
        ib = 15 - w;
        jb = u;
    }
}

// exponent e with x * 2^e in [0.5, 1) for x > 0; 0 for x == 0
__device__ __forceinline__ int unit_exp(float x) {
    if (!(x > 0.f)) return 0;
    return -__builtin_amdgcn_frexp_expf(x);   // x = m 2^e, m in [0.5, 1)
}

// DPP lane permutes inside a 16-lane row: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_ror:4, row_ror:8.  Applied in turn they give every lane of a row the value
// of every other lane.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float x) {   // sum over the 16 lanes sharing lane>>4
    x += dpp<0xb1>(x);
    x += dpp<0x4e>(x);
    x += dpp<0x124>(x);
    x += dpp<0x128>(x);
    return x;
}
__device__ __forceinline__ float rdl(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float wave_max(float x) {   // max over the wave
    x = fmaxf(x, dpp<0xb1>(x));
    x = fmaxf(x, dpp<0x4e>(x));
    x = fmaxf(x, dpp<0x124>(x));
    x = fmaxf(x, dpp<0x128>(x));
    return fmaxf(fmaxf(rdl(x, 0), rdl(x, 16)), fmaxf(rdl(x, 32), rdl(x, 48)));
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_m(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xf, true));
}
// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each 16-lane
// row, then the total of row 0 (row 2) is added to row 1 (row 3) and the total of
// rows 0-1 to rows 2-3.
__device__ __forceinline__ float wave_scan(float s) {
    s += dpp_m<0x111, 0xf>(s);
    s += dpp_m<0x112, 0xf>(s);
    s += dpp_m<0x114, 0xf>(s);
    s += dpp_m<0x118, 0xf>(s);
    s += dpp_m<0x142, 0xa>(s);
    s += dpp_m<0x143, 0xc>(s);
    return s;
}
// g = -softplus(z) from the hardware exp2/log2: for exp(-|z|) below 2^-24 the
// log1p term is dropped (an absolute error below 2^-24 in g).
__device__ __forceinline__ float decay_log_fast(float z) {
    const float y = fexp2(-fabsf(z) * kLog2e);
    return -(fmaxf(z, 0.f) + flog2(1.f + y) * 0.6931471805599453f);
}
// unit_exp of the largest |k| over this lane's 8 dims, 127 when all are 0 (no constraint)
__device__ __forceinline__ int8_t lane_kexp(const float* kv) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(kv[i]));
    return (int8_t)(m > 0.f ? max(-120, min(120, unit_exp(m))) : 127);
}
// Per-token key exponent of the state update's operands.  A key 2^-delta times the
// chunk's largest would, at the chunk's scale, give pair products near 2^-2delta: fp16
// subnormals with few bits left.  Half of delta goes onto the key (the phi(K)
// operand) and the other half stays on the weighted value and key operands, whose
// scale is 2^-e per key factor, so that both stay normal for delta up to about 20.
// The products, and with them the accumulators, do not change.
__device__ __forceinline__ int token_kexp(const int8_t (&row)[kWaves], int ek) {
    const uint2 u = *reinterpret_cast<const uint2*>(row);
    int m = 127;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = min(m, (int)(int8_t)((u.x >> (8 * i)) & 0xffu));
        m = min(m, (int)(int8_t)((u.y >> (8 * i)) & 0xffu));
    }
    return m == 127 ? ek : ek + ((max(m, ek) - ek) >> 1);
}

__device__ __forceinline__ float uni(float x) {   // wave-uniform value into a scalar register
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 8 bf16 values (one 16-byte load) to fp32
__device__ __forceinline__ void unpack8(const uint4 u, float* o) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return bf16x2_rne(a, b); }

// Number of end-state boundaries in (0, x]: the segment boundaries k seg_chunks
// (1 <= k <= nseg - 1, the last one ending the segment pass) and the piece
// boundaries p piece_chunks (1 <= p < pieces) that are not segment boundaries.
// For the chunk x where a virtual segment starts this is its index among the
// head's end states; for the start of segment s, the number of end states
// before it.
__host__ __device__ inline int vseg_index(int x, int seg_chunks, int nseg, int piece_chunks, int pieces) {
    if (x <= 0) return 0;
    int n = x / seg_chunks;
    n = n < nseg - 1 ? n : nseg - 1;
    for (int p = 1; p < pieces && p * piece_chunks <= x; ++p)
        if ((p * piece_chunks) % seg_chunks != 0) ++n;
    return n;
}

// Raw inputs of one chunk, one token per lane: lane t of wave w holds dims
// 8w..8w+7 of q and k of token t, waves 0..3 also value columns 8w..8w+7 of
// this workgroup's half, every wave the decay logit.  Tokens past T read as 0.
struct Raw {
    uint4 q, k, v;
    float z;
};

template <bool kWithQ>
__device__ __forceinline__ void fetch(Raw& r, const bf16* q, const bf16* k, const bf16* v, const float* z,
                                      size_t tok_base, int T, int t0, int lane, int w, int col0) {
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    r.q = r.k = r.v = z4;
    r.z = 0.f;
    if (t0 + lane < T) {
        // the logit first: the wait for the rows (before the maxima are published) then
        // retires it as well, and the next chunk's first use of it waits for nothing,
        // in particular not for the output stores issued after these loads
        r.z = z[tok_base + t0 + lane];
        const size_t row = (tok_base + t0 + lane) * kD;
        if (kWithQ) r.q = *reinterpret_cast<const uint4*>(q + row + 8 * w);
        r.k = *reinterpret_cast<const uint4*>(k + row + 8 * w);
        if (w < 4) r.v = *reinterpret_cast<const uint4*>(v + row + col0 + 8 * w);
    }
}

struct Smem {
    _Float16 Q[kC][kLS];        // q~ [t][d]
    _Float16 K[kC][kLS];        // k~ [t][d]
    _Float16 KT[kD][kLS];       // k~^T [d][t]
    _Float16 WKT[kD][kLS];      // normaliser update operand (w k)^T [d][t]
    _Float16 WVT[kDV][kLS];     // state update operand (w v)^T [n][t]
    __bf16 VT[kDV + 16][kLS];   // intra operand [v | 1]^T [n][t]; rows 32..47 are ones
    __bf16 A[kC][kLS];          // intra weights [t][s]; bf16 for fp32's exponent range
    _Float16 NT[kD][kLS];       // normaliser (fp16) [j][i]
    float Op[kWaves][kC][kDV + 4];   // per-wave readout partials
    float Oin[kC][kDV + 4];     // intra numerator
    float Dint[kC];             // intra denominator
    float Dinter[2][kC];        // normaliser readout partials
    float Gl[2][kC];            // chunk-local inclusive prefix of g, by chunk parity
    float qrow[kC][kWaves];     // per token, each wave's max |q scale| over its 8 dims
    alignas(8) int8_t kexp[kC][kWaves];   // per token, unit_exp of each wave's max |k| over its 8 dims (127: all 0)
    float red[2][kWaves][4];    // per-wave maxima of |k| [1], |v| [2], by chunk parity
    int erow[2][kC];            // per-token query exponent, by chunk parity
    int zero;
};

struct SmemSeg {
    _Float16 KT[kD][kLS];
    _Float16 WKT[kD][kLS];
    _Float16 WVT[kDV][kLS];
    alignas(8) int8_t kexp[kC][kWaves];
    float red[2][kWaves][4];
    int zero;
};

// ---------------------------------------------------------------------------
// Update of the 17 x 2 state tiles of this wave from the chunk's K^T and (w v)^T in
// LDS, tile by tile (kZero: start from zero).  The segment pre-pass uses this order:
// the token-half order of update_tiles below needs more registers than it has left.
template <bool kZero, typename SM>
__device__ __forceinline__ void update_tiles_seg(f4 (&S)[kTiles][2], const SM& sm, int wl, int kg, int gq, int bq4,
                                             _Float16 cslot, int l16) {
    const char* smb = reinterpret_cast<const char*>(&sm);
    h8 BV[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
            BV[kk][ct] = *reinterpret_cast<const h8*>(&sm.WVT[16 * ct + l16][32 * kk + 8 * kg]);
    // K^T byte addresses: per-lane bases for the two block rows, block column as immediate
    const int kt0 = (int)offsetof(SM, KT) + 16 * kg;
    const int aiA = kt0 + (4 * wl + gq) * kRow, ajA = kt0 + (4 * wl + bq4) * kRow;
    const int aiB = kt0 + (60 - 4 * wl + gq) * kRow, ajB = kt0 + bq4 * kRow;
    const int ajD = kt0 + (60 - 4 * wl + bq4) * kRow;
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
        int ai, aj;
        if (u == 0) {
            ai = aiA;
            aj = ajA;
        } else if (u == 16) {
            ai = aiB;
            aj = ajD;
        } else if (u <= 15 - wl) {
            ai = aiA;
            aj = ajA + u * 4 * kRow;
        } else {
            ai = aiB;
            aj = ajB + u * 4 * kRow;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const h8 ki = *reinterpret_cast<const h8*>(smb + ai + 64 * kk);
            const h8 kj = *reinterpret_cast<const h8*>(smb + aj + 64 * kk);
            h8 A = ki * kj;
            if (u == 0 || u == 16) A *= cslot;   // c * phi(k); zero on dead slots
            if (kZero && kk == 0) {
                S[u][0] = mfma(A, BV[0][0], f4{0.f, 0.f, 0.f, 0.f});
                S[u][1] = mfma(A, BV[0][1], f4{0.f, 0.f, 0.f, 0.f});
            } else {
                S[u][0] = mfma(A, BV[kk][0], S[u][0]);
                S[u][1] = mfma(A, BV[kk][1], S[u][1]);
            }
        }
    }
}

// The same update, token half (K = 32 tokens) outer: one half's (w v) operands and
// the row factors of the wave's two block rows are read once per half, and the two
// products into one accumulator are 17 tiles apart.  Used by the main kernel.
template <bool kZero, typename SM>
__device__ __forceinline__ void update_tiles(f4 (&S)[kTiles][2], const SM& sm, int wl, int kg, int gq, int bq4,
                                             _Float16 cslot, int l16) {
    const char* smb = reinterpret_cast<const char*>(&sm);
    // K^T byte addresses: per-lane bases for the two block rows, block column as immediate
    const int kt0 = (int)offsetof(SM, KT) + 16 * kg;
    const int aiA = kt0 + (4 * wl + gq) * kRow, ajA = kt0 + (4 * wl + bq4) * kRow;
    const int aiB = kt0 + (60 - 4 * wl + gq) * kRow, ajB = kt0 + bq4 * kRow;
    const int ajD = kt0 + (60 - 4 * wl + bq4) * kRow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const h8 BV0 = *reinterpret_cast<const h8*>(&sm.WVT[l16][32 * kk + 8 * kg]);
        const h8 BV1 = *reinterpret_cast<const h8*>(&sm.WVT[16 + l16][32 * kk + 8 * kg]);
        // row factors of block rows wl and 15 - wl; tiles 0..8 lie in row wl for every wave
        const h8 kiA = *reinterpret_cast<const h8*>(smb + aiA + 64 * kk);
        const h8 kiB = *reinterpret_cast<const h8*>(smb + aiB + 64 * kk);
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            h8 ki;
            int aj;
            if (u == 0) {
                ki = kiA;
                aj = ajA;
            } else if (u == 16) {
                ki = kiB;
                aj = ajD;
            } else if (u <= 8) {
                ki = kiA;
                aj = ajA + u * 4 * kRow;
            } else if (u <= 15 - wl) {
                ki = *reinterpret_cast<const h8*>(smb + aiA + 64 * kk);
                aj = ajA + u * 4 * kRow;
            } else {
                ki = *reinterpret_cast<const h8*>(smb + aiB + 64 * kk);
                aj = ajB + u * 4 * kRow;
            }
            const h8 kj = *reinterpret_cast<const h8*>(smb + aj + 64 * kk);
            h8 A = ki * kj;
            if (u == 0 || u == 16) A *= cslot;   // c * phi(k); zero on dead slots
            if (kZero && kk == 0) {
                S[u][0] = mfma(A, BV0, f4{0.f, 0.f, 0.f, 0.f});
                S[u][1] = mfma(A, BV1, f4{0.f, 0.f, 0.f, 0.f});
            } else {
                S[u][0] = mfma(A, BV0, S[u][0]);
                S[u][1] = mfma(A, BV1, S[u][1]);
            }
            // in pairs of tiles: left free, the scheduler hoists every tile's loads
            // and runs out of registers
            if (u & 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <typename SM>
__device__ __forceinline__ void update_norm(f4 (&N)[2], const SM& sm, int w, int l16, int kg) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int nt = 2 * w + x, nib = nt >> 2, njb = nt & 3;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const h8 a = *reinterpret_cast<const h8*>(&sm.KT[16 * nib + l16][32 * kk + 8 * kg]);
            const h8 b = *reinterpret_cast<const h8*>(&sm.WKT[16 * njb + l16][32 * kk + 8 * kg]);
            N[x] = mfma(a, b, N[x]);
        }
    }
}

// Frame choice for one accumulator family.  In: current frame lf, bound Mb of
// |acc| (<= 2^14), chunk log2 decay lg (<= 0), log2 of the bound of the chunk's
// new contribution in true units lc.  Out: new frame, multiplier of the old
// accumulators (1 = no multiply), zero-start flag, new bound.
struct Frame {
    float lf_new, ratio, mb_new;
    bool mul, zero;
};

__device__ __forceinline__ Frame choose_frame(float lf, float Mb, float lg, float lc) {
    Frame f;
    // Absorb the decay into the frame (no multiply) while the accumulator bound
    // stays within [2^10, 2^14]: large enough that the scaled operands keep fp16
    // precision, small enough that the readout's fp16 conversion cannot overflow.
    const float lf_d = lf + lg;
    const float e = lc - lf_d;   // log2 bound of the chunk's part in the decayed frame
    const float grow = (lc == -INFINITY) ? 0.f : fexp2(fminf(e, 64.f));
    const float mb_d = Mb + grow;
    if (mb_d <= 16384.f && mb_d >= 1024.f) {
        f.lf_new = lf_d;
        f.ratio = 1.f;
        f.mul = false;
        f.zero = false;
        f.mb_new = mb_d;
        return f;
    }
    // log2 of the whole bound in true units, log2(Mb 2^lf_d + 2^lc) = log2(mb_d) + lf_d
    // (the old part is negligible where grow was clamped)
    const float lt = (e > 64.f) ? lc : flog2(mb_d) + lf_d;
    float ln = (lt == -INFINITY) ? lf : ceilf(lt - kTarget);
    ln = fmaxf(ln, lf + lg - 100.f);
    f.lf_new = ln;
    f.ratio = fexp2(lf + lg - ln);
    f.zero = f.ratio < 0x1p-40f;
    f.mul = !f.zero;
    const float add = (lc == -INFINITY) ? 0.f : fexp2(lc - ln);
    f.mb_new = (f.zero ? 0.f : Mb * f.ratio) + add;
    return f;
}

// ---------------------------------------------------------------------------
// main kernel: one (head, segment, value half) per workgroup
__global__ void __launch_bounds__(kThreads, 1)
sq_main_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
               const float* __restrict__ z, bf16* __restrict__ out,
               const float* __restrict__ state_in, const float* __restrict__ norm_in,
               float* __restrict__ state_out, float* __restrict__ norm_out,
               const uint2* __restrict__ ws_state, const float* __restrict__ ws_norm,
               const float* __restrict__ ws_gam, int T, int nseg, int seg_chunks, float scale, int no_norm,
               float* __restrict__ row_stat, int scanned, const int* __restrict__ ws_exp, int pieces,
               int piece_chunks, int nvs) {
    __shared__ __attribute__((aligned(16))) Smem sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // All workgroups of one head (both value halves, every segment) go to the same
    // XCD (blocks b, b + 8, b + 16, ... are dispatched to one): the two halves read
    // the same q, k and z rows, and later segments read the same carry slots, so
    // most of those reads hit the L2 that the first reader filled.  A last group of
    // fewer than 8 heads keeps the plain order.
    int half, seg, bh;
    {
        const int b = blockIdx.x, per = 2 * nseg, nbh_ = (int)gridDim.x / per, grp = b / (8 * per);
        if ((grp + 1) * 8 <= nbh_) {
            const int within = b - grp * 8 * per, j = within >> 3;
            bh = grp * 8 + (within & 7);
            half = j & 1;
            seg = j >> 1;
        } else {
            half = b & 1;
            seg = (b >> 1) % nseg;
            bh = (b >> 1) / nseg;
        }
    }
    const int nc_total = (T + kC - 1) / kC;
    const int c_begin = seg * seg_chunks;
    const int c_end = min(nc_total, c_begin + seg_chunks);
    const int seg_T = min(T, c_end * kC);   // tokens past the segment's last read as zeros
    const size_t tok_base = (size_t)bh * T;
    const int col0 = half * kDV;

    f4 S[kTiles][2];
    f4 N[2];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) S[u][0] = S[u][1] = f4{0.f, 0.f, 0.f, 0.f};
    N[0] = N[1] = f4{0.f, 0.f, 0.f, 0.f};
    float lf = 0.f, lfn = 0.f;     // log2 frames: true value = acc * 2^lf
    float Mb = 0.f, Mn = 0.f;      // bounds on |acc|

    {
        const int lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
        float cacc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) cacc[b] = b < kg ? 0.f : (b == kg ? 1.f : 2.f);
        const bool from_abi = (seg == 0) && state_in != nullptr;
        if (from_abi || seg > 0) {
            float mx = 0.f, mnx = 0.f;
            if (from_abi) {
                const float* Sg = state_in + (size_t)bh * kPairs * kD;
#pragma unroll
                for (int u = 0; u < kTiles; ++u) {
                    int ib, jb;
                    tile_block(w, u, ib, jb);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const int i = 4 * ib + kg, j = 4 * jb + b;
                            float x = (i <= j) ? Sg[(size_t)pidx(i, j) * kD + col0 + 16 * ct + l16] : 0.f;
                            if (u == 0 || u == 16) x *= cacc[b];
                            S[u][ct][b] = x;
                            mx = fmaxf(mx, fabsf(x));
                        }
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int nt = 2 * w + x, nib = nt >> 2, njb = nt & 3;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int i = 16 * nib + 4 * kg + b, j = 16 * njb + l16;
                        N[x][b] = norm_in[(size_t)bh * kPairs + pidx(min(i, j), max(i, j))];
                        mnx = fmaxf(mnx, fabsf(N[x][b]));
                    }
                }
            } else {
                // carry into segment seg: sum over the virtual segments h before it of
                // exp(Gam_{h+1} + ... + Gam_{nv-1}) * dS_h (nv of them end at or before its start)
                const int ns1 = nvs;
                const int nv = vseg_index(seg * seg_chunks, seg_chunks, nseg, piece_chunks, pieces);
                float lw = 0.f;   // log2 weight of slot h, built from the newest one down
                // (scanned: slot nv-1 already holds the whole carry, see sq_carry_scan)
                const int h_end = scanned ? nv - 1 : 0;
                for (int h = nv - 1; h >= h_end; --h) {
                    const size_t slot = (size_t)(bh * ns1 + h) * 2 + half;
                    // fp16 slot with its own power-of-two scale, in two batches of loads,
                    // each all in flight before any is used
                    const float wgh = fexp2(lw - (float)ws_exp[slot]);
                    const uint2* Wh = ws_state + slot * (kStateHalf / 4) + (size_t)w * 64 * kTiles * 2;
#pragma unroll
                    for (int u0 = 0; u0 < kTiles; u0 += 9) {
                        uint2 xs[9][2];
#pragma unroll
                        for (int du = 0; du < 9; ++du)
#pragma unroll
                            for (int ct = 0; ct < 2; ++ct)
                                if (u0 + du < kTiles) xs[du][ct] = Wh[((u0 + du) * 2 + ct) * 64 + lane];
#pragma unroll
                        for (int du = 0; du < 9; ++du)
#pragma unroll
                            for (int ct = 0; ct < 2; ++ct)
                                if (u0 + du < kTiles) {
                                    const h4 hv = __builtin_bit_cast(h4, xs[du][ct]);
                                    S[u0 + du][ct] += wgh * f4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
                                }
                    }
                    const float wgt = fexp2(lw);   // the normaliser slots are fp32
                    const float* Ng = ws_norm + (size_t)(bh * ns1 + h) * kNormWG;
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int nt = 2 * w + x, nib = nt >> 2, njb = nt & 3;
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            N[x][b] += wgt * Ng[(16 * nib + 4 * kg + b) * kD + 16 * njb + l16];
                    }
                    lw += ws_gam[bh * ns1 + h] * kLog2e;
                }
#pragma unroll
                for (int u = 0; u < kTiles; ++u)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int b = 0; b < 4; ++b) mx = fmaxf(mx, fabsf(S[u][ct][b]));
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int b = 0; b < 4; ++b) mnx = fmaxf(mnx, fabsf(N[x][b]));
            }
            mx = wave_max(mx);
            mnx = wave_max(mnx);
            if (lane == 0) {
                sm.red[0][w][0] = mx;
                sm.red[0][w][1] = mnx;
            }
            __syncthreads();
            float a = 0.f, bb = 0.f;
            for (int i = 0; i < kWaves; ++i) {
                a = fmaxf(a, sm.red[0][i][0]);
                bb = fmaxf(bb, sm.red[0][i][1]);
            }
            __syncthreads();
            if (a > 0.f) {   // normalise the frames so the bounds start at 2^14
                lf = ceilf(log2f(a) - kTarget);
                const float f = exp2f(-lf);
#pragma unroll
                for (int u = 0; u < kTiles; ++u) {
                    S[u][0] *= f;
                    S[u][1] *= f;
                }
                Mb = a * f;
            }
            if (bb > 0.f) {
                lfn = ceilf(log2f(bb) - kTarget);
                const float f = exp2f(-lfn);
                N[0] *= f;
                N[1] *= f;
                Mn = bb * f;
            }
        }
    }

    // constant parts of LDS: ones rows of [V | 1]^T, the loop-opaque zero
    for (int e = tid; e < 16 * kLS; e += kThreads) sm.VT[kDV + e / kLS][e % kLS] = (__bf16)1.f;
    if (tid == 0) sm.zero = 0;

    Raw raw;
    // Per-wave maxima of |k|, |v| over the chunk rows in `raw` and of |scale q| per
    // token, published in red[c & 1] and qrow: the next barrier (the one that ends
    // the previous chunk) makes them visible to the scale and frame choice, so the
    // chunk needs no barrier of its own for them.
    auto publish_max = [&](int c_pub, int lane_, int wl_) {
        float qv[8], kv[8], vv[8];
        unpack8(raw.q, qv);
        unpack8(raw.k, kv);
        unpack8(raw.v, vv);
        float mq = 0.f, mk = 0.f, mv = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mq = fmaxf(mq, fabsf(qv[i]));
            mk = fmaxf(mk, fabsf(kv[i]));
            mv = fmaxf(mv, fabsf(vv[i]));
        }
        // max |q scale| = |scale| max |q| (rounding is monotone)
        sm.qrow[lane_][wl_] = mq * fabsf(scale);
        sm.kexp[lane_][wl_] = lane_kexp(kv);
        mk = wave_max(mk);
        mv = wave_max(mv);
        if (lane_ == 0) {
            sm.red[c_pub & 1][wl_][1] = mk;
            sm.red[c_pub & 1][wl_][2] = mv;
        }
    };
    if (c_begin < c_end) {
        fetch<true>(raw, q, k, v, z, tok_base, T, c_begin * kC, tid & 63, w, col0);
        publish_max(c_begin, tid & 63, w);
    }
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * kC;
        const int Lc = min(kC, T - t0);
        const int par = c & 1;
        // Lane-derived indices rebuilt from a value re-read from LDS every chunk (always
        // 0): address arithmetic then stays inside the loop instead of being hoisted
        // into registers.
        const int tidc = tid + sm.zero;
        const int lane = tidc & 63;
        const int l16 = lane & 15;
        const int kg = lane >> 4;
        const int gq = l16 >> 2, bq4 = l16 & 3;
        const int wl = __builtin_amdgcn_readfirstlane(tidc >> 6);

        // ------------------------------------------------ P1a: registers only (the chunk's
        // maxima were published before the barrier that ended the previous chunk)
        float qv[8], kv[8], vv[8];
        unpack8(raw.q, qv);
        unpack8(raw.k, kv);
        unpack8(raw.v, vv);
        const float g = (lane < Lc) ? decay_log_fast(raw.z) : 0.f;
        const float gl = wave_scan(g);                // Gl of token `lane`
        const float Gam = rdl(gl, 63);

        // ------------------------------------------------ P1b: scales, frames, operands
        float Mk = 0.f, Mv = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            Mk = fmaxf(Mk, sm.red[par][i][1]);
            if (i < 4) Mv = fmaxf(Mv, sm.red[par][i][2]);
        }
        // Per-token query scale: a row's weights, intra and inter, numerator and
        // denominator, all scale with the square of its query, so o_t does not depend
        // on it, and a query far smaller than the chunk's largest keeps its products
        // q_i q_j out of the fp16 subnormals.
        const f4 qm0 = *reinterpret_cast<const f4*>(&sm.qrow[lane][0]);
        const f4 qm1 = *reinterpret_cast<const f4*>(&sm.qrow[lane][4]);
        const float Mq = fmaxf(fmaxf(fmaxf(qm0[0], qm0[1]), fmaxf(qm0[2], qm0[3])),
                               fmaxf(fmaxf(qm1[0], qm1[1]), fmaxf(qm1[2], qm1[3])));
        Mk = uni(Mk);
        Mv = uni(Mv);
        const float lg = Gam * kLog2e;
        const int eq = max(-120, min(120, unit_exp(Mq)));   // per lane (token)
        const int ek = uni(max(-120, min(120, unit_exp(Mk))));
        const int evi = uni(max(-120, min(120, unit_exp(Mv) + 14)));
        const float lMk = (Mk > 0.f) ? flog2(Mk) : -INFINITY;
        const float lcs = (Mk > 0.f && Mv > 0.f) ? 7.f + 2.f * lMk + flog2(Mv) : -INFINITY;
        const float lcn = (Mk > 0.f) ? 6.f + 2.f * lMk : -INFINITY;
        const Frame fs = choose_frame(lf, Mb, lg, lcs);
        const Frame fn = choose_frame(lfn, Mn, lg, lcn);
        {
            // q scale 2^eq in one factor: the power of two is exact, so this rounds as
            // (q scale) 2^eq does
            const float sq = scale * ldexpf(1.f, eq), sk = ldexpf(1.f, ek);
            if (wl == 0) sm.erow[par][lane] = eq;
            const int et = token_kexp(sm.kexp[lane], ek);                      // the update's key exponent
            const float skt = ldexpf(1.f, et);
            const float wt = (lane < Lc) ? fexp2((Gam - gl) * kLog2e) : 0.f;   // w_t = exp(Gam - Gl_t)
            const float swk = wt * fexp2(-fn.lf_new - (float)et);             // (w k) operand, dN_acc = 2^-lfn dN
            const float swv = wt * fexp2(-fs.lf_new - 2.f * (float)et);       // (w v) operand, dS_acc = 2^-lf dS
            const float svi = ldexpf(1.f, evi);
            h8 q8, k8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qq = qv[i] * sq, kt = kv[i] * sk;
                q8[i] = (_Float16)qq;
                k8[i] = (_Float16)kt;
                sm.KT[8 * wl + i][lane] = (_Float16)(kv[i] * skt);
                sm.WKT[8 * wl + i][lane] = (_Float16)(kv[i] * swk);
            }
            *reinterpret_cast<h8*>(&sm.Q[lane][8 * wl]) = q8;
            *reinterpret_cast<h8*>(&sm.K[lane][8 * wl]) = k8;
            if (wl < 4) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    sm.WVT[8 * wl + i][lane] = (_Float16)(vv[i] * swv);
                    sm.VT[8 * wl + i][lane] = (__bf16)(vv[i] * svi);   // exact
                }
            }
            if (wl == 0) sm.Gl[par][lane] = gl;
            // normaliser of S_c to fp16 (|N| <= 2^14)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int nt = 2 * wl + x, nib = nt >> 2, njb = nt & 3;
                h4 t4;
#pragma unroll
                for (int b = 0; b < 4; ++b) t4[b] = (_Float16)N[x][b];
                *reinterpret_cast<h4*>(&sm.NT[16 * njb + l16][16 * nib + 4 * kg]) = t4;
            }
        }
        __syncthreads();   // B

        // ------------------------------------------------ P2: readout of S_c
        // Waves 4..7 share a SIMD with waves 0..3 and are the younger of each pair; left
        // to age order they finish the readout last and then run alone.  Raising their
        // issue priority for the readout evens the pair out.
        if (wl >= 4) __builtin_amdgcn_s_setprio(2);
        {
            f4 O[4][2];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) O[tb][0] = O[tb][1] = f4{0.f, 0.f, 0.f, 0.f};
            const char* smq = reinterpret_cast<const char*>(&sm);
            // The query factor q_i of a tile's rows depends only on the block row: read the
            // lane's two (dims 4 wl + kg and 4 (15 - wl) + kg, tokens 16 tb + l16) once per
            // chunk.  Off-diagonal tiles take 2 q_i (exact in fp16).
            const int rowq = kRow * l16;
            const int qrA = (int)offsetof(Smem, Q) + rowq + 8 * wl + 2 * kg;
            const int qrB = (int)offsetof(Smem, Q) + rowq + 8 * (15 - wl) + 2 * kg;
            h2 fA[2], fB[2];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int ro = 16 * kRow * tb;
                fA[tb >> 1][tb & 1] = *reinterpret_cast<const _Float16*>(smq + qrA + ro);
                fB[tb >> 1][tb & 1] = *reinterpret_cast<const _Float16*>(smq + qrB + ro);
            }
            const h2 fA2[2] = {fA[0] + fA[0], fA[1] + fA[1]};
            const h2 fB2[2] = {fB[0] + fB[0], fB[1] + fB[1]};
            const int qjA = (int)offsetof(Smem, Q) + rowq + 8 * wl;
            const int qjB = (int)offsetof(Smem, Q) + rowq;
            const int qjD = (int)offsetof(Smem, Q) + rowq + 8 * (15 - wl);
            // tile u: its row factors (packed by token block pairs) and the LDS address of
            // the four column factors q_j; tiles 1..8 lie in row wl for every wave
            auto tile_q = [&](int u, h2 (&f)[2], int& aj) {
                if (u == 0) {
                    f[0] = fA[0]; f[1] = fA[1];
                    aj = qjA;
                } else if (u == 16) {
                    f[0] = fB[0]; f[1] = fB[1];
                    aj = qjD;
                } else if (u <= 8 || u <= 15 - wl) {
                    f[0] = fA2[0]; f[1] = fA2[1];
                    aj = qjA + 8 * u;
                } else {
                    f[0] = fB2[0]; f[1] = fB2[1];
                    aj = qjB + 8 * u;
                }
            };
#pragma unroll
            for (int kp = 0; kp < 9; ++kp) {
                const int ua = 2 * kp, ub = 2 * kp + 1;
                h2 fa[2], fb[2] = {h2{0, 0}, h2{0, 0}};
                int aja, ajb = 0;
                tile_q(ua, fa, aja);
                if (ub < kTiles) tile_q(ub, fb, ajb);
                h8 B0, B1;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    B0[b] = (_Float16)S[ua][0][b];
                    B1[b] = (_Float16)S[ua][1][b];
                    B0[4 + b] = (ub < kTiles) ? (_Float16)S[ub][0][b] : (_Float16)0.f;
                    B1[4 + b] = (ub < kTiles) ? (_Float16)S[ub][1][b] : (_Float16)0.f;
                }
                // all LDS reads of this tile pair first, so one wait covers them
                h4 qja[4], qjb[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int ro = 16 * kRow * tb;
                    qja[tb] = *reinterpret_cast<const h4*>(smq + aja + ro);
                    if (ub < kTiles) qjb[tb] = *reinterpret_cast<const h4*>(smq + ajb + ro);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const _Float16 qa = fa[tb >> 1][tb & 1];
                    h8 A;
                    A[0] = qa * qja[tb][0]; A[1] = qa * qja[tb][1];
                    A[2] = qa * qja[tb][2]; A[3] = qa * qja[tb][3];
                    if (ub < kTiles) {
                        const _Float16 qb = fb[tb >> 1][tb & 1];
                        A[4] = qb * qjb[tb][0]; A[5] = qb * qjb[tb][1];
                        A[6] = qb * qjb[tb][2]; A[7] = qb * qjb[tb][3];
                    } else {
                        A[4] = A[5] = A[6] = A[7] = (_Float16)0.f;
                    }
                    // transposed product O^T = S^T phi_q^T: a lane ends with four consecutive
                    // value columns of one token (one 16-byte LDS write below)
                    O[tb][0] = mfma(B0, A, O[tb][0]);
                    O[tb][1] = mfma(B1, A, O[tb][1]);
                }
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    *reinterpret_cast<f4*>(&sm.Op[wl][16 * tb + l16][16 * ct + 4 * kg]) = O[tb][ct];
        }

        __builtin_amdgcn_s_setprio(0);
        // ------------------------------------------------ P3a: intra scores, den readout
        {
            // 16 tiles (tt, ts) of the 64 x 64 score matrix, two per wave; upper ones are zero
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int tile = 2 * wl + x, tt = tile >> 2, ts = tile & 3;
                // transposed scores X^T = K Q^T: a lane holds keys 4kg..4kg+3 of one query,
                // i.e. four consecutive entries of its row of A (one 8-byte LDS write)
                const int t = 16 * tt + l16;
                if (ts <= tt) {
                    f4 X = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const h8 a = *reinterpret_cast<const h8*>(&sm.Q[t][32 * kk + 8 * kg]);
                        const h8 b = *reinterpret_cast<const h8*>(&sm.K[16 * ts + l16][32 * kk + 8 * kg]);
                        X = mfma(b, a, X);
                    }
                    const float glt = sm.Gl[par][t];
                    const f4 gls = *reinterpret_cast<const f4*>(&sm.Gl[par][16 * ts + 4 * kg]);
                    bh4 av;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int s = 16 * ts + 4 * kg + b;
                        const float a = (s <= t) ? X[b] * X[b] * fexp2((glt - gls[b]) * kLog2e) : 0.f;
                        av[b] = (__bf16)a;
                    }
                    *reinterpret_cast<bh4*>(&sm.A[t][16 * ts + 4 * kg]) = av;
                } else {
                    *reinterpret_cast<bh4*>(&sm.A[t][16 * ts + 4 * kg]) = bh4{0, 0, 0, 0};
                }
            }
            // den readout: Y = Q N~, then sum_j Q[t][j] Y[t][j]
            const int tb = wl >> 1, jh = wl & 1;
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int jt = 2 * jh + c2;
                f4 Y = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const h8 a = *reinterpret_cast<const h8*>(&sm.Q[16 * tb + l16][32 * kk + 8 * kg]);
                    const h8 b = *reinterpret_cast<const h8*>(&sm.NT[16 * jt + l16][32 * kk + 8 * kg]);
                    Y = mfma(a, b, Y);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) part[b] += (float)sm.Q[16 * tb + 4 * kg + b][16 * jt + l16] * Y[b];
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float sred = sum16(part[b]);
                if (l16 == 0) sm.Dinter[jh][16 * tb + 4 * kg + b] = sred;
            }
        }
        __syncthreads();   // C

        // ------------------------------------------------ P3b: intra [A.V | rowsum A]
        {
            const int tb = wl & 3;
            const int nk = tb >= 2 ? 2 : 1;
            // transposed products (V^T A^T): a lane ends with four consecutive value columns of
            // one query
            if (wl < 4) {
                f4 Y0 = f4{0.f, 0.f, 0.f, 0.f}, Y1 = Y0;
                for (int kk = 0; kk < nk; ++kk) {
                    const bh8 a = *reinterpret_cast<const bh8*>(&sm.A[16 * tb + l16][32 * kk + 8 * kg]);
                    const bh8 b0 = *reinterpret_cast<const bh8*>(&sm.VT[l16][32 * kk + 8 * kg]);
                    const bh8 b1 = *reinterpret_cast<const bh8*>(&sm.VT[16 + l16][32 * kk + 8 * kg]);
                    Y0 = mfma(b0, a, Y0);
                    Y1 = mfma(b1, a, Y1);
                }
                *reinterpret_cast<f4*>(&sm.Oin[16 * tb + l16][4 * kg]) = Y0;
                *reinterpret_cast<f4*>(&sm.Oin[16 * tb + l16][16 + 4 * kg]) = Y1;
            } else {
                f4 Y = f4{0.f, 0.f, 0.f, 0.f};
                for (int kk = 0; kk < nk; ++kk) {
                    const bh8 a = *reinterpret_cast<const bh8*>(&sm.A[16 * tb + l16][32 * kk + 8 * kg]);
                    const bh8 b = *reinterpret_cast<const bh8*>(&sm.VT[kDV + l16][32 * kk + 8 * kg]);
                    Y = mfma(b, a, Y);
                }
                if (kg == 0) sm.Dint[16 * tb + l16] = Y[0];   // every row of the ones block is the row sum
            }
        }

        // ------------------------------------------------ P4: update (and next chunk's fetch)
        // Fetched and published in every chunk, the last one included (where nothing past
        // the segment is loaded and zeros are published that nothing reads): under a
        // branch of their own, the loads would count as possibly outstanding at the top
        // of the loop, and the waits there would also wait for this chunk's output stores.
        fetch<true>(raw, q, k, v, z, tok_base, seg_T, t0 + kC, lane, wl, col0);
        {
            const _Float16 cslot = (_Float16)(bq4 < gq ? 0.f : (bq4 == gq ? 1.f : 2.f));
            if (fs.mul) {
#pragma unroll
                for (int u = 0; u < kTiles; ++u) {
                    S[u][0] *= fs.ratio;
                    S[u][1] *= fs.ratio;
                }
            }
            if (fs.zero) update_tiles<true>(S, sm, wl, kg, gq, bq4, cslot, l16);
            else update_tiles<false>(S, sm, wl, kg, gq, bq4, cslot, l16);
            if (fn.zero) N[0] = N[1] = f4{0.f, 0.f, 0.f, 0.f};
            else if (fn.mul) {
                N[0] *= fn.ratio;
                N[1] *= fn.ratio;
            }
            update_norm(N, sm, wl, l16, kg);
        }
        publish_max(c + 1, lane, wl);   // rows fetched above
        __syncthreads();   // D

        // ------------------------------------------------ P5: combine and write out
        // o = (Oin 2^-evi + Osum r_num(t)) / (Dint + Dinter r_den(t)) after dropping the
        // common factor 2^-(2eq_t+2ek) of numerator and denominator.
        {
            const int t = tidc >> 3, n0 = (tidc & 7) * 4;
            if (t < Lc) {
                const float glt = sm.Gl[par][t] * kLog2e;
                const float r_num = fexp2(glt + lf + 2.f * (float)ek);
                const float r_den = fexp2(glt + lfn + 2.f * (float)ek);
                const float fin = ldexpf(1.f, -evi);
                const float den = fmaf(sm.Dinter[0][t] + sm.Dinter[1][t], r_den, sm.Dint[t]);
                const float back = fexp2(-2.f * (float)sm.erow[par][t] - 2.f * (float)ek);
                const float mul = no_norm ? back : (den == 0.f ? 0.f : __builtin_amdgcn_rcpf(den));
                f4 osum = *reinterpret_cast<const f4*>(&sm.Op[0][t][n0]);
#pragma unroll
                for (int ww = 1; ww < kWaves; ++ww) osum += *reinterpret_cast<const f4*>(&sm.Op[ww][t][n0]);
                const f4 oin = *reinterpret_cast<const f4*>(&sm.Oin[t][n0]);
                f4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = fmaf(oin[e], fin, osum[e] * r_num) * mul;
                *reinterpret_cast<uint2*>(out + (tok_base + t0 + t) * kD + col0 + n0) =
                    make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                // the weight sum in true units (the common factor dropped above put back)
                if (row_stat && half == 0 && n0 == 0) row_stat[tok_base + t0 + t] = den * back;
            }
        }
        lf = fs.lf_new;
        lfn = fn.lf_new;
        Mb = fs.mb_new;
        Mn = fn.mb_new;
    }

    // ---------------------------------------------------------------- state out
    if (state_out != nullptr && seg == nseg - 1) {
        const int lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
        const float f = exp2f(lf), fnn = exp2f(lfn);
        float* Sg = state_out + (size_t)bh * kPairs * kD;
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            int ib, jb;
            tile_block(w, u, ib, jb);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 4 * ib + kg, j = 4 * jb + b;
                    if (i <= j) {
                        float x = S[u][ct][b] * f;
                        if (u == 0 || u == 16) x = (b == kg) ? x : 0.5f * x;
                        Sg[(size_t)pidx(i, j) * kD + col0 + 16 * ct + l16] = x;
                    }
                }
        }
        if (half == 0) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int nt = 2 * w + x, nib = nt >> 2, njb = nt & 3;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 16 * nib + 4 * kg + b, j = 16 * njb + l16;
                    if (i <= j) norm_out[(size_t)bh * kPairs + pidx(i, j)] = N[x][b] * fnn;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Segment end states: one (head, segment < last, value half) per workgroup.
// dS_g = sum_{s in g} exp(g_{s+1} + ... + g_end) phi(k_s) v_s^T (plus the decayed
// caller state for g = 0), accumulated from the segment end backwards so that
// every weight is relative to the segment end and no accumulator is ever
// rescaled except when a chunk's contribution would overflow the frame.
template <bool kPieces>   // false: one piece per segment, no boundary inside a workgroup's range
__global__ void __launch_bounds__(kThreads, 1)
sq_segstate_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ z,
                   const float* __restrict__ state_in, const float* __restrict__ norm_in,
                   uint2* __restrict__ ws_state, float* __restrict__ ws_norm, float* __restrict__ ws_gam,
                   int* __restrict__ ws_exp, int T, int nseg, int seg_chunks, int pieces, int piece_chunks,
                   int nvs) {
    __shared__ __attribute__((aligned(16))) SmemSeg sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Both value halves of one (head, segment) go to the same XCD (blocks b and
    // b + 8 are dispatched to one), so the second half's reads of the rows both
    // halves use can hit the L2 that the first filled; a last group of fewer than 8 items
    // keeps the plain order.
    int half, rest;
    {
        const int b = blockIdx.x, nitems = (int)(gridDim.x >> 1), grp = b >> 4;
        if ((grp + 1) * 8 <= nitems) {
            rest = grp * 8 + (b & 7);
            half = (b >> 3) & 1;
        } else {
            rest = b >> 1;
            half = b & 1;
        }
    }
    const int piece = rest % pieces;
    const int bh = rest / pieces;
    const int span = (nseg - 1) * seg_chunks;   // segments before the last are full
    const int c_begin = piece * piece_chunks;
    const int c_end = min(span, c_begin + piece_chunks);
    // a segment boundary inside the piece (at most one, since piece_chunks <= seg_chunks)
    // ends the later virtual segment there: -1 if there is none
    const int c_next = (c_begin / seg_chunks + 1) * seg_chunks;
    const int split = kPieces && c_next < c_end ? c_next : -1;
    const size_t tok_base = (size_t)bh * T;
    const int col0 = half * kDV;

    f4 S[kTiles][2];
    f4 N[2];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) S[u][0] = S[u][1] = f4{0.f, 0.f, 0.f, 0.f};
    N[0] = N[1] = f4{0.f, 0.f, 0.f, 0.f};
    float lf = 0.f, lfn = 0.f, Mb = 0.f, Mn = 0.f;
    float lP = 0.f;   // log2 decay from the end of the current chunk to the segment end

    if (tid == 0) sm.zero = 0;
    Raw raw;
    fetch<false>(raw, k, k, v, z, tok_base, T, (c_end - 1) * kC, tid & 63, w, col0);
    __syncthreads();

    auto flush = [&](int x0, bool may_start) {
        // true end state (diagonal tiles weighted by c) of the virtual segment that starts at
        // chunk x0, plus the decayed caller state for the one at chunk 0 (may_start: x0 can
        // be 0; false where it cannot, so that the compiler drops that path there)
        const int lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
        const float f = exp2f(lf), fnn = exp2f(lfn), fin = exp2f(lP);
        const bool add_in = may_start && x0 == 0 && state_in != nullptr;
        float cacc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) cacc[b] = b < kg ? 0.f : (b == kg ? 1.f : 2.f);
        const size_t wsi = (size_t)bh * nvs + vseg_index(x0, seg_chunks, nseg, piece_chunks, pieces);
        const float* Sg = state_in ? state_in + (size_t)bh * kPairs * kD : nullptr;
        float mx = 0.f;
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            int ib, jb;
            tile_block(w, u, ib, jb);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f4 x = S[u][ct] * f;
                if (add_in) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int i = 4 * ib + kg, j = 4 * jb + b;
                        float s0 = (i <= j) ? Sg[(size_t)pidx(i, j) * kD + col0 + 16 * ct + l16] : 0.f;
                        if (u == 0 || u == 16) s0 *= cacc[b];
                        x[b] = fmaf(fin, s0, x[b]);
                    }
                }
                S[u][ct] = x;
#pragma unroll
                for (int b = 0; b < 4; ++b) mx = fmaxf(mx, fabsf(x[b]));
            }
        }
        // fp16 slot: values scaled by 2^e so that the largest stays below 2^14 (the
        // precision the readout's fp16 state operand has anyway); half the bytes for
        // the main kernel to read back
        mx = wave_max(mx);
        if (lane == 0) sm.red[0][w][0] = mx;
        __syncthreads();
        float M = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) M = fmaxf(M, sm.red[0][i][0]);
        // an all-zero slot takes the largest exponent, so that it adds next to nothing
        // to the bound the carry scan keeps
        const int e = uni(M > 0.f ? max(-120, min(120, unit_exp(M) + 14)) : 120);
        const float sc = ldexpf(1.f, e);
        uint2* Wh = ws_state + (wsi * 2 + half) * (kStateHalf / 4) + (size_t)w * 64 * kTiles * 2;
#pragma unroll
        for (int u = 0; u < kTiles; ++u)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const f4 x = S[u][ct] * sc;
                const h4 hv = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
                Wh[(u * 2 + ct) * 64 + lane] = __builtin_bit_cast(uint2, hv);
            }
        if (tid == 0) ws_exp[wsi * 2 + half] = e;
        if (half == 0) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int nt = 2 * w + x, nib = nt >> 2, njb = nt & 3;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 16 * nib + 4 * kg + b, j = 16 * njb + l16;
                    float val = N[x][b] * fnn;
                    if (add_in) val = fmaf(fin, norm_in[(size_t)bh * kPairs + pidx(min(i, j), max(i, j))], val);
                    ws_norm[wsi * kNormWG + i * kD + j] = val;
                }
            }
            if (tid == 0) ws_gam[wsi] = lP / kLog2e;
        }
        __syncthreads();   // the reductions above reuse LDS the next chunk writes
    };
    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * kC;
        const int par = c & 1;
        // re-derived from an LDS zero every chunk (kept out of registers across the loop),
        // masked to their ranges so that the address products stay 24-bit
        const int tidc = (tid + sm.zero) & (kThreads - 1);
        const int lane = tidc & 63;
        const int l16 = lane & 15;
        const int kg = lane >> 4;
        const int gq = l16 >> 2, bq4 = l16 & 3;
        const int wl = __builtin_amdgcn_readfirstlane(tidc >> 6) & (kWaves - 1);

        float kv[8], vv[8];
        unpack8(raw.k, kv);
        unpack8(raw.v, vv);
        const float g = decay_log_fast(raw.z);
        const float gl = wave_scan(g);
        const float Gam = rdl(gl, 63);
        float mk = 0.f, mv = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mk = fmaxf(mk, fabsf(kv[i]));
            mv = fmaxf(mv, fabsf(vv[i]));
        }
        sm.kexp[lane][wl] = lane_kexp(kv);
        mk = wave_max(mk);
        mv = wave_max(mv);
        if (lane == 0) {
            sm.red[par][wl][0] = mk;
            sm.red[par][wl][1] = mv;
        }
        __syncthreads();
        float Mk = 0.f, Mv = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            Mk = fmaxf(Mk, sm.red[par][i][0]);
            if (i < 4) Mv = fmaxf(Mv, sm.red[par][i][1]);
        }
        const int ek = max(-120, min(120, unit_exp(Mk)));
        const float lMk = (Mk > 0.f) ? flog2(Mk) : -INFINITY;
        // contributions of this chunk, relative to the segment end (decay lP folded in)
        const float lcs = (Mk > 0.f && Mv > 0.f) ? 7.f + 2.f * lMk + flog2(Mv) + lP : -INFINITY;
        const float lcn = (Mk > 0.f) ? 6.f + 2.f * lMk + lP : -INFINITY;
        const Frame fs = choose_frame(lf, Mb, 0.f, lcs);
        const Frame fn = choose_frame(lfn, Mn, 0.f, lcn);
        {
            const int et = token_kexp(sm.kexp[lane], ek);
            const float sk = ldexpf(1.f, et);
            const float lw = (Gam - gl) * kLog2e + lP;   // log2 weight of token `lane`
            const float swk = fexp2(lw - fn.lf_new - (float)et);
            const float swv = fexp2(lw - fs.lf_new - 2.f * (float)et);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sm.KT[8 * wl + i][lane] = (_Float16)(kv[i] * sk);
                sm.WKT[8 * wl + i][lane] = (_Float16)(kv[i] * swk);
            }
            if (wl < 4) {
#pragma unroll
                for (int i = 0; i < 8; ++i) sm.WVT[8 * wl + i][lane] = (_Float16)(vv[i] * swv);
            }
        }
        __syncthreads();
        if (c - 1 >= c_begin) fetch<false>(raw, k, k, v, z, tok_base, T, t0 - kC, lane, wl, col0);
        {
            const _Float16 cslot = (_Float16)(bq4 < gq ? 0.f : (bq4 == gq ? 1.f : 2.f));
            if (fs.mul) {
#pragma unroll
                for (int u = 0; u < kTiles; ++u) {
                    S[u][0] *= fs.ratio;
                    S[u][1] *= fs.ratio;
                }
            }
            if (fs.zero) update_tiles_seg<true>(S, sm, wl, kg, gq, bq4, cslot, l16);
            else update_tiles_seg<false>(S, sm, wl, kg, gq, bq4, cslot, l16);
            if (fn.zero) N[0] = N[1] = f4{0.f, 0.f, 0.f, 0.f};
            else if (fn.mul) {
                N[0] *= fn.ratio;
                N[1] *= fn.ratio;
            }
            update_norm(N, sm, wl, l16, kg);
        }
        lf = fs.lf_new;
        lfn = fn.lf_new;
        Mb = fs.mb_new;
        Mn = fn.mb_new;
        lP += Gam * kLog2e;
        if (kPieces && c == split) {   // [split, c_end) is complete: write it, start [c_begin, split) from zero
            flush(split, false);
#pragma unroll
            for (int u = 0; u < kTiles; ++u) S[u][0] = S[u][1] = f4{0.f, 0.f, 0.f, 0.f};
            N[0] = N[1] = f4{0.f, 0.f, 0.f, 0.f};
            lf = lfn = Mb = Mn = lP = 0.f;
        }
    }
    flush(c_begin, true);
}

// ---------------------------------------------------------------------------
// Inclusive scan of the segment end states, for heads split into many segments:
// slot h (h = 0..nseg-2) becomes the carry into segment h+1,
//     C_{h+1} = exp(Gam_h) C_h + dS_h,   C_1 = dS_0,
// so that each main-kernel workgroup reads one slot instead of summing all
// earlier ones (which costs a quadratic number of state reads).  One thread per
// four consecutive entries of a head's slots (both fp16 value halves, then the
// fp32 normaliser), sequential over the segments, the running carry in fp32.
// A state slot is stored as fp16 times 2^e with |entry| 2^e < 2^14; the carry's
// exponent comes from a bound every thread of the slot computes alike,
//     |C_{h+1}| <= 2^14 B_{h+1},   B_{h+1} = exp(Gam_h) B_h + 2^-e_h,
// and is written to its own array (the segment pass's exponents stay as read).
constexpr int kScanState = 2 * kStateHalf / 4;   // threads per head on the fp16 state
constexpr int kScanElems = kScanState + kNormWG / 4;

__global__ void __launch_bounds__(256)
sq_carry_scan(uint2* __restrict__ ws_state, float* __restrict__ ws_norm, const float* __restrict__ ws_gam,
              const int* __restrict__ ws_exp, int* __restrict__ ws_exps, int ns1, int etiles) {
    const int bh = blockIdx.x / etiles;
    const int e = (blockIdx.x % etiles) * 256 + threadIdx.x;
    if (e >= kScanElems) return;
    const float* gam = ws_gam + (size_t)bh * ns1;
    constexpr int U = 8;   // the chain is serial in h: loads run this many slots ahead
    if (e < kScanState) {
        const int half = (4 * e) / kStateHalf, off = (4 * e) % kStateHalf;
        uint2* p0 = ws_state + ((size_t)bh * ns1 * 2 + half) * (kStateHalf / 4) + off / 4;
        const size_t stride = (size_t)2 * kStateHalf / 4;   // uint2 per slot (two value halves)
        const int* ex = ws_exp + (size_t)bh * ns1 * 2 + half;
        int* exs = ws_exps + (size_t)bh * ns1 * 2 + half;
        const bool head = off == 0;   // one thread per half writes the exponents
        const auto unpack = [](uint2 u, float sc) {
            const h4 hv = __builtin_bit_cast(h4, u);
            return f4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]} * sc;
        };
        int e0 = ex[0];
        f4 c = unpack(p0[0], ldexpf(1.f, -e0));   // C_1 = dS_0, stored as it is
        float bnd = ldexpf(1.f, -e0);
        if (head) exs[0] = e0;
        const auto step = [&](int h, uint2 x, int eh, float g) {
            const float a = fexp2(g * kLog2e);
            const float sc = ldexpf(1.f, -eh);
            c = a * c + unpack(x, sc);
            bnd = fmaf(a, bnd, sc);
            const int en = max(-120, min(120, unit_exp(bnd)));
            const f4 y = c * ldexpf(1.f, en);
            const h4 hv = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
            p0[h * stride] = __builtin_bit_cast(uint2, hv);
            if (head) exs[(size_t)h * 2] = en;
        };
        int h = 1;
        for (; h + U <= ns1; h += U) {
            uint2 x[U];
            int eh[U];
            float g[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[u] = p0[(h + u) * stride];
                eh[u] = ex[(size_t)(h + u) * 2];
                g[u] = gam[h + u];   // segment h's own decay carries C_h across it
            }
#pragma unroll
            for (int u = 0; u < U; ++u) step(h + u, x[u], eh[u], g[u]);
        }
        for (; h < ns1; ++h) step(h, p0[h * stride], ex[(size_t)h * 2], gam[h]);
        return;
    }
    float* p0 = ws_norm + (size_t)bh * ns1 * kNormWG + 4 * (e - kScanState);
    const size_t stride = kNormWG;
    float4 c = *reinterpret_cast<const float4*>(p0);
    int h = 1;
    for (; h + U <= ns1; h += U) {
        float4 x[U];
        float g[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x[u] = *reinterpret_cast<const float4*>(p0 + (h + u) * stride);
            g[u] = gam[h + u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float a = fexp2(g[u] * kLog2e);
            c = make_float4(fmaf(a, c.x, x[u].x), fmaf(a, c.y, x[u].y), fmaf(a, c.z, x[u].z), fmaf(a, c.w, x[u].w));
            *reinterpret_cast<float4*>(p0 + (h + u) * stride) = c;
        }
    }
    for (; h < ns1; ++h) {
        const float4 x = *reinterpret_cast<const float4*>(p0 + h * stride);
        const float a = fexp2(gam[h] * kLog2e);
        c = make_float4(fmaf(a, c.x, x.x), fmaf(a, c.y, x.y), fmaf(a, c.z, x.z), fmaf(a, c.w, x.w));
        *reinterpret_cast<float4*>(p0 + h * stride) = c;
    }
}

// From this many segments on, the carries are scanned (sq_carry_scan) rather than
// summed by every workgroup.  Measured at 2x16x8192 (4 segments) the scan is not
// needed, at 1x16x32768 (8) the two cost the same, at 1x2x32768 (64) the scan
// takes the main kernel from 0.44 to 0.09 ms.
constexpr int kScanFrom = 9;

// The segment pass cuts the chunks before the last segment ((nseg - 1) seg_chunks
// of them) into `pieces` pieces of piece_chunks, one workgroup per (head, piece,
// value half): as many as fill the CUs, which the one-piece-per-segment split
// leaves partly idle (at 2x16x8192, 192 workgroups on 256 CUs).  A piece that
// crosses a segment boundary ends one end state there and starts the next, so
// the end states ("virtual segments") are the spans between consecutive
// boundaries of either kind; `nvs` of them per head, the carry into a segment is
// the decayed sum of those before its start.
struct Plan {
    int nseg, seg_chunks;
    int pieces, piece_chunks, nvs;
};

Plan plan_for(const FwdArgs& a) {
    const int nc = (a.T + kC - 1) / kC;
    const long nbh = (long)a.B * a.H;
    int want = (int)((256 + 2 * nbh - 1) / (2 * nbh));   // workgroups to fill 256 CUs
    want = std::max(1, std::min(want, nc / 4));             // at least 4 chunks per segment
    want = std::min(want, 64);
    const int sc = (nc + want - 1) / want;
    Plan p;
    p.seg_chunks = sc;
    p.nseg = (nc + sc - 1) / sc;
    const int ns1 = p.nseg - 1, span = ns1 * sc;
    p.pieces = ns1;
    p.piece_chunks = sc;
    if (ns1 > 0) {
        // pieces to fill the CUs (at most one boundary inside a piece: piece_chunks <= seg_chunks),
        // used when one piece per segment would leave at least a fifth of the CUs idle
        const int fill = (int)(256 / (2 * nbh));
        const int pc = fill > 0 ? (span + fill - 1) / fill : sc;
        if (fill * 4 >= ns1 * 5 && pc >= 4) {   // at least 4 chunks per piece, as per segment
            p.piece_chunks = pc;
            p.pieces = (span + pc - 1) / pc;
        }
    }
    p.nvs = ns1 > 0 ? vseg_index(span, sc, p.nseg, p.piece_chunks, p.pieces) : 0;
    return p;
}

// Workspace: the segment slots (when a head has more than one segment), then a
// staging copy of the caller's initial state for in-place resume.  With one
// segment only the normaliser needs staging: both value halves of a head read
// all of norm_in while half 0 writes norm_out; each half reads and writes only
// its own state columns, in the same threads.  With several segments the
// segment-0 workgroups read state_in and norm_in while the last segment's write
// state_out and norm_out, so both are staged.
struct WsLayout {
    size_t off_state, off_norm, off_gam, off_exp, off_exps, off_stage_s, off_stage_n, total;
};

WsLayout ws_layout(const FwdArgs& a, const Plan& p) {
    const size_t nbh = (size_t)a.B * a.H;
    const size_t ns1 = p.nseg > 1 ? (size_t)p.nvs : 0;   // end-state slots per head
    WsLayout L;
    L.off_state = 0;
    L.off_norm = align256(nbh * ns1 * 2 * kStateHalf * sizeof(_Float16));
    L.off_gam = align256(L.off_norm + nbh * ns1 * kNormWG * sizeof(float));
    L.off_exp = align256(L.off_gam + nbh * ns1 * sizeof(float));   // fp16 slots' scale exponents
    L.off_exps = align256(L.off_exp + nbh * ns1 * 2 * sizeof(int));   // the scanned carries' exponents
    L.off_stage_s = ns1 ? align256(L.off_exps + nbh * ns1 * 2 * sizeof(int)) : 0;
    const size_t stage_s = ns1 ? nbh * kPairs * kD * sizeof(float) : 0;
    L.off_stage_n = align256(L.off_stage_s + stage_s);
    L.total = align256(L.off_stage_n + nbh * kPairs * sizeof(float));
    return L;
}

int run(const FwdArgs& a) {
    const Plan p = plan_for(a);
    const WsLayout L = ws_layout(a, p);
    char* ws = (char*)a.ws;
    const bool slots = p.nseg > 1;
    uint2* wsS = slots ? (uint2*)(ws + L.off_state) : nullptr;   // fp16 x 4
    float* wsN = slots ? (float*)(ws + L.off_norm) : nullptr;
    float* wsG = slots ? (float*)(ws + L.off_gam) : nullptr;
    int* wsE = slots ? (int*)(ws + L.off_exp) : nullptr;
    int* wsEs = slots ? (int*)(ws + L.off_exps) : nullptr;
    // carries: scanned in place for many segments, else summed by each main workgroup
    const int scanned = p.nvs + 1 >= kScanFrom;
    const int nbh = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    const int no_norm = (a.flags & TWOMAMBA_FLAG_NO_NORM) != 0;
    const bf16* q = (const bf16*)a.q;
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    // in-place resume: read the caller's initial state from a staged copy (see WsLayout)
    const float* state_in = a.state_in;
    const float* norm_in = a.norm_in;
    if (a.state_in != nullptr && (a.state_in == a.state_out || a.norm_in == a.norm_out)) {
        const size_t nbh_ = (size_t)a.B * a.H;
        float* sn = (float*)(ws + L.off_stage_n);
        if (hipMemcpyAsync(sn, a.norm_in, nbh_ * kPairs * sizeof(float), hipMemcpyDeviceToDevice, st) != hipSuccess)
            return TWOMAMBA_ERR_DEVICE;
        norm_in = sn;
        if (p.nseg > 1) {
            float* ss = (float*)(ws + L.off_stage_s);
            if (hipMemcpyAsync(ss, a.state_in, nbh_ * kPairs * kD * sizeof(float), hipMemcpyDeviceToDevice, st) !=
                hipSuccess)
                return TWOMAMBA_ERR_DEVICE;
            state_in = ss;
        }
    }
    if (p.nseg > 1) {
        ktimer_begin(a.timer, "sq_segstate", a.stream);
        if (p.nvs > p.nseg - 1)
            hipLaunchKernelGGL(sq_segstate_kernel<true>, dim3(nbh * p.pieces * 2), dim3(kThreads), 0, st, k, v, a.z,
                               state_in, norm_in, wsS, wsN, wsG, wsE, a.T, p.nseg, p.seg_chunks, p.pieces,
                               p.piece_chunks, p.nvs);
        else
            hipLaunchKernelGGL(sq_segstate_kernel<false>, dim3(nbh * p.pieces * 2), dim3(kThreads), 0, st, k, v, a.z,
                               state_in, norm_in, wsS, wsN, wsG, wsE, a.T, p.nseg, p.seg_chunks, p.pieces,
                               p.piece_chunks, p.nvs);
        ktimer_end(a.timer, a.stream);
    }
    if (scanned) {
        const int etiles = (kScanElems + 255) / 256;
        ktimer_begin(a.timer, "sq_carry_scan", a.stream);
        hipLaunchKernelGGL(sq_carry_scan, dim3(nbh * etiles), dim3(256), 0, st, wsS, wsN, (const float*)wsG,
                           (const int*)wsE, wsEs, p.nvs, etiles);
        ktimer_end(a.timer, a.stream);
    }
    ktimer_begin(a.timer, "sq_mfma_main", a.stream);
    hipLaunchKernelGGL(sq_main_kernel, dim3(nbh * p.nseg * 2), dim3(kThreads), 0, st, q, k, v, a.z, (bf16*)a.out,
                       state_in, norm_in, a.state_out, a.norm_out, (const uint2*)wsS, (const float*)wsN,
                       (const float*)wsG, a.T, p.nseg, p.seg_chunks, a.scale, no_norm, a.row_stat, scanned,
                       (const int*)(scanned ? wsEs : wsE), p.pieces, p.piece_chunks, p.nvs);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

bool mfma_sq_supported(const FwdArgs& a) {
    return a.dtype == TWOMAMBA_BF16 && a.dk == 64 && a.dv == 64 && a.chunk == kC && a.T > 0 &&
           (size_t)a.B * a.H > 0;
}

size_t mfma_sq_workspace(const FwdArgs& a) { return ws_layout(a, plan_for(a)).total; }

int mfma_sq_fwd(const FwdArgs& a) { return run(a); }

}  // namespace twm
