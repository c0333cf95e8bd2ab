// MFMA kernels of the 2Mamba / 2Mamba-E backward pass for bf16 inputs and
// d_k = d_v = 64 ("2Mamba2Furious", App. C: gradients of the attention kernels
// with Q, K, V as inputs; C.1: the A-mask gradient from sums of the masked
// matrix along the key axis and along the query axis).
//
// The arithmetic per pair (t, s), s <= t, with x = q_t.k_s (bf16 products,
// fp32 sums), lambda2 = log2(e) (G_s - G_t) and dP = dout_t.v_s:
//   2Mamba:   u = 2^lambda2 x, P = scale^2 u x / den_t, dw = (dP - D_t) / den_t,
//             dS' = u dw;  dq_t = 2 scale^2 sum_s dS' k_s, dk_s = 2 scale^2
//             sum_t dS' q_t, dL/dlambda_ts = scale^2 x dS'   (den_t = scale^2
//             sum_s 2^lambda2 x^2; without normalisation 1/den_t = 1, D_t = 0);
//   2Mamba-E: P = 2^(log2(e) scale x + lambda2 - lse2_t), dS = P (dP - D_t);
//             dq_t = scale sum_s dS k_s, dk_s = scale sum_t dS q_t,
//             dL/dlambda_ts = dS;
//   first order: P = scale 2^lambda2 x, dS = 2^lambda2 dP; dq_t = scale
//             sum_s dS k_s, dk_s = scale sum_t dS q_t, dL/dlambda_ts = scale x dS
//             (no row statistic, so the first sweep is skipped);
// and dv_s = sum_t P dout_t.  D_t = dout_t.o_t comes from the preparation
// kernel together with the fp64 running sums G.
//
// Both kernels use 16x16x32 bf16 MFMAs.  A lane of a 16x16 accumulator holds
// four consecutive rows 4g..4g+3 (g = lane / 16) of one column (lane mod 16).
//  * bwd_q_kernel (64 queries per workgroup, 16 per wave, one query per lane
//    column): scores transposed, S^T = K Q^T and dP^T = V dout^T, over key
//    tiles of 64 from the first to the diagonal.  A first sweep gives the row
//    statistic (1/den_t or the log-sum-exp), a second one dq, through
//    dq^T = K^T dS^T, and the row sums of dL/dlambda.
//  * bwd_kv_kernel (64 keys per workgroup, 16 per wave, one key per lane
//    column): S = Q K^T and dP = dout V^T over query tiles of 64 from the
//    diagonal to the end; dv^T = dout^T P and dk^T = Q^T dS, and the column
//    sums of dL/dlambda.
// The probability / gradient accumulators leave the MFMA already in the B
// operand layout of the next product: two vertically adjacent 16x16 tiles give
// a lane the eight K-slots {4g..4g+3, 16+4g..16+4g+3}; the transposed A
// operands (K^T, Q^T, dout^T) are read in that order with gfx950's
// transposing LDS read.  Tiles reach LDS by buffer-to-LDS transfers as
// SwTiles (128-byte rows whose 16-byte chunks are permuted per row, so that the
// row reads and the transposing reads are free of bank conflicts),
// double-buffered, with the next tile's transfers in flight during the current
// tile's MFMAs.  The key-major kernel takes each lane's in-tile offsets once per
// kernel (it is held to 128 registers); the query-major one forms them where
// they are used, which it schedules better within its larger budget.
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "mfma_tiles.h"

namespace twm {
namespace {

using namespace tiles;
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kBlk = 64;               // queries or keys per workgroup
constexpr int kMinBlocks = 3;          // workgroups per CU the register budget is sized for
enum { kSq = 0, kExpV = 1, kLin = 2 };   // second order, exponentiated, first order

// ---------------------------------------------------------------------------
// query-major: D_t, row statistic, dq, row sums
// The key and value tiles are double-buffered in separate shared arrays (see the
// kernel), so that the compiler can tell a tile's reads from the transfers in flight
// into the other buffer.
struct QSmem {
    float A[2][kTile];      // log2(e) (G_s - G_ref) per key of the tile
};

__device__ __forceinline__ float dot8(uint4 a, uint4 b) {   // 8 bf16 x 8 bf16, fp32 sum
    const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), r);
        r = fmaf(__uint_as_float(x[i] & 0xffff0000u), __uint_as_float(y[i] & 0xffff0000u), r);
    }
    return r;
}

template <int kVar>
__global__ void __launch_bounds__(kThreads, kMinBlocks)
bwd_q_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
             const bf16* __restrict__ out, const bf16* __restrict__ dout, const double* __restrict__ G,
             const float* __restrict__ fstat, float* __restrict__ Dt, float* __restrict__ stat,
             float* __restrict__ rowsum, bf16* __restrict__ dq, int T, int nqb, float scale, int norm, int use_d,
             int by_xcd) {
    __shared__ __attribute__((aligned(16))) QSmem sm;
    __shared__ __attribute__((aligned(16))) SwTile sK0, sK1, sV0, sV1;
    int bh, blk;
    xcd_map(blockIdx.x, nqb, by_xcd, bh, blk);
    const int qb = nqb - 1 - blk;                  // longest rows first
    const int q0 = qb * kBlk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const int wu = __builtin_amdgcn_readfirstlane(w);   // the wave index as a scalar (tile transfers)
    const DmaOffsets dmo = dma_offsets(wu, lane);
    const size_t base = (size_t)bh * T;
    const int t = q0 + 16 * w + col;               // this lane's query
    const bool tv = t < T;
    const int tc = tv ? t : T - 1;
    const double gref = G[base + q0];
    const float b2 = (float)(G[base + tc] - gref) * kLog2e;
    const bf16* qrow = q + (base + tc) * kD;
    const bf16* orow = dout + (base + tc) * kD;
    const b8 Qb[2] = {own_op(qrow, g, 0), own_op(qrow, g, 1)};
    const b8 Ob[2] = {own_op(orow, g, 0), own_op(orow, g, 1)};
    // D_t = dout_t . out_t from the 16 dims each lane group holds
    float Dq = 0.f;
    if (use_d) {
        const bf16* yrow = out + (base + tc) * kD;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            Dq += dot8(*reinterpret_cast<const uint4*>(orow + 8 * g + 32 * kk),
                       *reinterpret_cast<const uint4*>(yrow + 8 * g + 32 * kk));
        Dq = xor_sum(Dq);
    }
    const float sl2 = scale * kLog2e;
    // Off the diagonal tile every key precedes every query of the block, so the
    // decay 2^(a_s - b_t) splits into a key factor 2^a_s and a query factor
    // 2^-b_t, each in (0, 1] (G rises along the sequence and the reference is the
    // block's first query): one multiply per pair instead of an exp2, and the
    // query factor, common to all of a lane's pairs, is applied to their sums
    // once.  The diagonal tile keeps the exact exponent.  2Mamba-E folds the
    // decay into its softmax exponent and always takes the log form.
    constexpr bool kSplit = kVar != kExpV;
    const float eb = kSplit ? fexp2(-b2) : 0.f;

    // The key terms of a tile: raw G loaded first (before the tile's transfers, so that
    // waiting for it does not wait for them), the terms written to LDS after the compute.
    const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(G + base), (short)0,
                                                                        T * 8, 0x00020000);
    auto load_a = [&](int s0) {
        return __builtin_amdgcn_raw_buffer_load_b64(rG, (uint32_t)(s0 + (tid & (kTile - 1))) * 8, 0, 0);
    };
    auto write_a = [&](int buf, int s0, bool split, v2u raw) {
        if (tid < kTile) {
            const int s = s0 + tid;
            const float a = s < T ? (float)(__builtin_bit_cast(double, raw) - gref) * kLog2e : -INFINITY;
            sm.A[buf][tid] = (kSplit && split) ? fexp2(a) : a;   // 2^a, or a
        }
    };
    auto stage_a = [&](int buf, int s0, bool split) { write_a(buf, s0, split, load_a(s0)); };
    // S^T[s][t] for the key tiles st = 2h, 2h+1 of 16
    auto scores = [&](const SwTile& K, int h, f4 (&S)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f4 c = {0.f, 0.f, 0.f, 0.f};
            c = mfma(row_op(K, 16 * (2 * h + u) + col, g, 0), Qb[0], c);
            c = mfma(row_op(K, 16 * (2 * h + u) + col, g, 1), Qb[1], c);
            S[u] = c;
        }
    };

    const __amdgpu_buffer_rsrc_t rk = head_tile_rsrc(k + base * kD, T), rv = head_tile_rsrc(v + base * kD, T);
    // ---------------------------------------------------------- sweep 1: statistic
    // (none for the first order; not needed without normalisation or when the
    // forward handed it over)
    const bool need_sweep1 = kVar != kLin && !fstat && !(kVar == kSq && !norm);
    float den = 0.f, m = -INFINITY, l = 0.f;
    auto sweep1 = [&](int kt, const SwTile& K, auto diag_tag) {
        constexpr bool kDiag = decltype(diag_tag)::value;
        const int cur = kt & 1, s0 = kt * kTile;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f4 S[2];
            scores(K, h, S);
            float y[8];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int st = 2 * h + u;
                const float4 a4 = *reinterpret_cast<const float4*>(&sm.A[cur][16 * st + 4 * g]);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool masked = kDiag && s0 + 16 * st + 4 * g + i > t;
                    if (kVar == kExpV) {
                        float yy = fmaf(S[u][i], sl2, av[i] - b2);
                        yy = masked ? -INFINITY : yy;
                        y[4 * u + i] = yy;
                        mx = fmaxf(mx, yy);
                    } else {
                        float L = kDiag ? fexp2(av[i] - b2) : av[i] * eb;
                        L = masked ? 0.f : L;
                        den = fmaf(L * S[u][i], S[u][i], den);
                    }
                }
            }
            if (kVar == kExpV) {
                if (mx > m) {
                    l *= fexp2(m - mx);
                    m = mx;
                }
                const float mref = (m == -INFINITY) ? 0.f : m;   // a lane group may see only masked keys so far
#pragma unroll
                for (int i = 0; i < 8; ++i) l += fexp2(y[i] - mref);
            }
        }
    };
    if (need_sweep1) {
        dma_tile(sK0, rk, 0, wu, dmo);
        stage_a(0, 0, 0 < qb);
        wait_vm();
        __syncthreads();
        // key tiles wholly before the queries, from Kc while the next goes into Kn
        auto round1 = [&](int kt, const SwTile& Kc, SwTile& Kn) {
            const int cur = kt & 1, s0 = kt * kTile;
            const v2u an = load_a(s0 + kTile);
            dma_tile(Kn, rk, s0 + kTile, wu, dmo);
            sweep1(kt, Kc, std::false_type{});
            write_a(cur ^ 1, s0 + kTile, kt + 1 < qb, an);
            wait_vm();
            __syncthreads();
        };
        for (int kt = 0; kt < qb; kt += 2) {
            round1(kt, sK0, sK1);
            if (kt + 1 < qb) round1(kt + 1, sK1, sK0);
        }
        if (qb & 1) sweep1(qb, sK1, std::true_type{});
        else sweep1(qb, sK0, std::true_type{});
        __syncthreads();
    }
    float st_v, cq;   // row statistic; cq: b2 + lse2 (2Mamba-E) or -D / den (2Mamba)
    const float given = fstat ? fstat[base + tc] : 0.f;   // lse_t (natural log) or den_t from the forward
    if (kVar == kLin) {
        st_v = 1.f;
        cq = 0.f;
    } else if (kVar == kExpV) {
        if (fstat) {
            st_v = given * kLog2e;
        } else {   // combine the four lane groups' (m, l)
            float M = fmaxf(m, __shfl_xor(m, 16));
            M = fmaxf(M, __shfl_xor(M, 32));
            const float lsc = (m == -INFINITY) ? 0.f : l * fexp2(m - M);
            const float L = xor_sum(lsc);
            st_v = M + flog2(L);
        }
        cq = b2 + st_v;
    } else {
        const float dn = fstat ? given : xor_sum(den) * scale * scale;
        st_v = norm ? (dn > 0.f ? 1.f / dn : 0.f) : 1.f;
        cq = -Dq * st_v;
    }

    // ---------------------------------------------------------- sweep 2: dq, row sums
    f4 dQ[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dQ[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float rs = 0.f;
    dma_tile(sK0, rk, 0, wu, dmo);
    dma_tile(sV0, rv, 0, wu, dmo);
    stage_a(0, 0, 0 < qb);
    wait_vm();
    __syncthreads();
    auto sweep2 = [&](int kt, const SwTile& K, const SwTile& V, auto diag_tag) {
        constexpr bool kDiag = decltype(diag_tag)::value;
        const int cur = kt & 1, s0 = kt * kTile;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f4 S[2], P[2];
            scores(K, h, S);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f4 c = {0.f, 0.f, 0.f, 0.f};
                c = mfma(row_op(V, 16 * (2 * h + u) + col, g, 0), Ob[0], c);
                c = mfma(row_op(V, 16 * (2 * h + u) + col, g, 1), Ob[1], c);
                P[u] = c;   // dP^T
            }
            float ds[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int st = 2 * h + u;
                const float4 a4 = *reinterpret_cast<const float4*>(&sm.A[cur][16 * st + 4 * g]);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = s0 + 16 * st + 4 * g + i;
                    const float x = S[u][i];
                    float d, Mv;
                    if (kVar == kExpV) {
                        const float p = fexp2(fmaf(x, sl2, av[i] - cq));
                        d = p * (P[u][i] - Dq);
                        Mv = d;
                    } else if (kVar == kSq) {
                        // off the diagonal the query factor eb is applied to the sums, once
                        const float uu = (kDiag ? fexp2(av[i] - b2) : av[i]) * x;
                        const float dw = fmaf(P[u][i], st_v, cq);
                        d = uu * dw;
                        Mv = x * d;
                    } else {
                        d = (kDiag ? fexp2(av[i] - b2) : av[i]) * P[u][i];
                        Mv = x * d;
                    }
                    if (kDiag) {
                        if (s < t) rs += Mv;
                        d = s <= t ? d : 0.f;
                    } else {
                        rs += Mv;
                    }
                    ds[4 * u + i] = d;
                }
            }
            // dq^T[d][t] += K^T[d][s] dS^T[s][t] over this 32-key half
            const b8 B = to_b(ds);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) dQ[dt] = mfma(tr_op(K, dt, 2 * h, lane), B, dQ[dt]);
        }
    };
    // from (Kc, Vc) while the next tile goes into (Kn, Vn), read last round
    auto round2 = [&](int kt, const SwTile& Kc, const SwTile& Vc, SwTile& Kn, SwTile& Vn) {
        const int cur = kt & 1, s0 = kt * kTile;
        const v2u an = load_a(s0 + kTile);
        dma_tile(Kn, rk, s0 + kTile, wu, dmo);
        dma_tile(Vn, rv, s0 + kTile, wu, dmo);
        sweep2(kt, Kc, Vc, std::false_type{});
        write_a(cur ^ 1, s0 + kTile, kt + 1 < qb, an);
        wait_vm();
        __syncthreads();
    };
    for (int kt = 0; kt < qb; kt += 2) {
        round2(kt, sK0, sV0, sK1, sV1);
        if (kt + 1 < qb) round2(kt + 1, sK1, sV1, sK0, sV0);
    }
    if (kSplit) {
        // the key tiles before the diagonal left out the query factor eb (in (0, 1]) of
        // every pair: it scales their sums before the diagonal tile adds its own terms
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dQ[dt] *= eb;
        rs *= eb;
    }
    if (qb & 1) sweep2(qb, sK1, sV1, std::true_type{});
    else sweep2(qb, sK0, sV0, std::true_type{});
    rs = xor_sum(rs);
    if (tv) {
        const float f = kVar == kSq ? 2.f * scale * scale : scale;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            uint2 o;
            o.x = pack2(dQ[dt][0] * f, dQ[dt][1] * f);
            o.y = pack2(dQ[dt][2] * f, dQ[dt][3] * f);
            *reinterpret_cast<uint2*>(dq + (base + t) * kD + 16 * dt + 4 * g) = o;
        }
        if (g == 0) {
            stat[base + t] = st_v;
            Dt[base + t] = Dq;
            rowsum[base + t] = kVar == kExpV ? rs : kVar == kSq ? rs * scale * scale : rs * scale;
        }
    }
}

// ---------------------------------------------------------------------------
// key-major: dk, dv, column sums
// The query and dout tiles are double-buffered in separate shared arrays (see the
// kernel), so that the compiler can tell a tile's reads from the transfers in flight
// into the other buffer; the per-row terms live here.
struct KVSmem {
    float B[2][kTile];      // per query of the tile: the decay term (see write_rows)
    float R[2][kTile];      // 2Mamba, diagonal tile: 1/den_t
    float C[2][kTile];      // 2Mamba: -D_t/den_t (times the query factor off the diagonal); 2Mamba-E: D_t
};

// The key-major kernel is held to four workgroups per CU (128 registers; 2Mamba's
// spills a few), which measured faster than three for 2Mamba; 2Mamba-E keeps three
template <int kVar>
__global__ void __launch_bounds__(kThreads, kVar == kExpV ? kMinBlocks : 4)
bwd_kv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
              const bf16* __restrict__ dout, const double* __restrict__ G, const float* __restrict__ Dt,
              const float* __restrict__ stat, float* __restrict__ colsum, bf16* __restrict__ dk,
              bf16* __restrict__ dv, int T, int nkb, float scale, int by_xcd) {
    __shared__ __attribute__((aligned(16))) KVSmem sm;
    __shared__ __attribute__((aligned(16))) SwTile sQ0, sQ1, sO0, sO1;
    int bh, kb;
    xcd_map(blockIdx.x, nkb, by_xcd, bh, kb);     // earliest keys (longest columns) first
    const int k0 = kb * kBlk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, col = lane & 15;
    const int wu = __builtin_amdgcn_readfirstlane(w);   // the wave index as a scalar (tile transfers)
    const DmaOffsets dmo = dma_offsets(wu, lane);
    const SwOffsets swo = sw_offsets(lane);
    const size_t base = (size_t)bh * T;
    const int s = k0 + 16 * w + col;               // this lane's key
    const bool sv_ok = s < T;
    const int sc = sv_ok ? s : T - 1;
    const double gref = G[base + k0];
    const float a2 = sv_ok ? (float)(G[base + sc] - gref) * kLog2e : -INFINITY;
    // Off the diagonal tile every query follows every key of the block, so the
    // decay splits into a key factor and a query factor, each in (0, 1], taken
    // against the block's last key (see the query-major kernel).
    constexpr bool kSplit = kVar != kExpV;
    const double gend = G[base + min(k0 + kBlk - 1, T - 1)];
    const float ea = (kSplit && sv_ok) ? fexp2((float)(G[base + sc] - gend) * kLog2e) : 0.f;
    const b8 Kb[2] = {own_op(k + (base + sc) * kD, g, 0), own_op(k + (base + sc) * kD, g, 1)};
    const b8 Vb[2] = {own_op(v + (base + sc) * kD, g, 0), own_op(v + (base + sc) * kD, g, 1)};
    const float sl2 = scale * kLog2e;

    // The query terms of a tile: raw G, statistic and D_t loaded first (before the tile's
    // transfers, so that waiting for them does not wait for those), the terms written to
    // LDS after the compute.  Rows past T read as zero and are marked by b.
    const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(G + base), (short)0,
                                                                        T * 8, 0x00020000),
                                 rS = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(stat + base), (short)0,
                                                                        T * 4, 0x00020000),
                                 rD = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Dt + base), (short)0,
                                                                        T * 4, 0x00020000);
    struct RowRaw {
        v2u g;
        float st, d;
    };
    auto load_rows = [&](int t0) {
        const uint32_t t = (uint32_t)(t0 + (tid & (kTile - 1)));
        RowRaw r;
        r.g = __builtin_amdgcn_raw_buffer_load_b64(rG, t * 8, 0, 0);
        r.st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, t * 4, 0, 0));
        r.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, t * 4, 0, 0));
        return r;
    };
    auto write_rows = [&](int buf, int t0, bool split, const RowRaw& raw) {
        if (tid < kTile) {
            const int t = t0 + tid;
            const bool lin = kSplit && split;   // B holds 2^-b (query factor) instead of b
            float b = lin ? 0.f : INFINITY, r = 0.f, c = 0.f;
            if (t < T) {
                const double gt = __builtin_bit_cast(double, raw.g);
                b = lin ? fexp2(-(float)(gt - gend) * kLog2e) : (float)(gt - gref) * kLog2e;
                const float st = raw.st, d = raw.d;
                if (kVar == kLin) {
                } else if (kVar == kExpV) {
                    b += st;
                    c = d;
                } else if (lin) {   // 2Mamba off the diagonal: B = q_f/den_t, C = -q_f D_t/den_t
                    c = -d * st * b;
                    b *= st;
                } else {
                    r = st;
                    c = -d * st;
                }
            }
            sm.B[buf][tid] = b;
            sm.R[buf][tid] = r;
            sm.C[buf][tid] = c;
        }
    };
    auto stage_rows = [&](int buf, int t0, bool split) { write_rows(buf, t0, split, load_rows(t0)); };

    f4 dK[4], dV[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dK[dt] = dV[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float cs = 0.f;
    const int nqt = (T - k0 + kTile - 1) / kTile;
    const __amdgpu_buffer_rsrc_t rq = head_tile_rsrc(q + base * kD, T), ro = head_tile_rsrc(dout + base * kD, T);
    dma_tile(sQ0, rq, k0, wu, dmo);
    dma_tile(sO0, ro, k0, wu, dmo);
    stage_rows(0, k0, false);   // the diagonal tile
    wait_vm();
    __syncthreads();
    auto tile = [&](int it, const SwTile& Q, const SwTile& O, auto diag_tag) {
        constexpr bool kDiag = decltype(diag_tag)::value;
        const int cur = it & 1, t0 = k0 + it * kTile;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f4 S[2], DP[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f4 c = {0.f, 0.f, 0.f, 0.f}, e = {0.f, 0.f, 0.f, 0.f};
                c = mfma(row_op(Q, swo, 2 * h + u, 0), Kb[0], c);
                c = mfma(row_op(Q, swo, 2 * h + u, 1), Kb[1], c);
                e = mfma(row_op(O, swo, 2 * h + u, 0), Vb[0], e);
                e = mfma(row_op(O, swo, 2 * h + u, 1), Vb[1], e);
                S[u] = c;
                DP[u] = e;
            }
            float p[8], ds[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = 2 * h + u;
                const float4 b4 = *reinterpret_cast<const float4*>(&sm.B[cur][16 * tt + 4 * g]);
                const float4 c4 = *reinterpret_cast<const float4*>(&sm.C[cur][16 * tt + 4 * g]);
                float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (kVar == kSq && kDiag) r4 = *reinterpret_cast<const float4*>(&sm.R[cur][16 * tt + 4 * g]);
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
                const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + 16 * tt + 4 * g + i;
                    const float x = S[u][i];
                    float pp, d, Mv;
                    if (kVar == kExpV) {
                        pp = fexp2(fmaf(x, sl2, a2 - bv[i]));
                        d = pp * (DP[u][i] - cv[i]);
                        Mv = d;
                    } else if (kVar == kSq) {
                        if (kDiag) {
                            const float uu = fexp2(a2 - bv[i]) * x;
                            pp = uu * x * rv[i];
                            d = uu * fmaf(DP[u][i], rv[i], cv[i]);
                        } else {   // the rows hold q_f/den_t and -q_f D_t/den_t
                            const float e = ea * x;
                            pp = e * x * bv[i];
                            d = e * fmaf(DP[u][i], bv[i], cv[i]);
                        }
                        Mv = x * d;
                    } else {
                        const float L = kDiag ? fexp2(a2 - bv[i]) : ea * bv[i];
                        pp = L * x;
                        d = L * DP[u][i];
                        Mv = x * d;
                    }
                    if (kDiag) {
                        if (t > s) cs += Mv;
                        pp = t >= s ? pp : 0.f;
                        d = t >= s ? d : 0.f;
                    } else {
                        cs += Mv;
                    }
                    p[4 * u + i] = pp;
                    ds[4 * u + i] = d;
                }
            }
            // dv^T[c][s] += dout^T[c][t] P[t][s];  dk^T[d][s] += Q^T[d][t] dS[t][s]
            const b8 BP = to_b(p), BD = to_b(ds);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                dV[dt] = mfma(tr_op(O, swo, dt, 2 * h), BP, dV[dt]);
                dK[dt] = mfma(tr_op(Q, swo, dt, 2 * h), BD, dK[dt]);
            }
        }
    };
    // one query tile from (Qc, Oc) while the next goes into (Qn, On), read last round
    auto step = [&](int it, const SwTile& Qc, const SwTile& Oc, SwTile& Qn, SwTile& On, auto diag_tag) {
        const int cur = it & 1, t0 = k0 + it * kTile;
        const bool more = it + 1 < nqt;
        const RowRaw rn = load_rows(t0 + kTile);   // past T when !more: reads as zero, unused
        if (more) {
            dma_tile(Qn, rq, t0 + kTile, wu, dmo);
            dma_tile(On, ro, t0 + kTile, wu, dmo);
        }
        tile(it, Qc, Oc, diag_tag);
        if (more) write_rows(cur ^ 1, t0 + kTile, true, rn);
        wait_vm();
        __syncthreads();
    };
    step(0, sQ0, sO0, sQ1, sO1, std::true_type{});   // the diagonal tile
    for (int it = 1; it < nqt; it += 2) {
        step(it, sQ1, sO1, sQ0, sO0, std::false_type{});
        if (it + 1 < nqt) step(it + 1, sQ0, sO0, sQ1, sO1, std::false_type{});
    }
    cs = xor_sum(cs);
    if (sv_ok) {
        const float fk = kVar == kSq ? 2.f * scale * scale : scale;
        const float fv = kVar == kSq ? scale * scale : kVar == kLin ? scale : 1.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            uint2 a, b;
            a.x = pack2(dK[dt][0] * fk, dK[dt][1] * fk);
            a.y = pack2(dK[dt][2] * fk, dK[dt][3] * fk);
            b.x = pack2(dV[dt][0] * fv, dV[dt][1] * fv);
            b.y = pack2(dV[dt][2] * fv, dV[dt][3] * fv);
            *reinterpret_cast<uint2*>(dk + (base + s) * kD + 16 * dt + 4 * g) = a;
            *reinterpret_cast<uint2*>(dv + (base + s) * kD + 16 * dt + 4 * g) = b;
        }
        if (g == 0) colsum[base + s] = kVar == kExpV ? cs : kVar == kSq ? cs * scale * scale : cs * scale;
    }
}

template <int kVar>
int launch(const BwdArgs& a, const BwdScratch& s) {
    hipStream_t st = (hipStream_t)a.stream;
    const int nb = (a.T + kBlk - 1) / kBlk;
    const int norm = !(a.flags & TWOMAMBA_FLAG_NO_NORM);
    const int use_d = kVar == kExpV || (kVar == kSq && norm);
    const int by_xcd = (a.B * a.H) % kXcd == 0;
    ktimer_begin(a.timer, "bwd_q", a.stream);
    hipLaunchKernelGGL((bwd_q_kernel<kVar>), dim3(a.B * a.H * nb), dim3(kThreads), 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.out, (const bf16*)a.dout, s.G, a.row_stat,
                       s.Dt, s.stat, s.rowsum, (bf16*)a.gq, a.T, nb, a.scale, norm, use_d, by_xcd);
    ktimer_end(a.timer, a.stream);
    ktimer_begin(a.timer, "bwd_kv", a.stream);
    hipLaunchKernelGGL((bwd_kv_kernel<kVar>), dim3(a.B * a.H * nb), dim3(kThreads), 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout, s.G, s.Dt, s.stat, s.colsum,
                       (bf16*)a.gk, (bf16*)a.gv, a.T, nb, a.scale, by_xcd);
    ktimer_end(a.timer, a.stream);
    return hipGetLastError() == hipSuccess ? TWOMAMBA_OK : TWOMAMBA_ERR_DEVICE;
}

}  // namespace

bool mfma_bwd_supported(const BwdArgs& a) {
    // tiles reach LDS through buffer transfers with 32-bit byte offsets into a head's rows
    return a.dtype == TWOMAMBA_BF16 && a.dk == kD && a.dv == kD && !(a.flags & TWOMAMBA_FLAG_REFERENCE_KERNELS) &&
           (size_t)a.T * kD * 2 < ((size_t)1 << 31);
}

int mfma_bwd(const BwdArgs& a) {
    if ((size_t)a.B * a.H * a.T == 0) return TWOMAMBA_OK;
    const BwdScratch s = bwd_scratch(a);
    int r = bwd_prep_launch(a, s, false);   // G only: D_t comes from the query-major kernel
    if (r != TWOMAMBA_OK) return r;
    r = a.variant == TWOMAMBA_EXP ? launch<kExpV>(a, s) : a.variant == TWOMAMBA_LIN ? launch<kLin>(a, s)
                                                                                    : launch<kSq>(a, s);
    if (r != TWOMAMBA_OK) return r;
    return bwd_dz_launch(a, s);
}

}  // namespace twm
