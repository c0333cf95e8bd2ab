// 16x16x32 bf16 MFMA tile helpers shared by the backward and first-order
// kernels (d = 64, bf16 operands, 64-row tiles staged through LDS).
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 used throughout: lane l of the
// A operand holds row l mod 16 and K-slots 8g..8g+7 (g = l / 16); lane l of
// the B operand holds column l mod 16 and the same K-slots; lane l of the
// accumulator holds rows 4g..4g+3 of column l mod 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace twm {
namespace tiles {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr int kD = 64;                 // head dim
constexpr int kW = 4;                  // waves per workgroup
constexpr int kThreads = 64 * kW;
constexpr int kTile = 64;              // rows per LDS tile
constexpr int kLS = 72;                // LDS row stride in bf16 (144 B)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f4 mfma(b8 a, b8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ b8 as_b8(uint4 u) { return __builtin_bit_cast(b8, u); }
// two fp32 -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2));
}
// two 16x16 accumulators (rows 4g..4g+3 and 16+4g..16+4g+3) as one B operand
__device__ __forceinline__ b8 to_b(const float (&x)[8]) {
    return as_b8(make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])));
}
// Workgroups are dealt to the 8 XCDs round-robin by index, block i to XCD
// i mod 8.  When the head count is a multiple of 8 the (head, block) pair of
// index i is chosen so that every block of a head runs on one XCD, where that
// head's tiles then stay in one L2: XCD x takes heads x, x + 8, ... in turn.
constexpr int kXcd = 8;
__device__ __forceinline__ void xcd_map(int i, int nb, bool by_xcd, int& bh, int& blk) {
    if (by_xcd) {
        const int x = i % kXcd, j = i / kXcd;
        bh = x + kXcd * (j / nb);
        blk = j % nb;
    } else {
        bh = i / nb;
        blk = i % nb;
    }
}

__device__ __forceinline__ float xor_sum(float x) {   // over the four lane groups g
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

struct Tile {
    uint16_t X[kTile][kLS];
};

// A operand of a row-major tile: row r, dims 8g + 32 kk .. + 7
__device__ __forceinline__ b8 row_op(const Tile& t, int r, int g, int kk) {
    return as_b8(*reinterpret_cast<const uint4*>(&t.X[r][8 * g + 32 * kk]));
}
// Operand of the transposed tile X^T (columns 16 dt .. 16 dt + 15 of X as rows)
// for the K-slots {16 tt + 4g + 0..3, 16 tt + 16 + 4g + 0..3}: inside a 16-lane
// group, lane 4j + r addresses columns 16 dt + 4r .. + 3 of row base + j and
// receives column 16 dt + (lane mod 16) of rows base .. base + 3 (gfx950's
// transposing LDS read).  The same values serve as an A operand (X^T rows) or
// as a B operand (X columns).
__device__ __forceinline__ b8 tr_op(const Tile& t, int dt, int tt, int lane) {
    const int g = lane >> 4, m = lane & 15, j = m >> 2, r = m & 3;
    const int row = 16 * tt + 4 * g + j, col = 16 * dt + 4 * r;
    const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)&t.X[row][col]);
    const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)&t.X[row + 16][col]);
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return as_b8(make_uint4(ua.x, ua.y, ub.x, ub.y));
}

// Global -> registers for one 64-row tile (two 16-byte chunks per thread of a
// 256-thread workgroup), rows past `rows` read as zero; registers -> LDS.
struct Stage {
    uint4 c[2];
};
__device__ __forceinline__ void fetch(Stage& s, const bf16* src, int rows, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, c = e & 7;
        s.c[n] = r < rows ? *reinterpret_cast<const uint4*>(src + (size_t)r * kD + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
}
__device__ __forceinline__ void store(const Stage& s, Tile& t, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + n * kThreads, r = e >> 3, c = e & 7;
        *reinterpret_cast<uint4*>(&t.X[r][8 * c]) = s.c[n];
    }
}

// a lane's own row (query or key) as a B operand: dims 8g + 32 kk .. + 7
__device__ __forceinline__ b8 own_op(const bf16* row, int g, int kk) {
    return as_b8(*reinterpret_cast<const uint4*>(row + 8 * g + 32 * kk));
}

}  // namespace tiles
}  // namespace twm
