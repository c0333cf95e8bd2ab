// Internal declarations shared by the host dispatcher and the HIP kernels of
// the 2Mamba library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/twomamba.h"

namespace twm {

// Optional per-launch timing: when a KTimer is attached to a call, every
// kernel launch is bracketed by a pair of HIP events (see twomamba_fwd_timed).
struct KTimer {
    static constexpr int kMax = 24;
    void* ev[2 * kMax];
    const char* names[kMax];
    int n;
    int error;
};
void ktimer_begin(KTimer* t, const char* name, void* stream);
void ktimer_end(KTimer* t, void* stream);
int ktimer_collect(KTimer* t, float* ms, const char** names, int cap);

// Everything the kernels need about one forward call, already validated.
struct FwdArgs {
    int B, H, T, dk, dv, chunk;
    float scale;
    int variant, dtype;
    unsigned flags;
    const void* q;
    const void* k;
    const void* v;
    const float* z;
    const float* state_in;
    const float* norm_in;
    void* out;
    float* state_out;
    float* norm_out;
    void* ws;
    size_t ws_bytes;
    void* stream;
    KTimer* timer;     // NULL unless called through twomamba_fwd_timed
    float* row_stat;   // NULL, or [B][H][T]: weight sum (2Mamba) / log-sum-exp (2Mamba-E) per query
    // size-2 input convolution applied by the kernels themselves while they load q, k, v
    // (twomamba_fwd_conv on the paths that fuse it): weights [3][H][d][2], bias [3][H][d]
    // or NULL, raw rows of the token before t = 0 [B][H][3][d] or NULL; conv_w NULL = none.
    // conv_q_only: only q is convolved in-kernel (k, v arrive convolved).
    const float* conv_w;
    const float* conv_b;
    const void* conv_prev;
    bool conv_q_only;
};

struct StepArgs {
    int B, H, dk, dv;
    float scale;
    int dtype;
    unsigned flags;
    const void* q;
    const void* k;
    const void* v;
    const float* z;
    float* state;
    float* norm;
    void* out;
    void* stream;
    // optional size-2 input convolution (twomamba_step_conv): weights
    // [3][H][d][2], bias [3][H][d] or NULL, cache [B][H][3][d] (input dtype)
    const float* conv_w;
    const float* conv_b;
    void* conv_state;
};

// size-2 input convolution (conv.hip)
struct ConvArgs {
    int B, H, T, d;
    int dtype;
    const void *q, *k, *v;
    const float* w;
    const float* b;
    const void* prev;
    void *qo, *ko, *vo;
    void* prev_out;
    void* stream;
    int first, count;   // the tensors convolved: first .. first + count - 1 of (q, k, v)
};
int conv2_launch(const ConvArgs& a);
// conv_state_out only: the raw rows of token T-1 (prev, or zeros, when T = 0)
int conv_tail_launch(const ConvArgs& a);

inline size_t num_pairs(int d) { return (size_t)d * (size_t)(d + 1) / 2; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- reference (plain fp32) kernels: any supported d, chunk 16/32/64 -------
size_t ref_sq_workspace(const FwdArgs& a);
int ref_sq_fwd(const FwdArgs& a);      // returns twomamba_status
int ref_exp_fwd(const FwdArgs& a);

// ---- MFMA kernels: bf16, dk = dv = 64 ---------------------------------------
bool mfma_sq_supported(const FwdArgs& a);
size_t mfma_sq_workspace(const FwdArgs& a);
int mfma_sq_fwd(const FwdArgs& a);
bool mfma_exp_supported(const FwdArgs& a);
int mfma_exp_fwd(const FwdArgs& a);

// ---- first-order variant (lin.hip) -----------------------------------------
size_t lin_workspace(const FwdArgs& a);
int lin_fwd(const FwdArgs& a);
bool lin_conv_fused(const FwdArgs& a);   // the path that applies conv_w in-kernel

// ---- library-owned workspace of twomamba_fwd_noalloc (noalloc.hip) ----------
// Device address of the current device's static scratch array (looked up once per
// device); `stream` must belong to the current device.  Returns a status.
int noalloc_scratch(void* stream, void** ptr);

// ---- decode step -------------------------------------------------------------
int step_launch(const StepArgs& a);

// 2Mamba-E decoding over a key/value cache (exp_step.hip)
struct ExpCacheArgs {
    int B, H, dk, dv, max_len, pos;
    float scale;
    int dtype;
    const void *q, *k, *v;
    const float* z;
    void *k_cache, *v_cache;
    double* g_cache;
    void* out;
    void* ws;
    size_t ws_bytes;
    void* stream;
};
size_t exp_step_workspace(const ExpCacheArgs& a);
int exp_step_launch(const ExpCacheArgs& a);
int exp_cache_fill_launch(const ExpCacheArgs& a);

// backward pass (bwd_ref.hip, bwd_mfma.hip)
struct BwdArgs {
    int B, H, T, dk, dv;
    float scale;
    int variant, dtype;
    unsigned flags;
    const void *q, *k, *v;
    const float* z;
    const void *out, *dout;
    const float* row_stat;   // the forward's per-row statistic, or NULL (recomputed)
    void *gq, *gk, *gv;   // dL/dq, dL/dk, dL/dv
    float* gz;            // dL/dz
    void* ws;
    size_t ws_bytes;
    void* stream;
    KTimer* timer;   // NULL unless called through twomamba_bwd_timed
};
// per-token scratch carved from the workspace
struct BwdScratch {
    double* G;       // running fp64 softplus sums
    float* stat;     // 1/den (2Mamba) or log-sum-exp (2Mamba-E) of each query row
    float* Dt;       // dout_t . out_t
    float* rowsum;   // sum_{s<t} dL/dlambda_ts
    float* colsum;   // sum_{t>s} dL/dlambda_ts
};
size_t bwd_workspace(const BwdArgs& a);
BwdScratch bwd_scratch(const BwdArgs& a);
int bwd_prep_launch(const BwdArgs& a, const BwdScratch& s, bool with_d);
int bwd_dz_launch(const BwdArgs& a, const BwdScratch& s);
int ref_bwd(const BwdArgs& a);
// 2Mamba backward in O(T) (sq_bwd_chunk.hip): chosen by TWOMAMBA_FLAG_CHUNKED_FORM,
// and by default from kSqChunkedMinT tokens per head on (where it overtakes the
// attention form, whose cost per token grows with T)
constexpr int kSqChunkedMinT = 20480;
bool sq_bwd_chunked_supported(const BwdArgs& a);
size_t sq_bwd_chunked_workspace(const BwdArgs& a);
int sq_bwd_chunked(const BwdArgs& a);
bool mfma_bwd_supported(const BwdArgs& a);
int mfma_bwd(const BwdArgs& a);
// first-order backward in O(T) through the segmented chunk kernels (lin.hip)
bool lin_bwd_chunked_supported(const BwdArgs& a);
size_t lin_bwd_chunked_workspace(const BwdArgs& a);
int lin_bwd_chunked(const BwdArgs& a);

}  // namespace twm
