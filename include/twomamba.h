/*
 * twomamba.h -- C ABI of the 2Mamba / 2Mamba-E sequence-mixing operator for
 * AMD MI355X (gfx950).
 *
 * The operator is defined in "2Mamba2Furious: Linear in Complexity, Competitive
 * in Accuracy" (paperlayer summary of arXiv 2602.17363), cited below as
 * [2M2F §n].  It is the attention kernel of that work: it takes queries, keys
 * and values and returns post-attention outputs, with no pre- or
 * post-processing (no convolution, gate, residual or output norm) [2M2F App. C].
 *
 * Per (batch b, head h), with g_t = -softplus(z_t) and L_ts = exp(g_{s+1}+...+g_t)
 * for s <= t (L_tt = 1):
 *
 *   2Mamba   (TWOMAMBA_SQ)  [2M2F §5]
 *       w_ts = L_ts * (scale * q_t . k_s)^2
 *       o_t  = sum_s w_ts v_s / sum_s w_ts          (o_t = 0 when the sum is 0)
 *     The mask multiplies the squared score; it is not itself squared.
 *   2Mamba-E (TWOMAMBA_EXP) [2M2F §6]
 *       o_t  = softmax_{s<=t}( scale * q_t . k_s + log L_ts ) . v
 *     i.e. softmax attention with the softplus A-mask as a log-bias.
 *
 * The second-order recurrent state of 2Mamba [2M2F §2, §5.1] is the symmetric
 * tensor sum_s L k_s (x) k_s (x) v_s, stored PACKED: D = dk*(dk+1)/2 rows, row
 * p(i,j) = i*dk - i*(i-1)/2 + (j-i) for 0 <= i <= j < dk (row-major upper
 * triangle), each row holding dv fp32 values of the UNSCALED products
 * k_i*k_j*v (the weight 2 of off-diagonal pairs is applied on the query side).
 * The normaliser state has the same D rows and one value per row
 * (sum_s L k_i k_j).  Layouts: state [B][H][D][dv], norm [B][H][D], fp32,
 * C-contiguous.  An initial state is the state before token 0; it is decayed by
 * g_0 like any earlier token.  A decode step consumes the decay logit of its
 * own token.
 *
 * Conventions shared by every entry point:
 *   - Every argument is checked on the host BEFORE any HIP call; an invalid
 *     call returns a status and touches neither the device nor the buffers.
 *   - Device pointers are caller-owned; the library allocates nothing and
 *     keeps no pointer after the call returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).  A launch failure returns
 *     TWOMAMBA_ERR_DEVICE; a fault inside a kernel surfaces at the caller's
 *     next synchronisation.
 *   - Outputs must not alias inputs, except that state_in == state_out and
 *     norm_in == norm_out are allowed (exact alias: in-place resume).
 *   - z may hold -inf (no decay for that token).  +inf and NaN in z, and
 *     non-finite q, k, v, are undefined.
 *   - Results are deterministic: identical inputs give bit-identical outputs
 *     (no floating-point atomics).
 */
#ifndef TWOMAMBA_H
#define TWOMAMBA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWOMAMBA_ABI_VERSION 5

typedef enum {
    TWOMAMBA_OK = 0,
    TWOMAMBA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    TWOMAMBA_ERR_SHAPE = 2,       /* negative size, or sizes that overflow size_t   */
    TWOMAMBA_ERR_DTYPE = 3,       /* dtype or variant value not in its enum         */
    TWOMAMBA_ERR_UNSUPPORTED = 4, /* valid request the library does not implement   */
    TWOMAMBA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required        */
    TWOMAMBA_ERR_DEVICE = 6,      /* a HIP call failed (launch, attribute, device)  */
    TWOMAMBA_ERR_ALIAS = 7,       /* an output overlaps an input it may not alias   */
    TWOMAMBA_ERR_SCRATCH = 8      /* twomamba_fwd_noalloc: the call needs more than *
                                   * TWOMAMBA_NOALLOC_SCRATCH_BYTES of workspace     */
} twomamba_status;

typedef enum { TWOMAMBA_F32 = 0, TWOMAMBA_BF16 = 1 } twomamba_dtype;   /* dtype of q, k, v and out */

typedef enum {
    TWOMAMBA_SQ = 0,   /* 2Mamba: squared score, normalised by the sum of weights  [2M2F §5] */
    TWOMAMBA_EXP = 1,  /* 2Mamba-E: exponentiated score (softmax) with the A-mask   [2M2F §6] */
    TWOMAMBA_LIN = 2   /* first order (Mamba-2S): o_t = sum_s L_ts (scale q_t.k_s) v_s, not
                          normalised (the output norm sits outside the kernel); the state
                          is the dk x dv matrix sum_s L k_s v_s^T, [B][H][dk][dv] fp32, with
                          no normaliser  [2M2F §2, §3-§4] */
} twomamba_variant;

enum {
    /* SQ only: return the numerator sum_s w_ts v_s instead of the normalised
       output, for callers that normalise themselves (e.g. an RMSNorm as in the
       Mamba-2 ablations, [2M2F §3]). */
    TWOMAMBA_FLAG_NO_NORM = 1u,
    /* Force the plain fp32 reference kernels instead of the MFMA kernels
       (testing aid; same results within fp32 rounding). */
    TWOMAMBA_FLAG_REFERENCE_KERNELS = 2u,
    /* twomamba_step / twomamba_step_conv: the first-order (TWOMAMBA_LIN) step,
       S <- e^g S + k v^T, o = scale q.S, on a [B][H][dk][dv] state; norm must
       be NULL. */
    TWOMAMBA_FLAG_FIRST_ORDER = 4u,
    /* twomamba_bwd / twomamba_bwd_workspace_size with TWOMAMBA_LIN: the
       attention (quadratic in T) form of the backward instead of the linear-in-T
       chunked form, for comparison; the same gradients within bf16 rounding.
       With TWOMAMBA_SQ it keeps the attention form at every T.  Ignored by the
       forward and by 2Mamba-E, whose backward is always the attention form. */
    TWOMAMBA_FLAG_ATTENTION_FORM = 8u,
    /* twomamba_bwd / twomamba_bwd_workspace_size with TWOMAMBA_SQ (bf16,
       dk = dv = 64, T < 2^24): the linear-in-T chunked form of the backward
       [2M2F App. C] at any T.  Without this flag that form is taken from
       20480 tokens per head on, where it overtakes the attention form (whose
       cost per token grows with T), and TWOMAMBA_FLAG_ATTENTION_FORM keeps
       the attention form.  The same gradients within bf16 rounding.  Ignored
       by the forward and by the other variants. */
    TWOMAMBA_FLAG_CHUNKED_FORM = 16u
};

typedef struct {
    int B, H, T;        /* batch, heads, tokens; B, H, T >= 0 (0 = nothing to do)     */
    int dk, dv;         /* head dims; supported: dk == dv, 16 or 64                   */
    int chunk;          /* chunk length of the chunked form: 0 = library choice, or   *
                         * 16, 32, 64 (reference kernels) / 64 (MFMA kernels, bf16,   *
                         * d = 64).  The result does not depend on it beyond fp32     *
                         * rounding.  Ignored by TWOMAMBA_EXP.                        */
    float scale;        /* multiplies q . k before squaring / exponentiating          */
    int variant;        /* twomamba_variant                                            */
    int dtype;          /* twomamba_dtype                                              */
    unsigned flags;     /* TWOMAMBA_FLAG_*                                             */
} twomamba_fwd_desc;

typedef struct {
    int B, H;           /* batch, heads                                                */
    int dk, dv;         /* head dims; supported: dk == dv, 16 or 64                   */
    float scale;
    int dtype;          /* dtype of q, k, v and out; the state is always fp32         */
    unsigned flags;     /* TWOMAMBA_FLAG_NO_NORM, TWOMAMBA_FLAG_FIRST_ORDER            */
} twomamba_step_desc;

/* ABI version of the loaded library (TWOMAMBA_ABI_VERSION it was built with). */
int twomamba_abi_version(void);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char* twomamba_status_str(int status);

/* Bytes of device workspace twomamba_fwd needs for *desc, written to *bytes.
   Returns the same status twomamba_fwd would return for the descriptor alone. */
int twomamba_fwd_workspace_size(const twomamba_fwd_desc* desc, size_t* bytes);

/*
 * Chunked/parallel forward of 2Mamba or 2Mamba-E over T tokens of every
 * (b, h)  [2M2F §5, §6; chunked evaluation of the recurrence by the SSD
 * duality, "Mamba-2 - State Space Duality" thread].
 *
 *   q, k      [B][H][T][dk]  dtype      device
 *   v         [B][H][T][dv]  dtype      device
 *   z         [B][H][T]      fp32       device   decay logits, g = -softplus(z)
 *   state_in  [B][H][D][dv]  fp32       device   SQ only; NULL = zero state
 *   norm_in   [B][H][D]      fp32       device   SQ only; NULL iff state_in NULL
 *   out       [B][H][T][dv]  dtype      device   written (round to nearest even for bf16)
 *   state_out [B][H][D][dv]  fp32       device   SQ only; NULL = not written
 *   norm_out  [B][H][D]      fp32       device   SQ only; NULL iff state_out NULL
 *   workspace                           device   >= twomamba_fwd_workspace_size bytes,
 *                                                 256-byte aligned; contents undefined after
 *
 * TWOMAMBA_EXP takes no state pointers (it needs a KV cache, [2M2F §1, §6]):
 * passing any returns TWOMAMBA_ERR_UNSUPPORTED.  TWOMAMBA_LIN takes
 * state_in / state_out of [B][H][dk][dv] (each optional on its own) and no
 * normaliser (norm_in and norm_out must be NULL); TWOMAMBA_FLAG_NO_NORM does
 * not change it.
 */
int twomamba_fwd(const twomamba_fwd_desc* desc,
                 const void* q, const void* k, const void* v, const float* z,
                 const float* state_in, const float* norm_in,
                 void* out, float* state_out, float* norm_out,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Profiling form of twomamba_fwd (same arguments and results).  Each kernel
 * launch of the call is bracketed by a pair of HIP events; the call then WAITS
 * for the stream and writes, for the first min(count, cap) launches, the
 * duration in milliseconds to kernel_ms[i] and a static kernel name to
 * kernel_names[i] (either array may be NULL).  *n_kernels receives the number
 * of launches.  Meant for benchmarks: it creates and destroys HIP events, so
 * it is not for use under graph capture.
 */
int twomamba_fwd_timed(const twomamba_fwd_desc* desc,
                       const void* q, const void* k, const void* v, const float* z,
                       const float* state_in, const float* norm_in,
                       void* out, float* state_out, float* norm_out,
                       void* workspace, size_t workspace_bytes, void* stream,
                       float* kernel_ms, const char** kernel_names, int cap, int* n_kernels);

/*
 * twomamba_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as twomamba_fwd, without the workspace: the
 * workspace twomamba_fwd_workspace_size reports comes from a buffer the library
 * owns, a static device array of TWOMAMBA_NOALLOC_SCRATCH_BYTES on each GPU,
 * held until the process ends.  A call whose workspace would exceed it returns
 * TWOMAMBA_ERR_SCRATCH before any HIP call (use twomamba_fwd with a workspace
 * of your own).  The call allocates nothing and leaves nothing behind that a
 * later call depends on.  `stream` must belong to the current device (else
 * TWOMAMBA_ERR_DEVICE).  All calls on one GPU share its buffer: calls that may
 * overlap on one GPU (other streams, other host threads) race on it and must
 * be serialised by the caller.
 */
#define TWOMAMBA_NOALLOC_SCRATCH_BYTES (128u << 20)

int twomamba_fwd_noalloc(const twomamba_fwd_desc* desc,
                         const void* q, const void* k, const void* v, const float* z,
                         const float* state_in, const float* norm_in,
                         void* out, float* state_out, float* norm_out, void* stream);

/*
 * twomamba_fwd that also writes each row's normalising statistic, the quantity
 * the backward otherwise recomputes with a pass over all earlier keys
 * [2M2F App. C: the gradient of a normalised kernel needs the row's
 * normaliser; storing it from the forward is the usual flash-attention
 * practice]:
 *
 *   row_stat  [B][H][T]  fp32  device  written, required (non-NULL) when B H T > 0
 *     TWOMAMBA_SQ:  den_t = sum_{s<=t} L_ts (scale q_t.k_s)^2 plus the initial
 *                   normaliser's term e^(g_0+..+g_t) phi_q(scale q_t).n0 when
 *                   norm_in is given (also written with TWOMAMBA_FLAG_NO_NORM);
 *     TWOMAMBA_EXP: lse_t = ln sum_{s<=t} exp(scale q_t.k_s + lambda_ts);
 *     TWOMAMBA_LIN: none; returns TWOMAMBA_ERR_UNSUPPORTED.
 * row_stat may not overlap any other argument.  The other arguments, results
 * and errors are those of twomamba_fwd.
 */
int twomamba_fwd_stats(const twomamba_fwd_desc* desc,
                       const void* q, const void* k, const void* v, const float* z,
                       const float* state_in, const float* norm_in,
                       void* out, float* state_out, float* norm_out, float* row_stat,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step of 2Mamba for every (b, h)  [2M2F §2 constant-size
 * hidden state; App. A inference]:
 *     S <- e^g S + phi(k) v^T,   n <- e^g n + phi(k),
 *     o  = phi_q(scale q) . S / phi_q(scale q) . n      (numerator only with NO_NORM)
 * with phi(k)_p(i,j) = k_i k_j and phi_q(q)_p(i,j) = (2 if i<j else 1) q_i q_j.
 *
 *   q, k   [B][H][dk]     dtype   device
 *   v      [B][H][dv]     dtype   device
 *   z      [B][H]         fp32    device
 *   state  [B][H][D][dv]  fp32    device   read and updated in place
 *   norm   [B][H][D]      fp32    device   read and updated in place
 *   out    [B][H][dv]     dtype   device
 */
int twomamba_step(const twomamba_step_desc* desc,
                  const void* q, const void* k, const void* v, const float* z,
                  float* state, float* norm, void* out, void* stream);

/*
 * 2Mamba-E decoding over a key/value cache  [2M2F §6: 2Mamba-E is softmax
 * attention with the softplus A-mask, so inference keeps every past key and
 * value; §1-§2: the KV cache grows with the sequence].
 *
 * The cache of every (b, h) holds, for each past token s, its key, its value
 * and G_s = softplus(z_0) + ... + softplus(z_s) in fp64.  At token t the decay
 * log-bias of key s <= t is G_s - G_t (= sum of g over s+1..t), so the output
 * is  o_t = softmax_{s<=t}(scale q_t . k_s + G_s - G_t) . v.
 *
 *   k_cache [B][H][max_len][dk]  dtype   device
 *   v_cache [B][H][max_len][dv]  dtype   device
 *   g_cache [B][H][max_len]      fp64    device
 */
typedef struct {
    int B, H;           /* batch, heads                                                */
    int dk, dv;         /* head dims; supported: dk == dv, 16 or 64                   */
    int max_len;        /* token capacity of the caches                                */
    int pos;            /* twomamba_exp_step: index of the new token (tokens 0..pos-1  *
                         * are cached).  twomamba_exp_cache_fill: number of tokens T   */
    float scale;        /* multiplies q . k                                            */
    int dtype;          /* dtype of q, k, v, out and of the K/V caches                 */
    unsigned flags;     /* must be 0                                                   */
} twomamba_exp_cache_desc;

/*
 * Fill positions 0..T-1 (T = desc->pos) of the caches from a prompt: keys and
 * values copied, G_s the running sum of softplus(z) (fp64, in token order).
 *
 *   k [B][H][T][dk], v [B][H][T][dv]  dtype   device
 *   z [B][H][T]                       fp32    device
 * T <= max_len; T = 0 does nothing.
 */
int twomamba_exp_cache_fill(const twomamba_exp_cache_desc* desc,
                            const void* k, const void* v, const float* z,
                            void* k_cache, void* v_cache, double* g_cache, void* stream);

/* Bytes of device workspace twomamba_exp_step needs for *desc, written to *bytes. */
int twomamba_exp_step_workspace_size(const twomamba_exp_cache_desc* desc, size_t* bytes);

/*
 * One 2Mamba-E decode step at position pos = desc->pos for every (b, h): the
 * new key and value are appended at row pos of the caches (with
 * G_pos = G_{pos-1} + softplus(z), G_{-1} = 0) and the new query attends over
 * rows 0..pos.  pos < max_len.
 *
 *   q, k   [B][H][dk]     dtype   device
 *   v      [B][H][dv]     dtype   device
 *   z      [B][H]         fp32    device
 *   out    [B][H][dv]     dtype   device
 *   workspace                     device   >= twomamba_exp_step_workspace_size bytes,
 *                                          256-byte aligned; contents undefined after
 * The caches are read for rows 0..pos-1 and written at row pos only.
 */
int twomamba_exp_step(const twomamba_exp_cache_desc* desc,
                      const void* q, const void* k, const void* v, const float* z,
                      void* k_cache, void* v_cache, double* g_cache,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Size-2 causal input convolution  [2M2F §3: a convolution of kernel size 2
 * along the sequence, without activation, in front of the attention kernel;
 * §4: kept in Mamba-2S; App. A: decoding then caches the raw query, key and
 * value of the one previous token].
 *
 * Each channel c of q, k and v (x below) is convolved separately:
 *     y_t[c] = w[c][1] * x_t[c] + w[c][0] * x_{t-1}[c] + b[c],
 * with x_{-1} the cached raw row of the token before the sequence (zeros when
 * none is given).  The outputs feed twomamba_fwd (or the reference forward)
 * in place of q, k, v; twomamba_step_conv does the same inside a decode step.
 */
typedef struct {
    int B, H, T;        /* batch, heads, tokens                                         */
    int d;              /* head dim of q, k and v (equal); supported: 16, 64            */
    int dtype;          /* dtype of q, k, v, the outputs and the cache                  */
    unsigned flags;     /* must be 0                                                    */
} twomamba_conv_desc;

/*
 *   q, k, v        [B][H][T][d]   dtype   device
 *   weight         [3][H][d][2]   fp32    device   q, k, v in that order; tap 0 multiplies
 *                                                  x_{t-1}, tap 1 multiplies x_t; 16-byte aligned
 *   bias           [3][H][d]      fp32    device   or NULL (no bias); 16-byte aligned
 *                                                  (a misaligned weight or bias returns
 *                                                  TWOMAMBA_ERR_UNSUPPORTED)
 *   conv_state_in  [B][H][3][d]   dtype   device   raw q, k, v rows of the token before
 *                                                  t = 0, or NULL (zeros)
 *   q_out, k_out, v_out  [B][H][T][d]  dtype  device   written (round to nearest even for bf16)
 *   conv_state_out [B][H][3][d]   dtype   device   the raw rows of token T-1 (conv_state_in
 *                                                  when T = 0), or NULL (not written)
 * Outputs must not overlap inputs or each other.
 */
int twomamba_conv2(const twomamba_conv_desc* desc,
                   const void* q, const void* k, const void* v,
                   const float* weight, const float* bias, const void* conv_state_in,
                   void* q_out, void* k_out, void* v_out, void* conv_state_out, void* stream);

/*
 * twomamba_fwd with the size-2 input convolution in front of the operator, in
 * one call: out = twomamba_fwd(conv2(q, k, v)) with conv2 as twomamba_conv2
 * defines it (same weights, bias and cached rows, same fp32 arithmetic, the
 * convolved values rounded to the input dtype before the operator uses them)
 * [2M2F §3: the kernel-2 convolution directly in front of the attention kernel;
 * §4: kept in Mamba-2S; App. A: decoding caches the one previous raw q, k, v].
 * Results are bit-identical to twomamba_conv2 followed by twomamba_fwd.
 *
 *   q, k, v         [B][H][T][d]   dtype   device   RAW inputs (d = dk = dv)
 *   z, state_in, norm_in, out, state_out, norm_out   as for twomamba_fwd
 *   conv_weight     [3][H][d][2]   fp32    device   as for twomamba_conv2; 16-byte aligned
 *   conv_bias       [3][H][d]      fp32    device   or NULL; 16-byte aligned
 *   conv_state_in   [B][H][3][d]   dtype   device   raw q, k, v rows of the token before t = 0,
 *                                                   or NULL (zeros); 16-byte aligned
 *   conv_state_out  [B][H][3][d]   dtype   device   the raw rows of token T-1 (conv_state_in, or
 *                                                   zeros, when T = 0), or NULL; may not overlap
 *                                                   any other argument or the workspace
 *   workspace                              device   >= twomamba_fwd_conv_workspace_size bytes
 * Where the path's kernels apply the convolution while loading their operands
 * (the first order at bf16, d = 64; the queries of 2Mamba-E at bf16, d = 64)
 * nothing convolved reaches HBM; otherwise the workspace holds the convolved
 * tensors, written by one pass in front of the forward.  Misaligned weight,
 * bias or cache returns TWOMAMBA_ERR_UNSUPPORTED; the other errors are those of
 * twomamba_fwd and twomamba_conv2.
 */
int twomamba_fwd_conv_workspace_size(const twomamba_fwd_desc* desc, size_t* bytes);

int twomamba_fwd_conv(const twomamba_fwd_desc* desc,
                      const void* q, const void* k, const void* v, const float* z,
                      const float* conv_weight, const float* conv_bias,
                      const void* conv_state_in, void* conv_state_out,
                      const float* state_in, const float* norm_in,
                      void* out, float* state_out, float* norm_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * twomamba_step with the size-2 input convolution in front: q, k, v are this
 * token's raw rows; each is convolved with the cached raw row of the previous
 * token (conv_state, [B][H][3][d] in the input dtype, read and then replaced
 * by this token's raw rows), then the step runs on the results.  weight and
 * bias as for twomamba_conv2 (bias may be NULL); dk == dv.
 */
int twomamba_step_conv(const twomamba_step_desc* desc,
                       const void* q, const void* k, const void* v, const float* z,
                       const float* weight, const float* bias, void* conv_state,
                       float* state, float* norm, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Backward pass of twomamba_fwd  [2M2F App. C: the gradients of each attention
 * kernel, with Q, K, V as inputs and the post-attention outputs as outputs;
 * C.1: the A-mask gradient is built from sums of the masked matrix along the
 * key axis and along the query axis].
 *
 * Given dout = dL/dout for out = twomamba_fwd(q, k, v, z) (no initial state),
 * writes dq, dk, dv (= dL/dq, dL/dk, dL/dv) and dz = dL/dz, the decay logits'
 * gradient (g = -softplus(z), so dz = -sigmoid(z) dL/dg).  The same descriptor
 * as the forward: variant, dtype, scale and TWOMAMBA_FLAG_NO_NORM (2Mamba only)
 * select the operator; desc->chunk is ignored (0 or a forward chunk size).  A
 * 2Mamba row whose weight sum is 0 has o_t = 0 and passes no gradient.
 *
 *   q, k      [B][H][T][dk]  dtype   device
 *   v         [B][H][T][dv]  dtype   device
 *   z         [B][H][T]      fp32    device
 *   out       [B][H][T][dv]  dtype   device   the forward's output for these inputs
 *                                             (only dout_t . out_t is used)
 *   dout      [B][H][T][dv]  dtype   device
 *   row_stat  [B][H][T]      fp32    device   the row statistics twomamba_fwd_stats wrote for
 *                                             these inputs (no initial state), or NULL: then
 *                                             the backward recomputes them (one more pass over
 *                                             the keys).  Ignored by TWOMAMBA_LIN and, being
 *                                             unused there, by TWOMAMBA_SQ with NO_NORM.
 *   dq, dk    [B][H][T][dk]  dtype   device   written
 *   dv        [B][H][T][dv]  dtype   device   written
 *   dz        [B][H][T]      fp32    device   written
 *   workspace                        device   >= twomamba_bwd_workspace_size bytes,
 *                                             256-byte aligned; contents undefined after
 * No output may overlap an input, another output or the workspace.
 */
int twomamba_bwd_workspace_size(const twomamba_fwd_desc* desc, size_t* bytes);

int twomamba_bwd(const twomamba_fwd_desc* desc,
                 const void* q, const void* k, const void* v, const float* z,
                 const void* out, const void* dout, const float* row_stat,
                 void* dq, void* dk, void* dv, float* dz,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Profiling form of twomamba_bwd, with the per-launch timings of
   twomamba_fwd_timed (the call waits for the stream). */
int twomamba_bwd_timed(const twomamba_fwd_desc* desc,
                       const void* q, const void* k, const void* v, const float* z,
                       const void* out, const void* dout, const float* row_stat,
                       void* dq, void* dk, void* dv, float* dz,
                       void* workspace, size_t workspace_bytes, void* stream,
                       float* kernel_ms, const char** kernel_names, int cap, int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* TWOMAMBA_H */
