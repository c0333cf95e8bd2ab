// Host side of the 2Mamba C ABI: argument validation (before any HIP call),
// path selection and status strings.  Kernels live in the .hip sources.
#include <stdint.h>
#include <string.h>

#include <initializer_list>

#include "internal.h"

using twm::FwdArgs;
using twm::StepArgs;

namespace {

bool mul_ok(size_t a, size_t b, size_t* r) { return !__builtin_mul_overflow(a, b, r); }

// product of non-negative ints into size_t, false on overflow
bool prod(size_t* r, std::initializer_list<size_t> xs) {
    size_t acc = 1;
    for (size_t x : xs)
        if (!mul_ok(acc, x, &acc)) return false;
    *r = acc;
    return true;
}

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

bool overlaps(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

Range rng(const void* p, size_t bytes) {
    uintptr_t u = (uintptr_t)p;
    return Range{u, p ? u + bytes : u};
}

bool supported_dims(int dk, int dv) { return dk == dv && (dk == 16 || dk == 64); }

// Validates everything but pointers/workspace; fills the byte sizes.
int check_desc(const twomamba_fwd_desc* d, size_t* qk_bytes, size_t* v_bytes, size_t* z_bytes,
               size_t* st_bytes, size_t* nm_bytes) {
    if (!d) return TWOMAMBA_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->T < 0 || d->dk <= 0 || d->dv <= 0) return TWOMAMBA_ERR_SHAPE;
    if (d->variant != TWOMAMBA_SQ && d->variant != TWOMAMBA_EXP && d->variant != TWOMAMBA_LIN)
        return TWOMAMBA_ERR_DTYPE;
    if (d->dtype != TWOMAMBA_F32 && d->dtype != TWOMAMBA_BF16) return TWOMAMBA_ERR_DTYPE;
    if (d->flags & ~(unsigned)(TWOMAMBA_FLAG_NO_NORM | TWOMAMBA_FLAG_REFERENCE_KERNELS | TWOMAMBA_FLAG_ATTENTION_FORM |
                               TWOMAMBA_FLAG_CHUNKED_FORM))
        return TWOMAMBA_ERR_UNSUPPORTED;
    if (d->variant == TWOMAMBA_EXP && (d->flags & TWOMAMBA_FLAG_NO_NORM)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!supported_dims(d->dk, d->dv)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
        return TWOMAMBA_ERR_SHAPE;
    if (d->chunk != 0 && d->chunk != 16 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128)
        return TWOMAMBA_ERR_UNSUPPORTED;
    const size_t es = d->dtype == TWOMAMBA_BF16 ? 2 : 4;
    const size_t B = d->B, H = d->H, T = d->T;
    const size_t D = d->variant == TWOMAMBA_LIN ? (size_t)d->dk : twm::num_pairs(d->dk);
    if (!prod(qk_bytes, {B, H, T, (size_t)d->dk, es}) || !prod(v_bytes, {B, H, T, (size_t)d->dv, es}) ||
        !prod(z_bytes, {B, H, T, 4}) || !prod(st_bytes, {B, H, D, (size_t)d->dv, 4}) || !prod(nm_bytes, {B, H, D, 4}))
        return TWOMAMBA_ERR_SHAPE;
    // grid limits: (B*H) * chunks or query tiles must fit a 31-bit grid
    size_t tiles = (T + 15) / 16, g;
    if (!prod(&g, {B, H, tiles}) || g > 0x7fffffffu) return TWOMAMBA_ERR_SHAPE;
    return TWOMAMBA_OK;
}

// Chooses the path and the effective chunk.  Returns a status.
int plan(const twomamba_fwd_desc* d, FwdArgs* a) {
    memset(a, 0, sizeof(*a));
    a->B = d->B; a->H = d->H; a->T = d->T; a->dk = d->dk; a->dv = d->dv;
    a->scale = d->scale; a->variant = d->variant; a->dtype = d->dtype; a->flags = d->flags;
    a->chunk = d->chunk;
    return TWOMAMBA_OK;
}

enum Path { REF, MFMA, LINP };

int choose(FwdArgs* a, Path* path) {
    const bool force_ref = (a->flags & TWOMAMBA_FLAG_REFERENCE_KERNELS) != 0;
    if (a->variant == TWOMAMBA_LIN) {
        a->chunk = 64;
        *path = LINP;
        return TWOMAMBA_OK;
    }
    if (a->variant == TWOMAMBA_EXP) {
        a->chunk = 0;
        *path = (!force_ref && twm::mfma_exp_supported(*a)) ? MFMA : REF;
        return TWOMAMBA_OK;
    }
    if (!force_ref) {
        FwdArgs t = *a;
        if (t.chunk == 0) t.chunk = 64;
        if (twm::mfma_sq_supported(t)) {
            *a = t;
            *path = MFMA;
            return TWOMAMBA_OK;
        }
    }
    if (a->chunk == 0) a->chunk = 64;
    if (a->chunk > 64) return TWOMAMBA_ERR_UNSUPPORTED;   // reference kernels stage <= 64 tokens
    *path = REF;
    return TWOMAMBA_OK;
}

size_t workspace_for(const FwdArgs& a, Path path) {
    if (a.variant == TWOMAMBA_EXP) return 0;
    if (path == LINP) return twm::lin_workspace(a);
    return path == MFMA ? twm::mfma_sq_workspace(a) : twm::ref_sq_workspace(a);
}

// Input convolution of twomamba_fwd_conv: which tensors go through the
// standalone pass into the workspace (after the path's own workspace) and which
// the path's kernels convolve while loading them.
struct ConvPlan {
    int first, count;   // tensors (of q, k, v) convolved by the pass
    bool fused_all;     // the first-order MFMA kernels convolve q, k and v themselves
    bool fused_q;       // the 2Mamba-E MFMA kernel convolves q itself
    size_t tensor_bytes, off, total;   // one convolved tensor; where the pass's outputs start; all bytes
};

ConvPlan conv_plan(const FwdArgs& a, Path path, size_t path_ws) {
    ConvPlan c{0, 3, false, false, 0, 0, path_ws};
    const size_t es = a.dtype == TWOMAMBA_BF16 ? 2 : 4;
    c.tensor_bytes = twm::align256((size_t)a.B * a.H * a.T * a.dk * es);
    if (path == LINP && twm::lin_conv_fused(a)) {
        c.count = 0;
        c.fused_all = true;
    } else if (path == MFMA && a.variant == TWOMAMBA_EXP) {
        c.first = 1;   // k and v: every query tile re-reads them, so they are convolved once up front
        c.count = 2;
        c.fused_q = true;
    }
    if ((size_t)a.B * a.H * a.T == 0) c.count = 0;
    c.off = twm::align256(path_ws);
    c.total = c.count ? c.off + (size_t)c.count * c.tensor_bytes : path_ws;
    return c;
}


}  // namespace

extern "C" {

int twomamba_abi_version(void) { return TWOMAMBA_ABI_VERSION; }

const char* twomamba_status_str(int s) {
    switch (s) {
        case TWOMAMBA_OK: return "ok";
        case TWOMAMBA_ERR_NULL: return "required pointer is NULL";
        case TWOMAMBA_ERR_SHAPE: return "invalid or overflowing shape/scale";
        case TWOMAMBA_ERR_DTYPE: return "invalid dtype or variant";
        case TWOMAMBA_ERR_UNSUPPORTED: return "unsupported configuration";
        case TWOMAMBA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case TWOMAMBA_ERR_DEVICE: return "HIP launch or device error";
        case TWOMAMBA_ERR_ALIAS: return "output overlaps an input";
        case TWOMAMBA_ERR_SCRATCH: return "workspace larger than the library's static scratch";
        default: return "unknown status";
    }
}

int twomamba_fwd_workspace_size(const twomamba_fwd_desc* d, size_t* bytes) {
    if (!bytes) return TWOMAMBA_ERR_NULL;
    *bytes = 0;
    size_t a1, a2, a3, a4, a5;
    int s = check_desc(d, &a1, &a2, &a3, &a4, &a5);
    if (s != TWOMAMBA_OK) return s;
    FwdArgs a;
    plan(d, &a);
    Path path;
    s = choose(&a, &path);
    if (s != TWOMAMBA_OK) return s;
    *bytes = workspace_for(a, path);
    return TWOMAMBA_OK;
}

// With `noalloc`, the workspace arguments are ignored and the call runs on the
// library's static scratch (twomamba_fwd_noalloc).
// The size-2 input convolution of twomamba_fwd_conv (NULL for the other forwards).
struct ConvIn {
    const float* w;
    const float* b;
    const void* prev;
    void* prev_out;
};

static int fwd_impl(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                    const float* state_in, const float* norm_in, void* out, float* state_out, float* norm_out,
                    float* row_stat, void* workspace, size_t workspace_bytes, void* stream, twm::KTimer* timer,
                    bool noalloc = false, const ConvIn* conv = nullptr) {
    size_t qkb, vb, zb, sb, nb;
    int s = check_desc(d, &qkb, &vb, &zb, &sb, &nb);
    if (s != TWOMAMBA_OK) return s;
    if (conv && d->dk != d->dv) return TWOMAMBA_ERR_UNSUPPORTED;
    const bool any = qkb != 0;   // B*H*T > 0
    const bool sq = d->variant == TWOMAMBA_SQ, lin = d->variant == TWOMAMBA_LIN;
    if (!sq && !lin && (state_in || norm_in || state_out || norm_out)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (lin && (norm_in || norm_out || row_stat)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (sq && (state_in == nullptr) != (norm_in == nullptr)) return TWOMAMBA_ERR_NULL;
    if (sq && (state_out == nullptr) != (norm_out == nullptr)) return TWOMAMBA_ERR_NULL;
    if (any && (!q || !k || !v || !z || !out)) return TWOMAMBA_ERR_NULL;

    // aliasing: out and the state outputs may not touch any input; the state
    // outputs may alias the state inputs only exactly (in-place resume).
    const Range rq = rng(q, qkb), rk = rng(k, qkb), rv = rng(v, vb), rz = rng(z, zb);
    const Range rsi = rng(state_in, sb), rni = rng(norm_in, nb), ro = rng(out, vb);
    const Range rso = rng(state_out, sb), rno = rng(norm_out, nb);
    for (const Range& in : {rq, rk, rv, rz, rsi, rni})
        if (overlaps(ro, in)) return TWOMAMBA_ERR_ALIAS;
    for (const Range& in : {rq, rk, rv, rz, ro})
        if (overlaps(rso, in) || overlaps(rno, in)) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rso, rno)) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rso, rsi) && state_out != state_in) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rno, rni) && norm_out != norm_in) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rso, rni) || overlaps(rno, rsi)) return TWOMAMBA_ERR_ALIAS;
    const Range rst = rng(row_stat, zb);   // [B][H][T] fp32, the size of z
    for (const Range& x : {rq, rk, rv, rz, rsi, rni, ro, rso, rno})
        if (overlaps(rst, x)) return TWOMAMBA_ERR_ALIAS;
    Range rcw{0, 0}, rcb{0, 0}, rcp{0, 0}, rcpo{0, 0};
    if (conv) {
        size_t wb, bb, cb;
        const size_t es = d->dtype == TWOMAMBA_BF16 ? 2 : 4;
        if (!prod(&wb, {3, (size_t)d->H, (size_t)d->dk, 2, 4}) || !prod(&bb, {3, (size_t)d->H, (size_t)d->dk, 4}) ||
            !prod(&cb, {(size_t)d->B, (size_t)d->H, 3, (size_t)d->dk, es}))
            return TWOMAMBA_ERR_SHAPE;
        if ((size_t)d->B * d->H > 0 && !conv->w) return TWOMAMBA_ERR_NULL;
        if (((uintptr_t)conv->w & 15u) || ((uintptr_t)conv->b & 15u) || ((uintptr_t)conv->prev & 15u))
            return TWOMAMBA_ERR_UNSUPPORTED;
        rcw = rng(conv->w, wb);
        rcb = rng(conv->b, bb);
        rcp = rng(conv->prev, cb);
        rcpo = rng(conv->prev_out, cb);
        for (const Range& o : {ro, rso, rno, rst})
            for (const Range& in : {rcw, rcb, rcp})
                if (overlaps(o, in)) return TWOMAMBA_ERR_ALIAS;
        for (const Range& x : {rq, rk, rv, rz, rsi, rni, ro, rso, rno, rst, rcw, rcb, rcp})
            if (overlaps(rcpo, x)) return TWOMAMBA_ERR_ALIAS;
    }

    FwdArgs a;
    plan(d, &a);
    Path path;
    s = choose(&a, &path);
    if (s != TWOMAMBA_OK) return s;
    const size_t path_need = workspace_for(a, path);
    const ConvPlan cp = conv ? conv_plan(a, path, path_need) : ConvPlan{0, 0, false, false, 0, 0, path_need};
    const size_t need = cp.total;
    if (noalloc) {
        // every check above has passed; the scratch lookup is the call's first HIP call
        if (need > (size_t)TWOMAMBA_NOALLOC_SCRATCH_BYTES) return TWOMAMBA_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            const int st = twm::noalloc_scratch(stream, &workspace);
            if (st != TWOMAMBA_OK) return st;
            workspace_bytes = TWOMAMBA_NOALLOC_SCRATCH_BYTES;
        }
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return TWOMAMBA_ERR_WORKSPACE;
        const Range rw = rng(workspace, need);
        for (const Range& o : {rq, rk, rv, rz, rsi, rni, ro, rso, rno, rst, rcw, rcb, rcp, rcpo})
            if (overlaps(rw, o)) return TWOMAMBA_ERR_ALIAS;
    }
    a.q = q; a.k = k; a.v = v; a.z = z;
    a.state_in = state_in; a.norm_in = norm_in;
    a.out = out; a.state_out = state_out; a.norm_out = norm_out;
    a.ws = workspace; a.ws_bytes = workspace_bytes; a.stream = stream;
    a.timer = timer;
    a.row_stat = row_stat;
    if (conv) {
        twm::ConvArgs ca;
        memset(&ca, 0, sizeof(ca));
        ca.B = d->B; ca.H = d->H; ca.T = d->T; ca.d = d->dk; ca.dtype = d->dtype;
        ca.q = q; ca.k = k; ca.v = v; ca.w = conv->w; ca.b = conv->b; ca.prev = conv->prev;
        ca.prev_out = conv->prev_out; ca.stream = stream;
        if (cp.count > 0) {
            // the pass's outputs: tensors first .. first + count - 1, one slot each
            void* conv_out[3] = {nullptr, nullptr, nullptr};
            for (int i = cp.first; i < cp.first + cp.count; ++i)
                conv_out[i] = (char*)workspace + cp.off + (size_t)(i - cp.first) * cp.tensor_bytes;
            ca.qo = conv_out[0]; ca.ko = conv_out[1]; ca.vo = conv_out[2];
            ca.first = cp.first;
            ca.count = cp.count;
            ca.prev_out = nullptr;   // written by the tail below, from the raw rows
            const int cs = twm::conv2_launch(ca);
            if (cs != TWOMAMBA_OK) return cs;
            if (cp.first <= 0) a.q = conv_out[0];
            a.k = conv_out[1];
            a.v = conv_out[2];
        }
        if (cp.fused_all || cp.fused_q) {
            a.conv_w = conv->w;
            a.conv_b = conv->b;
            a.conv_prev = conv->prev;
            a.conv_q_only = cp.fused_q;
        }
    }
    int rs;
    if (path == LINP) rs = twm::lin_fwd(a);
    else if (a.variant == TWOMAMBA_EXP) rs = path == MFMA ? twm::mfma_exp_fwd(a) : twm::ref_exp_fwd(a);
    else rs = path == MFMA ? twm::mfma_sq_fwd(a) : twm::ref_sq_fwd(a);
    if (rs != TWOMAMBA_OK || !conv || !conv->prev_out) return rs;
    twm::ConvArgs ct;
    memset(&ct, 0, sizeof(ct));
    ct.B = d->B; ct.H = d->H; ct.T = d->T; ct.d = d->dk; ct.dtype = d->dtype;
    ct.q = q; ct.k = k; ct.v = v; ct.prev = conv->prev; ct.prev_out = conv->prev_out; ct.stream = stream;
    return twm::conv_tail_launch(ct);
}

int twomamba_fwd(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                 const float* state_in, const float* norm_in, void* out, float* state_out, float* norm_out,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_impl(d, q, k, v, z, state_in, norm_in, out, state_out, norm_out, nullptr, workspace, workspace_bytes,
                    stream, nullptr);
}

int twomamba_fwd_conv_workspace_size(const twomamba_fwd_desc* d, size_t* bytes) {
    if (!bytes) return TWOMAMBA_ERR_NULL;
    *bytes = 0;
    size_t a1, a2, a3, a4, a5;
    int s = check_desc(d, &a1, &a2, &a3, &a4, &a5);
    if (s != TWOMAMBA_OK) return s;
    if (d->dk != d->dv) return TWOMAMBA_ERR_UNSUPPORTED;
    FwdArgs a;
    plan(d, &a);
    Path path;
    s = choose(&a, &path);
    if (s != TWOMAMBA_OK) return s;
    *bytes = conv_plan(a, path, workspace_for(a, path)).total;
    return TWOMAMBA_OK;
}

int twomamba_fwd_conv(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                      const float* conv_weight, const float* conv_bias, const void* conv_state_in,
                      void* conv_state_out, const float* state_in, const float* norm_in, void* out, float* state_out,
                      float* norm_out, void* workspace, size_t workspace_bytes, void* stream) {
    const ConvIn c{conv_weight, conv_bias, conv_state_in, conv_state_out};
    return fwd_impl(d, q, k, v, z, state_in, norm_in, out, state_out, norm_out, nullptr, workspace, workspace_bytes,
                    stream, nullptr, false, &c);
}

int twomamba_fwd_noalloc(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                         const float* state_in, const float* norm_in, void* out, float* state_out, float* norm_out,
                         void* stream) {
    return fwd_impl(d, q, k, v, z, state_in, norm_in, out, state_out, norm_out, nullptr, nullptr, 0, stream, nullptr,
                    true);
}

int twomamba_fwd_stats(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                       const float* state_in, const float* norm_in, void* out, float* state_out, float* norm_out,
                       float* row_stat, void* workspace, size_t workspace_bytes, void* stream) {
    size_t qkb, vb, zb, sb, nb;
    int s = check_desc(d, &qkb, &vb, &zb, &sb, &nb);
    if (s != TWOMAMBA_OK) return s;
    if (qkb != 0 && !row_stat) return TWOMAMBA_ERR_NULL;
    return fwd_impl(d, q, k, v, z, state_in, norm_in, out, state_out, norm_out, row_stat, workspace, workspace_bytes,
                    stream, nullptr);
}

int twomamba_fwd_timed(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                       const float* state_in, const float* norm_in, void* out, float* state_out, float* norm_out,
                       void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms,
                       const char** kernel_names, int cap, int* n_kernels) {
    if (!n_kernels) return TWOMAMBA_ERR_NULL;
    *n_kernels = 0;
    twm::KTimer t;
    memset(&t, 0, sizeof(t));
    int s = fwd_impl(d, q, k, v, z, state_in, norm_in, out, state_out, norm_out, nullptr, workspace, workspace_bytes,
                     stream, &t);
    const int c = twm::ktimer_collect(&t, kernel_ms, kernel_names, cap < 0 ? 0 : cap);
    *n_kernels = t.n;
    return s != TWOMAMBA_OK ? s : c;
}

static int step_impl(const twomamba_step_desc* d, const void* q, const void* k, const void* v, const float* z,
                     const float* conv_w, const float* conv_b, void* conv_state, float* state, float* norm,
                     void* out, void* stream) {
    if (!d) return TWOMAMBA_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->dk <= 0 || d->dv <= 0) return TWOMAMBA_ERR_SHAPE;
    if (d->dtype != TWOMAMBA_F32 && d->dtype != TWOMAMBA_BF16) return TWOMAMBA_ERR_DTYPE;
    if (d->flags & ~(unsigned)(TWOMAMBA_FLAG_NO_NORM | TWOMAMBA_FLAG_FIRST_ORDER)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!supported_dims(d->dk, d->dv)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
        return TWOMAMBA_ERR_SHAPE;
    const bool first = (d->flags & TWOMAMBA_FLAG_FIRST_ORDER) != 0;
    const size_t es = d->dtype == TWOMAMBA_BF16 ? 2 : 4;
    const size_t B = d->B, H = d->H, D = first ? (size_t)d->dk : twm::num_pairs(d->dk);
    size_t qkb, vb, zb, sb, nb;
    if (!prod(&qkb, {B, H, (size_t)d->dk, es}) || !prod(&vb, {B, H, (size_t)d->dv, es}) || !prod(&zb, {B, H, 4}) ||
        !prod(&sb, {B, H, D, (size_t)d->dv, 4}) || !prod(&nb, {B, H, D, 4}))
        return TWOMAMBA_ERR_SHAPE;
    if (B * H > 0x7fffffffu) return TWOMAMBA_ERR_SHAPE;
    if (B * H == 0) return TWOMAMBA_OK;
    if (first && norm) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !z || !state || (!first && !norm) || !out) return TWOMAMBA_ERR_NULL;
    const Range rq = rng(q, qkb), rk = rng(k, qkb), rv = rng(v, vb), rz = rng(z, zb);
    const Range rs = rng(state, sb), rn = rng(norm, nb), ro = rng(out, vb);
    for (const Range& w : {rs, rn, ro})
        for (const Range& in : {rq, rk, rv, rz})
            if (overlaps(w, in)) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rs, rn) || overlaps(rs, ro) || overlaps(rn, ro)) return TWOMAMBA_ERR_ALIAS;
    if (conv_w) {
        size_t cb, wb, bb;
        if (!prod(&cb, {B, H, 3, (size_t)d->dk, es}) || !prod(&wb, {3, H, (size_t)d->dk, 2, 4}) ||
            !prod(&bb, {3, H, (size_t)d->dk, 4}))
            return TWOMAMBA_ERR_SHAPE;
        const Range rc = rng(conv_state, cb), rw = rng(conv_w, wb), rb = rng(conv_b, bb);
        for (const Range& x : {rq, rk, rv, rz, rs, rn, ro, rw, rb})
            if (overlaps(rc, x)) return TWOMAMBA_ERR_ALIAS;
        for (const Range& w : {rs, rn, ro})
            if (overlaps(w, rw) || overlaps(w, rb)) return TWOMAMBA_ERR_ALIAS;
    }
    StepArgs a;
    memset(&a, 0, sizeof(a));
    a.B = d->B; a.H = d->H; a.dk = d->dk; a.dv = d->dv; a.scale = d->scale; a.dtype = d->dtype; a.flags = d->flags;
    a.q = q; a.k = k; a.v = v; a.z = z; a.state = state; a.norm = norm; a.out = out; a.stream = stream;
    a.conv_w = conv_w; a.conv_b = conv_b; a.conv_state = conv_state;
    return twm::step_launch(a);
}

int twomamba_step(const twomamba_step_desc* d, const void* q, const void* k, const void* v, const float* z,
                  float* state, float* norm, void* out, void* stream) {
    return step_impl(d, q, k, v, z, nullptr, nullptr, nullptr, state, norm, out, stream);
}

int twomamba_step_conv(const twomamba_step_desc* d, const void* q, const void* k, const void* v, const float* z,
                       const float* conv_w, const float* conv_b, void* conv_state, float* state, float* norm,
                       void* out, void* stream) {
    if (!d) return TWOMAMBA_ERR_NULL;
    if ((size_t)(d->B < 0 ? 0 : d->B) * (size_t)(d->H < 0 ? 0 : d->H) > 0 && (!conv_w || !conv_state))
        return TWOMAMBA_ERR_NULL;
    if (d->dk != d->dv) return TWOMAMBA_ERR_UNSUPPORTED;
    return step_impl(d, q, k, v, z, conv_w, conv_b, conv_state, state, norm, out, stream);
}

// ---------------------------------------------------------------------------
// size-2 input convolution
int twomamba_conv2(const twomamba_conv_desc* d, const void* q, const void* k, const void* v, const float* weight,
                   const float* bias, const void* conv_state_in, void* q_out, void* k_out, void* v_out,
                   void* conv_state_out, void* stream) {
    if (!d) return TWOMAMBA_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->T < 0 || d->d <= 0) return TWOMAMBA_ERR_SHAPE;
    if (d->dtype != TWOMAMBA_F32 && d->dtype != TWOMAMBA_BF16) return TWOMAMBA_ERR_DTYPE;
    if (d->flags != 0u) return TWOMAMBA_ERR_UNSUPPORTED;
    if (d->d != 16 && d->d != 64) return TWOMAMBA_ERR_UNSUPPORTED;
    const size_t es = d->dtype == TWOMAMBA_BF16 ? 2 : 4;
    const size_t B = d->B, H = d->H, T = d->T, D = d->d;
    size_t xb, cb, wb, bb, g;
    if (!prod(&xb, {B, H, T, D, es}) || !prod(&cb, {B, H, 3, D, es}) || !prod(&wb, {3, H, D, 2, 4}) ||
        !prod(&bb, {3, H, D, 4}) || T * (D / 8) + 255 > 0x7fffffffu ||
        !prod(&g, {B, H, (T * (D / 8) + 255) / 256}) || g > 0x7fffffffu)
        return TWOMAMBA_ERR_SHAPE;
    if (B * H == 0) return TWOMAMBA_OK;
    if (T > 0 && (!q || !k || !v || !weight || !q_out || !k_out || !v_out)) return TWOMAMBA_ERR_NULL;
    if (((uintptr_t)weight & 15u) || ((uintptr_t)bias & 15u)) return TWOMAMBA_ERR_UNSUPPORTED;
    const Range ins[] = {rng(q, xb), rng(k, xb), rng(v, xb), rng(weight, wb), rng(bias, bb), rng(conv_state_in, cb)};
    const Range outs[] = {rng(q_out, xb), rng(k_out, xb), rng(v_out, xb), rng(conv_state_out, cb)};
    for (const Range& o : outs)
        for (const Range& in : ins)
            if (overlaps(o, in)) return TWOMAMBA_ERR_ALIAS;
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return TWOMAMBA_ERR_ALIAS;
    twm::ConvArgs a;
    memset(&a, 0, sizeof(a));
    a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.dtype = d->dtype;
    a.q = q; a.k = k; a.v = v; a.w = weight; a.b = bias; a.prev = conv_state_in;
    a.qo = q_out; a.ko = k_out; a.vo = v_out; a.prev_out = conv_state_out; a.stream = stream;
    a.first = 0;
    a.count = 3;
    return twm::conv2_launch(a);
}

// ---------------------------------------------------------------------------
// 2Mamba-E key/value cache
static int check_cache(const twomamba_exp_cache_desc* d, bool fill, size_t* kb, size_t* vb, size_t* zb,
                       size_t* kcb, size_t* vcb, size_t* gcb) {
    if (!d) return TWOMAMBA_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->dk <= 0 || d->dv <= 0 || d->max_len < 0 || d->pos < 0) return TWOMAMBA_ERR_SHAPE;
    if (d->dtype != TWOMAMBA_F32 && d->dtype != TWOMAMBA_BF16) return TWOMAMBA_ERR_DTYPE;
    if (d->flags != 0u) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!supported_dims(d->dk, d->dv)) return TWOMAMBA_ERR_UNSUPPORTED;
    if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
        return TWOMAMBA_ERR_SHAPE;
    if (fill ? d->pos > d->max_len : d->pos >= d->max_len) return TWOMAMBA_ERR_SHAPE;
    const size_t es = d->dtype == TWOMAMBA_BF16 ? 2 : 4;
    const size_t B = d->B, H = d->H, L = d->max_len, T = fill ? (size_t)d->pos : 1;
    if (!prod(kb, {B, H, T, (size_t)d->dk, es}) || !prod(vb, {B, H, T, (size_t)d->dv, es}) ||
        !prod(zb, {B, H, T, 4}) || !prod(kcb, {B, H, L, (size_t)d->dk, es}) ||
        !prod(vcb, {B, H, L, (size_t)d->dv, es}) || !prod(gcb, {B, H, L, 8}))
        return TWOMAMBA_ERR_SHAPE;
    // grid: (B*H) * splits of 512 keys must fit a 31-bit grid
    size_t g;
    if (!prod(&g, {B, H, ((size_t)d->pos + 512) / 512}) || g > 0x7fffffffu) return TWOMAMBA_ERR_SHAPE;
    return TWOMAMBA_OK;
}

static twm::ExpCacheArgs cache_args(const twomamba_exp_cache_desc* d) {
    twm::ExpCacheArgs a;
    memset(&a, 0, sizeof(a));
    a.B = d->B; a.H = d->H; a.dk = d->dk; a.dv = d->dv; a.max_len = d->max_len; a.pos = d->pos;
    a.scale = d->scale; a.dtype = d->dtype;
    return a;
}

int twomamba_exp_cache_fill(const twomamba_exp_cache_desc* d, const void* k, const void* v, const float* z,
                            void* k_cache, void* v_cache, double* g_cache, void* stream) {
    size_t kb, vb, zb, kcb, vcb, gcb;
    int s = check_cache(d, true, &kb, &vb, &zb, &kcb, &vcb, &gcb);
    if (s != TWOMAMBA_OK) return s;
    if ((size_t)d->B * d->H == 0 || d->pos == 0) return TWOMAMBA_OK;
    if (!k || !v || !z || !k_cache || !v_cache || !g_cache) return TWOMAMBA_ERR_NULL;
    const Range rk = rng(k, kb), rv = rng(v, vb), rz = rng(z, zb);
    const Range rkc = rng(k_cache, kcb), rvc = rng(v_cache, vcb), rgc = rng(g_cache, gcb);
    for (const Range& w : {rkc, rvc, rgc})
        for (const Range& in : {rk, rv, rz})
            if (overlaps(w, in)) return TWOMAMBA_ERR_ALIAS;
    if (overlaps(rkc, rvc) || overlaps(rkc, rgc) || overlaps(rvc, rgc)) return TWOMAMBA_ERR_ALIAS;
    twm::ExpCacheArgs a = cache_args(d);
    a.k = k; a.v = v; a.z = z; a.k_cache = k_cache; a.v_cache = v_cache; a.g_cache = g_cache; a.stream = stream;
    return twm::exp_cache_fill_launch(a);
}

int twomamba_exp_step_workspace_size(const twomamba_exp_cache_desc* d, size_t* bytes) {
    if (!bytes) return TWOMAMBA_ERR_NULL;
    size_t kb, vb, zb, kcb, vcb, gcb;
    int s = check_cache(d, false, &kb, &vb, &zb, &kcb, &vcb, &gcb);
    if (s != TWOMAMBA_OK) return s;
    *bytes = twm::exp_step_workspace(cache_args(d));
    return TWOMAMBA_OK;
}

int twomamba_exp_step(const twomamba_exp_cache_desc* d, const void* q, const void* k, const void* v,
                      const float* z, void* k_cache, void* v_cache, double* g_cache, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    size_t kb, vb, zb, kcb, vcb, gcb;
    int s = check_cache(d, false, &kb, &vb, &zb, &kcb, &vcb, &gcb);
    if (s != TWOMAMBA_OK) return s;
    if ((size_t)d->B * d->H == 0) return TWOMAMBA_OK;
    if (!q || !k || !v || !z || !k_cache || !v_cache || !g_cache || !out) return TWOMAMBA_ERR_NULL;
    twm::ExpCacheArgs a = cache_args(d);
    const size_t need = twm::exp_step_workspace(a);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return TWOMAMBA_ERR_WORKSPACE;
    const Range rq = rng(q, kb), rk = rng(k, kb), rv = rng(v, vb), rz = rng(z, zb), ro = rng(out, vb);
    const Range rkc = rng(k_cache, kcb), rvc = rng(v_cache, vcb), rgc = rng(g_cache, gcb), rws = rng(workspace, need);
    for (const Range& w : {rkc, rvc, rgc, ro, rws})
        for (const Range& in : {rq, rk, rv, rz})
            if (overlaps(w, in)) return TWOMAMBA_ERR_ALIAS;
    const Range outs[] = {rkc, rvc, rgc, ro, rws};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j])) return TWOMAMBA_ERR_ALIAS;
    a.q = q; a.k = k; a.v = v; a.z = z; a.k_cache = k_cache; a.v_cache = v_cache; a.g_cache = g_cache; a.out = out;
    a.ws = workspace; a.ws_bytes = workspace_bytes; a.stream = stream;
    return twm::exp_step_launch(a);
}

// ---------------------------------------------------------------------------
// backward
static int check_bwd(const twomamba_fwd_desc* d, size_t* qkb, size_t* vb, size_t* zb) {
    size_t sb, nb;
    int s = check_desc(d, qkb, vb, zb, &sb, &nb);
    if (s != TWOMAMBA_OK) return s;
    size_t g;
    if (!prod(&g, {(size_t)d->B, (size_t)d->H, ((size_t)d->T + 63) / 64}) || g > 0x7fffffffu)
        return TWOMAMBA_ERR_SHAPE;
    if ((size_t)d->B * d->H > 0x7fffffffu) return TWOMAMBA_ERR_SHAPE;
    return TWOMAMBA_OK;
}

static twm::BwdArgs bwd_args(const twomamba_fwd_desc* d) {
    twm::BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.B = d->B; a.H = d->H; a.T = d->T; a.dk = d->dk; a.dv = d->dv;
    a.scale = d->scale; a.variant = d->variant; a.dtype = d->dtype; a.flags = d->flags;
    return a;
}

int twomamba_bwd_workspace_size(const twomamba_fwd_desc* d, size_t* bytes) {
    if (!bytes) return TWOMAMBA_ERR_NULL;
    *bytes = 0;
    size_t qkb, vb, zb;
    int s = check_bwd(d, &qkb, &vb, &zb);
    if (s != TWOMAMBA_OK) return s;
    const twm::BwdArgs ba = bwd_args(d);
    *bytes = twm::lin_bwd_chunked_supported(ba)  ? twm::lin_bwd_chunked_workspace(ba)
             : twm::sq_bwd_chunked_supported(ba) ? twm::sq_bwd_chunked_workspace(ba)
                                                 : twm::bwd_workspace(ba);
    return TWOMAMBA_OK;
}

static int bwd_impl(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                    const void* out, const void* dout, const float* row_stat, void* dq, void* dk, void* dv, float* dz,
                    void* workspace, size_t workspace_bytes, void* stream, twm::KTimer* timer) {
    size_t qkb, vb, zb;
    int s = check_bwd(d, &qkb, &vb, &zb);
    if (s != TWOMAMBA_OK) return s;
    if (qkb == 0) return TWOMAMBA_OK;
    if (!q || !k || !v || !z || !out || !dout || !dq || !dk || !dv || !dz) return TWOMAMBA_ERR_NULL;
    twm::BwdArgs a = bwd_args(d);
    const bool chunked = twm::lin_bwd_chunked_supported(a);
    const bool sq_chunked = !chunked && twm::sq_bwd_chunked_supported(a);
    const size_t need = chunked      ? twm::lin_bwd_chunked_workspace(a)
                        : sq_chunked ? twm::sq_bwd_chunked_workspace(a)
                                     : twm::bwd_workspace(a);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return TWOMAMBA_ERR_WORKSPACE;
    const Range ins[] = {rng(q, qkb), rng(k, qkb), rng(v, vb), rng(z, zb), rng(out, vb), rng(dout, vb),
                         rng(row_stat, zb)};
    const Range outs[] = {rng(dq, qkb), rng(dk, qkb), rng(dv, vb), rng(dz, zb), rng(workspace, need)};
    for (const Range& o : outs)
        for (const Range& in : ins)
            if (overlaps(o, in)) return TWOMAMBA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j])) return TWOMAMBA_ERR_ALIAS;
    a.q = q; a.k = k; a.v = v; a.z = z; a.out = out; a.dout = dout;
    a.row_stat = d->variant == TWOMAMBA_LIN ? nullptr : row_stat;   // the first order has none
    a.gq = dq; a.gk = dk; a.gv = dv; a.gz = dz;
    a.ws = workspace; a.ws_bytes = workspace_bytes; a.stream = stream; a.timer = timer;
    if (chunked) return twm::lin_bwd_chunked(a);
    if (sq_chunked) return twm::sq_bwd_chunked(a);
    return twm::mfma_bwd_supported(a) ? twm::mfma_bwd(a) : twm::ref_bwd(a);
}

int twomamba_bwd(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                 const void* out, const void* dout, const float* row_stat, void* dq, void* dk, void* dv, float* dz,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(d, q, k, v, z, out, dout, row_stat, dq, dk, dv, dz, workspace, workspace_bytes, stream, nullptr);
}

int twomamba_bwd_timed(const twomamba_fwd_desc* d, const void* q, const void* k, const void* v, const float* z,
                       const void* out, const void* dout, const float* row_stat, void* dq, void* dk, void* dv,
                       float* dz, void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms,
                       const char** kernel_names, int cap, int* n_kernels) {
    if (!n_kernels) return TWOMAMBA_ERR_NULL;
    *n_kernels = 0;
    twm::KTimer t;
    memset(&t, 0, sizeof(t));
    int s = bwd_impl(d, q, k, v, z, out, dout, row_stat, dq, dk, dv, dz, workspace, workspace_bytes, stream, &t);
    const int c = twm::ktimer_collect(&t, kernel_ms, kernel_names, cap < 0 ? 0 : cap);
    *n_kernels = t.n;
    return s != TWOMAMBA_OK ? s : c;
}

}  // extern "C"
