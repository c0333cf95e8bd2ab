"""fp64 CPU oracle for the 2Mamba / 2Mamba-E sequence-mixing operator.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, table or constant with the
HIP library and imports nothing from it.

Source: "2Mamba2Furious: Linear in Complexity, Competitive in Accuracy"
(paperlayer summary of arXiv 2602.17363), cited below as [2M2F §n].  The
pages describe the operator in prose only; where they leave a step open the
plainest reading is taken and named here (the same list sits in the design
notes):

* decay: g_t = -softplus(z_t) with the exact softplus max(x,0)+log1p(exp(-|x|))
  (softplus A-mask that drops the discretisation parameter, [2M2F §3, §4];
  equal to the forgetting transformer's log-sigmoid up to the sign of its
  argument, [2M2F §6]).
* mask: L_ts = exp(sum_{r=s+1..t} g_r) for s <= t, so the diagonal L_tt = 1 is
  kept (standard causal mask).
* 2Mamba: weight w_ts = L_ts * (scale * q_t.k_s)^2 -- the square is taken of
  the query-key product and the mask multiplies the squared score; the mask
  itself is not squared [2M2F §5].  "Softmax normalisation" [2M2F §5] is read
  as dividing by the sum of the same weights; o_t = 0 when that sum is 0.
* 2Mamba-E: softmax over s <= t of scale * q_t.k_s + log L_ts, i.e. softmax
  attention with the softplus A-mask as an additive log-bias [2M2F §6].
* second-order state: the symmetric k (x) k (x) v tensor [2M2F §2] packed as
  the row-major upper triangle p(i,j) = i*d - i*(i-1)/2 + (j-i), i <= j,
  holding the unscaled products k_i*k_j; the off-diagonal weight 2 lives on
  the query side.  A normaliser state n (same packing, sum of k (x) k) carries
  the softmax-normalisation denominator.
* an initial state enters as the state "before token 0" and is decayed by g_0
  like any earlier token (the Mamba-2 recurrence h_t = a_t h_{t-1} + ...,
  "Mamba-2 - State Space Duality" thread); a decode step consumes the decay
  logit of its own token.

Conv, time discretisation, gating and output norms are outside the operator:
the kernels of [2M2F App. C] take Q, K, V and return post-attention outputs
without pre- or post-processing.

Every function works on fp64 numpy arrays with leading batch/head axes
[B, H, ...] and treats each (b, h) independently.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softplus", "decay_log", "num_pairs", "pair_index", "pair_list",
    "phi_k", "phi_q", "fwd_quadratic", "fwd_quadratic_rows", "final_state_direct",
    "fwd_recurrent_full", "fwd_recurrent_packed", "step",
    "fwd_exp_quadratic", "fwd_exp_quadratic_rows", "fwd_exp_streaming",
    "state_elements", "memory_crossover_tokens",
    "sigmoid", "bwd_quadratic", "bwd_exp_quadratic", "conv2", "step_conv",
    "fwd_linear_quadratic", "fwd_linear_recurrent", "step_linear", "bwd_linear_quadratic", "bwd_blocked",
    "row_weight_sums", "row_logsumexp",
]


# ----------------------------------------------------------------------------
# decay  [2M2F §3 softplus A-mask; §6 log-sigmoid connection]
# ----------------------------------------------------------------------------

def softplus(x):
    """Exact softplus, log(1 + e^x), computed without overflow.

    softplus(-inf) = 0 exactly; no large-argument linearisation threshold.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        out = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    return np.where(np.isneginf(x), 0.0, out)


def decay_log(z):
    """Per-token log decay g = -softplus(z) <= 0 (so every L_ts lies in (0, 1])."""
    return -softplus(z)


# ----------------------------------------------------------------------------
# second-order features  [2M2F §2 higher-order state of about (dh^2, dh)]
# ----------------------------------------------------------------------------

def num_pairs(d: int) -> int:
    """Number of distinct entries of a symmetric d x d tensor, d(d+1)/2."""
    return d * (d + 1) // 2


def pair_index(i: int, j: int, d: int) -> int:
    """Packed position of the unordered pair (i, j), i <= j: row-major upper triangle."""
    if not (0 <= i <= j < d):
        raise ValueError("need 0 <= i <= j < d")
    return i * d - i * (i - 1) // 2 + (j - i)


def pair_list(d: int):
    """Arrays (I, J) with (I[p], J[p]) the pair stored at packed position p."""
    I = np.empty(num_pairs(d), dtype=np.int64)
    J = np.empty(num_pairs(d), dtype=np.int64)
    for i in range(d):
        for j in range(i, d):
            p = pair_index(i, j, d)
            I[p], J[p] = i, j
    return I, J


def phi_k(k):
    """Key-side features k_i k_j (i <= j), unscaled: [..., d] -> [..., D]."""
    I, J = pair_list(k.shape[-1])
    return k[..., I] * k[..., J]


def phi_q(q):
    """Query-side features c_ij q_i q_j with c = 2 off the diagonal, 1 on it.

    With phi_k this gives phi_q(q) . phi_k(k) = (q . k)^2.
    """
    I, J = pair_list(q.shape[-1])
    c = np.where(I == J, 1.0, 2.0)
    return c * q[..., I] * q[..., J]


# ----------------------------------------------------------------------------
# form (A): quadratic masked form, built row by row
# ----------------------------------------------------------------------------

def _row_log_mask(g_row_upto_t):
    """lambda_ts for s = 0..t from g_0..g_t, summed backward from the diagonal.

    lambda_tt = 0; lambda_t,s-1 = lambda_ts + g_s.  No global cumulative sum.
    """
    t = g_row_upto_t.shape[-1] - 1
    lam = np.zeros(g_row_upto_t.shape[:-1] + (t + 1,))
    if t > 0:
        # lambda_t,s = sum_{r=s+1}^{t} g_r  for s = 0..t-1
        tail = g_row_upto_t[..., 1:][..., ::-1]          # g_t, g_{t-1}, ..., g_1
        lam[..., :t] = np.cumsum(tail, axis=-1)[..., ::-1]
    return lam


def _sq_row(q_t, K, V, g_upto_t, scale, init_num=None, init_den=None, init_decay=None):
    lam = _row_log_mask(g_upto_t)                          # [..., t+1]
    score = scale * np.einsum("...d,...sd->...s", q_t, K)  # [..., t+1]
    w = np.exp(lam) * score * score
    num = np.einsum("...s,...sc->...c", w, V)
    den = w.sum(axis=-1)
    if init_num is not None:
        num = num + init_decay[..., None] * init_num
        den = den + init_decay * init_den
    return num, den


def _normalise(num, den, norm):
    if not norm:
        return num
    safe = np.where(den == 0.0, 1.0, den)
    return np.where(den[..., None] == 0.0, 0.0, num / safe[..., None])


def _init_terms(q, scale, state_in, norm_in):
    """phi_q(scale q_t) . S0 and phi_q(scale q_t) . n0 for every t."""
    fq = phi_q(scale * q)                                  # [B,H,T,D]
    num0 = np.einsum("bhtp,bhpc->bhtc", fq, state_in)
    den0 = np.einsum("bhtp,bhp->bht", fq, norm_in)
    return num0, den0


def fwd_quadratic(q, k, v, z, scale=1.0, norm=True, state_in=None, norm_in=None):
    """2Mamba output by the masked quadratic form, one query row at a time.

    o_t = sum_{s<=t} L_ts (scale q_t.k_s)^2 v_s / sum_{s<=t} L_ts (scale q_t.k_s)^2,
    plus the decayed initial-state term exp(g_0+...+g_t) phi_q(scale q_t).S0.
    [2M2F §5: squared QK product, A-mask on the squared score, softmax normalisation]
    """
    g = decay_log(z)
    B, H, T, _ = q.shape
    out = np.zeros(v.shape)
    has_init = state_in is not None
    if has_init:
        num0, den0 = _init_terms(q, scale, state_in, norm_in)
    for t in range(T):
        kw = {}
        if has_init:
            kw = dict(init_num=num0[:, :, t], init_den=den0[:, :, t],
                      init_decay=np.exp(g[:, :, :t + 1].sum(axis=-1)))
        num, den = _sq_row(q[:, :, t], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1], scale, **kw)
        out[:, :, t] = _normalise(num, den, norm)
    return out


def fwd_quadratic_rows(q, k, v, z, rows, scale=1.0, norm=True, state_in=None, norm_in=None):
    """Form (A) evaluated only at the query positions ``rows`` -> [B, H, len(rows), dv]."""
    g = decay_log(z)
    res = []
    for t in rows:
        kw = {}
        if state_in is not None:
            fq = phi_q(scale * q[:, :, t])
            kw = dict(init_num=np.einsum("bhp,bhpc->bhc", fq, state_in),
                      init_den=np.einsum("bhp,bhp->bh", fq, norm_in),
                      init_decay=np.exp(g[:, :, :t + 1].sum(axis=-1)))
        num, den = _sq_row(q[:, :, t], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1], scale, **kw)
        res.append(_normalise(num, den, norm))
    return np.stack(res, axis=2)


def final_state_direct(k, v, z, state_in=None, norm_in=None):
    """State after the last token, as a direct weighted sum over all tokens.

    S_T = exp(g_0+...+g_{T-1}) S0 + sum_s exp(g_{s+1}+...+g_{T-1}) phi_k(k_s) v_s^T,
    and the same for n with v replaced by 1.  Returns (S [B,H,D,dv], n [B,H,D]).
    """
    g = decay_log(z)
    B, H, T, d = k.shape
    # exponent for token s: sum_{r=s+1}^{T-1} g_r, summed backward from the end
    tail = np.zeros((B, H, T))
    tail[:, :, :T - 1] = np.cumsum(g[:, :, 1:][:, :, ::-1], axis=-1)[:, :, ::-1]
    w = np.exp(tail)
    fk = phi_k(k)                                            # [B,H,T,D]
    S = np.einsum("bhtp,bht,bhtc->bhpc", fk, w, v)
    n = np.einsum("bhtp,bht->bhp", fk, w)
    if state_in is not None:
        a = np.exp(g.sum(axis=-1))
        S = S + a[..., None, None] * state_in
        n = n + a[..., None] * norm_in
    return S, n


# ----------------------------------------------------------------------------
# forms (B) and (C): token-by-token recurrence  [SSD duality, "Mamba-2 - State
# Space Duality" thread: scalar-times-identity A makes the recurrence a causal
# linear attention]
# ----------------------------------------------------------------------------

def fwd_recurrent_full(q, k, v, z, scale=1.0, norm=True):
    """Form (B): recurrence over an explicit d^2 feature state vec(k k^T) v^T.

    Uses no packing and no pair table; tiny inputs only.
    """
    g = decay_log(z)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, d * d, dv))
    n = np.zeros((B, H, d * d))
    out = np.zeros(v.shape)
    for t in range(T):
        a = np.exp(g[:, :, t])
        fk = np.einsum("bhi,bhj->bhij", k[:, :, t], k[:, :, t]).reshape(B, H, d * d)
        qs = scale * q[:, :, t]
        fq = np.einsum("bhi,bhj->bhij", qs, qs).reshape(B, H, d * d)
        S = a[..., None, None] * S + fk[..., :, None] * v[:, :, t][..., None, :]
        n = a[..., None] * n + fk
        num = np.einsum("bhp,bhpc->bhc", fq, S)
        den = np.einsum("bhp,bhp->bh", fq, n)
        out[:, :, t] = _normalise(num, den, norm)
    return out


def step(q, k, v, z, state, norm_state, scale=1.0, norm=True):
    """One decode step of the packed recurrence (form (C) for a single token).

    S <- e^g S + phi_k(k) v^T ;  n <- e^g n + phi_k(k) ;  o = phi_q(scale q).S / phi_q(scale q).n
    Inputs q,k [B,H,d], v [B,H,dv], z [B,H], state [B,H,D,dv], norm_state [B,H,D].
    Returns (o, new_state, new_norm) without modifying the inputs.
    """
    a = np.exp(decay_log(z))
    fk = phi_k(k)
    S = a[..., None, None] * state + fk[..., :, None] * v[..., None, :]
    n = a[..., None] * norm_state + fk
    fq = phi_q(scale * q)
    num = np.einsum("bhp,bhpc->bhc", fq, S)
    den = np.einsum("bhp,bhp->bh", fq, n)
    return _normalise(num, den, norm), S, n


def fwd_recurrent_packed(q, k, v, z, scale=1.0, norm=True, state_in=None, norm_in=None):
    """Form (C): the packed D-feature recurrence, token by token.

    Returns (out, state_out, norm_out); the state is in the packed layout above.
    """
    B, H, T, d = q.shape
    dv = v.shape[-1]
    D = num_pairs(d)
    S = np.zeros((B, H, D, dv)) if state_in is None else np.array(state_in, dtype=np.float64)
    n = np.zeros((B, H, D)) if norm_in is None else np.array(norm_in, dtype=np.float64)
    out = np.zeros(v.shape)
    for t in range(T):
        out[:, :, t], S, n = step(q[:, :, t], k[:, :, t], v[:, :, t], z[:, :, t], S, n, scale, norm)
    return out, S, n


# ----------------------------------------------------------------------------
# 2Mamba-E  [2M2F §6: exponentiated QK product = softmax attention with the
# softplus A-mask]
# ----------------------------------------------------------------------------

def _exp_row(q_t, K, V, g_upto_t, scale):
    lam = _row_log_mask(g_upto_t)
    logit = scale * np.einsum("...d,...sd->...s", q_t, K) + lam
    m = logit.max(axis=-1, keepdims=True)
    p = np.exp(logit - m)
    return np.einsum("...s,...sc->...c", p, V) / p.sum(axis=-1)[..., None]


def fwd_exp_quadratic(q, k, v, z, scale=1.0):
    """Form (E-A): masked softmax, max-subtracted, one query row at a time."""
    g = decay_log(z)
    T = q.shape[2]
    out = np.zeros(v.shape)
    for t in range(T):
        out[:, :, t] = _exp_row(q[:, :, t], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1], scale)
    return out


def fwd_exp_quadratic_rows(q, k, v, z, rows, scale=1.0):
    g = decay_log(z)
    return np.stack([_exp_row(q[:, :, t], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1], scale)
                     for t in rows], axis=2)


def fwd_exp_streaming(q, k, v, z, scale=1.0):
    """Form (E-B): decode-style evaluation over a growing key/value cache.

    Each cached key carries a running log-decay bias; when token t arrives every
    existing bias is decreased by softplus(z_t) and the new key enters with bias
    0.  The query of token t then runs an online softmax (running max, running
    sum, running weighted value) over the cache in arrival order.
    """
    g = decay_log(z)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    out = np.zeros(v.shape)
    bias = np.zeros((B, H, 0))
    for t in range(T):
        bias = np.concatenate([bias + g[:, :, t:t + 1], np.zeros((B, H, 1))], axis=-1)
        m = np.full((B, H), -np.inf)
        l = np.zeros((B, H))
        acc = np.zeros((B, H, dv))
        for s in range(t + 1):
            x = scale * np.einsum("bhd,bhd->bh", q[:, :, t], k[:, :, s]) + bias[:, :, s]
            m_new = np.maximum(m, x)
            alpha = np.exp(m - m_new)
            p = np.exp(x - m_new)
            l = alpha * l + p
            acc = alpha[..., None] * acc + p[..., None] * v[:, :, s]
            m = m_new
        out[:, :, t] = acc / l[..., None]
    return out


# ----------------------------------------------------------------------------
# memory accounting  [2M2F §2 KV cache of 2*N*dh per head; §5.1 crossover;
# App. A window-1 cached q, k, v for the size-2 input convolution]
# ----------------------------------------------------------------------------

def state_elements(d: int, dv: int | None = None, conv_window: int = 2) -> int:
    """Elements one head keeps between tokens: packed state, normaliser, conv cache."""
    dv = d if dv is None else dv
    D = num_pairs(d)
    return D * dv + D + (conv_window - 1) * (2 * d + dv)


def memory_crossover_tokens(d: int, dv: int | None = None, conv_window: int = 2) -> float:
    """Sequence length above which the fixed state is smaller than a 2*N*dh KV cache."""
    return state_elements(d, dv, conv_window) / (2.0 * d)


# ----------------------------------------------------------------------------
# gradients  [2M2F App. C: each attention kernel is differentiated with Q, K, V
# as its inputs and the post-attention outputs as its outputs; C.1: the A-mask
# gradient is a sum of the masked matrix over the key axis and the query axis]
#
# Both functions return the gradients of  sum_t dout_t . o_t  with respect to
# q, k, v and the decay logits z, row by row over the quadratic form (A) or
# (E-A).  The A-mask enters through lambda_ts = g_{s+1} + ... + g_t, so an
# entry (t, s) of dL/dlambda reaches every g_r with s < r <= t; g = -softplus(z)
# gives dz = -sigmoid(z) dg.
# ----------------------------------------------------------------------------

def sigmoid(x):
    """Logistic function 1 / (1 + e^-x) without overflow; sigmoid(-inf) = 0."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _add_mask_grad(dg, dlam, t):
    """dg_r += sum_{s<r} dlam_s for r = 1..t (dlam over s = 0..t of row t)."""
    if t > 0:
        dg[..., 1:t + 1] += np.cumsum(dlam[..., :t], axis=-1)


def bwd_quadratic(q, k, v, z, dout, scale=1.0, norm=True):
    """Gradients (dq, dk, dv, dz) of the 2Mamba output, form (A), no initial state.

    Row t: a_s = scale q_t.k_s, w_s = L_ts a_s^2, num = sum w_s v_s,
    den = sum w_s, o_t = num / den.  With dnum = dout_t / den and
    dden = -dout_t.o_t / den:  dL/dw_s = dnum.v_s + dden, dv_s += w_s dnum,
    dL/da_s = dL/dw_s * 2 L_ts a_s, dq_t += scale sum_s dL/da_s k_s,
    dk_s += scale dL/da_s q_t and dL/dlambda_ts = dL/dw_s * w_s.  A row whose
    den is 0 has o_t = 0 by definition and passes no gradient.  Without
    normalisation o_t = num, dnum = dout_t and dden = 0.
    """
    g = decay_log(z)
    T = q.shape[2]
    dq, dk, dv, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(z.shape)
    for t in range(T):
        K, V = k[:, :, :t + 1], v[:, :, :t + 1]
        L = np.exp(_row_log_mask(g[:, :, :t + 1]))
        a = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], K)
        w = L * a * a
        do = dout[:, :, t]
        if norm:
            den = w.sum(axis=-1)
            rden = np.where(den > 0, 1.0 / np.where(den > 0, den, 1.0), 0.0)
            o = np.einsum("bhs,bhsc->bhc", w, V) * rden[..., None]
            dnum = do * rden[..., None]
            dden = -(do * o).sum(axis=-1) * rden
        else:
            dnum = do
            dden = np.zeros(w.shape[:-1])
        dw = np.einsum("bhsc,bhc->bhs", V, dnum) + dden[..., None]
        dv[:, :, :t + 1] += w[..., None] * dnum[:, :, None, :]
        da = dw * L * 2.0 * a
        dq[:, :, t] += scale * np.einsum("bhs,bhsd->bhd", da, K)
        dk[:, :, :t + 1] += scale * da[..., None] * q[:, :, t][:, :, None, :]
        _add_mask_grad(dg, dw * w, t)
    return dq, dk, dv, -sigmoid(z) * dg


def bwd_exp_quadratic(q, k, v, z, dout, scale=1.0):
    """Gradients (dq, dk, dv, dz) of the 2Mamba-E output, form (E-A).

    Row t: p = softmax_s(scale q_t.k_s + lambda_ts), o_t = sum p_s v_s.
    dp_s = dout_t.v_s, dL/dlogit_s = p_s (dp_s - dout_t.o_t), dv_s += p_s dout_t,
    dq_t += scale sum_s dL/dlogit_s k_s, dk_s += scale dL/dlogit_s q_t, and
    dL/dlambda_ts = dL/dlogit_s.
    """
    g = decay_log(z)
    T = q.shape[2]
    dq, dk, dv, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(z.shape)
    for t in range(T):
        K, V = k[:, :, :t + 1], v[:, :, :t + 1]
        logit = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], K) + _row_log_mask(g[:, :, :t + 1])
        p = np.exp(logit - logit.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        do = dout[:, :, t]
        o = np.einsum("bhs,bhsc->bhc", p, V)
        dp = np.einsum("bhsc,bhc->bhs", V, do)
        dl = p * (dp - (do * o).sum(axis=-1)[..., None])
        dv[:, :, :t + 1] += p[..., None] * do[:, :, None, :]
        dq[:, :, t] += scale * np.einsum("bhs,bhsd->bhd", dl, K)
        dk[:, :, :t + 1] += scale * dl[..., None] * q[:, :, t][:, :, None, :]
        _add_mask_grad(dg, dl, t)
    return dq, dk, dv, -sigmoid(z) * dg


# ----------------------------------------------------------------------------
# size-2 input convolution  [2M2F §3: a convolution of kernel size 2 over the
# sequence, no activation; §4: kept in Mamba-2S; App. A: decoding caches the
# window - 1 = 1 previous query, key and value]
#
# Reading: a causal depthwise convolution of each channel of q, k and v
# separately, y_t = w1 * x_t + w0 * x_{t-1} + b, with x_{-1} the cached raw
# row of the token before the sequence (zeros when there is none).
# ----------------------------------------------------------------------------

def conv2(x, w, b=None, prev=None):
    """Causal kernel-2 convolution along the token axis, channel by channel.

    x [B, H, T, d]; w [H, d, 2] with tap 0 on x_{t-1} and tap 1 on x_t;
    b [H, d] or None; prev [B, H, d] (the raw row before token 0) or None.
    """
    B, H, T, d = x.shape
    y = np.zeros(x.shape)
    for t in range(T):
        before = x[:, :, t - 1] if t > 0 else (np.zeros((B, H, d)) if prev is None else prev)
        y[:, :, t] = w[None, :, :, 1] * x[:, :, t] + w[None, :, :, 0] * before
        if b is not None:
            y[:, :, t] += b[None]
    return y


def step_conv(q, k, v, z, w, b, conv_state, state, norm_state, scale=1.0, norm=True):
    """One decode step with the input convolution in front of the recurrence.

    w [3, H, d, 2] and b [3, H, d] (or None) hold the q, k, v convolutions;
    conv_state [B, H, 3, d] holds the raw q, k, v of the previous token.
    Returns (out, state, norm, new conv_state = the raw q, k, v of this token).
    """
    xs = (q, k, v)
    ys = []
    for i in range(3):
        bi = None if b is None else b[i]
        ys.append(conv2(xs[i][:, :, None], w[i], bi, conv_state[:, :, i])[:, :, 0])
    out, S, n = step(ys[0], ys[1], ys[2], z, state, norm_state, scale=scale, norm=norm)
    return out, S, n, np.stack([q, k, v], axis=2)


# ----------------------------------------------------------------------------
# first-order variant (Mamba-2S)  [2M2F §2: first-order linear attention keeps a
# (dh, dh) state; §3-§4: the Mamba-2S base is output-norm linear attention with
# the softplus A-mask -- the norm sits outside the attention kernel, so the
# kernel returns the unnormalised sum]
#
#   o_t = sum_{s<=t} L_ts (scale q_t.k_s) v_s,   state S = sum_s L k_s v_s^T.
# ----------------------------------------------------------------------------

def fwd_linear_quadratic(q, k, v, z, scale=1.0, state_in=None):
    """First-order output by the masked quadratic form, one query row at a time,
    plus the decayed initial-state term exp(g_0+...+g_t) scale q_t.S0."""
    g = decay_log(z)
    T = q.shape[2]
    out = np.zeros(v.shape)
    for t in range(T):
        L = np.exp(_row_log_mask(g[:, :, :t + 1]))
        w = L * scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], k[:, :, :t + 1])
        out[:, :, t] = np.einsum("bhs,bhsc->bhc", w, v[:, :, :t + 1])
        if state_in is not None:
            out[:, :, t] += np.exp(g[:, :, :t + 1].sum(axis=-1))[..., None] * scale * np.einsum(
                "bhd,bhdc->bhc", q[:, :, t], state_in)
    return out


def step_linear(q, k, v, z, state, scale=1.0):
    """One first-order decode step: S <- e^g S + k v^T, o = scale q.S."""
    a = np.exp(decay_log(z))
    S = a[..., None, None] * state + k[..., :, None] * v[..., None, :]
    return scale * np.einsum("bhd,bhdc->bhc", q, S), S


def fwd_linear_recurrent(q, k, v, z, scale=1.0, state_in=None):
    """First-order recurrence token by token; returns (out, final state [B,H,dk,dv])."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state_in is None else state_in.copy()
    out = np.zeros(v.shape)
    for t in range(T):
        out[:, :, t], S = step_linear(q[:, :, t], k[:, :, t], v[:, :, t], z[:, :, t], S, scale)
    return out, S


def bwd_linear_quadratic(q, k, v, z, dout, scale=1.0):
    """Gradients (dq, dk, dv, dz) of the first-order output (no initial state).

    Row t: w_s = L_ts scale q_t.k_s, o_t = sum w_s v_s; dL/dw_s = dout_t.v_s,
    dv_s += w_s dout_t, dq_t += scale sum_s dL/dw_s L_ts k_s,
    dk_s += scale dL/dw_s L_ts q_t, dL/dlambda_ts = dL/dw_s w_s.
    """
    g = decay_log(z)
    T = q.shape[2]
    dq, dk, dv, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(z.shape)
    for t in range(T):
        K, V = k[:, :, :t + 1], v[:, :, :t + 1]
        L = np.exp(_row_log_mask(g[:, :, :t + 1]))
        w = L * scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], K)
        do = dout[:, :, t]
        dw = np.einsum("bhsc,bhc->bhs", V, do)
        dv[:, :, :t + 1] += w[..., None] * do[:, :, None, :]
        da = dw * L * scale
        dq[:, :, t] += np.einsum("bhs,bhsd->bhd", da, K)
        dk[:, :, :t + 1] += da[..., None] * q[:, :, t][:, :, None, :]
        _add_mask_grad(dg, dw * w, t)
    return dq, dk, dv, -sigmoid(z) * dg


def bwd_blocked(q, k, v, z, dout, variant="sq", scale=1.0, norm=True, block=512):
    """The same gradients as bwd_quadratic / bwd_exp_quadratic /
    bwd_linear_quadratic, written with whole score matrices for long sequences:
    query rows are taken `block` at a time against every key.  lambda_ts comes
    from the running sum G_t = g_0 + ... + g_t (fp64) as G_t - G_s.  Returns
    (dq, dk, dv, dz) for inputs [B, H, T, d] (one (b, h) at a time).
    """
    g = decay_log(z)
    B, H, T, _ = q.shape
    dq, dk, dv, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(z.shape)
    for b in range(B):
        for h in range(H):
            Q, K, V, DO = q[b, h], k[b, h], v[b, h], dout[b, h]
            G = np.cumsum(g[b, h])
            rows = np.zeros(T)      # strict row sums of dL/dlambda
            cols = np.zeros(T)      # strict column sums
            for r0 in range(0, T, block):
                r1 = min(T, r0 + block)
                t = np.arange(r0, r1)[:, None]
                s_ = np.arange(T)[None, :]
                causal = s_ <= t
                lam = np.where(causal, G[r0:r1, None] - G[None, :], -np.inf)
                x = scale * (Q[r0:r1] @ K.T)
                if variant == "exp":
                    logit = np.where(causal, x + lam, -np.inf)
                    P = np.exp(logit - logit.max(axis=1, keepdims=True))
                    P /= P.sum(axis=1, keepdims=True)
                    o = P @ V
                    dP = DO[r0:r1] @ V.T
                    dS = P * (dP - (DO[r0:r1] * o).sum(axis=1, keepdims=True))
                    dx, M, W = dS, dS, P
                else:
                    L = np.where(causal, np.exp(np.where(causal, lam, 0.0)), 0.0)
                    if variant == "sq":
                        w = L * x * x
                        den = w.sum(axis=1, keepdims=True)
                        if norm:
                            rden = np.where(den > 0, 1.0 / np.where(den > 0, den, 1.0), 0.0)
                            o = (w @ V) * rden
                            dw = (DO[r0:r1] @ V.T - (DO[r0:r1] * o).sum(axis=1, keepdims=True)) * rden
                            W = w * rden
                        else:
                            dw = DO[r0:r1] @ V.T
                            W = w
                        dx = dw * L * 2.0 * x
                    else:   # first order
                        w = L * x
                        dw = DO[r0:r1] @ V.T
                        W = w
                        dx = dw * L
                    M = dw * w
                dv[b, h] += W.T @ DO[r0:r1]
                dq[b, h, r0:r1] += scale * (dx @ K)
                dk[b, h] += scale * (dx.T @ Q[r0:r1])
                strict = s_ < t
                Ms = np.where(strict, M, 0.0)
                rows[r0:r1] += Ms.sum(axis=1)
                cols += Ms.sum(axis=0)
            # dg_r = sum over r' < r of (cols - rows)
            dg[b, h] = np.concatenate([[0.0], np.cumsum(cols - rows)[:-1]])
    return dq, dk, dv, -sigmoid(z) * dg


# ----------------------------------------------------------------------------
# per-row statistics a training forward hands to its backward: the 2Mamba
# weight sum (the normaliser of [2M2F §5]) and the 2Mamba-E log-sum-exp
# ----------------------------------------------------------------------------

def row_weight_sums(q, k, z, scale=1.0, state_in_norm=None, rows=None):
    """den_t = sum_{s<=t} L_ts (scale q_t.k_s)^2, plus exp(g_0+...+g_t)
    phi_q(scale q_t).n0 for an initial normaliser n0 -> [B, H, T] (or
    [B, H, len(rows)] for the listed rows t only)."""
    g = decay_log(z)
    rows = range(q.shape[2]) if rows is None else rows
    den = np.zeros(q.shape[:2] + (len(rows),))
    for i, t in enumerate(rows):
        L = np.exp(_row_log_mask(g[:, :, :t + 1]))
        a = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], k[:, :, :t + 1])
        den[:, :, i] = (L * a * a).sum(axis=-1)
        if state_in_norm is not None:
            den[:, :, i] += np.exp(g[:, :, :t + 1].sum(axis=-1)) * np.einsum(
                "bhp,bhp->bh", phi_q(scale * q[:, :, t]), state_in_norm)
    return den


def row_logsumexp(q, k, z, scale=1.0, rows=None):
    """lse_t = log sum_{s<=t} exp(scale q_t.k_s + lambda_ts) (natural log) -> [B, H, T]
    (or [B, H, len(rows)] for the listed rows t only)."""
    g = decay_log(z)
    rows = range(q.shape[2]) if rows is None else rows
    lse = np.zeros(q.shape[:2] + (len(rows),))
    for i, t in enumerate(rows):
        logit = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], k[:, :, :t + 1]) + _row_log_mask(g[:, :, :t + 1])
        m = logit.max(axis=-1)
        lse[:, :, i] = m + np.log(np.exp(logit - m[..., None]).sum(axis=-1))
    return lse
