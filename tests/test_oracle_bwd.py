"""Pins of the oracle's gradients (CPU only).

The gradient functions are checked against things other than themselves:
  * central finite differences of the oracle's forward forms, along random
    directions, for every input (q, k, v, z), both variants, with and without
    normalisation, strong and weak decay;
  * torch's autograd through its own causal scaled-dot-product attention
    (fp64, CPU) for 2Mamba-E with no decay (z = -inf), a library routine;
  * invariances that fix parts of the result exactly: the normalised 2Mamba
    output does not change when one q_t, or every k, is rescaled, so
    q_t.dq_t = 0 and sum_s k_s.dk_s = 0; both normalised outputs move by c
    when every v_s moves by c, so sum_s dv_s = sum_t dout_t; a common shift
    of every key adds a per-row constant to the 2Mamba-E logits, so
    sum_s dk_s = 0 there; z = -inf gives dz = 0.
Planted mistakes in the gradient code must fail at least one of these pins.
"""

import numpy as np
import pytest
import torch

from oracle import twomamba_oracle as O


def _inputs(seed, B=1, H=2, T=7, d=3, dv=2, z_mean=0.0):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, H, T, d))
    k = r.normal(size=(B, H, T, d))
    v = r.normal(size=(B, H, T, dv))
    z = r.normal(z_mean, 1.0, size=(B, H, T))
    do = r.normal(size=(B, H, T, dv))
    return q, k, v, z, do


def _fd_check(fwd, bwd, X, do, kw, seed, rtol=1e-6):
    """<grad_i, U> against (F(x + hU) - F(x - hU)) / 2h, F = sum dout . fwd."""
    r = np.random.default_rng(seed + 1000)
    grads = bwd(*X, do, **kw)
    for i in range(4):
        U = r.normal(size=X[i].shape)
        h = 1e-5
        Xp = list(X)
        Xm = list(X)
        Xp[i] = X[i] + h * U
        Xm[i] = X[i] - h * U
        fd = ((fwd(*Xp, **kw) - fwd(*Xm, **kw)) * do).sum() / (2 * h)
        an = (grads[i] * U).sum()
        assert abs(fd - an) <= rtol * max(1.0, abs(fd)), (i, fd, an)


FD_CASES = [(0, 0.0, 1.0), (1, -4.0, 0.7), (2, 2.0, 1.3)]


@pytest.mark.parametrize("seed,zm,scale", FD_CASES)
@pytest.mark.parametrize("norm", [True, False])
def test_sq_gradients_match_finite_differences(seed, zm, scale, norm):
    q, k, v, z, do = _inputs(seed, z_mean=zm)
    _fd_check(O.fwd_quadratic, O.bwd_quadratic, (q, k, v, z), do, dict(scale=scale, norm=norm), seed)


@pytest.mark.parametrize("seed,zm,scale", FD_CASES)
def test_exp_gradients_match_finite_differences(seed, zm, scale):
    q, k, v, z, do = _inputs(seed, z_mean=zm)
    _fd_check(O.fwd_exp_quadratic, O.bwd_exp_quadratic, (q, k, v, z), do, dict(scale=scale), seed)


def test_gradients_d16_longer_sequence():
    # wider heads and a longer row than the finite-difference cases above
    q, k, v, z, do = _inputs(5, B=1, H=1, T=40, d=16, dv=16, z_mean=-3.0)
    q, k = q / 4.0, k / 4.0
    _fd_check(O.fwd_quadratic, O.bwd_quadratic, (q, k, v, z), do, dict(scale=1.0), 5)
    _fd_check(O.fwd_exp_quadratic, O.bwd_exp_quadratic, (q, k, v, z), do, dict(scale=1.0), 5)


def test_exp_no_decay_gradients_match_torch_sdpa():
    q, k, v, _, do = _inputs(3, B=2, H=2, T=23, d=8, dv=5)
    z = np.full(q.shape[:3], -np.inf)
    dq, dk, dv, dz = O.bwd_exp_quadratic(q, k, v, z, do, scale=0.6)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.6)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(dz == 0.0)


def test_sq_no_decay_dz_is_zero():
    q, k, v, _, do = _inputs(4)
    z = np.full(q.shape[:3], -np.inf)
    assert np.all(O.bwd_quadratic(q, k, v, z, do)[3] == 0.0)


@pytest.mark.parametrize("zm", [0.0, -5.0])
def test_sq_scale_invariances(zm):
    q, k, v, z, do = _inputs(6, B=2, H=2, T=12, d=4, dv=3, z_mean=zm)
    dq, dk, dv, _ = O.bwd_quadratic(q, k, v, z, do, scale=0.9)
    # o_t depends on q_t only through its direction: q_t . dq_t = 0 per token
    assert np.max(np.abs((q * dq).sum(-1))) < 1e-10 * max(1.0, np.abs(dq).max())
    # a common scale of every k cancels: sum_s k_s . dk_s = 0 per head
    assert np.max(np.abs((k * dk).sum(axis=(-1, -2)))) < 1e-10 * max(1.0, np.abs(dk).max())
    # shifting every v by c shifts every o by c
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-10, atol=1e-10)


def test_exp_value_shift_and_logit_sum():
    q, k, v, z, do = _inputs(7, B=2, H=2, T=12, d=4, dv=3, z_mean=-1.0)
    dq, dk, dv, dz = O.bwd_exp_quadratic(q, k, v, z, do, scale=0.9)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-10, atol=1e-10)
    # a common shift u of every key adds scale q_t.u to every logit of row t,
    # a per-row constant the softmax removes
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-10 * max(1.0, np.abs(dk).max())


def test_no_norm_sq_is_linear_in_v():
    # without normalisation the output is linear in v: dv_s = sum_t w_ts dout_t
    q, k, v, z, do = _inputs(9, z_mean=-2.0)
    dv1 = O.bwd_quadratic(q, k, v, z, do, norm=False)[2]
    dv2 = O.bwd_quadratic(q, k, 3.0 * v - 1.0, z, do, norm=False)[2]
    np.testing.assert_allclose(dv1, dv2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

_orig_sq = O.bwd_quadratic
_orig_exp = O.bwd_exp_quadratic
_orig_add = O._add_mask_grad


def _mask_grad_includes_own_start(dg, dlam, t):
    # s <= r in place of s < r
    dg[..., :t + 1] += np.cumsum(dlam[..., :t + 1], axis=-1)


def _mask_grad_wrong_sign(dg, dlam, t):
    _orig_add(dg, -dlam, t)


def _sq_drop_dden(q, k, v, z, dout, scale=1.0, norm=True):
    # normalisation derivative dropped: as if den were a constant
    g = O.decay_log(z)
    T = q.shape[2]
    dq, dk, dv, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(z.shape)
    for t in range(T):
        K, V = k[:, :, :t + 1], v[:, :, :t + 1]
        L = np.exp(O._row_log_mask(g[:, :, :t + 1]))
        a = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], K)
        w = L * a * a
        den = w.sum(axis=-1)
        dnum = dout[:, :, t] / den[..., None]
        dw = np.einsum("bhsc,bhc->bhs", V, dnum)
        dv[:, :, :t + 1] += w[..., None] * dnum[:, :, None, :]
        da = dw * L * 2.0 * a
        dq[:, :, t] += scale * np.einsum("bhs,bhsd->bhd", da, K)
        dk[:, :, :t + 1] += scale * da[..., None] * q[:, :, t][:, :, None, :]
        O._add_mask_grad(dg, dw * w, t)
    return dq, dk, dv, -O.sigmoid(z) * dg


def _sq_no_factor_two(q, k, v, z, dout, scale=1.0, norm=True):
    dq, dk, dv, dz = _orig_sq(q, k, v, z, dout, scale, norm)
    return 0.5 * dq, 0.5 * dk, dv, dz


def _exp_swapped_qk_grads(q, k, v, z, dout, scale=1.0):
    dq, dk, dv, dz = _orig_exp(q, k, v, z, dout, scale)
    return dk, dq, dv, dz


def _dz_sigmoid_sign(q, k, v, z, dout, scale=1.0, norm=True):
    dq, dk, dv, dz = _orig_sq(q, k, v, z, dout, scale, norm)
    return dq, dk, dv, dz * O.sigmoid(-z) / np.maximum(O.sigmoid(z), 1e-300)


def _sq_fd():
    test_sq_gradients_match_finite_differences(0, 0.0, 1.0, True)


def _exp_fd():
    test_exp_gradients_match_finite_differences(1, -4.0, 0.7)


BWD_MUTATIONS = [
    ("mask gradient range s <= r", "_add_mask_grad", _mask_grad_includes_own_start, [_sq_fd, _exp_fd]),
    ("mask gradient sign", "_add_mask_grad", _mask_grad_wrong_sign, [_sq_fd, _exp_fd]),
    ("normalisation term dropped", "bwd_quadratic", _sq_drop_dden, [_sq_fd, lambda: test_sq_scale_invariances(0.0)]),
    ("factor 2 of the square dropped", "bwd_quadratic", _sq_no_factor_two, [_sq_fd]),
    ("q and k gradients swapped", "bwd_exp_quadratic", _exp_swapped_qk_grads, [_exp_fd,
                                                                              test_exp_no_decay_gradients_match_torch_sdpa]),
    ("sigmoid argument sign in dz", "bwd_quadratic", _dz_sigmoid_sign, [_sq_fd]),
]


@pytest.mark.parametrize("name,attr,patch,pins", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_planted_gradient_mistake_is_caught(monkeypatch, name, attr, patch, pins):
    monkeypatch.setattr(O, attr, patch)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


@pytest.mark.parametrize("variant,norm", [("sq", True), ("sq", False), ("exp", True), ("lin", True)])
def test_blocked_gradients_equal_the_row_loop(variant, norm):
    # the whole-matrix form used for long sequences, against the row loop,
    # with blocks that split the rows unevenly
    q, k, v, z, do = _inputs(11, B=2, H=2, T=37, d=5, dv=4, z_mean=-1.5)
    if variant == "sq":
        ref = O.bwd_quadratic(q, k, v, z, do, scale=0.8, norm=norm)
    elif variant == "exp":
        ref = O.bwd_exp_quadratic(q, k, v, z, do, scale=0.8)
    else:
        ref = O.bwd_linear_quadratic(q, k, v, z, do, scale=0.8)
    got = O.bwd_blocked(q, k, v, z, do, variant=variant, scale=0.8, norm=norm, block=10)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
