"""Pins of the oracle's first-order (Mamba-2S) forms (CPU only).

  * no decay: the output is a causal-masked product tril(Q K^T) V, computed
    with numpy matmuls;
  * the quadratic form equals the token-by-token recurrence, with and
    without an initial state, and split/resume through the state;
  * d = 1 is the second-order form's special case: (q k)^2 = q^2 k^2, so the
    unnormalised 2Mamba output on (q, k) equals the first-order one on
    (q^2, k^2) with the scale squared;
  * gradients match central finite differences of the forward;
plus planted mistakes that must trip one of these.
"""

import numpy as np
import pytest

from oracle import twomamba_oracle as O


def _in(seed, B=2, H=2, T=9, d=3, dv=2, zm=-1.0):
    r = np.random.default_rng(seed)
    return (r.normal(size=(B, H, T, d)), r.normal(size=(B, H, T, d)), r.normal(size=(B, H, T, dv)),
            r.normal(zm, 1.0, size=(B, H, T)))


def test_no_decay_is_masked_matmul():
    q, k, v, _ = _in(0)
    z = np.full(q.shape[:3], -np.inf)
    T = q.shape[2]
    ref = np.matmul(np.tril(np.matmul(q, np.swapaxes(k, -1, -2))) * 0.7, v)
    np.testing.assert_allclose(O.fwd_linear_quadratic(q, k, v, z, scale=0.7), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("with_state", [False, True])
def test_quadratic_equals_recurrence(with_state):
    q, k, v, z = _in(1, zm=0.5)
    S0 = np.random.default_rng(2).normal(size=(2, 2, 3, 2)) if with_state else None
    a = O.fwd_linear_quadratic(q, k, v, z, scale=1.3, state_in=S0)
    b, _ = O.fwd_linear_recurrent(q, k, v, z, scale=1.3, state_in=S0)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_split_resume_through_the_state():
    q, k, v, z = _in(3, T=12)
    whole, Sw = O.fwd_linear_recurrent(q, k, v, z)
    o1, S1 = O.fwd_linear_recurrent(q[:, :, :5], k[:, :, :5], v[:, :, :5], z[:, :, :5])
    o2 = O.fwd_linear_quadratic(q[:, :, 5:], k[:, :, 5:], v[:, :, 5:], z[:, :, 5:], state_in=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), whole, rtol=1e-11, atol=1e-12)


def test_d1_relation_to_the_second_order_form():
    q, k, v, z = _in(4, d=1, dv=3)
    lin = O.fwd_linear_quadratic(q * q, k * k, v, z, scale=0.8 ** 2)
    sq = O.fwd_quadratic(q, k, v, z, scale=0.8, norm=False)
    np.testing.assert_allclose(lin, sq, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,zm", [(5, 0.0), (6, -4.0)])
def test_linear_gradients_match_finite_differences(seed, zm):
    q, k, v, z = _in(seed, zm=zm)
    do = np.random.default_rng(seed + 100).normal(size=v.shape)
    grads = O.bwd_linear_quadratic(q, k, v, z, do, scale=0.9)
    X = [q, k, v, z]
    r = np.random.default_rng(seed + 200)
    for i in range(4):
        U = r.normal(size=X[i].shape)
        Xp, Xm = list(X), list(X)
        Xp[i] = X[i] + 1e-5 * U
        Xm[i] = X[i] - 1e-5 * U
        fd = ((O.fwd_linear_quadratic(*Xp, scale=0.9) - O.fwd_linear_quadratic(*Xm, scale=0.9)) * do).sum() / 2e-5
        an = (grads[i] * U).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (i, fd, an)


# ---------------------------------------------------------------- planted mistakes
_orig_step = O.step_linear
_orig_fwd = O.fwd_linear_quadratic
_orig_bwd = O.bwd_linear_quadratic


def _step_decay_after_add(q, k, v, z, state, scale=1.0):
    a = np.exp(O.decay_log(z))
    S = a[..., None, None] * (state + k[..., :, None] * v[..., None, :])
    return scale * np.einsum("bhd,bhdc->bhc", q, S), S


def _fwd_transposed_scores(q, k, v, z, scale=1.0, state_in=None):
    return _orig_fwd(k, q, v, z, scale, state_in)


def _bwd_no_mask_grad(q, k, v, z, dout, scale=1.0):
    dq, dk, dv, dz = _orig_bwd(q, k, v, z, dout, scale)
    return dq, dk, dv, np.zeros_like(dz)


@pytest.mark.parametrize("attr,patch,pins", [
    ("step_linear", _step_decay_after_add, [lambda: test_quadratic_equals_recurrence(False)]),
    ("fwd_linear_quadratic", _fwd_transposed_scores, [test_no_decay_is_masked_matmul,
                                                      lambda: test_quadratic_equals_recurrence(False)]),
    ("bwd_linear_quadratic", _bwd_no_mask_grad, [lambda: test_linear_gradients_match_finite_differences(5, 0.0)]),
], ids=["decay applied after the add", "scores transposed", "mask gradient dropped"])
def test_planted_linear_mistake_is_caught(monkeypatch, attr, patch, pins):
    monkeypatch.setattr(O, attr, patch)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
