"""Planted mistakes in the oracle must trip at least one pin (CPU only).

Each case patches one oracle function with a plausible slip (a dropped term, a
wrong sign, an off-by-one range, a transposed operand) and checks that a pin
from test_oracle_pins fails on it.  The patches live only inside the test.
"""

import numpy as np
import pytest

from oracle import twomamba_oracle as O
import test_oracle_pins as P


def _plus_softplus(z):
    return O.softplus(z)


def _mask_includes_own_token(g_row):
    t = g_row.shape[-1] - 1
    lam = np.zeros(g_row.shape)
    lam[..., :t + 1] = np.cumsum(g_row[..., ::-1], axis=-1)[..., ::-1]   # sums g_s..g_t
    return lam


def _mask_squared(g_row):
    return 2.0 * _orig_mask(g_row)


def _mask_drops_diagonal(g_row):
    lam = _orig_mask(g_row)
    lam[..., -1] = -np.inf
    return lam


def _phi_q_no_two(q):
    I, J = O.pair_list(q.shape[-1])
    return q[..., I] * q[..., J]


def _fwd_quadratic_qk_swapped(q, k, v, z, scale=1.0, norm=True, state_in=None, norm_in=None):
    # the score matrix transposed: (k_t . q_s)^2 in place of (q_t . k_s)^2
    return _orig_fwd(k, q, v, z, scale, norm, state_in, norm_in)


_orig_mask = O._row_log_mask
_orig_fwd = O.fwd_quadratic


def _exp_row_bias_sign(q_t, K, V, g_upto_t, scale):
    return _orig_exp_row(q_t, K, V, -g_upto_t, scale)


_orig_exp_row = O._exp_row


MUTATIONS = [
    ("decay sign", "decay_log", _plus_softplus, [P.test_softplus_is_negative_log_sigmoid,
                                                 lambda: P.test_d1_constant_decay_geometric_sum(0.0)]),
    ("mask range s..t", "_row_log_mask", _mask_includes_own_token, [P.test_d1_impulse_decays_by_following_tokens_only]),
    ("mask squared", "_row_log_mask", _mask_squared, [P.test_d1_impulse_decays_by_following_tokens_only]),
    ("diagonal dropped", "_row_log_mask", _mask_drops_diagonal, [P.test_quadratic_bruteforce_loops_tiny]),
    ("no factor 2", "phi_q", _phi_q_no_two, [lambda: P.test_feature_identity_bruteforce(3)]),
    ("score transposed", "fwd_quadratic", _fwd_quadratic_qk_swapped, [P.test_no_decay_unnormalised_is_masked_squared_matmul]),
    ("E bias sign", "_exp_row", _exp_row_bias_sign, [P.test_exp_zero_scores_closed_form]),
]


@pytest.mark.parametrize("name,attr,fn,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn, pins):
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught == len(pins), f"mutation '{name}' slipped past a pin"


def test_initial_state_without_decay_is_caught(monkeypatch):
    # Dropping the e^{g_0+...+g_t} factor on the carried state breaks split/resume.
    orig = O.fwd_quadratic

    def patched(q, k, v, z, scale=1.0, norm=True, state_in=None, norm_in=None):
        if state_in is None:
            return orig(q, k, v, z, scale, norm)
        g = O.decay_log(z)
        out = np.zeros(v.shape)
        num0, den0 = O._init_terms(q, scale, state_in, norm_in)
        for t in range(q.shape[2]):
            num, den = O._sq_row(q[:, :, t], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1], scale,
                                 init_num=num0[:, :, t], init_den=den0[:, :, t],
                                 init_decay=np.ones(q.shape[:2]))
            out[:, :, t] = O._normalise(num, den, norm)
        return out

    monkeypatch.setattr(O, "fwd_quadratic", patched)
    with pytest.raises(AssertionError):
        P.test_split_and_resume(6)


_orig_lse = O.row_logsumexp


def _lse_without_decay(q, k, z, scale=1.0, rows=None):
    return _orig_lse(q, k, np.full(z.shape, -np.inf), scale, rows)


def _lse_decay_sign_flipped(q, k, z, scale=1.0, rows=None):
    # lambda_ts entering with the wrong sign, e^{-lambda}: the mask of logits -z'
    # with softplus(z') = -softplus(z) is not available, so build it from the rows
    g = O.decay_log(z)
    rows_ = range(q.shape[2]) if rows is None else rows
    out = np.zeros(q.shape[:2] + (len(rows_),))
    for i, t in enumerate(rows_):
        logit = scale * np.einsum("bhd,bhsd->bhs", q[:, :, t], k[:, :, :t + 1]) - O._row_log_mask(g[:, :, :t + 1])
        out[:, :, i] = np.log(np.exp(logit).sum(axis=-1))
    return out


@pytest.mark.parametrize("fn", [_lse_without_decay, _lse_decay_sign_flipped], ids=["lse decay dropped",
                                                                                   "lse decay sign"])
def test_planted_mistake_in_row_logsumexp_is_caught(monkeypatch, fn):
    monkeypatch.setattr(O, "row_logsumexp", fn)
    for pin in (P.test_row_logsumexp_zero_scores_geometric_closed_form,
                P.test_row_logsumexp_zero_scores_follow_the_one_token_recursion,
                P.test_row_logsumexp_decay_gradient_is_softmax_mass_before_the_token):
        with pytest.raises(AssertionError):
            pin()
