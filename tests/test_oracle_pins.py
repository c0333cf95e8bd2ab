"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties an oracle function to something it cannot agree with by
construction: a closed form, a library routine, brute-force sums on tiny
inputs, an independent evaluation order, an invariant of the mathematics, or a
number the pages print.  Source of the method: "2Mamba2Furious: Linear in
Complexity, Competitive in Accuracy" (paperlayer summary), cited [2M2F §n].
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import twomamba_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.Generator(np.random.PCG64(1000 + seed))


def rand_inputs(seed, B=1, H=2, T=7, d=3, dv=2, z_mean=0.0):
    r = rng(seed)
    q = r.standard_normal((B, H, T, d)) / math.sqrt(d)
    k = r.standard_normal((B, H, T, d)) / math.sqrt(d)
    v = r.standard_normal((B, H, T, dv))
    z = r.standard_normal((B, H, T)) + z_mean
    return q, k, v, z


def relerr(a, b):
    """max over (b,h) of ||a-b||_inf / ||b||_inf (per-head inf norm)."""
    a = np.asarray(a); b = np.asarray(b)
    B, H = b.shape[:2]
    num = np.abs(a - b).reshape(B, H, -1).max(-1)
    den = np.abs(b).reshape(B, H, -1).max(-1)
    return float((num / np.where(den == 0, 1, den)).max())


# --------------------------------------------------------------------------- decay

def test_softplus_is_negative_log_sigmoid():
    # [2M2F §6]: the softplus mask matches the forgetting transformer's log-sigmoid
    # up to the sign of the argument: -softplus(z) = log sigmoid(-z).
    z = np.concatenate([np.linspace(-60, 60, 2001), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    ref = scipy.special.log_expit(-z)
    got = O.decay_log(z)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    assert O.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert O.decay_log(-np.inf) == 0.0                      # no decay at all
    assert np.all(O.decay_log(z) <= 0.0)                    # L_ts in (0, 1]


def test_softplus_matches_torch_below_threshold():
    z = np.linspace(-30, 19.9, 997)
    ref = torch.nn.functional.softplus(torch.from_numpy(z)).numpy()
    assert np.allclose(O.softplus(z), ref, rtol=1e-13, atol=0)


# --------------------------------------------------------------------------- features

@pytest.mark.parametrize("d", [1, 2, 3, 5, 16, 64])
def test_pair_layout_row_major_upper_triangle(d):
    D = O.num_pairs(d)
    assert D == d * (d + 1) // 2
    # enumerate the upper triangle row by row; positions must be 0,1,2,...
    expect = 0
    for i in range(d):
        for j in range(i, d):
            assert O.pair_index(i, j, d) == expect
            expect += 1
    assert expect == D
    I, J = O.pair_list(d)
    assert np.all(I <= J) and len(set(zip(I.tolist(), J.tolist()))) == D
    assert O.pair_index(d - 1, d - 1, d) == D - 1
    if d > 1:
        assert O.pair_index(1, 1, d) == d


@pytest.mark.parametrize("d", [1, 2, 3, 16])
def test_feature_identity_bruteforce(d):
    r = rng(d)
    for _ in range(5):
        q = r.standard_normal(d)
        k = r.standard_normal(d)
        dot = sum(q[i] * k[i] for i in range(d))
        explicit = sum(q[i] * q[j] * k[i] * k[j] for i in range(d) for j in range(d))   # vec(qq^T).vec(kk^T)
        got = float(O.phi_q(q) @ O.phi_k(k))
        assert got == pytest.approx(dot * dot, rel=1e-12, abs=1e-14)
        assert got == pytest.approx(explicit, rel=1e-12, abs=1e-14)


def test_features_are_symmetric_halves():
    # phi_k holds each unordered product once and unscaled; phi_q carries the 2.
    q = np.array([1.0, 2.0, 3.0])
    assert O.phi_k(q).tolist() == [1, 2, 3, 4, 6, 9]
    assert O.phi_q(q).tolist() == [1, 4, 6, 4, 12, 9]


# --------------------------------------------------------------------------- 2Mamba closed forms

@pytest.mark.parametrize("zval", [-3.0, 0.0, 1.5])
def test_d1_constant_decay_geometric_sum(zval):
    # d = 1, q = k = 1, v = 1, constant decay a = e^g: the unnormalised output is
    # the geometric sum of a^0..a^t (the diagonal weight is 1; the exponent of the
    # term s is the number of tokens after s up to t).
    T = 12
    one = np.ones((1, 1, T, 1))
    z = np.full((1, 1, T), zval)
    a = math.exp(-math.log1p(math.exp(zval)))
    num = O.fwd_quadratic(one, one, one, z, norm=False)[0, 0, :, 0]
    for t in range(T):
        assert num[t] == pytest.approx((1 - a ** (t + 1)) / (1 - a), rel=1e-13)
    normed = O.fwd_quadratic(one, one, one, z, norm=True)
    assert np.allclose(normed, 1.0, rtol=1e-14)


def test_d1_impulse_decays_by_following_tokens_only():
    # One value impulse at s0: the output at t >= s0 is exp(g_{s0+1}+...+g_t) and
    # 0 before s0 (causality).  Pins the summation range s+1..t and the sign of g.
    T, s0 = 10, 3
    r = rng(7)
    z = r.standard_normal((1, 1, T))
    g = [-math.log1p(math.exp(x)) for x in z[0, 0]]
    one = np.ones((1, 1, T, 1))
    v = np.zeros((1, 1, T, 1)); v[0, 0, s0, 0] = 1.0
    num = O.fwd_quadratic(one, one, v, z, norm=False)[0, 0, :, 0]
    for t in range(T):
        expect = 0.0 if t < s0 else math.exp(sum(g[s0 + 1:t + 1]))
        assert num[t] == pytest.approx(expect, rel=1e-13, abs=1e-300)


def test_quadratic_bruteforce_loops_tiny():
    # Pure-Python term-by-term evaluation of the definition on a tiny case.
    q, k, v, z = rand_inputs(11, B=1, H=1, T=5, d=2, dv=2)
    scale = 0.8
    got = O.fwd_quadratic(q, k, v, z, scale=scale)
    got_nn = O.fwd_quadratic(q, k, v, z, scale=scale, norm=False)
    g = [-(max(x, 0) + math.log1p(math.exp(-abs(x)))) for x in z[0, 0]]
    for t in range(5):
        num = [0.0, 0.0]; den = 0.0
        for s in range(t + 1):
            lam = 0.0
            for r_ in range(s + 1, t + 1):
                lam += g[r_]
            sc = scale * (q[0, 0, t, 0] * k[0, 0, s, 0] + q[0, 0, t, 1] * k[0, 0, s, 1])
            w = math.exp(lam) * sc * sc
            den += w
            for c in range(2):
                num[c] += w * v[0, 0, s, c]
        for c in range(2):
            assert got[0, 0, t, c] == pytest.approx(num[c] / den, rel=1e-12)
            assert got_nn[0, 0, t, c] == pytest.approx(num[c], rel=1e-12, abs=1e-15)


def test_no_decay_unnormalised_is_masked_squared_matmul():
    # z = -inf gives L = 1 on and below the diagonal: squared linear attention.
    q, k, v, z = rand_inputs(3, T=9, d=4, dv=3)
    z[...] = -np.inf
    scores = np.matmul(q, np.swapaxes(k, -1, -2)) ** 2 * np.tril(np.ones((9, 9)))
    ref = np.matmul(scores, v)
    assert relerr(O.fwd_quadratic(q, k, v, z, norm=False), ref) < 1e-13


def test_single_token_returns_value():
    q, k, v, z = rand_inputs(4, T=1, d=5, dv=4)
    assert relerr(O.fwd_quadratic(q, k, v, z), v) < 1e-14
    assert relerr(O.fwd_exp_quadratic(q, k, v, z), v) < 1e-14


def test_strong_decay_returns_own_value():
    q, k, v, z = rand_inputs(5, T=20, d=4, dv=3)
    z[...] = 60.0                        # every earlier token weighted by < e^-60
    assert relerr(O.fwd_quadratic(q, k, v, z), v) < 1e-12
    assert relerr(O.fwd_exp_quadratic(q, k, v, z), v) < 1e-12


# --------------------------------------------------------------------------- independent forms agree

Z_REGIMES = [0.0, -6.0, 3.0, "ninf"]


@pytest.mark.parametrize("zreg", Z_REGIMES)
@pytest.mark.parametrize("norm", [True, False])
def test_quadratic_equals_recurrences(zreg, norm):
    q, k, v, z = rand_inputs(21, B=2, H=2, T=17, d=3, dv=2, z_mean=0.0 if zreg == "ninf" else zreg)
    if zreg == "ninf":
        z[...] = -np.inf
    for scale in (1.0, 0.6):
        a = O.fwd_quadratic(q, k, v, z, scale=scale, norm=norm)
        b = O.fwd_recurrent_full(q, k, v, z, scale=scale, norm=norm)
        c, S, n = O.fwd_recurrent_packed(q, k, v, z, scale=scale, norm=norm)
        assert relerr(b, a) < 1e-10
        assert relerr(c, a) < 1e-10
        S2, n2 = O.final_state_direct(k, v, z)
        assert relerr(S, S2) < 1e-10 and relerr(n, n2) < 1e-10


@pytest.mark.parametrize("zreg", Z_REGIMES)
def test_exp_forms_agree(zreg):
    q, k, v, z = rand_inputs(31, B=1, H=2, T=15, d=4, dv=3, z_mean=0.0 if zreg == "ninf" else zreg)
    if zreg == "ninf":
        z[...] = -np.inf
    for scale in (1.0, 2.5):
        a = O.fwd_exp_quadratic(q, k, v, z, scale=scale)
        b = O.fwd_exp_streaming(q, k, v, z, scale=scale)
        assert relerr(b, a) < 1e-10


def test_exp_no_decay_is_causal_softmax_attention():
    # [2M2F §6]: with the A-mask switched off (z=-inf) 2Mamba-E is softmax attention.
    q, k, v, z = rand_inputs(41, B=2, H=3, T=13, d=8, dv=5)
    z[...] = -np.inf
    scale = 0.9
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=scale).numpy()
    assert relerr(O.fwd_exp_quadratic(q, k, v, z, scale=scale), ref) < 1e-12
    assert relerr(O.fwd_exp_streaming(q, k, v, z, scale=scale), ref) < 1e-12


def test_exp_zero_scores_closed_form():
    # q = k = 0: the softmax weights are exp(lambda_ts) alone.  With a constant decay
    # a and a value that is 1 only at s = t, o_t = 1 / (1 + a + ... + a^t).
    T = 9
    zero = np.zeros((1, 1, T, 2))
    v = np.zeros((1, 1, T, T)); v[0, 0, np.arange(T), np.arange(T)] = 1.0
    z = np.full((1, 1, T), -0.5)
    a = math.exp(-math.log1p(math.exp(-0.5)))
    o = O.fwd_exp_quadratic(zero, zero, v, z)
    for t in range(T):
        assert o[0, 0, t, t] == pytest.approx((1 - a) / (1 - a ** (t + 1)), rel=1e-13)
        # the weight on the oldest token is a^t times the weight on the newest
        if t > 0:
            assert o[0, 0, t, 0] == pytest.approx(o[0, 0, t, t] * a ** t, rel=1e-12)


# --------------------------------------------------------------------------- invariants

def test_normalised_output_is_scale_invariant_and_convex():
    q, k, v, z = rand_inputs(51, B=2, H=2, T=16, d=4, dv=3, z_mean=-2.0)
    o1 = O.fwd_quadratic(q, k, v, z, scale=1.0)
    o2 = O.fwd_quadratic(q, k, v, z, scale=3.7)
    assert relerr(o2, o1) < 1e-12
    for t in range(16):
        lo = v[:, :, :t + 1].min(axis=2)
        hi = v[:, :, :t + 1].max(axis=2)
        assert np.all(o1[:, :, t] >= lo - 1e-12) and np.all(o1[:, :, t] <= hi + 1e-12)


def test_homogeneity_and_linearity():
    q, k, v, z = rand_inputs(61, B=1, H=2, T=11, d=4, dv=3, z_mean=-1.0)
    base = O.fwd_quadratic(q, k, v, z, norm=False)
    assert relerr(O.fwd_quadratic(1.7 * q, k, v, z, norm=False), 1.7 ** 2 * base) < 1e-12
    assert relerr(O.fwd_quadratic(q, -0.4 * k, v, z, norm=False), 0.16 * base) < 1e-12
    v2 = rng(62).standard_normal(v.shape)
    lin = O.fwd_quadratic(q, k, 2 * v - 3 * v2, z, norm=False)
    assert relerr(lin, 2 * base - 3 * O.fwd_quadratic(q, k, v2, z, norm=False)) < 1e-12
    normed = O.fwd_quadratic(q, k, v, z)
    assert relerr(O.fwd_quadratic(5 * q, 0.3 * k, v, z), normed) < 1e-12


def test_head_permutation_equivariance():
    q, k, v, z = rand_inputs(71, B=2, H=3, T=8, d=3, dv=2)
    perm = [2, 0, 1]
    o = O.fwd_quadratic(q, k, v, z)
    op = O.fwd_quadratic(q[:, perm], k[:, perm], v[:, perm], z[:, perm])
    assert relerr(op, o[:, perm]) < 1e-15
    e = O.fwd_exp_quadratic(q, k, v, z)
    ep = O.fwd_exp_quadratic(q[:, perm], k[:, perm], v[:, perm], z[:, perm])
    assert relerr(ep, e[:, perm]) < 1e-15


@pytest.mark.parametrize("split", [1, 6, 13])
def test_split_and_resume(split):
    # Running the first part, carrying its final state, then the rest equals one run.
    q, k, v, z = rand_inputs(81, B=1, H=2, T=19, d=3, dv=2, z_mean=-3.0)
    full = O.fwd_quadratic(q, k, v, z)
    S, n = O.final_state_direct(k[:, :, :split], v[:, :, :split], z[:, :, :split])
    a = O.fwd_quadratic(q[:, :, :split], k[:, :, :split], v[:, :, :split], z[:, :, :split])
    b = O.fwd_quadratic(q[:, :, split:], k[:, :, split:], v[:, :, split:], z[:, :, split:],
                        state_in=S, norm_in=n)
    assert relerr(np.concatenate([a, b], axis=2), full) < 1e-10
    # the recurrence resumes the same way, and its final state matches the direct sum
    c, S2, n2 = O.fwd_recurrent_packed(q[:, :, split:], k[:, :, split:], v[:, :, split:], z[:, :, split:],
                                       state_in=S, norm_in=n)
    assert relerr(c, b) < 1e-10
    Sf, nf = O.final_state_direct(k, v, z)
    assert relerr(S2, Sf) < 1e-10 and relerr(n2, nf) < 1e-10
    Sd, nd = O.final_state_direct(k[:, :, split:], v[:, :, split:], z[:, :, split:], state_in=S, norm_in=n)
    assert relerr(Sd, Sf) < 1e-10 and relerr(nd, nf) < 1e-10


def test_decode_steps_continue_the_forward():
    q, k, v, z = rand_inputs(91, B=2, H=2, T=14, d=4, dv=3, z_mean=-2.0)
    T0 = 9
    full = O.fwd_quadratic(q, k, v, z)
    S, n = O.final_state_direct(k[:, :, :T0], v[:, :, :T0], z[:, :, :T0])
    for t in range(T0, 14):
        o, S, n = O.step(q[:, :, t], k[:, :, t], v[:, :, t], z[:, :, t], S, n)
        assert relerr(o[:, :, None], full[:, :, t:t + 1]) < 1e-10


def test_rows_form_matches_full_form():
    q, k, v, z = rand_inputs(95, B=1, H=2, T=12, d=3, dv=2)
    S, n = O.final_state_direct(k[:, :, :4], v[:, :, :4], z[:, :, :4])
    rows = [0, 5, 11]
    full = O.fwd_quadratic(q, k, v, z, state_in=S, norm_in=n)
    assert relerr(O.fwd_quadratic_rows(q, k, v, z, rows, state_in=S, norm_in=n), full[:, :, rows]) < 1e-13
    e = O.fwd_exp_quadratic(q, k, v, z)
    assert relerr(O.fwd_exp_quadratic_rows(q, k, v, z, rows), e[:, :, rows]) < 1e-13


def test_zero_denominator_gives_zero():
    # q_t orthogonal to every key: all weights vanish and the output is 0 by convention.
    T = 4
    q = np.zeros((1, 1, T, 2)); q[..., 0] = 1.0
    k = np.zeros((1, 1, T, 2)); k[..., 1] = 1.0
    v = np.ones((1, 1, T, 3))
    z = np.zeros((1, 1, T))
    assert np.all(O.fwd_quadratic(q, k, v, z) == 0.0)
    o, _, _ = O.fwd_recurrent_packed(q, k, v, z)
    assert np.all(o == 0.0)


# --------------------------------------------------------------------------- a number the pages print

def test_memory_crossover_matches_the_page():
    # [2M2F §5.1]: at dh = 64 the squared state beats a softmax KV cache beyond about
    # 1058 tokens.  The packed symmetric state plus its normaliser plus the window-2
    # convolution cache reproduces it; other layouts do not.
    with open(os.path.join(GOLDEN, "memory_crossover.json")) as f:
        gold = json.load(f)
    d = gold["head_dim"]
    n_star = O.memory_crossover_tokens(d, conv_window=gold["conv_window"])
    assert math.ceil(n_star) == gold["crossover_tokens_approx"]
    # counting only the state (no normaliser), or an unsymmetrised d^2 state, misses it
    assert math.ceil(O.num_pairs(d) * d / (2 * d)) != gold["crossover_tokens_approx"]
    assert math.ceil((d * d * d + d * d) / (2 * d)) != gold["crossover_tokens_approx"]


def test_model_shapes_fixture_consistent():
    with open(os.path.join(GOLDEN, "model_shapes.json")) as f:
        s = json.load(f)
    for m in ("small_300M", "medium_700M"):
        assert s[m]["hidden"] == s[m]["heads"] * s[m]["head_dim"]


# ---------------------------------------------------------------- row statistics
def test_row_weight_sums_relate_the_two_normalisations():
    # o_t (normalised) * den_t = o_t without normalisation, row by row
    r = np.random.default_rng(61)
    q, k, v = (r.normal(size=(2, 2, 19, 4)) for _ in range(3))
    z = r.normal(-1.0, 1.0, size=(2, 2, 19))
    n0 = np.abs(r.normal(size=(2, 2, 10)))
    S0 = r.normal(size=(2, 2, 10, 4))
    den = O.row_weight_sums(q, k, z, scale=0.7, state_in_norm=n0)
    o = O.fwd_quadratic(q, k, v, z, scale=0.7, state_in=S0, norm_in=n0)
    num = O.fwd_quadratic(q, k, v, z, scale=0.7, norm=False, state_in=S0, norm_in=n0)
    np.testing.assert_allclose(o * den[..., None], num, rtol=1e-10, atol=1e-12)


def test_row_logsumexp_matches_torch_without_decay():
    r = np.random.default_rng(62)
    q, k = (r.normal(size=(2, 3, 17, 5)) for _ in range(2))
    z = np.full((2, 3, 17), -np.inf)
    s = 0.8 * np.matmul(q, np.swapaxes(k, -1, -2))
    s = np.where(np.tril(np.ones((17, 17), dtype=bool)), s, -np.inf)
    ref = torch.logsumexp(torch.tensor(s), dim=-1).numpy()
    np.testing.assert_allclose(O.row_logsumexp(q, k, z, scale=0.8), ref, rtol=1e-12, atol=1e-12)


def test_row_statistics_on_a_row_subset_are_those_rows():
    r = np.random.default_rng(63)
    q, k = (r.normal(size=(1, 2, 23, 4)) for _ in range(2))
    z = r.normal(-1.0, 1.0, size=(1, 2, 23))
    rows = [0, 5, 22]
    np.testing.assert_array_equal(O.row_weight_sums(q, k, z, scale=0.9, rows=rows),
                                  O.row_weight_sums(q, k, z, scale=0.9)[:, :, rows])
    np.testing.assert_array_equal(O.row_logsumexp(q, k, z, scale=0.9, rows=rows),
                                  O.row_logsumexp(q, k, z, scale=0.9)[:, :, rows])


def test_row_logsumexp_zero_scores_geometric_closed_form():
    # With zero scores only the A-mask is left [2M2F §6]: for a constant decay logit c
    # every row is a geometric series, lse_t = log sum_{m=0..t} e^{m g} with
    # g = -softplus(c).  A dropped mask gives log(t+1), a mask of the wrong sign a
    # growing series, a mask that includes the query's own token a shift by g.
    T = 40
    t = np.arange(T)
    for c in (-3.0, -1.0, 0.0, 0.7, 2.5):
        g = -math.log1p(math.exp(c))
        q = np.zeros((1, 1, T, 3))
        k = np.random.default_rng(64).normal(size=(1, 1, T, 3))
        z = np.full((1, 1, T), c)
        ref = np.log(-np.expm1((t + 1) * g) / -math.expm1(g))
        np.testing.assert_allclose(O.row_logsumexp(q, k, z)[0, 0], ref, rtol=1e-13, atol=1e-13)
    # no decay at all: t + 1 equal terms
    z = np.full((1, 1, T), -np.inf)
    np.testing.assert_allclose(O.row_logsumexp(np.zeros((1, 1, T, 3)), k, z)[0, 0], np.log(t + 1.0), rtol=1e-14)


def test_row_logsumexp_zero_scores_follow_the_one_token_recursion():
    # Zero scores with a varying decay: the row sum of token t is e^{g_t} times the row
    # sum of token t-1 plus the diagonal's 1, so lse_t = log(1 + e^{g_t + lse_{t-1}}).
    r = np.random.default_rng(65)
    z = r.normal(-1.0, 1.0, size=(2, 2, 31))
    g = -np.logaddexp(0.0, z)
    ref = np.zeros_like(z)
    for t in range(1, 31):
        ref[..., t] = np.logaddexp(0.0, g[..., t] + ref[..., t - 1])
    got = O.row_logsumexp(np.zeros((2, 2, 31, 4)), r.normal(size=(2, 2, 31, 4)), z)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def _lse_fd_inputs():
    r = np.random.default_rng(66)
    q, k = (r.normal(size=(1, 2, 13, 3)) for _ in range(2))
    z = r.normal(-1.0, 1.0, size=(1, 2, 13))
    return q, k, z


def test_row_logsumexp_decay_gradient_is_softmax_mass_before_the_token():
    # d lse_t / d g_r is the softmax mass on keys s < r <= t (those whose mask sums g_r),
    # and dg_r/dz_r = -sigmoid(z_r).  The 2Mamba-E forward with values 1(s < r) returns
    # exactly that mass, so a central difference of lse in z_r must match
    # -sigmoid(z_r) * o_t.  The forward is pinned on its own (causal SDPA without decay,
    # the zero-score closed form with decay, the streaming form).
    q, k, z = _lse_fd_inputs()
    T = q.shape[2]
    h = 1e-6
    for r_ in (1, 5, 12):
        v = (np.arange(T) < r_).astype(float)[None, None, :, None] * np.ones((1, 2, T, 1))
        o = O.fwd_exp_quadratic(q, k, v, z, scale=0.9)[..., 0]
        zp, zm = z.copy(), z.copy()
        zp[..., r_] += h
        zm[..., r_] -= h
        fd = (O.row_logsumexp(q, k, zp, scale=0.9) - O.row_logsumexp(q, k, zm, scale=0.9)) / (2 * h)
        ref = -O.sigmoid(z[..., r_])[..., None] * o
        ref[..., :r_] = 0.0     # rows before r do not contain g_r
        np.testing.assert_allclose(fd, ref, rtol=1e-6, atol=1e-8)
        assert np.abs(ref[..., r_:]).max() > 1e-3


def test_row_logsumexp_query_gradient_is_softmax_mean_key():
    # d lse_t / d q_t = scale * sum_s p_ts k_s: the 2Mamba-E forward with the keys as values
    q, k, z = _lse_fd_inputs()
    o = O.fwd_exp_quadratic(q, k, k, z, scale=0.9)
    h = 1e-6
    for t in (0, 4, 12):
        for i in range(3):
            qp, qm = q.copy(), q.copy()
            qp[:, :, t, i] += h
            qm[:, :, t, i] -= h
            fd = (O.row_logsumexp(qp, k, z, scale=0.9, rows=[t]) - O.row_logsumexp(qm, k, z, scale=0.9, rows=[t]))
            np.testing.assert_allclose(fd[..., 0] / (2 * h), 0.9 * o[:, :, t, i], rtol=1e-6, atol=1e-8)
