"""Pins of the oracle's size-2 input convolution (CPU only).

  * torch.nn.functional.conv1d with one group per channel, left-padded by
    the cached row, is the library definition the oracle's loop must match;
  * an impulse on one channel leaves exactly the two taps behind it;
  * running a sequence in two pieces, the second started from the first's
    last raw row, equals running it whole;
  * decode steps with the convolution cache, from a state the packed
    recurrence built over a convolved prompt, equal the quadratic form on the
    convolved whole sequence.
"""

import numpy as np
import torch

from oracle import twomamba_oracle as O


def _data(seed, B=2, H=3, T=9, d=4):
    r = np.random.default_rng(seed)
    return r.normal(size=(B, H, T, d)), r.normal(size=(H, d, 2)), r.normal(size=(H, d)), r.normal(size=(B, H, d))


def test_conv2_matches_torch_grouped_conv1d():
    x, w, b, prev = _data(0)
    B, H, T, d = x.shape
    y = O.conv2(x, w, b, prev)
    xt = torch.tensor(np.concatenate([prev[:, :, None], x], axis=2))        # [B,H,T+1,d]
    xt = xt.permute(0, 1, 3, 2).reshape(B, H * d, T + 1)
    wt = torch.tensor(w.reshape(H * d, 1, 2))
    yt = torch.nn.functional.conv1d(xt, wt, torch.tensor(b.reshape(-1)), groups=H * d)
    yt = yt.reshape(B, H, d, T).permute(0, 1, 3, 2).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)
    # no cached row: zero padding
    y0 = O.conv2(x, w, b)
    xt0 = torch.tensor(x).permute(0, 1, 3, 2).reshape(B, H * d, T)
    yt0 = torch.nn.functional.conv1d(torch.nn.functional.pad(xt0, (1, 0)), wt, torch.tensor(b.reshape(-1)),
                                     groups=H * d).reshape(B, H, d, T).permute(0, 1, 3, 2).numpy()
    np.testing.assert_allclose(y0, yt0, rtol=1e-12, atol=1e-12)


def test_conv2_impulse():
    _, w, _, _ = _data(1)
    x = np.zeros((1, 3, 6, 4))
    x[0, 1, 2, 3] = 1.0
    y = O.conv2(x, w)
    expect = np.zeros_like(x)
    expect[0, 1, 2, 3] = w[1, 3, 1]
    expect[0, 1, 3, 3] = w[1, 3, 0]
    np.testing.assert_array_equal(y, expect)


def test_conv2_split_resume():
    x, w, b, prev = _data(2, T=11)
    whole = O.conv2(x, w, b, prev)
    a = O.conv2(x[:, :, :5], w, b, prev)
    c = O.conv2(x[:, :, 5:], w, b, x[:, :, 4])
    np.testing.assert_allclose(np.concatenate([a, c], axis=2), whole, rtol=1e-14, atol=1e-14)


def test_step_conv_continues_the_convolved_sequence():
    r = np.random.default_rng(3)
    B, H, T0, N, d = 1, 2, 6, 4, 3
    T = T0 + N
    q, k, v = (r.normal(size=(B, H, T, d)) for _ in range(3))
    z = r.normal(-1.0, 1.0, size=(B, H, T))
    w = r.normal(size=(3, H, d, 2))
    b = r.normal(size=(3, H, d))
    qc, kc, vc = (O.conv2(x, w[i], b[i]) for i, x in enumerate((q, k, v)))
    ref = O.fwd_quadratic(qc, kc, vc, z, scale=0.8)
    # state after the convolved prompt, then steps carrying the raw last row
    S, n = O.final_state_direct(kc[:, :, :T0], vc[:, :, :T0], z[:, :, :T0])
    cs = np.stack([q[:, :, T0 - 1], k[:, :, T0 - 1], v[:, :, T0 - 1]], axis=2)
    for t in range(T0, T):
        o, S, n, cs = O.step_conv(q[:, :, t], k[:, :, t], v[:, :, t], z[:, :, t], w, b, cs, S, n, scale=0.8)
        np.testing.assert_allclose(o, ref[:, :, t], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
import pytest

_orig_conv2 = O.conv2


def _taps_swapped(x, w, b=None, prev=None):
    return _orig_conv2(x, w[..., ::-1], b, prev)


def _prev_ignored(x, w, b=None, prev=None):
    return _orig_conv2(x, w, b, None)


@pytest.mark.parametrize("patch,pins", [
    (_taps_swapped, [test_conv2_impulse, test_conv2_matches_torch_grouped_conv1d]),
    (_prev_ignored, [test_conv2_split_resume, test_conv2_matches_torch_grouped_conv1d,
                     test_step_conv_continues_the_convolved_sequence]),
], ids=["taps swapped", "cached row ignored"])
def test_planted_conv_mistake_is_caught(monkeypatch, patch, pins):
    monkeypatch.setattr(O, "conv2", patch)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
