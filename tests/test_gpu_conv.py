"""GPU parity of the size-2 input convolution (twomamba_conv2) and of the decode
step with its one-token cache (twomamba_step_conv) against the oracle.

  * conv2 alone vs oracle.conv2 (with and without bias and cached row, ragged
    T, T = 0), and its cache output;
  * conv2 followed by the MFMA forward vs the oracle's quadratic form on the
    convolved inputs;
  * prompt (conv2 + forward with state) then decode steps through
    twomamba_step_conv vs the oracle's quadratic form on the whole convolved
    sequence, and the cache after the steps.

Tolerance: per-head inf-norm relative error <= 2e-2 (bf16) or 1e-4 (fp32).
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def weights(H, d, seed, bias=True):
    r = np.random.default_rng(seed + 900)
    w = r.normal(0.0, 0.7, size=(3, H, d, 2)).astype(np.float32)
    b = r.normal(0.0, 0.1, size=(3, H, d)).astype(np.float32) if bias else None
    return w, b


def cast(x, dtype):
    t = torch.from_numpy(np.asarray(x))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


@pytest.mark.parametrize("dtype,d,T,bias,cached", [
    ("bf16", 64, 200, True, True), ("bf16", 64, 77, False, False), ("f32", 16, 130, True, False),
    ("f32", 64, 1, True, True),
])
def test_conv2_matches_oracle(dtype, d, T, bias, cached):
    announce(f"conv2 {dtype} d={d} T={T} bias={bias} cached={cached}")
    B, H = 2, 3
    q, k, v, _ = SI.draw(B, H, T, d, seed=31, dtype=dtype)
    w, b = weights(H, d, 31, bias)
    prev = cast(np.random.default_rng(32).normal(size=(B, H, 3, d)), dtype) if cached else None
    qd, kd, vd = dev(q, k, v)
    wd = torch.from_numpy(w).cuda()
    bd = None if b is None else torch.from_numpy(b).cuda()
    yq, yk, yv, st = tmb.conv2(qd, kd, vd, wd, bd, None if prev is None else prev.cuda(), want_state=True)
    torch.cuda.synchronize()
    pv = None if prev is None else SI.to_f64(prev)
    for i, (x, y) in enumerate(((q, yq), (k, yk), (v, yv))):
        ref = O.conv2(SI.to_f64(x), w[i].astype(np.float64), None if b is None else b[i].astype(np.float64),
                      None if pv is None else pv[:, :, i])
        assert relerr(host64(y), ref) < TOL[dtype]
    last = torch.stack([q[:, :, -1], k[:, :, -1], v[:, :, -1]], dim=2)
    assert torch.equal(st.cpu(), last)


def test_conv2_empty_sequence_passes_the_cache_through():
    announce("conv2 T=0")
    B, H, d = 2, 3, 16
    z = torch.zeros(B, H, 0, d, device="cuda")
    w = torch.ones(3, H, d, 2, device="cuda")
    prev = torch.randn(B, H, 3, d, device="cuda")
    *_, st = tmb.conv2(z, z, z, w, None, prev, want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(st, prev)
    *_, st0 = tmb.conv2(z, z, z, w, None, None, want_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st0) == 0


@pytest.mark.parametrize("variant", ["sq", "exp"])
def test_conv_then_forward(variant):
    announce(f"conv2 + {variant} forward bf16 2x4x300")
    B, H, T, d = 2, 4, 300, 64
    q, k, v, z = SI.draw(B, H, T, d, seed=33, dtype="bf16", z_mean=-4.0)
    w, b = weights(H, d, 33)
    qd, kd, vd, zd = dev(q, k, v, z)
    yq, yk, yv = tmb.conv2(qd, kd, vd, torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda())
    out = tmb.fwd(yq, yk, yv, zd, variant=variant)
    torch.cuda.synchronize()
    xs = [O.conv2(SI.to_f64(x), w[i].astype(np.float64), b[i].astype(np.float64)) for i, x in enumerate((q, k, v))]
    zz = SI.to_f64(z)
    ref = O.fwd_quadratic(*xs, zz) if variant == "sq" else O.fwd_exp_quadratic(*xs, zz)
    assert relerr(host64(out), ref) < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prompt_then_conv_steps(dtype):
    B, H, d, T0, N = 2, 2, 64, 150, 24
    T = T0 + N
    announce(f"conv prompt T0={T0} + {N} conv steps {dtype}")
    q, k, v, z = SI.draw(B, H, T, d, seed=34, dtype=dtype, z_mean=-3.0)
    w, b = weights(H, d, 34)
    qd, kd, vd, zd = dev(q, k, v, z)
    wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    yq, yk, yv, cs = tmb.conv2(qd[:, :, :T0].contiguous(), kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(),
                               wd, bd, want_state=True)
    _, S, n = tmb.fwd(yq, yk, yv, zd[:, :, :T0].contiguous(), want_state=True)
    outs = []
    for t in range(T0, T):
        outs.append(tmb.step_conv(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                  zd[:, :, t].contiguous(), wd, bd, cs, S, n))
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=2)
    xs = [O.conv2(SI.to_f64(x), w[i].astype(np.float64), b[i].astype(np.float64)) for i, x in enumerate((q, k, v))]
    ref = O.fwd_quadratic_rows(*xs, SI.to_f64(z), list(range(T0, T)))
    e = relerr(got, ref)
    print(f"  out err {e:.2e}")
    assert e < TOL[dtype]
    assert torch.equal(cs.cpu(), torch.stack([q[:, :, -1], k[:, :, -1], v[:, :, -1]], dim=2))
