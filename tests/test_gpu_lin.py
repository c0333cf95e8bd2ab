"""GPU parity of the first-order (Mamba-2S) variant against the oracle.

  * chunked forward (TWOMAMBA_LIN) vs the quadratic form, with and without an
    initial state, the final state vs the recurrence, ragged T, T = 0;
  * the full workload size 2 x 16 x 8192 (bf16) vs the token recurrence
    (pinned equal to the quadratic form), every row;
  * prompt then first-order decode steps (TWOMAMBA_FLAG_FIRST_ORDER), plain
    and through the input convolution;
  * backward (reference and MFMA kernels) vs the oracle's gradients.

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


@pytest.mark.parametrize("dtype,B,H,T,d,zm,scale,with_state", [
    ("f32", 1, 2, 150, 16, 0.0, 1.0, False), ("f32", 2, 2, 130, 64, -4.0, 0.8, True),
    ("bf16", 2, 3, 300, 64, -6.0, 1.0, True), ("bf16", 1, 2, 1, 64, 0.0, 1.0, False),
])
def test_lin_forward_matches_oracle(dtype, B, H, T, d, zm, scale, with_state):
    announce(f"lin fwd {dtype} {B}x{H}x{T} d={d} z_mean={zm} state={with_state}")
    q, k, v, z = SI.draw(B, H, T, d, seed=41, dtype=dtype, z_mean=zm)
    S0 = np.random.default_rng(42).normal(0, 0.3, size=(B, H, d, d)) if with_state else None
    qd, kd, vd, zd = dev(q, k, v, z)
    s_in = None if S0 is None else torch.from_numpy(S0.astype(np.float32)).cuda()
    out, S, _ = tmb.fwd(qd, kd, vd, zd, variant="lin", scale=scale, state_in=s_in, want_state=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = (SI.to_f64(t) for t in (q, k, v, z))
    S0r = None if S0 is None else S0.astype(np.float32).astype(np.float64)
    ref = O.fwd_linear_quadratic(qq, kk, vv, zz, scale=scale, state_in=S0r)
    _, Sref = O.fwd_linear_recurrent(qq, kk, vv, zz, scale=scale, state_in=S0r)
    eo, es = relerr(host64(out), ref), relerr(host64(S), Sref)
    print(f"  out err {eo:.2e} state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


def test_lin_forward_empty_sequence_copies_the_state():
    announce("lin fwd T=0")
    z4 = torch.zeros(2, 3, 0, 16, device="cuda")
    s_in = torch.randn(2, 3, 16, 16, device="cuda")
    out, S, _ = tmb.fwd(z4, z4, z4, torch.zeros(2, 3, 0, device="cuda"), variant="lin", state_in=s_in,
                        want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S, s_in)


def test_lin_full_size_every_row():
    B, H, T, d = 2, 16, 8192, 64
    announce(f"lin fwd bf16 {B}x{H}x{T} vs the token recurrence")
    q, k, v, z = SI.draw(B, H, T, d, seed=3, dtype="bf16", z_mean=-4.0)
    out, S, _ = tmb.fwd(*dev(q, k, v, z), variant="lin", want_state=True)
    torch.cuda.synchronize()
    ref, Sref = O.fwd_linear_recurrent(*(SI.to_f64(t) for t in (q, k, v, z)))
    eo, es = relerr(host64(out), ref), relerr(host64(S), Sref)
    print(f"  out err {eo:.2e} state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# B*H not a multiple of 4 leaves dead waves in the last workgroup of the d = 64 step
@pytest.mark.parametrize("dtype,conv,B,H", [("f32", False, 2, 2), ("bf16", False, 1, 3), ("f32", True, 2, 2),
                                            ("f32", True, 1, 5), ("bf16", True, 2, 3)])
def test_lin_prompt_then_steps(dtype, conv, B, H):
    d, T0, N = 64, 130, 20
    T = T0 + N
    announce(f"lin prompt T0={T0} + {N} first-order steps {dtype} conv={conv} B={B} H={H}")
    q, k, v, z = SI.draw(B, H, T, d, seed=43, dtype=dtype, z_mean=-3.0)
    qd, kd, vd, zd = dev(q, k, v, z)
    qq, kk, vv, zz = (SI.to_f64(t) for t in (q, k, v, z))
    if conv:
        r = np.random.default_rng(44)
        w = r.normal(0, 0.7, size=(3, H, d, 2)).astype(np.float32)
        b = r.normal(0, 0.1, size=(3, H, d)).astype(np.float32)
        wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
        yq, yk, yv, cs = tmb.conv2(qd[:, :, :T0].contiguous(), kd[:, :, :T0].contiguous(),
                                   vd[:, :, :T0].contiguous(), wd, bd, want_state=True)
        _, S, _ = tmb.fwd(yq, yk, yv, zd[:, :, :T0].contiguous(), variant="lin", want_state=True)
        qq, kk, vv = (O.conv2(x, w[i].astype(np.float64), b[i].astype(np.float64)) for i, x in enumerate((qq, kk, vv)))
    else:
        _, S, _ = tmb.fwd(qd[:, :, :T0].contiguous(), kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(),
                          zd[:, :, :T0].contiguous(), variant="lin", want_state=True)
    outs = []
    for t in range(T0, T):
        args = [x[:, :, t].contiguous() for x in (qd, kd, vd, zd)]
        if conv:
            outs.append(tmb.step_conv(*args, wd, bd, cs, S, None, first_order=True))
        else:
            outs.append(tmb.step(*args, S, None, first_order=True))
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=2)
    ref = O.fwd_linear_quadratic(qq, kk, vv, zz)[:, :, T0:]
    e = relerr(got, ref)
    print(f"  out err {e:.2e}")
    assert e < TOL[dtype]


def _dout(B, H, T, d, dtype, seed):
    t = torch.from_numpy(np.random.default_rng(seed + 500).standard_normal((B, H, T, d)))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


@pytest.mark.parametrize("dtype,B,H,T,d,zm,scale", [
    ("f32", 1, 2, 150, 16, 0.0, 1.0), ("bf16", 2, 2, 200, 64, -3.0, 0.8), ("bf16", 2, 4, 300, 64, -1.0, 1.0),
])
@pytest.mark.parametrize("reference", [True, False])
def test_lin_backward_matches_oracle(dtype, B, H, T, d, zm, scale, reference):
    announce(f"lin bwd {dtype} {B}x{H}x{T} d={d} z_mean={zm} reference={reference}")
    q, k, v, z = SI.draw(B, H, T, d, seed=45, dtype=dtype, z_mean=zm)
    do = _dout(B, H, T, d, dtype, 45)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant="lin", scale=scale)
    g = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin", scale=scale, reference_kernels=reference)
    torch.cuda.synchronize()
    ref = O.bwd_linear_quadratic(*(SI.to_f64(t) for t in (q, k, v, z, do)), scale=scale)
    for name, a, r in zip(("dq", "dk", "dv", "dz"), g, ref):
        e = relerr(host64(a), r)
        print(f"  {name} {e:.2e}")
        assert e < TOL[dtype]
