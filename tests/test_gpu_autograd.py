"""The autograd wrapper (second_order_ssm_amd.twomamba): its gradients are the
library backward's, fed with the forward's row statistics, and they chain into
surrounding torch operations.  Compared with the oracle's gradients at the
bf16 / fp32 tolerances (per-head inf-norm relative error)."""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant,dtype,d", [("sq", "bf16", 64), ("exp", "bf16", 64), ("lin", "bf16", 64),
                                             ("sq", "f32", 16)])
def test_autograd_matches_oracle(variant, dtype, d):
    B, H, T = 1, 2, 150
    announce(f"autograd {variant} {dtype} {B}x{H}x{T} d={d}")
    q, k, v, z = SI.draw(B, H, T, d, seed=95, dtype=dtype, z_mean=-2.0)
    do = torch.from_numpy(np.random.default_rng(96).standard_normal((B, H, T, d)))
    do = do.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    leaves = [t.clone().requires_grad_(True) for t in dev(q, k, v, z)]
    out = tmb.twomamba(*leaves, variant=variant)
    out.backward(do.cuda())
    torch.cuda.synchronize()
    qq, kk, vv, zz, dd = (SI.to_f64(t) for t in (q, k, v, z, do))
    if variant == "sq":
        ref = O.bwd_quadratic(qq, kk, vv, zz, dd)
    elif variant == "exp":
        ref = O.bwd_exp_quadratic(qq, kk, vv, zz, dd)
    else:
        ref = O.bwd_linear_quadratic(qq, kk, vv, zz, dd)
    for name, leaf, r in zip(("dq", "dk", "dv", "dz"), leaves, ref):
        e = relerr(host64(leaf.grad), r)
        print(f"  {name} {e:.2e}")
        assert e < TOL[dtype]


def test_autograd_chains_through_projections():
    # x -> (q, k, v) by linear maps, then the operator: torch's chain rule on the
    # projections must see the operator's gradients
    B, H, T, d, C = 1, 2, 130, 16, 24
    announce(f"autograd through projections {B}x{H}x{T} d={d}")
    r = np.random.default_rng(97)
    x = torch.from_numpy(r.standard_normal((B, H, T, C)) / np.sqrt(C)).float().cuda()
    W = [torch.from_numpy(r.standard_normal((C, d)) / np.sqrt(C)).float().cuda().requires_grad_(True)
         for _ in range(3)]
    z = torch.from_numpy(r.standard_normal((B, H, T)) - 2.0).float().cuda()
    q, k, v = (x @ w for w in W)
    out = tmb.twomamba(q, k, v, z)
    loss = (out * out).sum()
    loss.backward()
    # the same chain by hand: dL/dout = 2 out, operator backward, then x^T d(.)
    dq, dk, dv, _ = tmb.bwd(q.detach().contiguous(), k.detach().contiguous(), v.detach().contiguous(), z,
                            out.detach(), 2 * out.detach())
    for w, g in zip(W, (dq, dk, dv)):
        ref = torch.einsum("bhtc,bhtd->cd", x, g)
        assert torch.allclose(w.grad, ref, rtol=1e-4, atol=1e-5)
