"""GPU parity of the first-order (Mamba-2S) forward across the layouts of its
segmented bf16 d = 64 path, against the fp64 oracle on every row.

The path cuts each head into segments (about two workgroups per CU, at least
two chunks each), computes their end states, scans them into carries and then
runs every segment from its carry.  The shapes reach one segment per head at
many heads, sixteen segments with a ragged last chunk, odd head counts with a
caller state, and a long head of 157 two-chunk segments (the scan's unrolled
and remainder parts).  Slow decay, z ~ N(-8, 1), so that the carries reach far.
The reference is the oracle's token-by-token recurrence (pinned to its
quadratic form on the CPU), for all rows and for the final state.  At 157
segments the O(T) backward is also compared with the quadratic MFMA kernels
(TWOMAMBA_FLAG_ATTENTION_FORM), which tests/test_gpu_bwd.py pins to the oracle.
Tolerance: per-head inf-norm relative error <= 2e-2.
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, T, caller state
    (1, 1, 64, False),       # one chunk
    (2, 16, 130, True),      # 32 heads of three chunks: one segment each
    (1, 1, 3000, False),     # sixteen segments of three chunks, ragged last chunk
    (3, 5, 777, True),       # fifteen heads, a caller state folded into the first segment
    (1, 3, 20000, True),     # 157 segments of two chunks, ragged last chunk
]


@pytest.mark.parametrize("B,H,T,with_state", SHAPES)
def test_lin_plan_forward(B, H, T, with_state):
    announce(f"first-order fwd layout B={B} H={H} T={T} state={with_state}")
    d = 64
    q, k, v, z = SI.draw(B, H, T, d, seed=900 + T, dtype="bf16", z_mean=-8.0)
    S0 = np.random.default_rng(901).normal(0, 0.3, size=(B, H, d, d)).astype(np.float32) if with_state else None
    qd, kd, vd, zd = dev(q, k, v, z)
    s_in = None if S0 is None else torch.from_numpy(S0).cuda()
    out, S, _ = tmb.fwd(qd, kd, vd, zd, variant="lin", state_in=s_in, want_state=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = (SI.to_f64(t) for t in (q, k, v, z))
    ref, Sref = O.fwd_linear_recurrent(qq, kk, vv, zz, state_in=None if S0 is None else S0.astype(np.float64))
    eo, es = relerr(host64(out), ref), relerr(host64(S), Sref)
    print(f"  out err {eo:.2e} state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_lin_plan_backward_many_segments():
    B, H, T, d = 1, 3, 20000, 64
    announce(f"first-order O(T) bwd against the attention form B={B} H={H} T={T}")
    q, k, v, z = SI.draw(B, H, T, d, seed=920, dtype="bf16", z_mean=-8.0)
    do = torch.from_numpy(np.random.default_rng(921).standard_normal((B, H, T, d))).to(torch.bfloat16)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant="lin")
    a = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin")
    b = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin", attention_form=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dz"), a, b):
        e = relerr(host64(x), host64(y))
        print(f"  {name} {e:.2e}")
        assert e < TOL["bf16"]
