"""GPU parity of the MFMA 2Mamba-E forward (bf16 inputs, d = 64) against the fp64 oracle.

Cases span several 256-query workgroup tiles and 64-key tiles with ragged tails,
strong and weak decay (the bias spans thousands of log units in the first,
nearly nothing in the second), no decay at all (plain causal softmax), query
scales, logits large enough that the running max has to move, and sampled rows
of the full 2 x 16 x 8192 workload.  Tolerance: per-head inf-norm relative error
<= 2e-2 (bf16 inputs and probabilities, fp32 accumulation).
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def o64(*ts):
    return tuple(SI.to_f64(t) for t in ts)


CASES = [
    # B, H, T, z_mean, z_neg_inf, scale
    (1, 2, 64, 0.0, False, 1.0),
    (2, 3, 200, 0.0, False, 1.0),
    (1, 2, 1000, -6.0, False, 1.0),     # 4 query tiles, ragged tail
    (1, 1, 777, -10.0, False, 0.125),   # slow decay, small scale
    (2, 1, 333, 0.0, True, 1.0),        # no decay: plain causal softmax
    (1, 2, 1, 0.0, False, 1.0),         # single token
    (1, 1, 2500, 4.0, False, 1.0),      # very strong decay: bias of thousands
    (1, 1, 4096, -12.0, False, 2.0),    # long, weak decay
]


@pytest.mark.parametrize("B,H,T,zm,zinf,scale", CASES)
def test_mfma_exp_matches_oracle(B, H, T, zm, zinf, scale):
    announce(f"MFMA EXP B={B} H={H} T={T} z_mean={zm} ninf={zinf} scale={scale}")
    q, k, v, z = SI.draw(B, H, T, 64, seed=200 + T, dtype="bf16", z_mean=zm, z_neg_inf=zinf)
    out = tmb.fwd(*dev(q, k, v, z), variant="exp", scale=scale)
    torch.cuda.synchronize()
    ref = O.fwd_exp_quadratic(*o64(q, k, v, z), scale=scale)
    e = relerr(host64(out), ref)
    print(f"  err out {e:.2e}")
    assert e < TOL["bf16"]


def test_mfma_exp_large_logits():
    # |q.k| of tens to hundreds: the running max moves many times along a row
    announce("MFMA EXP q*8, k*4 (large logits)")
    q, k, v, z = SI.draw(1, 2, 600, 64, seed=11, dtype="f32", z_mean=-8.0)
    q, k, v = (q * 8).bfloat16(), (k * 4).bfloat16(), v.bfloat16()
    out = tmb.fwd(*dev(q, k, v, z), variant="exp")
    torch.cuda.synchronize()
    assert relerr(host64(out), O.fwd_exp_quadratic(*o64(q, k, v, z))) < TOL["bf16"]


def test_mfma_exp_no_decay_is_causal_softmax():
    # with z = -inf the operator is causal softmax attention: check against torch's
    announce("MFMA EXP z=-inf vs torch causal SDPA (fp32, CPU)")
    q, k, v, z = SI.draw(1, 2, 300, 64, seed=12, dtype="bf16", z_neg_inf=True)
    out = tmb.fwd(*dev(q, k, v, z), variant="exp", scale=0.7)
    torch.cuda.synchronize()
    ref = torch.nn.functional.scaled_dot_product_attention(q.float(), k.float(), v.float(), is_causal=True, scale=0.7)
    assert relerr(host64(out), ref.double().numpy()) < TOL["bf16"]


def test_mfma_exp_matches_reference_kernel():
    announce("MFMA EXP vs reference kernel, B=2 H=2 T=2048")
    q, k, v, z = dev(*SI.draw(2, 2, 2048, 64, seed=13, dtype="bf16", z_mean=-7.0))
    a = tmb.fwd(q, k, v, z, variant="exp")
    b = tmb.fwd(q, k, v, z, variant="exp", reference_kernels=True)
    torch.cuda.synchronize()
    assert relerr(host64(a), host64(b)) < TOL["bf16"]


def test_mfma_exp_deterministic():
    announce("MFMA EXP bitwise determinism")
    q, k, v, z = dev(*SI.draw(2, 2, 777, 64, seed=14, dtype="bf16", z_mean=-3.0))
    a = tmb.fwd(q, k, v, z, variant="exp")
    b = tmb.fwd(q, k, v, z, variant="exp")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("zm", [0.0, -9.0])
def test_mfma_exp_full_size_sampled_rows(zm):
    # the benchmark shape, checked on rows at tile boundaries and at the end of
    # the sequence for a few heads (the oracle computes single rows directly)
    B, H, T = 2, 16, 8192
    announce(f"MFMA EXP full size B={B} H={H} T={T} z_mean={zm}, sampled rows")
    q, k, v, z = SI.draw(B, H, T, 64, seed=3, dtype="bf16", z_mean=zm)
    out = host64(tmb.fwd(*dev(q, k, v, z), variant="exp"))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 255, 256, 257, 4095, 4096, 5000, 8127, 8128, 8191]
    heads = [(0, 0), (1, 7), (1, 15)]
    for b, h in heads:
        qq, kk, vv, zz = (SI.to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v, z))
        ref = O.fwd_exp_quadratic_rows(qq, kk, vv, zz, rows)
        e = relerr(out[b:b + 1, h:h + 1, rows], ref)
        print(f"  head ({b},{h}) err {e:.2e}")
        assert e < TOL["bf16"]


def test_mfma_exp_decay_resets():
    # no decay except a near-total reset (bias about -50) every 97 tokens
    announce("MFMA EXP decay resets B=1 H=2 T=1000")
    q, k, v, z = SI.draw(1, 2, 1000, 64, seed=230, dtype="bf16")
    z = torch.full_like(z, float("-inf"))
    z[:, :, ::97] = 50.0
    out = tmb.fwd(*dev(q, k, v, z), variant="exp")
    torch.cuda.synchronize()
    e = relerr(host64(out), O.fwd_exp_quadratic(*o64(q, k, v, z)))
    print(f"  err out {e:.2e}")
    assert e < TOL["bf16"]
