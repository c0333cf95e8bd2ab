"""GPU parity of the backward pass (twomamba_bwd) against the oracle's gradients.

For seeded inputs (synth_inputs) and a seeded output gradient, the HIP
backward's dq, dk, dv and dz are compared with the fp64 oracle (bwd_quadratic /
bwd_exp_quadratic, themselves pinned by finite differences and torch SDPA
autograd) on the same cast inputs.  The forward output handed to the backward
is the library's own forward.

Tolerance: per-head inf-norm relative error <= 2e-2 (bf16) or 1e-4 (fp32),
for each of the four gradients.
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def _dout(B, H, T, dv, dtype, seed):
    g = np.random.default_rng(seed + 500).standard_normal((B, H, T, dv))
    t = torch.from_numpy(g)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def run_bwd(variant, dtype, B, H, T, d, zm, scale, no_norm=False, reference=False, seed=11, z_neg_inf=False):
    q, k, v, z = SI.draw(B, H, T, d, seed=seed, dtype=dtype, z_mean=zm, z_neg_inf=z_neg_inf)
    do = _dout(B, H, T, d, dtype, seed)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant=variant, scale=scale, no_norm=no_norm)
    g = tmb.bwd(qd, kd, vd, zd, out, dod, variant=variant, scale=scale, no_norm=no_norm,
                reference_kernels=reference)
    torch.cuda.synchronize()
    return [host64(x) for x in g], (q, k, v, z, do)


def oracle_grads(variant, inputs, scale, no_norm=False):
    q, k, v, z, do = (SI.to_f64(t) for t in inputs)
    if variant == "sq":
        return O.bwd_quadratic(q, k, v, z, do, scale=scale, norm=not no_norm)
    return O.bwd_exp_quadratic(q, k, v, z, do, scale=scale)


def check(got, ref, tol, label):
    names = ("dq", "dk", "dv", "dz")
    errs = {n: relerr(g, r) for n, g, r in zip(names, got, ref)}
    print(f"  {label}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e < tol, f"{n} error {e:.3e}"


CASES = [
    # variant, dtype, B, H, T, d, z_mean, scale, no_norm
    ("sq", "f32", 1, 2, 150, 16, 0.0, 1.0, False),
    ("sq", "f32", 1, 2, 130, 64, -4.0, 0.8, False),
    ("sq", "bf16", 2, 2, 200, 64, -6.0, 1.0, False),
    ("sq", "f32", 1, 2, 100, 16, -2.0, 1.0, True),
    ("sq", "bf16", 1, 2, 129, 64, 0.0, 1.0, True),
    ("exp", "f32", 1, 2, 150, 16, 0.0, 1.0, False),
    ("exp", "bf16", 2, 2, 200, 64, -3.0, 1.0, False),
    ("exp", "f32", 1, 1, 65, 64, -8.0, 0.5, False),
    ("sq", "bf16", 1, 2, 1000, 64, -3.0, 1.0, False),
    ("exp", "bf16", 1, 2, 1000, 64, -1.0, 0.7, False),
    ("sq", "bf16", 1, 1, 64, 64, -12.0, 1.0, False),
    ("exp", "bf16", 1, 1, 63, 64, 0.0, 1.0, False),
    # head counts that are multiples of 8 take the XCD-grouped block order
    ("sq", "bf16", 2, 4, 300, 64, -2.0, 1.0, False),
    ("exp", "bf16", 1, 8, 257, 64, -1.0, 1.0, False),
    # strong decay (a bias near -4, for 2Mamba-E -2, per token): only the nearest
    # pairs count.  Stronger decay leaves each output nearly its own value: dq and
    # dk then shrink to the size of the bf16 rounding of the forward output that
    # the backward is given, and the comparison measures that rounding.
    ("sq", "bf16", 1, 2, 300, 64, 4.0, 1.0, False),
    ("exp", "bf16", 1, 2, 300, 64, 2.0, 1.0, False),
]


@pytest.mark.parametrize("variant,dtype,B,H,T,d,zm,scale,no_norm", CASES)
@pytest.mark.parametrize("reference", [True, False])
def test_bwd_matches_oracle(variant, dtype, B, H, T, d, zm, scale, no_norm, reference):
    announce(f"bwd {variant} {dtype} {B}x{H}x{T} d={d} z_mean={zm} scale={scale} no_norm={no_norm} "
             f"reference={reference}")
    got, inputs = run_bwd(variant, dtype, B, H, T, d, zm, scale, no_norm, reference)
    ref = oracle_grads(variant, inputs, scale, no_norm)
    check(got, ref, TOL[dtype], variant)


@pytest.mark.parametrize("variant", ["sq", "exp"])
def test_bwd_no_decay(variant):
    announce(f"bwd {variant} with z = -inf")
    got, inputs = run_bwd(variant, "bf16", 1, 2, 96, 64, 0.0, 1.0, z_neg_inf=True)
    ref = oracle_grads(variant, inputs, 1.0)
    check(got[:3], ref[:3], TOL["bf16"], variant)
    assert np.all(got[3] == 0.0)


@pytest.mark.parametrize("variant", ["sq", "exp"])
def test_bwd_single_token_and_empty(variant):
    announce(f"bwd {variant} T=1 and T=0")
    got, inputs = run_bwd(variant, "f32", 2, 3, 1, 16, 0.0, 1.0)
    # one token: o_0 = v_0 whatever q, k and z, so dv = dout and the rest is 0
    # (up to the rounding of the weight ratio, which the relative bar would
    # measure against the oracle's own rounding noise)
    np.testing.assert_allclose(got[2], SI.to_f64(inputs[4]), rtol=1e-6, atol=1e-6)
    for x in (got[0], got[1], got[3]):
        assert np.max(np.abs(x)) < 1e-5
    z4 = torch.zeros(1, 1, 0, 16, device="cuda")
    g = tmb.bwd(z4, z4, z4, torch.zeros(1, 1, 0, device="cuda"), z4, z4, variant=variant)
    assert all(x.numel() == 0 for x in g)


def test_bwd_deterministic():
    announce("bwd bitwise determinism")
    a, _ = run_bwd("exp", "bf16", 1, 2, 300, 64, -2.0, 1.0)
    b, _ = run_bwd("exp", "bf16", 1, 2, 300, 64, -2.0, 1.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("variant", ["sq", "exp", "lin"])
def test_bwd_full_size_two_heads(variant):
    # the benchmark workload 2 x 16 x 8192 bf16, in the launch configuration the
    # benchmark times; two whole heads against the oracle's whole-matrix form
    B, H, T, d = 2, 16, 8192, 64
    announce(f"bwd {variant} full size {B}x{H}x{T}")
    q, k, v, z = SI.draw(B, H, T, d, seed=3, dtype="bf16")
    do = _dout(B, H, T, d, "bf16", 3)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant=variant)
    g = tmb.bwd(qd, kd, vd, zd, out, dod, variant=variant)
    torch.cuda.synchronize()
    got = [host64(x) for x in g]
    for b, h in [(0, 0), (1, 15)]:
        sl = lambda t: SI.to_f64(t[b:b + 1, h:h + 1])
        ref = O.bwd_blocked(sl(q), sl(k), sl(v), sl(z), sl(do), variant=variant)
        check([x[b:b + 1, h:h + 1] for x in got], ref, TOL["bf16"], f"{variant} head ({b},{h})")


@pytest.mark.parametrize("B,H,T,heads", [(2, 16, 8192, [(0, 3), (1, 12)]), (1, 16, 32768, [(0, 7)])])
def test_lin_bwd_linear_in_T_full_size(B, H, T, heads):
    # the first order's O(T) backward (three segmented forwards, two of them in reverse
    # time) at the workload sizes, with slow decay (z_mean -8) so that the carried
    # states of the reverse passes reach across chunks and segments
    d = 64
    announce(f"first-order chunked bwd {B}x{H}x{T} z_mean -8")
    q, k, v, z = SI.draw(B, H, T, d, seed=3, dtype="bf16", z_mean=-8.0)
    do = _dout(B, H, T, d, "bf16", 3)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant="lin")
    g = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin")
    torch.cuda.synchronize()
    got = [host64(x) for x in g]
    for b, h in heads:
        sl = lambda t: SI.to_f64(t[b:b + 1, h:h + 1])
        ref = O.bwd_blocked(sl(q), sl(k), sl(v), sl(z), sl(do), variant="lin")
        check([x[b:b + 1, h:h + 1] for x in got], ref, TOL["bf16"], f"lin head ({b},{h})")


@pytest.mark.parametrize("T", [1, 64, 65, 700])
def test_lin_bwd_linear_form_matches_attention_form(T):
    # the same gradients from the O(T) path, the quadratic reference kernels and the quadratic MFMA kernels
    announce(f"first-order bwd: chunked vs reference kernels T={T}")
    q, k, v, z = SI.draw(2, 3, T, 64, seed=60 + T, dtype="bf16", z_mean=-6.0)
    do = _dout(2, 3, T, 64, "bf16", 61)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out = tmb.fwd(qd, kd, vd, zd, variant="lin")
    a = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin")
    b = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin", reference_kernels=True)
    c = tmb.bwd(qd, kd, vd, zd, out, dod, variant="lin", attention_form=True)   # the MFMA attention form
    torch.cuda.synchronize()
    for nm, x, y, w in zip(("dq", "dk", "dv", "dz"), a, b, c):
        e, e2 = relerr(host64(x), host64(y)), relerr(host64(w), host64(y))
        print(f"  {nm} {e:.2e} (attention form {e2:.2e})")
        assert e < TOL["bf16"] and e2 < TOL["bf16"], nm
