"""GPU parity of the per-row statistics (twomamba_fwd_stats) and of the backward
that takes them instead of recomputing them.

  * the row statistic against the oracle: 2Mamba's weight sum den_t (with and
    without an initial normaliser, also under NO_NORM) and 2Mamba-E's natural
    log-sum-exp lse_t, on the MFMA and the reference kernels, ragged T;
  * the output of twomamba_fwd_stats is bit-identical to twomamba_fwd's;
  * twomamba_bwd with the statistics against the oracle's gradients;
  * the full workload size 2 x 16 x 8192 (bf16): sampled rows of the
    statistic, and two whole heads of the backward fed with them, which is
    the configuration the benchmark times.

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


def o64(*ts):
    return tuple(SI.to_f64(t) for t in ts)


def initial_state(B, H, d, seed):
    _, k0, v0, z0 = SI.draw(B, H, 40, d, seed=seed, dtype="f32", z_mean=-2.0)
    S0, n0 = O.final_state_direct(*o64(k0, v0, z0))
    return (torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(n0, dtype=np.float32)).cuda())


STAT_CASES = [
    # variant, dtype, B, H, T, d, z_mean, scale, reference, with_state, no_norm
    ("sq", "bf16", 2, 3, 300, 64, -2.0, 1.0, False, False, False),
    ("sq", "bf16", 1, 2, 1000, 64, -6.0, 0.8, False, True, False),
    ("sq", "bf16", 1, 2, 130, 64, 0.0, 1.0, False, False, True),
    ("sq", "f32", 1, 2, 150, 16, 0.0, 1.0, True, True, False),
    ("sq", "bf16", 2, 2, 77, 64, -3.0, 1.0, True, False, False),
    ("exp", "bf16", 2, 3, 300, 64, -2.0, 1.0, False, False, False),
    ("exp", "bf16", 1, 2, 1000, 64, -1.0, 0.7, False, False, False),
    ("exp", "bf16", 1, 1, 1, 64, 0.0, 1.0, False, False, False),
    ("exp", "f32", 1, 2, 150, 16, 0.0, 1.0, True, False, False),
]


@pytest.mark.parametrize("variant,dtype,B,H,T,d,zm,scale,reference,with_state,no_norm", STAT_CASES)
def test_forward_row_statistics(variant, dtype, B, H, T, d, zm, scale, reference, with_state, no_norm):
    announce(f"fwd stats {variant} {dtype} {B}x{H}x{T} d={d} z_mean={zm} scale={scale} reference={reference} "
             f"state={with_state} no_norm={no_norm}")
    q, k, v, z = SI.draw(B, H, T, d, seed=70 + T, dtype=dtype, z_mean=zm)
    qd, kd, vd, zd = dev(q, k, v, z)
    kw = dict(variant=variant, scale=scale, reference_kernels=reference, no_norm=no_norm)
    n0 = None
    if with_state:
        S0d, n0d = initial_state(B, H, d, seed=T)
        kw.update(state_in=S0d, norm_in=n0d)
        n0 = host64(n0d)
    plain = tmb.fwd(qd, kd, vd, zd, **kw)
    out, stat = tmb.fwd(qd, kd, vd, zd, want_stats=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    qq, kk, _, zz = o64(q, k, v, z)
    if variant == "sq":
        ref = O.row_weight_sums(qq, kk, zz, scale=scale, state_in_norm=n0)
    else:
        ref = O.row_logsumexp(qq, kk, zz, scale=scale)
    e = relerr(host64(stat), ref)
    print(f"  stat err {e:.2e}")
    assert e < TOL[dtype]


BWD_CASES = [
    # variant, dtype, B, H, T, d, z_mean, scale, no_norm
    ("sq", "bf16", 2, 2, 200, 64, -6.0, 1.0, False),
    ("sq", "bf16", 1, 2, 1000, 64, -3.0, 0.8, False),
    ("sq", "bf16", 1, 2, 129, 64, 0.0, 1.0, True),
    ("sq", "f32", 1, 2, 130, 64, -4.0, 0.8, False),
    ("exp", "bf16", 2, 2, 200, 64, -3.0, 1.0, False),
    ("exp", "bf16", 1, 8, 257, 64, -1.0, 0.7, False),
    ("exp", "f32", 1, 2, 150, 16, 0.0, 1.0, False),
]


def _dout(B, H, T, d, dtype, seed):
    t = torch.from_numpy(np.random.default_rng(seed + 500).standard_normal((B, H, T, d)))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


@pytest.mark.parametrize("variant,dtype,B,H,T,d,zm,scale,no_norm", BWD_CASES)
@pytest.mark.parametrize("reference", [True, False])
def test_backward_with_forward_statistics(variant, dtype, B, H, T, d, zm, scale, no_norm, reference):
    announce(f"bwd with stats {variant} {dtype} {B}x{H}x{T} d={d} z_mean={zm} scale={scale} no_norm={no_norm} "
             f"reference={reference}")
    q, k, v, z = SI.draw(B, H, T, d, seed=80 + T, dtype=dtype, z_mean=zm)
    do = _dout(B, H, T, d, dtype, 80)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    kw = dict(variant=variant, scale=scale, no_norm=no_norm, reference_kernels=reference)
    out, stat = tmb.fwd(qd, kd, vd, zd, want_stats=True, **kw)
    g = tmb.bwd(qd, kd, vd, zd, out, dod, row_stat=stat, **kw)
    torch.cuda.synchronize()
    qq, kk, vv, zz, dd = o64(q, k, v, z, do)
    if variant == "sq":
        ref = O.bwd_quadratic(qq, kk, vv, zz, dd, scale=scale, norm=not no_norm)
    else:
        ref = O.bwd_exp_quadratic(qq, kk, vv, zz, dd, scale=scale)
    for name, a, r in zip(("dq", "dk", "dv", "dz"), g, ref):
        e = relerr(host64(a), r)
        print(f"  {name} {e:.2e}")
        assert e < TOL[dtype], f"{name} error {e:.3e}"


@pytest.mark.parametrize("variant", ["sq", "exp"])
def test_full_size_statistics_and_backward(variant):
    B, H, T, d = 2, 16, 8192, 64
    announce(f"fwd stats + bwd {variant} full size {B}x{H}x{T}")
    q, k, v, z = SI.draw(B, H, T, d, seed=3, dtype="bf16")
    do = _dout(B, H, T, d, "bf16", 3)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    out, stat = tmb.fwd(qd, kd, vd, zd, variant=variant, want_stats=True)
    g = tmb.bwd(qd, kd, vd, zd, out, dod, variant=variant, row_stat=stat)
    torch.cuda.synchronize()
    # sampled rows of the statistic on every head: both ends, chunk and
    # segment boundaries, the ragged middle
    rows = [0, 1, 63, 64, 1000, 4095, 4096, 8190, 8191]
    qq, kk, zz = o64(q, k, z)
    if variant == "sq":
        ref = O.row_weight_sums(qq, kk, zz, rows=rows)
    else:
        ref = O.row_logsumexp(qq, kk, zz, rows=rows)
    e = relerr(host64(stat)[:, :, rows], ref)
    print(f"  stat err {e:.2e}")
    assert e < TOL["bf16"]
    got = [host64(x) for x in g]
    for b, h in [(0, 3), (1, 12)]:
        sl = lambda t: SI.to_f64(t[b:b + 1, h:h + 1])
        gref = O.bwd_blocked(sl(q), sl(k), sl(v), sl(z), sl(do), variant=variant)
        for name, a, r in zip(("dq", "dk", "dv", "dz"), got, gref):
            e = relerr(a[b:b + 1, h:h + 1], r)
            print(f"  head ({b},{h}) {name} {e:.2e}")
            assert e < TOL["bf16"], f"{name} error {e:.3e}"
