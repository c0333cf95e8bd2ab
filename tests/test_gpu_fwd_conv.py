"""GPU parity of twomamba_fwd_conv, the forward with the size-2 input
convolution in front ("2Mamba2Furious", §3-§4, App. A).

* bit-identical to twomamba_conv2 followed by twomamba_fwd on every path
  (2Mamba and first order MFMA, 2Mamba-E MFMA, the fp32 reference kernels),
  ragged token counts, with and without a cached raw row and a bias;
* against the fp64 oracle (its conv2, then its forward forms) at small ragged
  sizes, and on sampled rows of the B=2 H=16 T=8192 bf16 workload;
* a prompt split in two, carried through the convolution cache and the state,
  equals the whole prompt.
Tolerances: per-head inf-norm relative error <= 2e-2 (bf16), 1e-4 (fp32).
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu

ORACLE_FWD = {"sq": O.fwd_quadratic, "exp": O.fwd_exp_quadratic, "lin": O.fwd_linear_quadratic}


def conv_params(B, H, d, dtype, seed, bias=True, prev=True):
    r = np.random.default_rng(seed)
    w = torch.from_numpy((0.5 + 0.5 * r.standard_normal((3, H, d, 2))).astype(np.float32))
    b = torch.from_numpy((0.1 * r.standard_normal((3, H, d))).astype(np.float32)) if bias else None
    p = torch.from_numpy((r.standard_normal((B, H, 3, d)) / np.sqrt(d)).astype(np.float32)).to(
        SI.torch_dtype(dtype)) if prev else None
    return w, b, p


def oracle_conv(q, k, v, w, b, p):
    """The oracle's conv2 of each tensor (from the library's [3][H][d][2] layout),
    rounded to the input dtype: the operation defines the convolved values as
    rounded to it before the operator uses them (with a bias the outputs can be
    ill-conditioned in q', so the unrounded values would not be the reference)."""
    outs = []
    for i, x in enumerate((q, k, v)):
        y = O.conv2(SI.to_f64(x), SI.to_f64(w[i]), None if b is None else SI.to_f64(b[i]),
                    None if p is None else SI.to_f64(p[:, :, i]))
        outs.append(torch.from_numpy(y).to(x.dtype).to(torch.float64).numpy())
    return outs


CASES = [("sq", "bf16", 64), ("exp", "bf16", 64), ("lin", "bf16", 64),
         ("sq", "f32", 16), ("exp", "f32", 16), ("lin", "f32", 64)]


@pytest.mark.parametrize("variant,dtype,d", CASES)
@pytest.mark.parametrize("T", [1, 65, 300])
@pytest.mark.parametrize("bias_prev", [(False, False), (True, True)])
def test_fwd_conv_bit_identical_to_conv_then_fwd(variant, dtype, d, T, bias_prev):
    announce(f"fwd_conv == conv2 + fwd: {variant} {dtype} d={d} T={T} bias/prev={bias_prev}")
    B, H = 2, 3
    q, k, v, z = dev(*SI.draw(B, H, T, d, seed=500 + T, dtype=dtype, z_mean=-6.0))
    w, b, p = (x.cuda() if x is not None else None for x in conv_params(B, H, d, dtype, 501, *bias_prev))
    kw = dict(want_state=True) if variant != "exp" else {}
    got = tmb.fwd_conv(q, k, v, z, w, b, p, variant=variant, want_conv_state=True, **kw)
    qc, kc, vc, cs = tmb.conv2(q, k, v, w, b, p, want_state=True)
    ref = tmb.fwd(qc, kc, vc, z, variant=variant, **kw)
    torch.cuda.synchronize()
    got = got if isinstance(got, tuple) else (got,)
    ref = (ref if isinstance(ref, tuple) else (ref,)) + (cs,)
    for i, (a, r) in enumerate(zip(got, ref)):
        assert (a is None and r is None) or torch.equal(a, r), f"result {i} differs"


@pytest.mark.parametrize("variant,dtype,d", CASES)
@pytest.mark.parametrize("T", [1, 63, 200])
def test_fwd_conv_matches_oracle(variant, dtype, d, T):
    announce(f"fwd_conv vs oracle: {variant} {dtype} d={d} T={T}")
    B, H = 1, 2
    q, k, v, z = SI.draw(B, H, T, d, seed=510 + T, dtype=dtype, z_mean=-6.0)
    w, b, p = conv_params(B, H, d, dtype, 511)
    out = tmb.fwd_conv(*dev(q, k, v, z), w.cuda(), b.cuda(), p.cuda(), variant=variant)
    torch.cuda.synchronize()
    qq, kk, vv = oracle_conv(q, k, v, w, b, p)
    ref = ORACLE_FWD[variant](qq, kk, vv, SI.to_f64(z))
    e = relerr(host64(out), ref)
    print(f"  err {e:.2e}")
    assert e < TOL[dtype]


@pytest.mark.parametrize("variant", ["sq", "exp", "lin"])
def test_fwd_conv_full_size_sampled_rows(variant):
    B, H, T, d = 2, 16, 8192, 64
    announce(f"fwd_conv bf16 {B}x{H}x{T} {variant}, sampled rows")
    q, k, v, z = SI.draw(B, H, T, d, seed=3, dtype="bf16", z_mean=-8.0)
    w, b, p = conv_params(B, H, d, "bf16", 520)
    qd, kd, vd, zd = dev(q, k, v, z)
    out = tmb.fwd_conv(qd, kd, vd, zd, w.cuda(), b.cuda(), p.cuda(), variant=variant)
    qc, kc, vc = tmb.conv2(qd, kd, vd, w.cuda(), b.cuda(), p.cuda())
    assert torch.equal(out, tmb.fwd(qc, kc, vc, zd, variant=variant))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 2047, 2048, 4095, 4096, 8191]
    qq, kk, vv = oracle_conv(q, k, v, w, b, p)
    zz = SI.to_f64(z)
    if variant == "sq":
        ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows)
    elif variant == "exp":
        ref = O.fwd_exp_quadratic_rows(qq, kk, vv, zz, rows)
    else:
        ref = np.stack([O.fwd_linear_quadratic(qq[:, :, :r + 1], kk[:, :, :r + 1], vv[:, :, :r + 1],
                                               zz[:, :, :r + 1])[:, :, r] for r in rows[:6]], axis=2)
        rows = rows[:6]
    e = relerr(host64(out)[:, :, rows], ref)
    print(f"  rows err {e:.2e}")
    assert e < TOL["bf16"]


@pytest.mark.parametrize("variant,dtype,d", [("sq", "bf16", 64), ("lin", "bf16", 64), ("sq", "f32", 16)])
def test_prompt_split_through_the_convolution_cache(variant, dtype, d):
    announce(f"fwd_conv split prompt {variant} {dtype} d={d}")
    B, H, T, T1 = 1, 2, 700, 257
    q, k, v, z = dev(*SI.draw(B, H, T, d, seed=530, dtype=dtype, z_mean=-8.0))
    w, b, _ = (x.cuda() if x is not None else None for x in conv_params(B, H, d, dtype, 531, prev=False))
    full = tmb.fwd_conv(q, k, v, z, w, b, variant=variant, want_state=True)
    sl = lambda x, a, c: x[:, :, a:c].contiguous()
    o1, S1, n1, c1 = tmb.fwd_conv(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(z, 0, T1), w, b, variant=variant,
                                  want_state=True, want_conv_state=True)
    o2, S2, n2 = tmb.fwd_conv(sl(q, T1, T), sl(k, T1, T), sl(v, T1, T), sl(z, T1, T), w, b, c1, variant=variant,
                              state_in=S1, norm_in=n1, want_state=True)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert relerr(host64(torch.cat([o1, o2], 2)), host64(full[0])) < tol
    assert relerr(host64(S2), host64(full[1])) < tol
    # the cache holds the raw rows of the first part's last token
    assert torch.equal(c1, torch.stack([q[:, :, T1 - 1], k[:, :, T1 - 1], v[:, :, T1 - 1]], dim=2))
