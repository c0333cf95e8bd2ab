"""GPU parity of 2Mamba-E decoding over a key/value cache against the fp64 oracle.

A prompt of T0 tokens goes into the caches (twomamba_exp_cache_fill), then N
tokens are decoded one at a time (twomamba_exp_step).  Every decoded output is
compared with the oracle's quadratic 2Mamba-E form evaluated on the whole
sequence (prompt + decoded tokens) at that row; the E quadratic and streaming
forms are pinned to each other and to causal softmax by the oracle tests.  The
caches are checked too: key/value rows bit-exact, G against the oracle's running
sum of softplus(z) (= -sum of g).

Tolerance: per-head inf-norm relative error <= 2e-2 (bf16), <= 1e-4 (fp32).
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from oracle import twomamba_oracle as O
from gpu_util import TOL, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def run_decode(B, H, d, T0, N, dtype, zm=0.0, scale=1.0, max_len=None, seed=7):
    """Returns (per-step outputs [B,H,N,d] float64, the full inputs, the caches)."""
    T = T0 + N
    max_len = max_len or T
    q, k, v, z = SI.draw(B, H, T, d, seed=seed, dtype=dtype, z_mean=zm)
    qd, kd, vd, zd = dev(q, k, v, z)
    kc, vc, gc = tmb.exp_cache(B, H, d, max_len, dtype=qd.dtype)
    if T0 > 0:
        tmb.exp_cache_fill(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), zd[:, :, :T0].contiguous(),
                           kc, vc, gc)
    outs = []
    for i in range(N):
        t = T0 + i
        o = tmb.exp_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                         zd[:, :, t].contiguous(), kc, vc, gc, t, scale=scale)
        outs.append(o)
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=2)
    return got, (q, k, v, z), (kc, vc, gc)


CASES = [
    # B, H, d, T0, N, dtype, z_mean
    (1, 2, 64, 0, 40, "bf16", 0.0),        # from an empty cache
    (2, 3, 64, 1000, 40, "bf16", -6.0),    # crosses the 1024-key split boundary
    (1, 2, 64, 511, 4, "bf16", -10.0),     # 512-key split boundary, weak decay
    (1, 2, 16, 300, 20, "f32", -4.0),      # d = 16, fp32
    (1, 1, 64, 2047, 3, "f32", -8.0),      # fp32, long
]


@pytest.mark.parametrize("B,H,d,T0,N,dtype,zm", CASES)
def test_exp_decode_matches_oracle(B, H, d, T0, N, dtype, zm):
    announce(f"E decode B={B} H={H} d={d} T0={T0} N={N} {dtype} z_mean={zm}")
    got, (q, k, v, z), (kc, vc, gc) = run_decode(B, H, d, T0, N, dtype, zm=zm, scale=0.9)
    qq, kk, vv, zz = (SI.to_f64(t) for t in (q, k, v, z))
    ref = O.fwd_exp_quadratic_rows(qq, kk, vv, zz, list(range(T0, T0 + N)), scale=0.9)
    e = relerr(got, ref)
    print(f"  out err {e:.2e}")
    assert e < TOL[dtype]
    # caches: rows 0..T-1 hold the keys / values, g the running softplus sums
    T = T0 + N
    assert torch.equal(kc[:, :, :T].cpu(), k) and torch.equal(vc[:, :, :T].cpu(), v)
    g_ref = -np.cumsum(O.decay_log(zz), axis=-1)
    g_got = host64(gc[:, :, :T])
    assert np.max(np.abs(g_got - g_ref) / np.maximum(1.0, np.abs(g_ref))) < 1e-12


def test_exp_decode_no_decay_is_softmax_attention():
    announce("E decode with z = -inf vs torch causal SDPA on the full sequence")
    B, H, d, T0, N = 1, 2, 64, 200, 8
    q, k, v, z = SI.draw(B, H, T0 + N, d, seed=17, dtype="bf16", z_neg_inf=True)
    qd, kd, vd, zd = dev(q, k, v, z)
    kc, vc, gc = tmb.exp_cache(B, H, d, T0 + N)
    tmb.exp_cache_fill(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), zd[:, :, :T0].contiguous(), kc, vc, gc)
    outs = [tmb.exp_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                         zd[:, :, t].contiguous(), kc, vc, gc, t) for t in range(T0, T0 + N)]
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=2)
    ref = torch.nn.functional.scaled_dot_product_attention(q.float(), k.float(), v.float(), is_causal=True,
                                                         scale=1.0)
    assert relerr(got, ref[:, :, T0:].double().numpy()) < TOL["bf16"]


def test_exp_decode_bench_shape_sampled_heads():
    # the benchmark shape: 64 x 32 heads, 2048-token prompt, a few decode steps;
    # the oracle follows three heads
    B, H, d, T0, N = 64, 32, 64, 2048, 3
    announce(f"E decode bench shape B={B} H={H} T0={T0} N={N}")
    got, (q, k, v, z), _ = run_decode(B, H, d, T0, N, "bf16", max_len=T0 + 64, seed=4)
    for b, h in [(0, 0), (31, 17), (63, 31)]:
        qq, kk, vv, zz = (SI.to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v, z))
        ref = O.fwd_exp_quadratic_rows(qq, kk, vv, zz, list(range(T0, T0 + N)))
        e = relerr(got[b:b + 1, h:h + 1], ref)
        print(f"  head ({b},{h}) err {e:.2e}")
        assert e < TOL["bf16"]


def test_exp_decode_deterministic():
    announce("E decode bitwise determinism")
    a, _, _ = run_decode(2, 2, 64, 700, 5, "bf16", seed=23)
    b, _, _ = run_decode(2, 2, 64, 700, 5, "bf16", seed=23)
    assert np.array_equal(a, b)
