"""GPU parity of the MFMA 2Mamba forward (bf16 inputs, d = 64) against the fp64 oracle.

Cases span several 64-token chunks with ragged tails, the multi-segment path
(few heads and long sequences are split into segments chained by a scan), the
weak-decay regimes where the carried state dominates, a carried initial state,
the unnormalised numerator and the query scale.  Tolerance: per-head inf-norm
relative error <= 2e-2 (bf16 inputs, fp32 accumulation), for outputs and for the
final state and normaliser.
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


def oracle_state(B, H, d, seed, z_mean):
    _, k0, v0, z0 = SI.draw(B, H, 48, d, seed=seed, dtype="f32", z_mean=z_mean)
    S0, n0 = O.final_state_direct(SI.to_f64(k0), SI.to_f64(v0), SI.to_f64(z0))
    S0 = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    n0 = torch.from_numpy(np.ascontiguousarray(n0, dtype=np.float32)).cuda()
    return S0, n0


CASES = [
    # B, H, T, z_mean, z_neg_inf
    (1, 2, 64, 0.0, False),
    (2, 3, 200, 0.0, False),
    (1, 2, 1000, -6.0, False),     # 4 segments, ragged tail
    (1, 1, 1024, -10.0, False),    # 4 segments, slow decay: the carry matters
    (2, 1, 333, 0.0, True),        # no decay at all
    (1, 2, 1, 0.0, False),         # single token
    (1, 2, 1000, 20.0, False),     # very strong decay: the carry vanishes every chunk
]


@pytest.mark.parametrize("B,H,T,zm,zinf", CASES)
@pytest.mark.parametrize("with_state", [False, True])
def test_mfma_sq_matches_oracle(B, H, T, zm, zinf, with_state):
    announce(f"MFMA SQ B={B} H={H} T={T} z_mean={zm} ninf={zinf} state={with_state}")
    d = 64
    q, k, v, z = SI.draw(B, H, T, d, seed=100 + T, dtype="bf16", z_mean=zm, z_neg_inf=zinf)
    kw, S0, n0 = {}, None, None
    if with_state:
        S0d, n0d = oracle_state(B, H, d, seed=T, z_mean=zm)
        kw = dict(state_in=S0d, norm_in=n0d)
        S0, n0 = host64(S0d), host64(n0d)
    out, S, n = tmb.fwd(*dev(q, k, v, z), want_state=True, **kw)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    ref = O.fwd_quadratic(qq, kk, vv, zz, state_in=S0, norm_in=n0)
    S_ref, n_ref = O.final_state_direct(kk, vv, zz, state_in=S0, norm_in=n0)
    e_out, e_s, e_n = relerr(host64(out), ref), relerr(host64(S), S_ref), relerr(host64(n), n_ref)
    print(f"  err out {e_out:.2e} state {e_s:.2e} norm {e_n:.2e}")
    assert e_out < TOL["bf16"]
    assert e_s < TOL["bf16"] and e_n < TOL["bf16"]


def test_mfma_sq_no_norm_and_scale():
    announce("MFMA SQ NO_NORM, scale 0.5")
    q, k, v, z = SI.draw(1, 2, 300, 64, seed=5, dtype="bf16", z_mean=-4.0)
    out = tmb.fwd(*dev(q, k, v, z), no_norm=True, scale=0.5)
    torch.cuda.synchronize()
    ref = O.fwd_quadratic(*o64(q, k, v, z), scale=0.5, norm=False)
    assert relerr(host64(out), ref) < TOL["bf16"]


def test_mfma_sq_large_magnitudes():
    # inputs far from unit scale exercise the per-chunk power-of-two scaling
    announce("MFMA SQ q*300, k/500, v*1e4")
    q, k, v, z = SI.draw(1, 2, 260, 64, seed=6, dtype="f32", z_mean=-5.0)
    q, k, v = (q * 300).bfloat16(), (k / 500).bfloat16(), (v * 1e4).bfloat16()
    out, S, n = tmb.fwd(*dev(q, k, v, z), want_state=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    assert relerr(host64(out), O.fwd_quadratic(qq, kk, vv, zz)) < TOL["bf16"]
    S_ref, n_ref = O.final_state_direct(kk, vv, zz)
    assert relerr(host64(S), S_ref) < TOL["bf16"] and relerr(host64(n), n_ref) < TOL["bf16"]


def test_mfma_matches_reference_kernels():
    # the two HIP paths agree with each other on a mid-size multi-segment case
    announce("MFMA SQ vs reference kernels, B=2 H=2 T=2048")
    q, k, v, z = dev(*SI.draw(2, 2, 2048, 64, seed=8, dtype="bf16", z_mean=-7.0))
    a, Sa, na = tmb.fwd(q, k, v, z, want_state=True)
    b, Sb, nb = tmb.fwd(q, k, v, z, want_state=True, reference_kernels=True)
    torch.cuda.synchronize()
    assert relerr(host64(a), host64(b)) < TOL["bf16"]
    assert relerr(host64(Sa), host64(Sb)) < TOL["bf16"]


def test_mfma_split_resume():
    announce("MFMA SQ split/resume T=700 = 300 + 400")
    q, k, v, z = dev(*SI.draw(1, 2, 700, 64, seed=9, dtype="bf16", z_mean=-8.0))
    full, Sf, nf = tmb.fwd(q, k, v, z, want_state=True)
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, S1, n1 = tmb.fwd(sl(q, 0, 300), sl(k, 0, 300), sl(v, 0, 300), sl(z, 0, 300), want_state=True)
    o2, S2, n2 = tmb.fwd(sl(q, 300, 700), sl(k, 300, 700), sl(v, 300, 700), sl(z, 300, 700),
                         state_in=S1, norm_in=n1, want_state=True)
    torch.cuda.synchronize()
    assert relerr(host64(torch.cat([o1, o2], 2)), host64(full)) < TOL["bf16"]
    assert relerr(host64(S2), host64(Sf)) < TOL["bf16"]


def test_mfma_deterministic():
    announce("MFMA SQ bitwise determinism")
    q, k, v, z = dev(*SI.draw(2, 2, 777, 64, seed=10, dtype="bf16", z_mean=-3.0))
    a = tmb.fwd(q, k, v, z, want_state=True)
    b = tmb.fwd(q, k, v, z, want_state=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,H,T,with_state", [
    (1, 1, 16384, False),      # 64 segments of 4 chunks: the carries go through the segment scan
    (1, 2, 6000 - 37, True),   # 19 segments, ragged last chunk, caller state folded into the first
    (1, 1, 32768, False),      # 126 segment-pass pieces of 4 chunks (two per segment), scanned
    (2, 16, 2048 - 37, True),  # 4 segments of 8 chunks, pieces of 6 crossing them, caller state
])
def test_mfma_sq_many_segments(B, H, T, with_state):
    # few heads and a long sequence split into many segments, with slow decay so
    # that every carry matters; sampled rows against the oracle, and the final state
    announce(f"MFMA SQ many segments B={B} H={H} T={T} state={with_state}")
    d = 64
    q, k, v, z = SI.draw(B, H, T, d, seed=110, dtype="bf16", z_mean=-10.0)
    kw, S0, n0 = {}, None, None
    if with_state:
        S0d, n0d = oracle_state(B, H, d, seed=111, z_mean=-10.0)
        kw = dict(state_in=S0d, norm_in=n0d)
        S0, n0 = host64(S0d), host64(n0d)
    out, S, n = tmb.fwd(*dev(q, k, v, z), want_state=True, **kw)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    rows = sorted({0, 1, 255, 256, 257, 1023, 1024, T // 3, T // 2, T - 300, T - 65, T - 64, T - 1})
    ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows, state_in=S0, norm_in=n0)
    e = relerr(host64(out)[:, :, rows], ref)
    S_ref, n_ref = O.final_state_direct(kk, vv, zz, state_in=S0, norm_in=n0)
    es, en = relerr(host64(S), S_ref), relerr(host64(n), n_ref)
    print(f"  rows err {e:.2e} state {es:.2e} norm {en:.2e}")
    assert e < TOL["bf16"] and es < TOL["bf16"] and en < TOL["bf16"]


@pytest.mark.parametrize("B,H,T", [
    (1, 1, 4096),   # 16 segments: carries through the segment scan
    (1, 4, 2048),   # 8 segments: carries summed in the main kernel's prologue
    (2, 16, 4096),  # 4 segments, 4 segment-pass pieces crossing them: 6 end states per head
])
@pytest.mark.parametrize("mode", ["blocks", "huge", "tiny", "zero_then_tiny"])
def test_mfma_sq_carry_magnitudes(B, H, T, mode):
    # The segment end states are stored as fp16 with one power-of-two scale per
    # slot.  Values far from unit scale, and slots whose magnitudes differ by up
    # to 2^60 from one segment to the next, must come through the slots and the
    # scan without overflow or loss.  Slow decay, so that every carry matters.
    announce(f"MFMA SQ carry magnitudes B={B} H={H} T={T} mode={mode}")
    d = 64
    q, k, v, z = SI.draw(B, H, T, d, seed=120, dtype="f32", z_mean=-10.0)
    if mode == "blocks":
        # v scaled by 2^u per 256-token block, u in [-30, 30]
        u = np.random.default_rng(121).integers(-30, 31, size=(T + 255) // 256)
        f = torch.from_numpy(np.repeat(2.0 ** u, 256)[:T].astype(np.float32))
        v = v * f[None, None, :, None]
    elif mode == "huge":
        v = v * 1e20
    elif mode == "tiny":
        k, v = k * 1e-6, v * 1e-20
    else:
        # a quarter of the sequence with k = 0 (all-zero segment states), the rest
        # tiny: the zero slots must not swamp the scaling of the tiny carries
        k = k.clone()
        k[:, :, : T // 4] = 0
        v = v * 1e-20
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    out, S, n = tmb.fwd(*dev(q, k, v, z), want_state=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    rows = sorted({0, 255, 256, 511, 1023, 1024, T // 2 + 7, T - 257, T - 1})
    ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows)
    got = host64(out)[:, :, rows]
    assert np.isfinite(got).all()
    e = relerr(got, ref)
    S_ref, n_ref = O.final_state_direct(kk, vv, zz)
    es, en = relerr(host64(S), S_ref), relerr(host64(n), n_ref)
    print(f"  rows err {e:.2e} state {es:.2e} norm {en:.2e}")
    assert e < TOL["bf16"] and es < TOL["bf16"] and en < TOL["bf16"]


@pytest.mark.parametrize("B,H,T", [(1, 2, 1000), (1, 1, 4096)])
def test_mfma_sq_decay_resets(B, H, T):
    # no decay at all except a near-total reset (g about -50) every 97 tokens:
    # the accumulators restart inside chunks, segments and across the scan
    announce(f"MFMA SQ decay resets B={B} H={H} T={T}")
    q, k, v, z = SI.draw(B, H, T, 64, seed=130, dtype="bf16")
    z = torch.full_like(z, float("-inf"))
    z[:, :, ::97] = 50.0
    out, S, n = tmb.fwd(*dev(q, k, v, z), want_state=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    rows = sorted({0, 1, 96, 97, 98, 500, T // 2, T - 98, T - 97, T - 2, T - 1})
    ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows)
    e = relerr(host64(out)[:, :, rows], ref)
    S_ref, n_ref = O.final_state_direct(kk, vv, zz)
    es, en = relerr(host64(S), S_ref), relerr(host64(n), n_ref)
    print(f"  rows err {e:.2e} state {es:.2e} norm {en:.2e}")
    assert e < TOL["bf16"] and es < TOL["bf16"] and en < TOL["bf16"]


@pytest.mark.parametrize("no_norm", [False, True])
def test_mfma_sq_small_query_rows(no_norm):
    # Every 7th query is 1000x smaller than the rest, with weak decay, so that the
    # carried state dominates.  A normalised output does not depend on its query's
    # size, so those rows must be as accurate as the others (their products q_i q_j
    # would sit in the fp16 subnormals under a chunk-wide query scale); without
    # normalisation, and for the row statistic, they are compared on their own scale.
    announce(f"MFMA SQ small query rows no_norm={no_norm}")
    B, H, T = 1, 2, 1000
    q, k, v, z = SI.draw(B, H, T, 64, seed=140, dtype="f32", z_mean=-10.0)
    q = q.clone()
    q[:, :, ::7] *= 1e-3
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    out, st = tmb.fwd(*dev(q, k, v, z), no_norm=no_norm, want_stats=True)
    torch.cuda.synchronize()
    qq, kk, vv, zz = o64(q, k, v, z)
    rows = list(range(0, T, 7))
    ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows, norm=not no_norm)
    e = relerr(host64(out)[:, :, rows], ref)
    den_ref = O.row_weight_sums(qq, kk, zz, rows=rows)
    es = relerr(host64(st)[:, :, rows], den_ref)
    print(f"  small rows err {e:.2e} statistic {es:.2e}")
    assert e < TOL["bf16"] and es < TOL["bf16"]


# one segment per head; four segments per head; four segments and segment-pass pieces
@pytest.mark.parametrize("B,H,T", [(1, 2, 300), (1, 2, 1000), (2, 16, 2048)])
def test_mfma_sq_in_place_resume(B, H, T):
    # state_out == state_in and norm_out == norm_in (exact alias, in-place resume): the
    # result must equal the call with separate output buffers, bit for bit, and the oracle.
    announce(f"MFMA SQ in-place resume B={B} H={H} T={T}")
    q, k, v, z = SI.draw(B, H, T, 64, seed=11 + T, dtype="bf16", z_mean=-8.0)
    S0d, n0d = oracle_state(B, H, 64, seed=12, z_mean=-8.0)
    qd, kd, vd, zd = dev(q, k, v, z)
    o_sep, S_sep, n_sep = tmb.fwd(qd, kd, vd, zd, state_in=S0d, norm_in=n0d, want_state=True)
    S, n = S0d.clone(), n0d.clone()
    o_alias, S_a, n_a = tmb.fwd(qd, kd, vd, zd, state_in=S, norm_in=n, state_out=S, norm_out=n, want_state=True)
    torch.cuda.synchronize()
    assert S_a.data_ptr() == S.data_ptr() and n_a.data_ptr() == n.data_ptr()
    assert torch.equal(o_alias, o_sep) and torch.equal(S, S_sep) and torch.equal(n, n_sep)
    qq, kk, vv, zz = o64(q, k, v, z)
    S0, n0 = host64(S0d), host64(n0d)
    if B * H <= 4:
        assert relerr(host64(o_alias), O.fwd_quadratic(qq, kk, vv, zz, state_in=S0, norm_in=n0)) < TOL["bf16"]
    else:   # rows at chunk, piece and segment boundaries
        rows = sorted({0, 1, 383, 384, 511, 512, 767, 768, 1023, 1024, 1151, 1152, 1535, 1536, T - 1})
        ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows, state_in=S0, norm_in=n0)
        assert relerr(host64(o_alias)[:, :, rows], ref) < TOL["bf16"]
    S_ref, n_ref = O.final_state_direct(kk, vv, zz, state_in=S0, norm_in=n0)
    assert relerr(host64(S), S_ref) < TOL["bf16"] and relerr(host64(n), n_ref) < TOL["bf16"]
