"""Out-of-bounds canaries and run-to-run determinism on the GPU.

Canaries: every output buffer is a view into a larger allocation whose guard
words before and after it hold a fixed NaN bit pattern; after the call (ragged
token counts, several kernel paths) the guards must be bit-for-bit unchanged.
Key/value cache rows past the newest position, and the parts of the caches a
prompt fill does not cover, are checked the same way.

Determinism: each entry point runs ten times, interleaved with the other
entry points in changing orders, and every result must be bit-identical to
the first (no floating-point atomics anywhere in the library)."""

import math

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

G = 1024   # guard elements on each side (keeps 256-byte alignment for 2- and 4-byte types)
PAT = {torch.float32: (torch.int32, 0x7FC0BEEF), torch.bfloat16: (torch.int16, 0x7FC1),
       torch.float64: (torch.int64, 0x7FF8DEADBEEF0001)}


class Guarded:
    """A device view of `shape` with guard words on both sides."""

    def __init__(self, shape, dtype):
        self.n = math.prod(shape)
        self.buf = torch.empty(self.n + 2 * G, dtype=dtype, device="cuda")
        it, pat = PAT[dtype]
        self.ibuf = self.buf.view(it)
        self.ibuf.fill_(pat if pat < 2 ** (8 * self.ibuf.element_size() - 1) else pat - 2 ** (8 * self.ibuf.element_size()))
        self.ref = self.ibuf.clone()
        self.t = self.buf[G:G + self.n].view(shape)

    def intact(self):
        return torch.equal(self.ibuf[:G], self.ref[:G]) and torch.equal(self.ibuf[G + self.n:], self.ref[G + self.n:])


def _inputs(B, H, T, d, dtype, seed, zm=-6.0):
    return dev(*SI.draw(B, H, T, d, seed=seed, dtype=dtype, z_mean=zm))


FWD_CASES = [
    # variant, dtype, d, B, H, T
    ("sq", "bf16", 64, 1, 3, 1), ("sq", "bf16", 64, 1, 3, 65), ("sq", "bf16", 64, 1, 2, 1000),
    ("sq", "bf16", 64, 2, 1, 2085), ("sq", "f32", 16, 1, 2, 100), ("sq", "f32", 64, 1, 1, 70),
    ("exp", "bf16", 64, 1, 2, 300), ("exp", "f32", 16, 1, 2, 70),
    ("lin", "bf16", 64, 1, 2, 700), ("lin", "f32", 16, 1, 2, 77),
]


@pytest.mark.parametrize("variant,dtype,d,B,H,T", FWD_CASES)
def test_forward_writes_stay_in_bounds(variant, dtype, d, B, H, T):
    announce(f"canaries forward {variant} {dtype} d={d} {B}x{H}x{T}")
    td = SI.torch_dtype(dtype)
    q, k, v, z = _inputs(B, H, T, d, dtype, seed=400 + T)
    D = d if variant == "lin" else d * (d + 1) // 2
    out = Guarded((B, H, T, d), td)
    kw = {}
    so = no = rs = None
    if variant != "exp":
        so = Guarded((B, H, D, d), torch.float32)
        kw.update(state_out=so.t)
        if variant == "sq":
            no = Guarded((B, H, D), torch.float32)
            kw.update(norm_out=no.t)
    if variant != "lin":
        rs = Guarded((B, H, T), torch.float32)
        kw.update(row_stat=rs.t)
    tmb.fwd(q, k, v, z, variant=variant, out=out.t, **kw)
    torch.cuda.synchronize()
    for name, g in (("out", out), ("state_out", so), ("norm_out", no), ("row_stat", rs)):
        if g is not None:
            assert g.intact(), f"{name} guard overwritten"
    if variant == "sq":
        o2 = Guarded((B, H, T, d), td)
        tmb.fwd_noalloc(q, k, v, z, out=o2.t)
        torch.cuda.synchronize()
        assert o2.intact()


@pytest.mark.parametrize("dtype,d,T", [("bf16", 64, 77), ("f32", 16, 1), ("bf16", 16, 130)])
def test_convolution_writes_stay_in_bounds(dtype, d, T):
    announce(f"canaries conv2 {dtype} d={d} T={T}")
    td = SI.torch_dtype(dtype)
    B, H = 2, 3
    q, k, v, _ = _inputs(B, H, T, d, dtype, seed=410)
    r = np.random.default_rng(411)
    w = torch.from_numpy(r.standard_normal((3, H, d, 2)).astype(np.float32)).cuda()
    b = torch.from_numpy(r.standard_normal((3, H, d)).astype(np.float32)).cuda()
    outs = [Guarded((B, H, T, d), td) for _ in range(3)]
    st = Guarded((B, H, 3, d), td)
    tmb.conv2(q, k, v, w, b, outs=[o.t for o in outs], state_out=st.t)
    torch.cuda.synchronize()
    assert all(o.intact() for o in outs) and st.intact()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_writes_stay_in_bounds(dtype):
    announce(f"canaries decode steps {dtype}")
    td = SI.torch_dtype(dtype)
    B, H, d, T0 = 2, 3, 64, 40
    D = d * (d + 1) // 2
    q, k, v, z = _inputs(B, H, T0 + 6, d, dtype, seed=420)
    # 2Mamba decode: state and normaliser updated in place inside guards, output guarded
    S = Guarded((B, H, D, d), torch.float32)
    n = Guarded((B, H, D), torch.float32)
    S.t.zero_()
    n.t.zero_()
    cs = Guarded((B, H, 3, d), td)
    cs.t.zero_()
    wc = torch.ones((3, H, d, 2), dtype=torch.float32, device="cuda")
    for t in range(T0, T0 + 3):
        o = Guarded((B, H, d), td)
        tmb.step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), z[:, :, t].contiguous(),
                 S.t, n.t, out=o.t)
        o2 = Guarded((B, H, d), td)
        tmb.step_conv(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                      z[:, :, t].contiguous(), wc, None, cs.t, S.t, n.t, out=o2.t)
        torch.cuda.synchronize()
        assert o.intact() and o2.intact() and S.intact() and n.intact() and cs.intact()
    # first-order decode (B*H = 6: the second workgroup of four heads has two without a head)
    S1 = Guarded((B, H, d, d), torch.float32)
    S1.t.zero_()
    cs1 = Guarded((B, H, 3, d), td)
    cs1.t.zero_()
    for t in range(T0, T0 + 3):
        o = Guarded((B, H, d), td)
        tmb.step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), z[:, :, t].contiguous(),
                 S1.t, None, first_order=True, out=o.t)
        o2 = Guarded((B, H, d), td)
        tmb.step_conv(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                      z[:, :, t].contiguous(), wc, None, cs1.t, S1.t, None, first_order=True, out=o2.t)
        torch.cuda.synchronize()
        assert o.intact() and o2.intact() and S1.intact() and cs1.intact()
    # 2Mamba-E decode: cache rows past the newest position keep their pattern
    L = T0 + 8
    kc, vc, gc = Guarded((B, H, L, d), td), Guarded((B, H, L, d), td), Guarded((B, H, L), torch.float64)
    tmb.exp_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), z[:, :, :T0].contiguous(),
                       kc.t, vc.t, gc.t)
    for pos in range(T0, T0 + 4):
        o = Guarded((B, H, d), td)
        tmb.exp_step(q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous(),
                     z[:, :, pos].contiguous(), kc.t, vc.t, gc.t, pos, out=o.t)
        torch.cuda.synchronize()
        assert o.intact() and kc.intact() and vc.intact() and gc.intact()
        for c, it in ((kc, PAT[td][0]), (vc, PAT[td][0]), (gc, torch.int64)):
            tail = c.t[:, :, pos + 1:].contiguous().view(it)
            assert bool((tail == c.ref[G:G + 1][0]).all()), f"cache rows past {pos} written"


# "sq_chunked": 2Mamba's linear-in-T backward (TWOMAMBA_FLAG_CHUNKED_FORM)
@pytest.mark.parametrize("variant,dtype,d", [("sq", "bf16", 64), ("exp", "bf16", 64), ("lin", "bf16", 64),
                                             ("sq", "f32", 16), ("sq_chunked", "bf16", 64)])
def test_backward_writes_stay_in_bounds(variant, dtype, d):
    announce(f"canaries backward {variant} {dtype} d={d}")
    td = SI.torch_dtype(dtype)
    B, H, T = 1, 2, 130
    chunked = variant == "sq_chunked"
    variant = "sq" if chunked else variant
    q, k, v, z = _inputs(B, H, T, d, dtype, seed=430)
    out = tmb.fwd(q, k, v, z, variant=variant)
    do = torch.randn_like(out)
    gs = [Guarded((B, H, T, d), td) for _ in range(3)] + [Guarded((B, H, T), torch.float32)]
    tmb.bwd(q, k, v, z, out, do, variant=variant, chunked_form=chunked, grads=[g.t for g in gs])
    torch.cuda.synchronize()
    assert all(g.intact() for g in gs)


def test_bitwise_determinism_ten_runs_interleaved():
    announce("determinism: 10 runs, interleaved launch orders")
    q, k, v, z = _inputs(1, 2, 2085, 64, "bf16", seed=440, zm=-8.0)
    qf, kf, vf, zf = _inputs(1, 2, 300, 16, "f32", seed=441, zm=-4.0)
    S0 = torch.zeros((1, 2, 2080, 64), dtype=torch.float32, device="cuda")
    n0 = torch.zeros((1, 2, 2080), dtype=torch.float32, device="cuda")
    calls = {
        "sq": lambda: tmb.fwd(q, k, v, z, want_state=True, want_stats=True),
        "sq_ref": lambda: tmb.fwd(qf, kf, vf, zf, want_state=True),
        "exp": lambda: tmb.fwd(q, k, v, z, variant="exp", want_stats=True),
        "lin": lambda: tmb.fwd(q, k, v, z, variant="lin", want_state=True),
        "bwd": lambda: tmb.bwd(q, k, v, z, q, v, variant="sq"),
        "exp_bwd": lambda: tmb.bwd(q, k, v, z, q, v, variant="exp"),
        "sq_bwd_chunked": lambda: tmb.bwd(q, k, v, z, q, v, variant="sq", chunked_form=True),
        "step": lambda: (lambda S, n: (tmb.step(q[:, :, 7].contiguous().float(), k[:, :, 7].contiguous().float(),
                                                v[:, :, 7].contiguous().float(), z[:, :, 7].contiguous(), S, n),
                                       S, n))(S0.clone(), n0.clone()),
    }
    names = list(calls)
    first = {}
    rng = np.random.default_rng(442)
    for run in range(10):
        order = list(rng.permutation(names))
        for nm in order:
            res = calls[nm]()
            res = res if isinstance(res, tuple) else (res,)
            res = [r.clone() for r in res if r is not None]
            if run == 0:
                first[nm] = res
            else:
                for a, b in zip(first[nm], res):
                    assert torch.equal(a, b), f"{nm} differs in run {run} (order {order})"
        torch.cuda.synchronize()
