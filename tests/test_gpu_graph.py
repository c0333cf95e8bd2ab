"""HIP graph capture of the entry points.

The library allocates nothing, issues no memset and never synchronises, so a
sequence of calls can be captured on the caller's stream and replayed.  Each
captured graph here is replayed several times, with eager work and
synchronisations between the replays, and every replay is compared bit for bit
with the same calls made eagerly (the kernels are deterministic):

  * a run of 2Mamba decode steps on a prefilled state (state updated in place);
  * a 2Mamba forward with row statistics followed by its backward (MFMA
    kernels, caller-owned workspaces);
  * a run of 2Mamba-E decode steps over a key/value cache (positions fixed at
    capture).
"""

import numpy as np
import pytest
import torch

import second_order_ssm_amd as tmb
import synth_inputs as SI
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _eager_noise():
    # unrelated eager work between replays, on the same stream
    x = torch.randn(4096, device="cuda")
    return float((x * x).sum())


def test_graph_decode_steps():
    B, H, d, T0, N = 4, 4, 64, 100, 8
    announce(f"graph: {N} 2Mamba decode steps {B}x{H} d={d}")
    q, k, v, z = SI.draw(B, H, T0 + N, d, seed=91, dtype="bf16", z_mean=-2.0)
    qd, kd, vd, zd = dev(q, k, v, z)
    pre = [x[:, :, :T0].contiguous() for x in (qd, kd, vd, zd)]
    _, S0, n0 = tmb.fwd(*pre, want_state=True)
    steps = [tuple(x[:, :, t].contiguous() for x in (qd, kd, vd, zd)) for t in range(T0, T0 + N)]
    Se, ne = S0.clone(), n0.clone()
    outs_e = [tmb.step(*a, Se, ne) for a in steps]
    torch.cuda.synchronize()

    Sg, ng = S0.clone(), n0.clone()
    outs_g = [torch.empty_like(o) for o in outs_e]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for a, o in zip(steps, outs_g):
            tmb.step(*a, Sg, ng, out=o)
    for _ in range(REPLAYS):
        Sg.copy_(S0)
        ng.copy_(n0)
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        for oe, og in zip(outs_e, outs_g):
            assert torch.equal(oe, og)
        assert torch.equal(Sg, Se) and torch.equal(ng, ne)


@pytest.mark.parametrize("variant", ["sq", "exp"])
def test_graph_forward_and_backward(variant):
    B, H, T, d = 2, 4, 700, 64
    announce(f"graph: {variant} forward with statistics + backward {B}x{H}x{T}")
    q, k, v, z = SI.draw(B, H, T, d, seed=92, dtype="bf16", z_mean=-1.0)
    do = torch.from_numpy(np.random.default_rng(93).standard_normal((B, H, T, d))).to(torch.bfloat16)
    qd, kd, vd, zd, dod = dev(q, k, v, z, do)
    desc = tmb.make_desc(B, H, T, d, d, variant=variant, dtype=torch.bfloat16)
    ws = torch.empty(max(tmb.workspace_size(desc), 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(tmb.bwd_workspace_size(desc), 1), dtype=torch.uint8, device="cuda")

    out_e, st_e = tmb.fwd(qd, kd, vd, zd, variant=variant, want_stats=True, workspace=ws)
    g_e = tmb.bwd(qd, kd, vd, zd, out_e, dod, variant=variant, row_stat=st_e, workspace=wsb)
    torch.cuda.synchronize()

    out_g, st_g = torch.empty_like(out_e), torch.empty_like(st_e)
    g_g = tuple(torch.empty_like(x) for x in g_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tmb.fwd(qd, kd, vd, zd, variant=variant, out=out_g, row_stat=st_g, workspace=ws)
        tmb.bwd(qd, kd, vd, zd, out_g, dod, variant=variant, row_stat=st_g, grads=g_g, workspace=wsb)
    for _ in range(REPLAYS):
        for x in (out_g, st_g, *g_g):
            x.fill_(float("nan"))
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(st_g, st_e)
        for a, b in zip(g_g, g_e):
            assert torch.equal(a, b)


def test_graph_exp_decode_steps():
    B, H, d, T0, N, L = 4, 4, 64, 300, 6, 512
    announce(f"graph: {N} 2Mamba-E decode steps over a {T0}-token cache {B}x{H}")
    q, k, v, z = SI.draw(B, H, T0 + N, d, seed=94, dtype="bf16", z_mean=-1.0)
    qd, kd, vd, zd = dev(q, k, v, z)
    kc, vc, gc = tmb.exp_cache(B, H, d, L)
    tmb.exp_cache_fill(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), zd[:, :, :T0].contiguous(), kc, vc, gc)
    nws = max(tmb.exp_step_workspace_size(B, H, d, L, p) for p in range(T0, T0 + N))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    steps = [tuple(x[:, :, t].contiguous() for x in (qd, kd, vd, zd)) for t in range(T0, T0 + N)]
    outs_e = [tmb.exp_step(*a, kc, vc, gc, T0 + i, workspace=ws) for i, a in enumerate(steps)]
    torch.cuda.synchronize()
    cache_e = (kc.clone(), vc.clone(), gc.clone())

    outs_g = [torch.empty_like(o) for o in outs_e]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i, (a, o) in enumerate(zip(steps, outs_g)):
            tmb.exp_step(*a, kc, vc, gc, T0 + i, out=o, workspace=ws)
    for _ in range(REPLAYS):
        for o in outs_g:
            o.fill_(float("nan"))
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        for oe, og in zip(outs_e, outs_g):
            assert torch.equal(oe, og)
        # the steps rewrite rows T0.. with the same values
        for a, b in zip((kc, vc, gc), cache_e):
            assert torch.equal(a, b)
