"""GPU parity of the MFMA 2Mamba forward across the branches of its launch plan.

How a call is laid out depends on the number of heads and the length: one
segment or several, the segment pre-pass cut into pieces or one piece per
segment, pieces that cross a segment boundary (two end states from one
workgroup), carries summed in the main kernel or scanned first, and a last
segment shorter than the others.  Each shape below is the smallest found that
reaches one combination of those branches (slow decay, z ~ N(-10, 1), so that
every carry matters).  Every head is compared with the plain fp32 reference
kernels on the GPU (an independent path, itself pinned to the oracle by
tests/test_gpu_parity.py), and the first and last heads with the fp64 oracle at
the rows on both sides of every chunk boundary, together with their final
state and normaliser.  Tolerance: per-head inf-norm relative error <= 2e-2.
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
    # B, H, T                     what the shape reaches
    (1, 1, 1),        # one token, one segment
    (1, 1, 511),      # two segments, one end state, ragged last chunk
    (2, 8, 3000),     # eight segments summed in the main kernel, last segment shorter
    (1, 1, 4097),     # thirteen segments, carries scanned, one-token last chunk
    (1, 1, 3000),     # ten segments scanned, last segment of two chunks
    (4, 16, 1000),    # two segments, the pre-pass cut into pieces that end on chunk boundaries
    (4, 16, 3000),    # two segments, pieces, last segment one chunk shorter
    (2, 16, 1500),    # four segments, pieces crossing segment boundaries (six end states)
    (2, 16, 3000),    # the same with a shorter last segment
    (1, 5, 6000),     # nineteen segments, pieces crossing them, 36 end states scanned
]


def _rows(T):
    rows = {0, T - 1}
    for c in range(64, T, 64):
        rows.update((c - 1, c))
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("B,H,T", SHAPES)
def test_plan_branch(B, H, T):
    announce(f"MFMA SQ plan branch B={B} H={H} T={T}")
    d = 64
    q, k, v, z = SI.draw(B, H, T, d, seed=700 + T + 13 * B * H, dtype="bf16", z_mean=-10.0)
    qd, kd, vd, zd = dev(q, k, v, z)
    out, S, n = tmb.fwd(qd, kd, vd, zd, want_state=True)
    out_r, S_r, n_r = tmb.fwd(qd, kd, vd, zd, want_state=True, reference_kernels=True)
    torch.cuda.synchronize()
    e_all = relerr(host64(out), host64(out_r))
    e_all_s = relerr(host64(S), host64(S_r))
    e_all_n = relerr(host64(n), host64(n_r))
    print(f"  all heads against the reference kernels: out {e_all:.2e} state {e_all_s:.2e} norm {e_all_n:.2e}")
    assert e_all < TOL["bf16"] and e_all_s < TOL["bf16"] and e_all_n < TOL["bf16"]

    rows = _rows(T)
    o = host64(out)
    Sg, ng = host64(S), host64(n)
    heads = sorted({(0, 0), (B - 1, H - 1)})
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qq, kk, vv, zz = (SI.to_f64(t[sl]) for t in (q, k, v, z))
        ref = O.fwd_quadratic_rows(qq, kk, vv, zz, rows)
        e = relerr(o[sl][:, :, rows], ref)
        S_ref, n_ref = O.final_state_direct(kk, vv, zz)
        es, en = relerr(Sg[sl], S_ref), relerr(ng[sl], n_ref)
        print(f"  head ({b}, {h}) against the oracle: {len(rows)} rows {e:.2e} state {es:.2e} norm {en:.2e}")
        assert e < TOL["bf16"] and es < TOL["bf16"] and en < TOL["bf16"]
