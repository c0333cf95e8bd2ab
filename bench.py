"""Benchmark of the 2Mamba operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--legs sq,sq_4x16x2048,sq_1x16x32768,exp,step,exp_step,bwd,exp_bwd,conv,fwd_conv,
                            lin,lin_step,lin_bwd,sq_bwd_chunked]
                    [--cpu-seconds S]

A timed step is one 2Mamba chunked forward (decay prep, features, intra-chunk,
chunk state, inter-chunk scan, readout, normalisation) over one batch of the
long-context workload B=2, H=16, T=8192, d_k=d_v=64, bf16 inputs, seeded
synthetic data.  ``value`` is its whole-job throughput in head-tokens/s with
all inputs resident in HBM.  The same run also measures, each in its own timed
loop, the 2Mamba forward at B=4 H=16 T=2048 and at B=1 H=16 T=32768, the
2Mamba-E forward on the headline shape and the recurrent decode step
(batch 64, 32 heads, fp32 packed state of 1.09 GB, 256 sequential steps after
a T=2048 prefill) and the 2Mamba-E decode over a bf16 key/value cache (batch
64, 32 heads, 256 sequential steps after a 2048-token prompt), and the
backward pass of both variants, the size-2 input convolution and the
first-order (Mamba-2S) forward on the forward's workload, the first-order
decode step and backward, and the 2Mamba backward in its O(T) chunked form at
B=2 H=16 T=8192 and B=1 H=16 T=32768 beside its attention form; they are
reported under ``legs``.

The roofline entry is for the dominant kernel of the timed step: algorithmic
work attributed to that kernel per launch divided by its average duration,
measured with HIP events on the stream the kernel runs on (a second loop over
the same inputs through twomamba_fwd_timed).  ``cpu_baseline`` times the fp64
oracle (packed recurrent form) on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd tokens/s (B·H·T, d=64, bf16) + % MFMA peak; decode step HBM GB/s"
PEAK_BF16_FLOPS = 2.5e15        # MI355X dense bf16/fp16 MFMA
PEAK_FP32_VALU_FLOPS = 157.3e12 # MI355X fp32 vector
PEAK_HBM = 8.0e12               # MI355X HBM3E bytes/s

SQ_SHAPE = dict(B=2, H=16, T=8192, d=64, seed=3)
EXP_SHAPE = dict(B=2, H=16, T=8192, d=64, seed=3)
# the other two 2Mamba workloads of the pages' shapes, reported beside the headline
SQ_SHAPES_EXTRA = {"sq_4x16x2048": dict(B=4, H=16, T=2048, d=64, seed=1),
                   "sq_1x16x32768": dict(B=1, H=16, T=32768, d=64, seed=2)}
STEP_SHAPE = dict(B=64, H=32, d=64, prefill_T=2048, prefill_seed=4, steps=256)
EXP_STEP_SHAPE = dict(B=64, H=32, d=64, prompt_T=2048, seed=4, steps=256)


def sq_flops_per_head_token(d=64, dv=64, c0=64):
    """Algorithmic 2Mamba work: two state contractions (update and readout,
    2*D*dv each) plus the causal intra-chunk part at a fixed 64-token chunk."""
    D = d * (d + 1) // 2
    return 4 * D * dv + c0 * (d + dv)


def exp_flops_per_head(T, d=64, dv=64):
    """Causal softmax attention work: QK^T and PV over the lower triangle incl. diagonal."""
    return T * (T + 1) * (d + dv)


def step_bytes_per_head(d=64, dv=64):
    """Decode step HBM bytes: read+write the fp32 state and normaliser, read q,k,z,v, write out (fp32)."""
    D = d * (d + 1) // 2
    return 2 * (D * dv + D) * 4 + (3 * d + 1) * 4 + dv * 4


def exp_step_bytes_per_head(pos, d=64, dv=64, esize=2):
    """2Mamba-E decode step at position `pos`: read the pos cached key/value rows
    and their fp64 running decay sums, append row pos, read q, k, v (input dtype)
    and z (fp32), write the output row."""
    row = (d + dv) * esize + 8
    return pos * row + row + (2 * d + dv) * esize + 4 + dv * esize


def bwd_flops_per_head(T, d=64, dv=64):
    """Algorithmic backward work over the causal pairs T(T+1)/2: recompute the
    score (2d), dP = dout.v (2dv), dv (2dv), dk (2d), dq (2d)."""
    return T * (T + 1) // 2 * 2 * (3 * d + 2 * dv)


def bwd_kernel_work(name, T, d=64, dv=64):
    """Share of the backward work credited to one kernel per head: the
    key-major kernel does the score, dP, dv and dk products, the query-major one
    dq (its score / dP recomputation and the row-statistic sweep are counted as
    overhead, not work)."""
    pairs = T * (T + 1) // 2
    if name == "bwd_kv":
        return pairs * 2 * (2 * d + 2 * dv)
    if name == "bwd_q":
        return pairs * 2 * d
    return 0


def kernel_work(name, leg_work):
    """Algorithmic work credited to the dominant kernel per launch: the whole
    leg's work, since each forward kernel executes every algorithmic step of its
    variant itself (the segment-state pre-pass of the 2Mamba forward is extra
    work on top)."""
    return leg_work


KERNEL_SOURCES = {"sq_mfma_main": "sq_mfma.hip", "exp_mfma": "exp_mfma.hip", "step_kernel": "step.hip",
                  "exp_decode_partial": "exp_step.hip", "exp_decode_combine": "exp_step.hip",
                  "bwd_q": "bwd_mfma.hip", "bwd_kv": "bwd_mfma.hip", "exp_bwd_q": "bwd_mfma.hip",
                  "exp_bwd_kv": "bwd_mfma.hip", "conv2_kernel": "conv.hip", "lin_seg": "lin.hip",
                  "lin_scan": "lin.hip", "lin_main": "lin.hip", "step_first_order64_kernel": "step.hip",
                  "sq_segstate": "sq_mfma.hip", "bwd_prep": "bwd_ref.hip", "bwd_dz": "bwd_ref.hip",
                  "sqc_walk_q": "sq_bwd_chunk.hip", "sqc_walk_k": "sq_bwd_chunk.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def source_digest(kernel):
    import hashlib

    src = KERNEL_SOURCES.get(kernel)
    if src is None:
        return None
    with open(os.path.join(ROOT, "second_order_ssm_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    counter summary (already scaled by the copy-kernel calibration), or None when
    there is none or the kernel's source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_digest(kernel)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("kernel="):
                continue
            kv = dict(x.split("=", 1) for x in line.split())
            if kv.get("kernel") == kernel and kv.get("src_sha256") == want:
                return float(kv["traffic_bytes"])
    return None


def traffic_sum(*kernels):
    """Summed counter traffic of kernels that together make one step, or None if any is missing."""
    t = [measured_traffic(k) for k in kernels]
    return None if any(x is None for x in t) else sum(t)


def time_loop(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def dominant_kernel(fn_timed, calls):
    """Average per-kernel durations over `calls` timed invocations; returns (name, ms, all)."""
    acc = {}
    for _ in range(calls):
        kt = []
        fn_timed(kt)
        for name, ms in kt:
            acc.setdefault(name, []).append(ms)
    avg = {n: sum(v) / len(v) for n, v in acc.items()}
    name = max(avg, key=avg.get)
    return name, avg[name], avg


def leg_sq(steps, warmup, variant="sq", shape=None):
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = shape or (SQ_SHAPE if variant == "sq" else EXP_SHAPE)
    B, H, T, d = shp["B"], shp["H"], shp["T"], shp["d"]
    q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=shp["seed"], dtype="bf16"))
    out = torch.empty_like(v)
    desc = tmb.make_desc(B, H, T, d, d, variant=variant, dtype=torch.bfloat16)
    nws = tmb.workspace_size(desc)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    fn = lambda: tmb.fwd(q, k, v, z, variant=variant, out=out, workspace=ws)
    ms = time_loop(fn, steps, warmup)
    name, kms, allk = dominant_kernel(lambda kt: tmb.fwd(q, k, v, z, variant=variant, out=out, workspace=ws,
                                                         kernel_times=kt), max(3, min(steps, 10)))
    ht = B * H * T
    if variant == "sq":
        work = ht * sq_flops_per_head_token(d, d)
    else:
        work = B * H * exp_flops_per_head(T, d, d)
    mfma = not name.startswith("ref_")
    peak = PEAK_BF16_FLOPS if mfma else PEAK_FP32_VALU_FLOPS
    achieved = kernel_work(name, work) / (kms * 1e-3)
    return dict(
        workload=f"{'2Mamba' if variant == 'sq' else '2Mamba-E'} fwd B={B} H={H} T={T} d={d} bf16",
        ms=ms, head_tokens_per_s=ht / (ms * 1e-3), flops_per_call=work,
        tflops=work / (ms * 1e-3) / 1e12, frac_peak_bf16=work / (ms * 1e-3) / PEAK_BF16_FLOPS,
        kernels_ms=allk,
        roofline=dict(bound="mfma" if mfma else "alu", kernel=name, achieved=achieved / 1e12, peak=peak / 1e12,
                      unit="TFLOP/s", frac=achieved / peak,
                      # the counter summary covers the headline shape only
                      traffic=measured_traffic(name) if shape is None else None),
    )


def leg_bwd(steps, warmup, variant="sq"):
    """Backward (dq, dk, dv, dz) of the forward on the same workload, with a
    seeded N(0,1) output gradient; the forward output and its per-row
    statistics (as a training step keeps them) are computed once, untimed."""
    import numpy as np
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = SQ_SHAPE
    B, H, T, d = shp["B"], shp["H"], shp["T"], shp["d"]
    q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=shp["seed"], dtype="bf16"))
    dout = torch.from_numpy(np.random.default_rng(shp["seed"] + 500).standard_normal((B, H, T, d))).to(
        torch.bfloat16).cuda()
    out, stat = tmb.fwd(q, k, v, z, variant=variant, want_stats=True)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z))
    desc = tmb.make_desc(B, H, T, d, d, variant=variant, dtype=torch.bfloat16)
    ws = torch.empty(tmb.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    fn = lambda: tmb.bwd(q, k, v, z, out, dout, variant=variant, grads=grads, workspace=ws, row_stat=stat)
    ms = time_loop(fn, steps, warmup)
    name, kms, allk = dominant_kernel(lambda kt: tmb.bwd(q, k, v, z, out, dout, variant=variant, grads=grads,
                                                         workspace=ws, row_stat=stat, kernel_times=kt),
                                      max(3, min(steps, 10)))
    work = B * H * bwd_flops_per_head(T, d, d)
    # the work splits over two MFMA kernels (and two small ones); the roofline
    # entry covers all of them: the op's work over the summed kernel durations
    ktot = sum(allk.values())
    achieved = work / (ktot * 1e-3)
    return dict(
        workload=f"{'2Mamba' if variant == 'sq' else '2Mamba-E'} bwd B={B} H={H} T={T} d={d} bf16",
        ms=ms, head_tokens_per_s=B * H * T / (ms * 1e-3), flops_per_call=work,
        tflops=work / (ms * 1e-3) / 1e12, frac_peak_bf16=work / (ms * 1e-3) / PEAK_BF16_FLOPS,
        kernels_ms=allk,
        kernel_work_tflops={n: B * H * bwd_kernel_work(n, T, d, d) / (ms_ * 1e-3) / 1e12 for n, ms_ in allk.items()
                            if bwd_kernel_work(n, T, d, d)},
        roofline=dict(bound="mfma", kernel="+".join(allk), achieved=achieved / 1e12, peak=PEAK_BF16_FLOPS / 1e12,
                      unit="TFLOP/s", frac=achieved / PEAK_BF16_FLOPS,
                      # counter traffic of the two MFMA kernels (the decay scan and dz kernels are small)
                      traffic=traffic_sum(*[("" if variant == "sq" else "exp_") + n for n in ("bwd_q", "bwd_kv")])),
    )


def sqc_walk_flops_per_head_token(d=64, dv=64):
    """Work of one chunk walk of the 2Mamba O(T) backward per head-token: the
    update S[i, c, j] += (lambda b_i e_c) b_j and the readout A_j += (a_i c_c) S[i, c, j]
    over the unpacked state, d x (dv + 1) x d each (the 65th column included)."""
    return 4 * d * d * (dv + 1)


def sq_bwd_chunked_flops_per_head_token(d=64, dv=64):
    """The O(T) backward's work per head-token: two walks (dq forward in time, dk
    reversed) and the reversed-time forward that gives dv."""
    return 2 * sqc_walk_flops_per_head_token(d, dv) + sq_flops_per_head_token(d, dv)


def leg_sq_bwd_chunked(steps, warmup):
    """2Mamba backward in O(T) (TWOMAMBA_FLAG_CHUNKED_FORM; the default from 20480 tokens
    per head) at the forward's workload and at the long-context one (B=1 H=16 T=32768),
    beside the attention form of the same backward on the same inputs.  Roofline: the chunk-walk kernel, over the
    walk's contractions (sqc_walk_flops_per_head_token) per launch."""
    import numpy as np
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    res = {}
    for B, H, T in ((SQ_SHAPE["B"], SQ_SHAPE["H"], SQ_SHAPE["T"]), (1, 16, 32768)):
        d = SQ_SHAPE["d"]
        q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=SQ_SHAPE["seed"], dtype="bf16"))
        dout = torch.from_numpy(np.random.default_rng(SQ_SHAPE["seed"] + 500).standard_normal((B, H, T, d))).to(
            torch.bfloat16).cuda()
        out, stat = tmb.fwd(q, k, v, z, want_stats=True)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z))
        desc = tmb.make_desc(B, H, T, d, d, dtype=torch.bfloat16, flags=tmb.FLAG_CHUNKED_FORM)
        ws = torch.empty(tmb.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
        fn = lambda: tmb.bwd(q, k, v, z, out, dout, chunked_form=True, grads=grads, workspace=ws, row_stat=stat)
        ms = time_loop(fn, steps, warmup)
        per = {}
        calls = max(3, min(steps, 10))
        for _ in range(calls):
            kt = []
            tmb.bwd(q, k, v, z, out, dout, chunked_form=True, grads=grads, workspace=ws, row_stat=stat,
                    kernel_times=kt)
            for n, x in kt:
                per[n] = per.get(n, 0.0) + x / calls
        del ws
        desc_a = tmb.make_desc(B, H, T, d, d, dtype=torch.bfloat16, flags=tmb.FLAG_ATTENTION_FORM)
        ws_a = torch.empty(tmb.bwd_workspace_size(desc_a), dtype=torch.uint8, device="cuda")
        fn_a = lambda: tmb.bwd(q, k, v, z, out, dout, attention_form=True, grads=grads, workspace=ws_a,
                               row_stat=stat)
        ms_att = time_loop(fn_a, max(3, steps // 5), 1)
        del ws_a
        walk_ms = (per.get("sqc_walk_q", 0.0) + per.get("sqc_walk_k", 0.0)) / 2
        walk_work = B * H * T * sqc_walk_flops_per_head_token(d, d)
        work = B * H * T * sq_bwd_chunked_flops_per_head_token(d, d)
        res[f"{B}x{H}x{T}"] = dict(ms=ms, head_tokens_per_s=B * H * T / (ms * 1e-3), flops_per_call=work,
                                   tflops=work / (ms * 1e-3) / 1e12, kernels_ms=per,
                                   walk_kernel_ms=walk_ms, walk_kernel_tflops=walk_work / (walk_ms * 1e-3) / 1e12,
                                   attention_form_ms=ms_att, speedup_over_attention_form=ms_att / ms)
        del q, k, v, z, dout, out, stat, grads
        torch.cuda.empty_cache()
    head = res["1x16x32768"]
    wt = head["walk_kernel_tflops"] * 1e12
    return dict(workload="2Mamba bwd in O(T) (chunked form), bf16 d=64: B=2 H=16 T=8192 and B=1 H=16 T=32768",
                ms=res[f"{SQ_SHAPE['B']}x{SQ_SHAPE['H']}x{SQ_SHAPE['T']}"]["ms"], shapes=res,
                roofline=dict(bound="mfma", kernel="sqc_walk_kernel (main walk, 1x16x32768)", achieved=wt / 1e12,
                              peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s", frac=wt / PEAK_BF16_FLOPS, traffic=None))


def lin_bwd_bytes_per_head_token(d=64, dv=64, esize=2):
    """Algorithmic bytes of the first-order backward per head-token: read q, k, v
    and dout, write dq, dk and dv (input dtype), read z and write dz (fp32)."""
    return (4 * d + 3 * dv) * esize + 8 if d == dv else (2 * d + 2 * dv + 2 * d + dv) * esize + 8


def leg_lin_bwd(steps, warmup):
    """First-order backward in O(T) (three segmented chunk passes, two in reverse
    time, and the dz scan) at the forward's workload and at the long-context one
    (B=1 H=16 T=32768), beside the attention (quadratic) form of the same backward.  Its arithmetic is small (about 12 d dv FLOP per
    head-token in the state contractions), so the roofline is HBM, over the
    algorithmic bytes of the backward (inputs read and gradients written once)."""
    import numpy as np
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    res = {}
    for B, H, T in ((SQ_SHAPE["B"], SQ_SHAPE["H"], SQ_SHAPE["T"]), (1, 16, 32768)):
        d = SQ_SHAPE["d"]
        q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=SQ_SHAPE["seed"], dtype="bf16"))
        dout = torch.from_numpy(np.random.default_rng(SQ_SHAPE["seed"] + 500).standard_normal((B, H, T, d))).to(
            torch.bfloat16).cuda()
        out = tmb.fwd(q, k, v, z, variant="lin")
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z))
        desc = tmb.make_desc(B, H, T, d, d, variant="lin", dtype=torch.bfloat16)
        ws = torch.empty(tmb.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
        fn = lambda: tmb.bwd(q, k, v, z, out, dout, variant="lin", grads=grads, workspace=ws)
        ms = time_loop(fn, steps, warmup)
        # the attention (quadratic) form of the same backward, for comparison
        desc_a = tmb.make_desc(B, H, T, d, d, variant="lin", dtype=torch.bfloat16, flags=tmb.FLAG_ATTENTION_FORM)
        ws_a = torch.empty(tmb.bwd_workspace_size(desc_a), dtype=torch.uint8, device="cuda")
        fn_a = lambda: tmb.bwd(q, k, v, z, out, dout, variant="lin", attention_form=True, grads=grads, workspace=ws_a)
        ms_att = time_loop(fn_a, max(3, steps // 5), 1)
        del ws_a
        byts = B * H * T * lin_bwd_bytes_per_head_token(d, d)
        bw = byts / (ms * 1e-3)
        kt = []
        tmb.bwd(q, k, v, z, out, dout, variant="lin", grads=grads, workspace=ws, kernel_times=kt)
        per = {}
        for n, x in kt:
            per[n] = per.get(n, 0.0) + x
        res[f"{B}x{H}x{T}"] = dict(ms=ms, head_tokens_per_s=B * H * T / (ms * 1e-3), bytes_per_call=byts,
                                   kernels_ms=per, GBps=bw / 1e9, frac_hbm=bw / PEAK_HBM,
                                   attention_form_ms=ms_att, speedup_over_attention_form=ms_att / ms)
        del q, k, v, z, dout, out, grads, ws
        torch.cuda.empty_cache()
    head = res[f"{SQ_SHAPE['B']}x{SQ_SHAPE['H']}x{SQ_SHAPE['T']}"]
    return dict(workload="first-order (Mamba-2S) bwd in O(T), bf16 d=64: B=2 H=16 T=8192 and B=1 H=16 T=32768",
                ms=head["ms"], shapes=res,
                roofline=dict(bound="hbm", kernel="lin_seg+lin_scan+lin_main (x3)+bwd_dz",
                              achieved=head["GBps"], peak=PEAK_HBM / 1e9, unit="GB/s", frac=head["frac_hbm"],
                              traffic=None))


def leg_conv(steps, warmup):
    """Size-2 input convolution of q, k and v on the forward's workload (bf16,
    with bias and a cached row): HBM-bound, three tensors read and written."""
    import numpy as np
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = SQ_SHAPE
    B, H, T, d = shp["B"], shp["H"], shp["T"], shp["d"]
    q, k, v, _ = (t.cuda() for t in SI.draw(B, H, T, d, seed=shp["seed"], dtype="bf16"))
    r = np.random.default_rng(shp["seed"] + 900)
    w = torch.from_numpy(r.normal(0.0, 0.7, size=(3, H, d, 2)).astype(np.float32)).cuda()
    b = torch.from_numpy(r.normal(0.0, 0.1, size=(3, H, d)).astype(np.float32)).cuda()
    prev = torch.zeros(B, H, 3, d, dtype=torch.bfloat16, device="cuda")
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    st = torch.empty_like(prev)
    ms = time_loop(lambda: tmb.conv2(q, k, v, w, b, prev, outs=outs, state_out=st), steps, warmup)
    byts = 2 * 3 * B * H * T * d * 2 + 2 * B * H * 3 * d * 2 + w.numel() * 4 + b.numel() * 4
    bw = byts / (ms * 1e-3)
    return dict(workload=f"size-2 input convolution of q, k, v B={B} H={H} T={T} d={d} bf16", ms=ms,
                bytes_per_call=byts,
                roofline=dict(bound="hbm", kernel="conv2_kernel", achieved=bw / 1e9, peak=PEAK_HBM / 1e9,
                              unit="GB/s", frac=bw / PEAK_HBM, traffic=measured_traffic("conv2_kernel")))


def leg_fwd_conv(steps, warmup):
    """The forward with the size-2 input convolution in front (twomamba_fwd_conv)
    on the forward's workload (bf16, with bias and a cached row), for each
    variant beside the forward alone and the unfused sequence (twomamba_conv2,
    then twomamba_fwd).  Timed interleaved, median of rounds.  The first order
    convolves in its kernels, 2Mamba-E convolves its queries in its kernel and
    k, v in one pass, 2Mamba runs the pass over q, k, v into its workspace."""
    import statistics

    import numpy as np
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = SQ_SHAPE
    B, H, T, d = shp["B"], shp["H"], shp["T"], shp["d"]
    q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=shp["seed"], dtype="bf16"))
    r = np.random.default_rng(shp["seed"] + 900)
    w = torch.from_numpy(r.normal(0.0, 0.7, size=(3, H, d, 2)).astype(np.float32)).cuda()
    b = torch.from_numpy(r.normal(0.0, 0.1, size=(3, H, d)).astype(np.float32)).cuda()
    prev = torch.zeros(B, H, 3, d, dtype=torch.bfloat16, device="cuda")
    cbuf = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    res = {}
    for variant in ("sq", "exp", "lin"):
        out = torch.empty_like(v)
        desc = tmb.make_desc(B, H, T, d, d, variant=variant, dtype=torch.bfloat16)
        ws = torch.empty(max(1, tmb.workspace_size(desc)), dtype=torch.uint8, device="cuda")
        wsc = torch.empty(max(1, tmb.conv_workspace_size(desc)), dtype=torch.uint8, device="cuda")
        fns = {
            "fwd": lambda: tmb.fwd(q, k, v, z, variant=variant, out=out, workspace=ws),
            "conv_then_fwd": lambda: (tmb.conv2(q, k, v, w, b, prev, outs=cbuf),
                                      tmb.fwd(*cbuf, z, variant=variant, out=out, workspace=ws)),
            "fwd_conv": lambda: tmb.fwd_conv(q, k, v, z, w, b, prev, variant=variant, out=out, workspace=wsc),
        }
        t = {n: [] for n in fns}
        for _ in range(max(3, steps // 5)):
            for n, fn in fns.items():
                t[n].append(time_loop(fn, 5, 1))
        med = {n: statistics.median(x) for n, x in t.items()}
        res[variant] = dict(ms=med, fused_over_fwd=med["fwd_conv"] / med["fwd"],
                            fused_over_unfused=med["fwd_conv"] / med["conv_then_fwd"])
    return dict(workload=f"forward with the size-2 input convolution, B={B} H={H} T={T} d={d} bf16", variants=res)


def leg_lin(steps, warmup):
    """First-order (Mamba-2S) chunked forward on the forward's workload.  Its
    work is small (4 d dv flops per head-token), so the roofline is HBM: q, k,
    v and out in bf16, z in fp32 (516 bytes per head-token)."""
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = SQ_SHAPE
    B, H, T, d = shp["B"], shp["H"], shp["T"], shp["d"]
    q, k, v, z = (t.cuda() for t in SI.draw(B, H, T, d, seed=shp["seed"], dtype="bf16"))
    out = torch.empty_like(v)
    desc = tmb.make_desc(B, H, T, d, d, variant="lin", dtype=torch.bfloat16)
    ws = torch.empty(max(tmb.workspace_size(desc), 1), dtype=torch.uint8, device="cuda")
    ms = time_loop(lambda: tmb.fwd(q, k, v, z, variant="lin", out=out, workspace=ws), steps, warmup)
    _, _, allk = dominant_kernel(lambda kt: tmb.fwd(q, k, v, z, variant="lin", out=out, workspace=ws,
                                                    kernel_times=kt), max(3, min(steps, 10)))
    ht = B * H * T
    byts = ht * (3 * d * 2 + 4 + d * 2)
    ktot = sum(allk.values())
    bw = byts / (ktot * 1e-3)
    return dict(workload=f"first-order (Mamba-2S) fwd B={B} H={H} T={T} d={d} bf16", ms=ms,
                head_tokens_per_s=ht / (ms * 1e-3), bytes_per_call=byts, kernels_ms=allk,
                roofline=dict(bound="hbm", kernel="+".join(allk), achieved=bw / 1e9, peak=PEAK_HBM / 1e9,
                              unit="GB/s", frac=bw / PEAK_HBM, traffic=traffic_sum(*allk)))


def leg_lin_step(warmup):
    """First-order decode step at batch 64, 32 heads: the dk x dv fp32 state is
    read and written once per step."""
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    B, H, d, nsteps = STEP_SHAPE["B"], STEP_SHAPE["H"], STEP_SHAPE["d"], STEP_SHAPE["steps"]
    S = torch.zeros(B, H, d, d, device="cuda")
    qs, ks, vs, zs = (t.cuda() for t in SI.draw(B, H, nsteps + warmup, d, seed=STEP_SHAPE["prefill_seed"] + 200,
                                                 dtype="f32"))
    steps_in = [tuple(x[:, :, i].contiguous() for x in (qs, ks, vs, zs)) for i in range(nsteps + warmup)]
    out = torch.empty(B, H, d, device="cuda")
    for i in range(warmup):
        tmb.step(*steps_in[i], S, None, first_order=True, out=out)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(warmup, warmup + nsteps):
        tmb.step(*steps_in[i], S, None, first_order=True, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / nsteps
    # the same steps captured once as a HIP graph and replayed: a 16 us step
    # otherwise pays a launch gap each time
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(warmup, warmup + nsteps):
            tmb.step(*steps_in[i], S, None, first_order=True, out=out)
    graph.replay()
    torch.cuda.synchronize()
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms_graph = a.elapsed_time(b) / nsteps
    byts = B * H * (2 * d * d * 4 + (3 * d + 1) * 4 + d * 4)
    # the kernel runs shorter than one Python-side launch: the eager loop measures
    # launch gaps, the replay of the captured steps measures the kernels back to back
    bw = byts / (ms_graph * 1e-3)
    return dict(workload=f"first-order decode step B={B} H={H} d={d} fp32 state, {nsteps} sequential steps",
                ms=ms, bytes_per_step=byts, ms_graph_replay=ms_graph,
                GBps_graph_replay=byts / (ms_graph * 1e-3) / 1e9,
                roofline=dict(bound="hbm", kernel="step_first_order64_kernel", timed="graph replay",
                              achieved=bw / 1e9,
                              peak=PEAK_HBM / 1e9, unit="GB/s", frac=bw / PEAK_HBM,
                              traffic=measured_traffic("step_first_order64_kernel")))


def leg_step(warmup):
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    B, H, d, TP = STEP_SHAPE["B"], STEP_SHAPE["H"], STEP_SHAPE["d"], STEP_SHAPE["prefill_T"]
    nsteps = STEP_SHAPE["steps"]
    # prefill (setup, untimed): bf16 T=2048 forward, its final state is the decode state
    q, k, v, z = (t.cuda() for t in SI.draw(B, H, TP, d, seed=STEP_SHAPE["prefill_seed"], dtype="bf16"))
    _, S, n = tmb.fwd(q, k, v, z, want_state=True)
    del q, k, v, z
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # fresh per-step inputs drawn up front, resident in HBM
    qs, ks, vs, zs = (t.cuda() for t in SI.draw(B, H, nsteps + warmup, d, seed=STEP_SHAPE["prefill_seed"] + 100,
                                                 dtype="f32"))
    steps_in = [tuple(x[:, :, i].contiguous() for x in (qs, ks, vs, zs)) for i in range(nsteps + warmup)]
    out = torch.empty(B, H, d, device="cuda")
    for i in range(warmup):
        tmb.step(*steps_in[i], S, n, out=out)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(warmup, warmup + nsteps):
        tmb.step(*steps_in[i], S, n, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / nsteps
    byts = B * H * step_bytes_per_head(d, d)
    bw = byts / (ms * 1e-3)
    return dict(workload=f"decode step B={B} H={H} d={d} fp32 state, {nsteps} sequential steps",
                ms=ms, bytes_per_step=byts,
                roofline=dict(bound="hbm", kernel="step_kernel", achieved=bw / 1e9, peak=PEAK_HBM / 1e9,
                              unit="GB/s", frac=bw / PEAK_HBM, traffic=measured_traffic("step_kernel")))


def leg_exp_step(warmup):
    """2Mamba-E decode over a key/value cache: a bf16 prompt of 2048 tokens goes
    into the caches (untimed), `warmup` untimed steps, then 256 timed sequential
    steps, each attending over every cached position (split over 512-key blocks,
    then one combine launch)."""
    import torch

    import second_order_ssm_amd as tmb
    import synth_inputs as SI

    shp = EXP_STEP_SHAPE
    B, H, d, T0, nsteps = shp["B"], shp["H"], shp["d"], shp["prompt_T"], shp["steps"]
    L = T0 + warmup + nsteps
    kc, vc, gc = tmb.exp_cache(B, H, d, L, dtype=torch.bfloat16)
    _, k, v, z = SI.draw(B, H, T0, d, seed=shp["seed"], dtype="bf16")
    k, v, z = k.cuda(), v.cuda(), z.cuda()
    tmb.exp_cache_fill(k, v, z, kc, vc, gc)
    del k, v, z
    torch.cuda.synchronize()
    qs, ks, vs, zs = (t.cuda() for t in SI.draw(B, H, warmup + nsteps, d, seed=shp["seed"] + 100, dtype="bf16"))
    steps_in = [tuple(x[:, :, i].contiguous() for x in (qs, ks, vs, zs)) for i in range(warmup + nsteps)]
    out = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(tmb.exp_step_workspace_size(B, H, d, L, L - 1), dtype=torch.uint8, device="cuda")
    for i in range(warmup):
        tmb.exp_step(*steps_in[i], kc, vc, gc, T0 + i, out=out, workspace=ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(warmup, warmup + nsteps):
        tmb.exp_step(*steps_in[i], kc, vc, gc, T0 + i, out=out, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / nsteps
    byts = B * H * sum(exp_step_bytes_per_head(T0 + i, d, d) for i in range(warmup, warmup + nsteps)) / nsteps
    bw = byts / (ms * 1e-3)
    return dict(workload=f"2Mamba-E decode B={B} H={H} d={d} bf16 key/value cache, positions "
                         f"{T0 + warmup}..{T0 + warmup + nsteps - 1}",
                ms=ms, bytes_per_step=byts,
                roofline=dict(bound="hbm", kernel="exp_decode_partial+exp_decode_combine", achieved=bw / 1e9,
                              peak=PEAK_HBM / 1e9, unit="GB/s", frac=bw / PEAK_HBM,
                              traffic=traffic_sum("exp_decode_partial", "exp_decode_combine")))


_ORACLE_INPUTS = None   # (q, k, v, z) fp64 [B*H, T, ...], set before the pool forks


def _oracle_heads(args):
    """Worker of the CPU baseline: form (C) over the first n tokens of a subset of heads."""
    from oracle import twomamba_oracle as O

    heads, n = args
    sel = lambda x: x[heads][None, :, :n]
    q, k, v, z = _ORACLE_INPUTS
    t0 = time.perf_counter()
    O.fwd_recurrent_packed(sel(q), sel(k), sel(v), sel(z))
    return time.perf_counter() - t0


def cpu_baseline_worker(seconds):
    """fp64 oracle (packed recurrent form, form C) on the host cores: the 32 heads of
    the 2Mamba workload split over a process pool (heads are independent), over
    the first n tokens, n sized to about `seconds` of wall time.  Runs in a child
    process that never touches the GPU; prints one JSON object."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import platform

    global _ORACLE_INPUTS
    import synth_inputs as SI

    shp = SQ_SHAPE
    nh = shp["B"] * shp["H"]
    q, k, v, z = SI.draw(shp["B"], shp["H"], shp["T"], shp["d"], seed=shp["seed"], dtype="bf16")
    _ORACLE_INPUTS = tuple(SI.to_f64(t).reshape((nh,) + tuple(t.shape[2:])) for t in (q, k, v, z))
    procs = max(1, min(os.cpu_count() or 1, 16, nh))
    groups = [list(range(i, nh, procs)) for i in range(procs)]
    ctx = mp.get_context("fork")
    with cf.ProcessPoolExecutor(procs, mp_context=ctx) as ex:
        # calibration: 16 tokens of every group at once, then the sized run
        t0 = time.perf_counter()
        list(ex.map(_oracle_heads, [(g, 16) for g in groups]))
        per_tok = (time.perf_counter() - t0) / 16
        n = int(max(32, min(shp["T"], seconds / max(per_tok, 1e-9))))
        t0 = time.perf_counter()
        list(ex.map(_oracle_heads, [(g, n) for g in groups]))
        dt = time.perf_counter() - t0
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    print(json.dumps(dict(value=nh * n / dt, unit="head-tokens/s", cores=procs, kind="oracle",
                          sample=f"packed recurrent fp64 oracle (form C), all {shp['B']}x{shp['H']} heads of the "
                                 f"B=2 H=16 T=8192 d=64 workload over {procs} processes (heads split between "
                                 f"them, one thread each), first {n} of {shp['T']} tokens, {dt:.1f} s wall; "
                                 f"host {cpu}, {os.cpu_count()} logical CPUs")))


def cpu_baseline(seconds):
    """The CPU baseline, run in a child process (it never touches the GPU)."""
    import subprocess

    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-worker", str(seconds)],
                       capture_output=True, text=True, env=env, timeout=max(120.0, 8 * seconds))
    if r.returncode != 0:
        print(f"[bench] cpu baseline failed: {r.stderr[-500:]}", file=sys.stderr)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def achievable_peaks():
    """Measured ceilings on this GPU, with the library's own microbenchmark kernels:
    a 1 GiB streaming device copy (bytes read + written per second) and a loop of
    16 independent chains of 16x16x32 f16 MFMAs per wave on register operands,
    with the shader clock it ran at; beside them a large bf16
    library GEMM (8192^3, hipBLASLt via torch.matmul).  Context for the roofline
    fractions, which stay against the published peaks."""
    import torch

    import second_order_ssm_amd as tmb

    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = time_loop(lambda: tmb.ceiling_copy(src, dst), 20, 3)
    copy_bw = 2 * src.numel() * 4 / (ms * 1e-3)
    assert torch.equal(dst[:: 1 << 20], src[:: 1 << 20])
    del src, dst
    wgs, iters = 256 * 8, 500
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros((wgs, 2), dtype=torch.int64, device="cuda")
    ms = time_loop(lambda: tmb.ceiling_mfma(wgs, iters, sink, clocks), 10, 2)
    mfma = wgs * 4 * iters * 16 * 16384 / (ms * 1e-3)
    ck = clocks.cpu().double()
    mhz = float((ck[:, 0] / ck[:, 1].clamp(min=1)).median()) * 100.0
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms = time_loop(lambda: torch.matmul(a, b), 20, 3)
    gemm = 2 * n ** 3 / (ms * 1e-3)
    del a, b
    torch.cuda.empty_cache()
    return dict(copy_GBps=copy_bw / 1e9, copy_frac_of_peak=copy_bw / PEAK_HBM,
                mfma_loop_TFLOPs=mfma / 1e12, mfma_loop_frac_of_peak=mfma / PEAK_BF16_FLOPS,
                mfma_loop_clock_MHz=mhz,
                bf16_gemm_TFLOPs=gemm / 1e12, bf16_gemm_frac_of_peak=gemm / PEAK_BF16_FLOPS,
                device=device_facts())


def device_facts():
    """What the device reports about itself: the published peaks assume 256
    compute units at 2.4 GHz and 288 GB of HBM."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(0)
    facts = dict(name=p.name, arch=getattr(p, "gcnArchName", None), compute_units=p.multi_processor_count,
                 hbm_GB=round(p.total_memory / 1e9, 1))
    facts["max_clock_MHz"] = None
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        # one block per agent; the GPU agent's block names gfx950 (CPU agents report their own clocks)
        for block in txt.split("*******"):
            if "gfx950" not in block:
                continue
            for line in block.splitlines():
                if "Max Clock Freq" in line:
                    facts["max_clock_MHz"] = int(line.split(":")[1].split()[0])
                if "Compute Unit:" in line:
                    facts["rocminfo_compute_units"] = int(line.split(":")[1].split()[0])
            break
    except (OSError, subprocess.SubprocessError, ValueError, IndexError):
        pass
    return facts


def copy_calibration(nbytes=1 << 30, reps=5):
    """The library's streaming copy kernel on a buffer of known size, run under
    rocprofv3 --pmc to calibrate FETCH_SIZE / WRITE_SIZE (each dispatch moves
    nbytes each way)."""
    import torch

    import second_order_ssm_amd as tmb

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        tmb.ceiling_copy(src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="sq,sq_4x16x2048,sq_1x16x32768,exp,step,exp_step,bwd,exp_bwd,conv,fwd_conv,"
                                      "lin,lin_step,lin_bwd,sq_bwd_chunked")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the copy / GEMM ceiling measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--cpu-baseline-worker", type=float, default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_worker is not None:
        cpu_baseline_worker(args.cpu_baseline_worker)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (each head is independent, "
              "so several GPUs would shard B*H with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    legs = args.legs.split(",")
    res = {}
    if "sq" in legs:
        res["sq"] = leg_sq(args.steps, args.warmup, "sq")
        print(f"[bench] sq leg done: {res['sq']['ms']:.3f} ms/step", file=sys.stderr, flush=True)
    for name, shp in SQ_SHAPES_EXTRA.items():
        if name in legs:
            res[name] = leg_sq(args.steps, args.warmup, "sq", shp)
            print(f"[bench] {name} leg done: {res[name]['ms']:.3f} ms/call", file=sys.stderr, flush=True)
    if "exp" in legs:
        res["exp"] = leg_sq(args.steps, args.warmup, "exp")
        print(f"[bench] exp leg done: {res['exp']['ms']:.3f} ms/call", file=sys.stderr, flush=True)
    if "step" in legs:
        res["step"] = leg_step(args.warmup)
        print(f"[bench] step leg done: {res['step']['ms']:.4f} ms/step", file=sys.stderr, flush=True)
    if "bwd" in legs:
        res["bwd"] = leg_bwd(args.steps, args.warmup, "sq")
        print(f"[bench] bwd leg done: {res['bwd']['ms']:.3f} ms/call", file=sys.stderr, flush=True)
    if "exp_bwd" in legs:
        res["exp_bwd"] = leg_bwd(args.steps, args.warmup, "exp")
        print(f"[bench] exp_bwd leg done: {res['exp_bwd']['ms']:.3f} ms/call", file=sys.stderr, flush=True)
    if "conv" in legs:
        res["conv"] = leg_conv(args.steps, args.warmup)
        print(f"[bench] conv leg done: {res['conv']['ms']:.4f} ms/call", file=sys.stderr, flush=True)
    if "sq_bwd_chunked" in legs:
        res["sq_bwd_chunked"] = leg_sq_bwd_chunked(args.steps, args.warmup)
        print(f"[bench] sq_bwd_chunked leg done: {res['sq_bwd_chunked']['ms']:.3f} ms/call", file=sys.stderr,
              flush=True)
    if "lin_bwd" in legs:
        res["lin_bwd"] = leg_lin_bwd(args.steps, args.warmup)
        print(f"[bench] lin_bwd leg done: {res['lin_bwd']['ms']:.4f} ms/call", file=sys.stderr, flush=True)
    if "fwd_conv" in legs:
        res["fwd_conv"] = leg_fwd_conv(args.steps, args.warmup)
        print(f"[bench] fwd_conv leg done", file=sys.stderr, flush=True)
    if "lin" in legs:
        res["lin"] = leg_lin(args.steps, args.warmup)
        print(f"[bench] lin leg done: {res['lin']['ms']:.4f} ms/call", file=sys.stderr, flush=True)
    if "lin_step" in legs:
        res["lin_step"] = leg_lin_step(args.warmup)
        print(f"[bench] lin_step leg done: {res['lin_step']['ms']:.4f} ms/step", file=sys.stderr, flush=True)
    if "exp_step" in legs:
        res["exp_step"] = leg_exp_step(args.warmup)
        print(f"[bench] exp_step leg done: {res['exp_step']['ms']:.4f} ms/step", file=sys.stderr, flush=True)
    peaks = achievable_peaks() if args.peaks else None
    if peaks:
        for leg in res.values():
            rf = leg.get("roofline")
            if rf is None:
                continue
            if rf["unit"] == "GB/s":
                rf["frac_of_measured_copy"] = rf["achieved"] / peaks["copy_GBps"]
            elif rf["bound"] == "mfma":
                rf["frac_of_measured_mfma"] = rf["achieved"] / peaks["mfma_loop_TFLOPs"]
    cpu = cpu_baseline(args.cpu_seconds) if args.cpu_seconds > 0 else None
    # the headline is the 2Mamba forward; a run of other legs only reports the first
    # leg that has a roofline, or none
    head = res.get("sq") or next((leg for leg in res.values() if "roofline" in leg), None) or {}
    line = {
        "metric": METRIC,
        "value": head.get("head_tokens_per_s"),
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.get("ms"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(d) q,k,v and N(0,1) decay logits)",
        "config": {"workload": head.get("workload"), "B": SQ_SHAPE["B"], "H": SQ_SHAPE["H"], "T": SQ_SHAPE["T"],
                   "d": SQ_SHAPE["d"], "chunk": 64},
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "legs": res,
        "measured_peaks": peaks,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
