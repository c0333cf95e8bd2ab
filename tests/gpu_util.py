"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def relerr(got, ref):
    """max over (b,h) of ||got-ref||_inf / ||ref||_inf, as float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    B, H = ref.shape[:2]
    num = np.abs(got - ref).reshape(B, H, -1).max(-1)
    den = np.abs(ref).reshape(B, H, -1).max(-1)
    return float((num / np.where(den == 0, 1.0, den)).max())


def dev(*ts):
    out = tuple(t.to("cuda") for t in ts)
    return out if len(out) > 1 else out[0]


def host64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def announce(msg):
    print(f"[case] {msg}", flush=True)
