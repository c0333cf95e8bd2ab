"""Seeded synthetic inputs for the 2Mamba operator (shared by tests, bench and smoke).

This module only draws random numbers and casts them. It holds none of the
operator's arithmetic, so the fp64 oracle and the HIP path can both consume it
without sharing any part of the method.

Recipe (stand-in for the language-model activations of the 300M/700M Llama-2
ablation models in "2Mamba2Furious: Linear in Complexity, Competitive in
Accuracy", App. B; no dataset or trained weight is used):

* generator ``numpy.random.Generator(PCG64(seed))``, fp64 draws;
* draw order q, k, v (each standard normal divided by sqrt(d), shape
  [B, H, T, d], C order), then z (normal with mean ``z_mean`` and std 1,
  shape [B, H, T]);
* q, k, v are cast to the requested dtype (fp32 or bf16, round to nearest
  even); z always stays fp32.  Consumers that need the exact values upcast the
  cast tensors, so both sides see bit-identical inputs.
"""

from __future__ import annotations

import math

import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def draw(B: int, H: int, T: int, d: int, dv: int | None = None, *, seed: int,
         dtype: str = "bf16", z_mean: float = 0.0, z_neg_inf: bool = False):
    """Return CPU tensors (q, k, v, z) drawn with the recipe above.

    ``z_neg_inf`` replaces every decay logit with -inf (no decay at all);
    ``z_mean`` shifts the logits (e.g. -10 gives a chunk decay near 0.995).
    """
    dv = d if dv is None else dv
    rng = np.random.Generator(np.random.PCG64(seed))
    s = 1.0 / math.sqrt(d)
    q = rng.standard_normal((B, H, T, d)) * s
    k = rng.standard_normal((B, H, T, d)) * s
    v = rng.standard_normal((B, H, T, dv)) * s
    z = rng.standard_normal((B, H, T)) + z_mean
    if z_neg_inf:
        z[...] = -np.inf
    td = _DTYPES[dtype]
    cast = lambda a: torch.from_numpy(a.astype(np.float32)).to(td).contiguous()
    return cast(q), cast(k), cast(v), torch.from_numpy(z.astype(np.float32)).contiguous()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (possibly bf16) tensor to an fp64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
