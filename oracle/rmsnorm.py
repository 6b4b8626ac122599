"""Plain fp64 CPU residual-add + RMS normalisation -- the oracle. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
this module; the HIP library never does. It shares no code with the HIP path.

What it computes ("Kernel and Operator Fusion -- Inference Optimization", §4 "Tiny example"
and §5 "Why add_rms_norm returns two things"): for every row of x and of the residual stream,
  t   = x + residual                      (the new residual, which the next layer's add needs)
  out = t / sqrt(mean(t^2) + eps) * weight
with the mean taken over the row's d elements and weight broadcast along the row. Both t and
out are returned, in that page's order (normalised output first). eps defaults to 1e-6, the
value in that page's unfused listing.

Everything is evaluated in float64 on values that arrive as float32 (bfloat16-exact for the
bf16 workloads), so the only rounding is fp64's.
"""
from __future__ import annotations

import numpy as np


def add_rms_norm(x, residual, weight, eps=1e-6):
    """x, residual [M, d]; weight [d]. Returns (out [M, d], t [M, d]) in float64."""
    t = np.asarray(x, dtype=np.float64) + np.asarray(residual, dtype=np.float64)
    ms = np.mean(t * t, axis=-1, keepdims=True)          # mean of squares over the row
    out = t / np.sqrt(ms + float(eps)) * np.asarray(weight, dtype=np.float64)
    return out, t
