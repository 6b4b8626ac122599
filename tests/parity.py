"""Tolerances and helpers for comparing the HIP path with the fp64 oracle.

Tolerances (absolute unless stated), on inputs rounded to bfloat16 before either side sees
them:
  * bf16 output O:  max |O - O*| <= 2e-2 and mean |O - O*| <= 2e-3 over all elements;
  * fp32 output O:  max |O - O*| / max |O*| <= 1e-5;
  * LSE:            max |LSE - LSE*| <= 1e-3 over finite entries; -inf where the oracle
                    has -inf (rows that see no key), exactly.
The bf16 bound is dominated by the final rounding of O to bfloat16 (half an ulp is 2^-8
relative, 0.0156 for |O| in [4, 8)), plus the bfloat16 rounding of the probabilities that
feed the second matrix product; the fp32 accumulation and exp2 error are far below it.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_REL = 1e-5
LSE_ABS = 1e-3


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_lse(lse, ref, tol=LSE_ABS, what="LSE"):
    lse = np.asarray(lse, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert lse.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: finite pattern differs"
    assert np.all(lse[~fin] == ref[~fin]), f"{what}: -inf rows differ"
    if fin.any():
        err = np.max(np.abs(lse[fin] - ref[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
        return float(err)
    return 0.0


def check_bf16(o, ref, what="O", max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS):
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert o.shape == ref.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    d = np.abs(o - ref)
    mx, mn = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    assert mx <= max_abs, f"{what}: max abs err {mx:.3e} > {max_abs}"
    assert mn <= mean_abs, f"{what}: mean abs err {mn:.3e} > {mean_abs}"
    return mx, mn


def check_f32(o, ref, what="O", rel=F32_REL):
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert o.shape == ref.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    err = float(np.max(np.abs(o - ref))) / scale
    assert err <= rel, f"{what}: norm-wise relative err {err:.3e} > {rel}"
    return err
