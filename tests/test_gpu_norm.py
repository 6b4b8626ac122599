"""Fused residual add + RMS norm on the GPU (attn_add_rms_norm) against the fp64 oracle.

Bar (derived from the arithmetic; the pages give no tolerance for this kernel): the GPU adds,
squares and scales in fp32 and rounds each output to bfloat16 once, so
  * the new residual must be x + residual rounded to nearest: within half a bf16 ulp of the
    exact sum (the fp32 sum of two bf16 values is exact at these magnitudes);
  * the normalised output must be within half a bf16 ulp of the exact result, plus a
    relative 1e-5 for the fp32 sum of squares and reciprocal square root.
"""
import numpy as np
import pytest
import torch

import exact_attention_42_amd as A
import oracle
import workloads as W
from tests.parity import to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)


def half_ulp(v):
    """Half a bfloat16 ulp at |v| (8 significant bits): 2^(floor(log2|v|) - 8)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def check_norm(g_out, g_t, ref_out, ref_t, what):
    g_out = np.asarray(g_out, dtype=np.float64)
    g_t = np.asarray(g_t, dtype=np.float64)
    et = np.abs(g_t - ref_t)
    assert np.all(et <= half_ulp(ref_t)), f"{what}: residual off by {et.max():.3e}"
    eo = np.abs(g_out - ref_out)
    bound = half_ulp(ref_out) + 1e-5 * np.abs(ref_out) + 1e-30
    bad = eo > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs beyond half an ulp + 1e-5 rel, "
                           f"worst {eo[bad].max():.3e}")
    return float(eo.max()), float(eo.mean())


@pytest.mark.parametrize("M,d", [(1, 8), (3, 24), (5, 4104), (33, 5120), (2, 8192),
                                 (7, 65536), (1000, 4096), (64, 2048)])
def test_norm_shapes(M, d, dev):
    x, r, w = W.norm_inputs(M, d, seed=M * 7 + d)
    out, t = A.add_rms_norm(bf(x, dev), bf(r, dev), bf(w, dev))
    torch.cuda.synchronize()
    ref_out, ref_t = oracle.add_rms_norm(x, r, w, eps=1e-6)
    check_norm(to_np(out), to_np(t), ref_out, ref_t, f"M={M} d={d}")


@pytest.mark.parametrize("name", list(W.NORM_CONFIGS))
def test_norm_configs(name, dev):
    cfg = W.NORM_CONFIGS[name]
    x, r, w = W.norm_inputs_for(cfg)
    out, t = A.add_rms_norm(bf(x, dev), bf(r, dev), bf(w, dev), eps=cfg.eps)
    torch.cuda.synchronize()
    go, gt = to_np(out), to_np(t)
    if cfg.M * cfg.d > (1 << 24):          # check sampled rows of the largest shape
        rows = np.unique(np.r_[0, cfg.M - 1, np.random.default_rng(1).integers(0, cfg.M, 96)])
        x, r, go, gt = x[rows], r[rows], go[rows], gt[rows]
    ref_out, ref_t = oracle.add_rms_norm(x, r, w, eps=cfg.eps)
    mx, mn = check_norm(go, gt, ref_out, ref_t, name)
    print(f"{name}: out max|err| {mx:.3e} mean {mn:.3e}")


def test_norm_in_place_and_eps(dev):
    M, d = 9, 3072
    x, r, w = W.norm_inputs(M, d, seed=99)
    x[2] = 0.0
    r[2] = 0.0                                   # a zero row: out = 0 (eps keeps it finite)
    gx, gr, gw = bf(x, dev), bf(r, dev), bf(w, dev)
    for eps in (1e-6, 0.5):
        ref_out, ref_t = oracle.add_rms_norm(x, r, w, eps=eps)
        ax, ar = gx.clone(), gr.clone()
        out, t = A.add_rms_norm(ax, ar, gw, eps=eps, out=ax, residual_out=ar)
        torch.cuda.synchronize()
        assert out.data_ptr() == ax.data_ptr() and t.data_ptr() == ar.data_ptr()
        check_norm(to_np(ax), to_np(ar), ref_out, ref_t, f"in place, eps={eps}")
        assert bool((ax[2] == 0).all())
        o2, t2 = A.add_rms_norm(gx, gr, gw, eps=eps)
        torch.cuda.synchronize()
        assert torch.equal(o2, ax) and torch.equal(t2, ar)


def test_norm_rows_are_independent(dev):
    """A row's result does not depend on the other rows or on the batch size."""
    x, r, w = W.norm_inputs(40, 4096, seed=5)
    o_all, t_all = A.add_rms_norm(bf(x, dev), bf(r, dev), bf(w, dev))
    o_one, t_one = A.add_rms_norm(bf(x[17:18], dev), bf(r[17:18], dev), bf(w, dev))
    torch.cuda.synchronize()
    assert torch.equal(o_all[17:18], o_one) and torch.equal(t_all[17:18], t_one)
