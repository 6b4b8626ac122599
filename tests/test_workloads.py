"""Input generators: determinism, bfloat16 rounding, the paged layout, and the workload
shapes against the sizes the pages print (tests/golden/page_workloads.json)."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_workloads.json")


def _golden():
    with open(GOLDEN) as f:
        return {it["id"]: it for it in json.load(f)["items"]}


def test_bf16_round_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32),
        (r.standard_normal(1000) * 1e30).astype(np.float32),
        (r.standard_normal(1000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895e38, -3.3895e38, 1.00390625,
                  1.01171875, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32),
        # every tie pattern in the low 16 bits around a few exponents
        (np.arange(0x3F800000, 0x3F820000, 0x1000, dtype=np.uint32) | 0x8000).view(np.float32),
    ])
    ours = W.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    nan = W.bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(W.bits_to_f32(nan)).all()


def test_generators_are_deterministic_and_bf16_exact():
    a = W.fwd_inputs(1, 4, 2, 33, 65, 64, seed=7)
    b = W.fwd_inputs(1, 4, 2, 33, 65, 64, seed=7)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
        assert np.array_equal(W.bf16_round(x), x)
    c = W.fwd_inputs(1, 4, 2, 33, 65, 64, seed=8)
    assert not np.array_equal(a[0], c[0])
    f = W.fwd_inputs(1, 1, 1, 8, 8, 64, seed=1, dtype="f32")
    assert not np.array_equal(W.bf16_round(f[0]), f[0])


def test_decode_layout_is_a_permutation_with_poisoned_tails():
    d = W.decode_inputs(B=9, Hq=8, Hkv=2, D=16, block_size=16, ctx_lo=1, ctx_hi=70, seed=3)
    nblk = (d.ctx_lens + 15) // 16
    used = np.concatenate([d.block_table[b, :nblk[b]] for b in range(9)])
    assert sorted(used.tolist()) == list(range(d.k_cache.shape[0]))   # each block used once
    for b in range(9):
        assert np.all(d.block_table[b, nblk[b]:] == -1)
        tail = d.ctx_lens[b] - (nblk[b] - 1) * 16
        last = d.block_table[b, nblk[b] - 1]
        assert np.all(d.k_cache[last, :, tail:, :] == W.POISON_FINITE)
        assert np.all(d.v_cache[last, :, tail:, :] == W.POISON_FINITE)
        assert np.all(np.abs(d.k_cache[last, :, :tail, :]) < 100)
    d2 = W.decode_inputs(B=9, Hq=8, Hkv=2, D=16, block_size=16, ctx_lo=1, ctx_hi=70, seed=3)
    assert d2.k_cache.tobytes() == d.k_cache.tobytes()


def test_decode_config_recipe_seed_1004():
    """The paged-decode recipe: context lengths uniform in [512, 4096], 16-token blocks."""
    cfg = W.CONFIGS["paged_decode_b64"]
    rng = np.random.default_rng(cfg.seed)
    ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi, size=cfg.B, endpoint=True)
    assert ctx.min() >= 512 and ctx.max() <= 4096
    nblk = (ctx + 15) // 16
    assert int(ctx.sum()) == 152235 and int(nblk.sum()) == 9545 and int(nblk.max()) == 256


def test_workload_shapes_match_the_pages():
    g = _golden()
    c3 = W.CONFIGS["batched_b8_s4096"]
    it = g["batched_score_tensor"]
    assert (c3.B, c3.Hq, c3.Sq) == (it["B"], it["H"], it["S"])
    assert c3.B * c3.Hq * c3.Sq * c3.Sk > it["elements_more_than"]
    c5 = W.CONFIGS["long_s32768"]
    it = g["long_context_score_matrix"]
    assert c5.Sq >= it["T"] and it["T"] * it["T"] > it["entries_more_than"]
    it = g["llama3_8b_projection_widths"]
    for name in ("llama3_8b_prefill", "paged_decode_b64"):
        c = W.CONFIGS[name]
        assert c.Hq * c.D == it["q_out"] and c.Hkv * c.D == it["k_out"] == it["v_out"]
        assert (c.Hq + 2 * c.Hkv) * c.D == it["qkv_out"]
    rows = g["llama3_8b_fusion_table"]["rows"]
    for r in rows:   # the table's TPS column is 1000 / ms: a per-token (decode-step) time
        assert abs(1000.0 / r["ms"] - r["tps"]) < 0.06


def test_sample_rows_cover_edges():
    rows = W.sample_rows(2, 4, 100, 20, seed=1, must=(63, 64, 99))
    assert len(rows) == 20 and (0, 0, 0) in rows and (1, 3, 99) in rows
    assert {63, 64}.issubset({i for _, _, i in rows})


def test_norm_inputs_are_bf16_exact_and_seeded():
    x, r, w = W.norm_inputs(5, 24, seed=3)
    assert x.shape == (5, 24) and r.shape == (5, 24) and w.shape == (24,)
    for a in (x, r, w):
        assert a.dtype == np.float32
        assert np.array_equal(W.bf16_round(a), a)
    x2, r2, w2 = W.norm_inputs(5, 24, seed=3)
    assert np.array_equal(x, x2) and np.array_equal(r, r2) and np.array_equal(w, w2)
    assert abs(float(w.mean()) - 1.0) < 0.2
    cfg = W.NORM_CONFIGS["add_rms_norm_64x8192"]
    assert (cfg.M, cfg.d, cfg.eps) == (64, 8192, 1e-6)


def test_norm_workload_is_the_pages_tensor():
    it = _golden()["add_rms_norm_tensor"]
    c = W.NORM_CONFIGS["add_rms_norm_64x8192"]
    assert (c.M, c.d, c.eps) == (it["M"], it["d"], it["eps"]) and it["dtype"] == "bf16"
