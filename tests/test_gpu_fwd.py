"""Forward parity on the GPU: the HIP kernels behind attn_fwd / attn_fwd_f32 against the
fp64 oracle on identical seeded inputs (rounded to bf16 first for the bf16 path).

Small shapes are compared element by element over every output and span several 128-query
and 64-key tiles plus ragged tails. Of the full-size workloads, the Llama-3-8B-shaped prefill
and the batched B=8, S=4096 one are compared on every element; the 32K-token one on one row
of every 32-row slice of every head (every unit of work), and everywhere on properties that
hold at any size.
"""
import numpy as np
import pytest
import torch

import exact_attention_42_amd as A
import oracle
import workloads as W
from tests.parity import check_bf16, check_f32, check_lse, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _gpu(x, dev, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dtype)


def run_bf16(q, k, v, causal, scale, dev):
    o, lse = A.attn_fwd(_gpu(q, dev, torch.bfloat16), _gpu(k, dev, torch.bfloat16),
                        _gpu(v, dev, torch.bfloat16), causal=causal, scale=float(scale))
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


SMALL = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 1, 1, 128, 128, 128, False),
    (1, 1, 1, 128, 128, 128, True),
    (2, 4, 2, 200, 200, 128, True),       # ragged q and k tails, GQA 2:1
    (2, 4, 2, 200, 200, 128, False),
    (1, 8, 2, 333, 333, 64, True),        # D = 64, GQA 4:1
    (1, 2, 2, 257, 257, 64, False),
    (1, 2, 1, 100, 300, 128, True),       # Sq < Sk: bottom-right causal alignment
    (1, 2, 1, 300, 100, 128, True),       # Sq > Sk: the first 200 rows see no key
    (1, 2, 2, 1, 777, 128, True),         # one query, a decode-like row
    (1, 2, 2, 70, 1, 128, False),         # one key
    (3, 2, 1, 129, 63, 64, False),        # Sk below one tile
    (1, 4, 4, 512, 512, 128, True),       # several full tiles, MHA (key-range splits)
    # with this few query tiles, causal calls split their key ranges when there are enough key
    # tiles (the first, third and fourth here) and run the paired-tile kernel otherwise
    (1, 2, 1, 1100, 1100, 128, True),     # 9 tiles
    (1, 2, 1, 900, 400, 128, True),       # Sq > Sk: whole light tiles see no key (paired)
    (1, 8, 2, 1000, 1000, 64, True),      # D = 64, GQA 4:1
    (2, 2, 2, 640, 700, 128, True),       # Sq < Sk, ragged heavy tail
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_fwd_bf16_small(shape, dev):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed=hash(shape) % 2**31)
    scale = np.float32(1 / np.sqrt(D))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    check_bf16(o, O)
    check_lse(lse, L)


def random_pair_shape(seed):
    """A causal shape that runs the paired-tile kernel: at most 64 query tiles per head and
    enough query tiles in all (B * Hq * tiles >= 1.5 x the CUs) that the call does not split
    its key ranges. Drawn from a seeded generator: odd and even tile counts, Sq above or below
    Sk (both signs of the diagonal offset), ragged tails, D = 64 or 128, GQA 1:1 to 4:1."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.choice([4, 8]))
    Hkv = int(rng.choice([4, 8]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    min_tiles = -(-3 * cus // (2 * B * Hq))          # ceil(1.5 CUs / (B Hq))
    Sq = int(rng.integers(128 * (min_tiles - 1) + 1, 128 * (min_tiles + 3) + 1))
    Sk = int(rng.integers(1, 2 * Sq + 64))
    return B, Hq, Hkv, Sq, Sk, D


@pytest.mark.parametrize("seed", range(12))
def test_fwd_pair_kernel_random_shapes(seed, dev):
    """Sampled rows (every query tile's first and last rows among them) against the oracle."""
    B, Hq, Hkv, Sq, Sk, D = random_pair_shape(seed)
    ntq = -(-Sq // 128)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ntq <= 64 and 2 * B * Hq * ntq >= 3 * cus     # the paired-tile kernel runs
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed=900 + seed)
    scale = np.float32(1 / np.sqrt(D))
    o, lse = run_bf16(q, k, v, True, scale, dev)
    edges = [e for t in range(ntq) for e in (128 * t, 128 * t + 31, 128 * t + 32, 128 * t + 127)]
    rows = W.sample_rows(B, Hq, Sq, 96 + len(edges), seed=seed, must=edges)
    O, L = oracle.attention_rows(q, k, v, rows, causal=True, scale=scale)
    idx = tuple(np.array(rows).T)
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D}"
    check_bf16(o[idx], O, what=what + " sampled O")
    check_lse(lse[idx], L, what=what + " sampled LSE")


def random_split_shape(seed):
    """Seeds 0-6: few query tiles against up to 3000 keys, causal or not -- calls with fewer
    query tiles than the CUs can take split their key ranges (a second kernel merges the
    ranges). Seeds 7-9: enough query tiles (B=2, 16 heads, ~1600 rows) for the one-range-per-
    tile kernel, non-causal."""
    rng = np.random.default_rng(700 + seed)
    if seed >= 7:
        return (2, 16, 4, int(rng.integers(1536, 1800)), int(rng.integers(100, 1200)),
                int(rng.choice([64, 128])), False)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    Sq = int(rng.integers(1, 700))
    Sk = int(rng.integers(1, 3000))
    causal = bool(rng.integers(0, 2))
    return B, Hq, Hkv, Sq, Sk, D, causal


@pytest.mark.parametrize("seed", range(10))
def test_fwd_split_and_tile_random_shapes(seed, dev):
    B, Hq, Hkv, Sq, Sk, D, causal = random_split_shape(seed)
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed=1100 + seed)
    scale = np.float32(1 / np.sqrt(D))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal}"
    check_bf16(o, O, what=what + " O")
    check_lse(lse, L, what=what + " LSE")


@pytest.mark.parametrize("shape", [(1, 1, 1, 128, 128, 64, False), (2, 4, 2, 200, 150, 128, True),
                                   (1, 2, 1, 77, 300, 64, True), (1, 2, 2, 300, 90, 128, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fwd_f32_small(shape, dev):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed=7 + Sq, dtype="f32")
    scale = np.float32(1 / np.sqrt(D))
    o, lse = A.attn_fwd_f32(_gpu(q, dev, torch.float32), _gpu(k, dev, torch.float32),
                            _gpu(v, dev, torch.float32), causal=causal, scale=float(scale))
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    check_f32(to_np(o), O)
    check_lse(to_np(lse), L, tol=1e-5)


def test_config_tiny_f32(dev):
    """B=1, H=1, S=128, D=64, fp32, non-causal: every output element."""
    cfg = W.CONFIGS["tiny_f32"]
    q, k, v = W.fwd_inputs_for(cfg)
    o, lse = A.attn_fwd_f32(_gpu(q, dev, torch.float32), _gpu(k, dev, torch.float32),
                            _gpu(v, dev, torch.float32), causal=cfg.causal, scale=float(cfg.scale))
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, causal=cfg.causal, scale=cfg.scale)
    check_f32(to_np(o), O)
    check_lse(to_np(lse), L, tol=1e-5)


def test_config_llama3_8b_prefill_full(dev):
    """B=1, Hq=32, Hkv=8, S=2048, D=128, bf16, causal: every output element."""
    cfg = W.CONFIGS["llama3_8b_prefill"]
    q, k, v = W.fwd_inputs_for(cfg)
    o, lse = run_bf16(q, k, v, cfg.causal, cfg.scale, dev)
    O, L = oracle.attention(q, k, v, causal=cfg.causal, scale=cfg.scale)
    mx, mn = check_bf16(o, O)
    err = check_lse(lse, L)
    print(f"llama3_8b_prefill: O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}")


def test_config_chunked_prefill_full(dev):
    """A chunked-prefill step: the last 512 of 4096 tokens (Hq=32, Hkv=8, D=128, bf16)
    against the whole prefix, bottom-right causal: every output element."""
    cfg = W.CONFIGS["chunked_prefill_512_of_4096"]
    q, k, v = W.fwd_inputs_for(cfg)
    o, lse = run_bf16(q, k, v, cfg.causal, cfg.scale, dev)
    O, L = oracle.attention(q, k, v, causal=cfg.causal, scale=cfg.scale)
    mx, mn = check_bf16(o, O)
    err = check_lse(lse, L)
    print(f"chunked_prefill_512_of_4096: O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}")


def _oracle_threads(fn, jobs, threads=8):
    """Runs independent oracle evaluations on a pool of host threads (numpy releases the GIL
    in its kernels), each with a small BLAS thread count so the pool does not oversubscribe
    the host."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=2):
        with ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(lambda j: fn(*j), jobs))


def _run_full_size(cfg, dev):
    q, k, v = W.fwd_inputs_for(cfg)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    o, lse = A.attn_fwd(qg, kg, vg, causal=cfg.causal, scale=float(cfg.scale))
    torch.cuda.synchronize()
    # properties at every position: finite; each O row is a convex combination of V rows
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    g = cfg.Hq // cfg.Hkv
    vmax = vg.float().amax(dim=2).repeat_interleave(g, dim=1)    # [B, Hq, D]
    vmin = vg.float().amin(dim=2).repeat_interleave(g, dim=1)
    assert bool((o.float() <= vmax[:, :, None, :] + 2e-2).all())
    assert bool((o.float() >= vmin[:, :, None, :] - 2e-2).all())
    # causal row 0 sees key 0 only: O = V_0 exactly (one weight of 1), LSE = scale q_0 . k_0
    if cfg.causal and cfg.Sq == cfg.Sk:
        assert torch.equal(o[:, :, 0], vg.repeat_interleave(g, dim=1)[:, :, 0])
        s0 = np.float64(cfg.scale) * np.einsum(
            "bhd,bhd->bh", q[:, :, 0].astype(np.float64),
            np.repeat(k[:, :, 0], g, axis=1).astype(np.float64))
        assert np.max(np.abs(lse[:, :, 0].cpu().numpy() - s0)) <= 1e-3
    return q, k, v, o, lse


def test_config_batched_b8_s4096_full(dev):
    """B=8, H=32, S=4096, D=128, bf16, causal: every output element against the oracle (the
    oracle runs batch entry by batch entry on a pool of host threads)."""
    cfg = W.CONFIGS["batched_b8_s4096"]
    q, k, v, o, lse = _run_full_size(cfg, dev)
    res = _oracle_threads(
        lambda b: oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=cfg.causal,
                                   scale=cfg.scale), [(b,) for b in range(cfg.B)])
    O = np.concatenate([r[0] for r in res])
    L = np.concatenate([r[1] for r in res])
    mx, mn = check_bf16(to_np(o), O, what="batched_b8_s4096 O")
    err = check_lse(to_np(lse), L, what="batched_b8_s4096 LSE")
    print(f"batched_b8_s4096: every element: O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}")


def test_config_long_s32768_every_wave_slice(dev):
    """B=1, Hq=32, Hkv=8, S=32768, D=128, bf16 x0.5, causal: one row out of every 32-row slice
    of every head (a seeded random row in each slice; 32,768 rows, every (head, 32-row) unit
    of work), plus the last row of every head, against the oracle."""
    cfg = W.CONFIGS["long_s32768"]
    q, k, v, o, lse = _run_full_size(cfg, dev)
    rng = np.random.default_rng(cfg.seed)
    rows = []
    for h in range(cfg.Hq):
        picks = np.arange(0, cfg.Sq, 32) + rng.integers(0, 32, size=cfg.Sq // 32)
        rows.extend((0, h, int(i)) for i in picks)
        rows.append((0, h, cfg.Sq - 1))
    heads = [[r for r in rows if r[1] == h] for h in range(cfg.Hq)]
    res = _oracle_threads(
        lambda rr: oracle.attention_rows(q, k, v, rr, causal=cfg.causal, scale=cfg.scale),
        [(rr,) for rr in heads])
    rows = [r for rr in heads for r in rr]
    O = np.concatenate([r[0] for r in res])
    L = np.concatenate([r[1] for r in res])
    idx = tuple(np.array(rows).T)
    mx, mn = check_bf16(to_np(o)[idx], O, what="long_s32768 O (one row per 32-row slice)")
    err = check_lse(to_np(lse)[idx], L, what="long_s32768 LSE")
    print(f"long_s32768: {len(rows)} rows: O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}")


def test_long_causal_head_full(dev):
    """A causal shape with more than 64 query tiles of 128 rows per head, enough work that the
    keys are not split (B=1, Hq=6, Hkv=3, S=8320): every output element."""
    q, k, v = W.fwd_inputs(1, 6, 3, 8320, 8320, 128, seed=8320)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, True, scale, dev)
    res = _oracle_threads(
        lambda h: oracle.attention(q[:, h:h + 1], k[:, h // 2:h // 2 + 1],
                                   v[:, h // 2:h // 2 + 1], causal=True, scale=scale),
        [(h,) for h in range(6)])
    O = np.concatenate([r[0] for r in res], axis=1)
    L = np.concatenate([r[1] for r in res], axis=1)
    mx, mn = check_bf16(o, O, what="S=8320 O")
    check_lse(lse, L, what="S=8320 LSE")


@pytest.mark.parametrize("ntiles", [64, 65])
def test_causal_kernel_switch_sampled(ntiles, dev):
    """Causal launches with up to 64 query tiles of 128 rows per head run the paired-tile kernel,
    longer ones the one-tile-per-workgroup kernel; both sides of the switch, on sampled rows."""
    S = 128 * ntiles
    # six query heads: 64 x 6 query tiles are enough that the call does not split key ranges
    Hq = 6
    assert 2 * Hq * ntiles >= 3 * torch.cuda.get_device_properties(0).multi_processor_count
    q, k, v = W.fwd_inputs(1, Hq, 3, S, S, 128, seed=1000 + ntiles)
    o, lse = run_bf16(q, k, v, True, np.float32(1 / np.sqrt(128)), dev)
    edges = [0, 1, 127, 128, S // 2 - 1, S // 2, S // 2 + 127, S - 129, S - 128, S - 1]
    rows = W.sample_rows(1, Hq, S, 96, seed=ntiles, must=edges)
    O, L = oracle.attention_rows(q, k, v, rows, causal=True, scale=np.float32(1 / np.sqrt(128)))
    idx = tuple(np.array(rows).T)
    check_bf16(o[idx], O, what=f"{ntiles} tiles sampled O")
    check_lse(lse[idx], L, what=f"{ntiles} tiles sampled LSE")


def test_scale_zero_and_no_keys(dev):
    q, k, v = W.fwd_inputs(1, 2, 1, 130, 90, 128, seed=5)
    o, lse = run_bf16(q, k, v, True, np.float32(0.0), dev)
    O, L = oracle.attention(q, k, v, causal=True, scale=0.0)
    check_bf16(o, O)
    check_lse(lse, L)
    # Sk = 0: every row sees nothing
    qg = _gpu(q, dev, torch.bfloat16)
    e = torch.empty((1, 1, 0, 128), dtype=torch.bfloat16, device=dev)
    o, lse = A.attn_fwd(qg, e, e, causal=False)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_empty_problems(dev):
    e = torch.empty((0, 4, 16, 128), dtype=torch.bfloat16, device=dev)
    o, lse = A.attn_fwd(e, e[:, :2], e[:, :2])
    assert o.shape == (0, 4, 16, 128)
    q = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 2, 5, 64), dtype=torch.bfloat16, device=dev)
    o, lse = A.attn_fwd(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 4, 0, 64)


def test_fwd_is_deterministic(dev):
    """Repeated launches give identical bits (guards the LDS double buffer against races)."""
    q, k, v = W.fwd_inputs(2, 8, 2, 640, 640, 128, seed=9)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    ref, ref_l = A.attn_fwd(qg, kg, vg, causal=True)
    for _ in range(30):
        o, l = A.attn_fwd(qg, kg, vg, causal=True)
        assert torch.equal(o, ref) and torch.equal(l, ref_l)


def test_gqa_equals_repeated_heads(dev):
    q, k, v = W.fwd_inputs(1, 8, 2, 300, 300, 128, seed=10)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    o1, l1 = A.attn_fwd(qg, kg, vg, causal=True)
    o2, l2 = A.attn_fwd(qg, kg.repeat_interleave(4, 1).contiguous(),
                        vg.repeat_interleave(4, 1).contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_row0_is_v0(dev):
    q, k, v = W.fwd_inputs(2, 4, 2, 256, 256, 128, seed=11)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    o, lse = A.attn_fwd(qg, kg, vg, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], vg.repeat_interleave(2, 1)[:, :, 0])


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", [
    (2, 32, 8, 768, 300, False),   # 384 query tiles: one pass over the keys per tile
    (1, 8, 2, 768, 300, False),    # 48 query tiles: key ranges split, then merged
    (2, 32, 8, 768, 2000, True),
    (1, 4, 4, 300, 5000, True),    # a short chunk over a long prefix, heavily split
])
def test_key_split_and_whole_paths(B, Hq, Hkv, Sq, Sk, causal, dev):
    """The forward splits each query tile's keys when the tiles alone cannot fill the device;
    both the split and the whole-range paths match the oracle, with and without the mask."""
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=B * 1000 + Sq + Sk)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    check_bf16(o, O)
    check_lse(lse, L)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", [
    (1, 2, 1, 257, 3001, True),    # a ragged query tile and a partial last key tile
    (1, 2, 2, 513, 2050, False),
    (2, 4, 1, 256, 1000, True),    # 4 query heads per KV head
    (1, 8, 2, 1000, 6000, True),   # eight ranges per query tile
    (1, 3, 3, 600, 600, True),     # Sq = Sk: the last range holds the diagonal
])
def test_wide_key_splits(B, Hq, Hkv, Sq, Sk, causal, dev):
    """Few 256-row query tiles with D = 128: the wide kernel takes the key ranges (one per
    workgroup) and a second kernel merges them; every element against the oracle."""
    assert A.attn_fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, 128, causal) > 0   # (splits)
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=B * 7 + Sq * 3 + Sk)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} causal={causal}"
    check_bf16(o, O, what=what + " O")
    check_lse(lse, L, what=what + " LSE")


@pytest.mark.parametrize("seed", range(6))
def test_wide_key_splits_random(seed, dev):
    """Random few-tile shapes with D = 128 and Sq >= 256 (the wide kernel's key-range splits):
    ragged query and key ends, Sq above and below Sk, both masks, GQA."""
    rng = np.random.default_rng(900 + seed)
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    Sq = int(rng.integers(256, 900))
    Sk = int(rng.integers(1000, 5000))     # (at least 16 key tiles: always split)
    causal = bool(rng.integers(0, 2))
    assert A.attn_fwd_workspace_bytes(1, Hq, Hkv, Sq, Sk, 128, causal) > 0
    q, k, v = W.fwd_inputs(1, Hq, Hkv, Sq, Sk, 128, seed=950 + seed)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    what = f"Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} causal={causal}"
    check_bf16(o, O, what=what + " O")
    check_lse(lse, L, what=what + " LSE")


# ---- the wide kernel (one wave per SIMD, 256-row workgroups) ----

@pytest.fixture
def forced_wide():
    prev = A.attn_fwd_force_mapping("wide")
    yield
    A.attn_fwd_force_mapping(prev)


WIDE_SMALL = [
    # B, Hq, Hkv, Sq, Sk, causal: ragged query and key tails, Sq above and below Sk, GQA, one
    # query, one key, shapes whose waves end 1-3 tiles before their workgroup's last tile
    (1, 1, 1, 256, 256, True), (1, 1, 1, 256, 256, False), (1, 2, 1, 300, 300, True),
    (2, 4, 2, 200, 200, False), (1, 2, 1, 100, 300, True), (1, 2, 1, 300, 100, True),
    (1, 2, 2, 1, 777, True), (1, 2, 2, 70, 1, False), (1, 4, 4, 1000, 1000, True),
    (2, 2, 1, 640, 700, True), (1, 2, 1, 2048, 2048, True), (1, 2, 2, 513, 2000, False),
    (1, 3, 1, 1200, 900, True), (1, 2, 2, 2100, 2100, True), (1, 8, 1, 257, 1025, True),
    (3, 2, 2, 511, 65, True), (1, 1, 1, 64, 64, True), (1, 2, 1, 320, 3000, False),
]


@pytest.mark.parametrize("shape", WIDE_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_fwd_wide_small(shape, dev, forced_wide):
    B, Hq, Hkv, Sq, Sk, causal = shape
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=1234 + Sq + Sk)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    check_bf16(o, O, what=f"{shape} O")
    check_lse(lse, L, what=f"{shape} LSE")


def random_wide_shape(seed):
    """Seeded shapes for the wide kernel: 1-3 batch entries, GQA 1:1 to 8:1, 1-1800 queries
    and 1-3000 keys (both signs of the causal offset), causal or not."""
    rng = np.random.default_rng(4200 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    Sq = int(rng.integers(1, 1800))
    Sk = int(rng.integers(1, 3000))
    causal = bool(rng.integers(0, 2))
    return B, Hq, Hkv, Sq, Sk, causal


@pytest.mark.parametrize("seed", range(12))
def test_fwd_wide_random_shapes(seed, dev, forced_wide):
    B, Hq, Hkv, Sq, Sk, causal = random_wide_shape(seed)
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=5200 + seed)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} causal={causal}"
    check_bf16(o, O, what=what + " O")
    check_lse(lse, L, what=what + " LSE")


# More 256-row items than compute units (B, Hq, Hkv, Sq, Sk, causal), compared in full: two or
# more rounds of workgroups per CU, the last partial; both masks; queries ending before and after
# the keys (the first items of the last case see no key at all); a ragged last query tile; KV
# heads that split evenly over the 8 XCDs (per-XCD bundles) and ones that do not (12).
WIDE_MANY_ITEMS = [
    (2, 48, 8, 768, 768, True), (3, 48, 8, 640, 1088, False), (1, 60, 12, 1280, 1280, True),
    (2, 72, 8, 512, 1216, True), (1, 96, 16, 900, 640, True),
]


@pytest.mark.parametrize("shape", WIDE_MANY_ITEMS, ids=lambda s: "x".join(map(str, s)))
def test_fwd_wide_many_items(shape, dev, forced_wide):
    B, Hq, Hkv, Sq, Sk, causal = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ((Sq + 255) // 256) * B * Hq > cus and Sk % 64 == 0
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=7700 + Sq + Sk + Hq)
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run_bf16(q, k, v, causal, scale, dev)
    O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
    check_bf16(o, O, what=f"{shape} O")
    check_lse(lse, L, what=f"{shape} LSE")


def test_fwd_wide_many_items_is_deterministic(dev, forced_wide):
    """A many-item problem gives identical bits on repeated launches, and each batch entry the
    bits of that entry alone (144 items, a different placement of its items on the XCDs)."""
    q, k, v = W.fwd_inputs(2, 48, 8, 768, 768, 128, seed=21)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    ref, ref_l = A.attn_fwd(qg, kg, vg, causal=True)
    for _ in range(10):
        o, l = A.attn_fwd(qg, kg, vg, causal=True)
        assert torch.equal(o, ref) and torch.equal(l, ref_l)
    o1, l1 = A.attn_fwd(qg[1:].contiguous(), kg[1:].contiguous(), vg[1:].contiguous(),
                        causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[0], ref[1]) and torch.equal(l1[0], ref_l[1])


def test_fwd_wide_many_items_sizes_in_turn(dev, forced_wide):
    """Many-item problems of different sizes launched one after another on one stream with no
    synchronisation between them (fewer items, then more, then fewer again): each output
    matches the oracle's."""
    shapes = [(2, 72, 8, 512, 1216, True), (1, 96, 16, 900, 640, True),
              (2, 48, 8, 768, 768, True), (3, 48, 8, 640, 1088, False),
              (1, 60, 12, 1280, 1280, True)]
    scale = np.float32(1 / np.sqrt(128))
    runs = []
    for i, (B, Hq, Hkv, Sq, Sk, causal) in enumerate(shapes):
        q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, 128, seed=7900 + i)
        o, lse = A.attn_fwd(_gpu(q, dev, torch.bfloat16), _gpu(k, dev, torch.bfloat16),
                            _gpu(v, dev, torch.bfloat16), causal=causal, scale=float(scale))
        runs.append((q, k, v, causal, o, lse))
    torch.cuda.synchronize()
    for (q, k, v, causal, o, lse), shape in zip(runs, shapes):
        O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
        check_bf16(to_np(o), O, what=f"{shape} O")
        check_lse(to_np(lse), L, what=f"{shape} LSE")


def test_fwd_wide_many_items_two_streams(dev, forced_wide):
    """The same many-item problem launched alternately on two streams without synchronising
    between them: every launch gives the bits of a launch alone."""
    q, k, v = W.fwd_inputs(1, 60, 12, 1280, 1280, 128, seed=22)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    ref, ref_l = A.attn_fwd(qg, kg, vg, causal=True)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(6):
        with torch.cuda.stream(streams[i % 2]):
            outs.append(A.attn_fwd(qg, kg, vg, causal=True))
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref) and torch.equal(l, ref_l)


def test_fwd_wide_is_deterministic(dev, forced_wide):
    """Repeated launches give identical bits (the four LDS stages and the spread loads leave no
    race)."""
    q, k, v = W.fwd_inputs(2, 8, 2, 1100, 1100, 128, seed=19)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    ref, ref_l = A.attn_fwd(qg, kg, vg, causal=True)
    for _ in range(30):
        o, l = A.attn_fwd(qg, kg, vg, causal=True)
        assert torch.equal(o, ref) and torch.equal(l, ref_l)


@pytest.mark.parametrize("Sq", [768, 769])
def test_wide_default_switch(Sq, dev):
    """D=128 problems with at least four 256-row work items per CU run the wide kernel by
    default: 4 x 64 heads x ceil(769/256) = 1024 items does (its output equals the forced wide
    kernel's bit for bit), 768 rows (768 items) does not; both sides against the oracle on
    sampled rows."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"the switch point is sized for 256 CUs (this device has {cus})")
    B, Hq, Hkv = 4, 64, 8
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sq, 128, seed=Sq)
    qg, kg, vg = (_gpu(x, dev, torch.bfloat16) for x in (q, k, v))
    scale = float(np.float32(1 / np.sqrt(128)))
    o, lse = A.attn_fwd(qg, kg, vg, causal=True, scale=scale)
    prev = A.attn_fwd_force_mapping("wide")
    try:
        ow, lw = A.attn_fwd(qg, kg, vg, causal=True, scale=scale)
    finally:
        A.attn_fwd_force_mapping(prev)
    torch.cuda.synchronize()
    same = torch.equal(o, ow) and torch.equal(lse, lw)
    assert same == (Sq == 769)
    rows = W.sample_rows(B, Hq, Sq, 128, seed=Sq, must=[0, 255, 256, 511, 512, Sq - 1])
    O, L = oracle.attention_rows(q, k, v, rows, causal=True, scale=np.float32(scale))
    idx = tuple(np.array(rows).T)
    check_bf16(to_np(o)[idx], O, what=f"Sq={Sq} sampled O")
    check_lse(to_np(lse)[idx], L, what=f"Sq={Sq} sampled LSE")


def test_forced_mapping_falls_back(dev):
    """A forced wide mapping with D=64, and a forced pair mapping on a non-causal call, run the
    tile kernel (both still match the oracle)."""
    for mapping, D, causal in (("wide", 64, True), ("pair", 128, False)):
        prev = A.attn_fwd_force_mapping(mapping)
        try:
            q, k, v = W.fwd_inputs(1, 4, 2, 300, 300, D, seed=D)
            scale = np.float32(1 / np.sqrt(D))
            o, lse = run_bf16(q, k, v, causal, scale, dev)
        finally:
            A.attn_fwd_force_mapping(prev)
        O, L = oracle.attention(q, k, v, causal=causal, scale=scale)
        check_bf16(o, O)
        check_lse(lse, L)
