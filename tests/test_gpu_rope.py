"""Fused RoPE + paged KV-cache store on the GPU (attn_rope_cache_write) against the fp64
oracle, and the decode reading what it wrote.

Bar (derived from the arithmetic; the pages give no tolerance for this step): the angle and
its sine and cosine are evaluated in fp64, rounded to fp32, the rotation runs in fp32 and each
output is rounded to bfloat16 once. So a rotated element must be within half a bf16 ulp of
the exact value plus 1e-6 of its pair's magnitude (fp32 cos/sin and products); values are
copied exactly; cache slots that no token maps to must be untouched, bit for bit.
"""
import numpy as np
import pytest
import torch

import exact_attention_42_amd as A
import oracle
import workloads as W
from tests.parity import check_bf16, check_lse, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def half_ulp(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def check_rotated(g, ref, x, what):
    """g, ref, x: [..., D] (GPU result, exact result, unrotated input)."""
    g = np.asarray(g, dtype=np.float64)
    D = x.shape[-1]
    pair = np.abs(x[..., :D // 2]) + np.abs(x[..., D // 2:])
    pair = np.concatenate([pair, pair], axis=-1)
    err = np.abs(g - ref)
    bad = err > half_ulp(ref) + 1e-6 * pair + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {err[bad].max():.3e}"
    return float(err.max())


def run_case(dev, T, Hq, Hkv, D, positions, seq_ids, table, nb, seed, base=10000.0,
             check=True, in_place=False):
    q, k, v = W.rope_inputs(T, Hq, Hkv, D, seed)
    rng = np.random.default_rng(seed + 1)
    kc = W.bf16_round(rng.standard_normal((nb, Hkv, 16, D), dtype=np.float32))
    vc = W.bf16_round(rng.standard_normal((nb, Hkv, 16, D), dtype=np.float32))
    gq, gk, gv, gkc, gvc = bf(q, dev), bf(k, dev), bf(v, dev), bf(kc, dev), bf(vc, dev)
    gout = A.rope_cache_write(gq, gk, gv, i32(positions, dev), gkc, gvc, i32(table, dev),
                              seq_ids=None if seq_ids is None else i32(seq_ids, dev),
                              base=base, check_blocks=check, q_out=gq if in_place else None)
    torch.cuda.synchronize()
    qr, kc2, vc2 = oracle.rope_cache_write(q, k, v, positions, kc, vc, table, seq_ids=seq_ids,
                                           base=base, num_blocks=nb if check else 0)
    check_rotated(to_np(gout), qr, q, "rotated queries")
    gkc_np, gvc_np = to_np(gkc), to_np(gvc)
    # the value cache: copies and untouched slots, exactly
    assert np.array_equal(gvc_np, vc2), "value cache"
    # the key cache: untouched slots exactly, stored slots within the rotation bar
    changed = np.any(kc2 != kc, axis=-1) | np.any(vc2 != vc, axis=-1)      # [nb, Hkv, 16]
    assert np.array_equal(gkc_np[~changed], kc2[~changed]), "untouched key slots"
    if changed.any():
        kx = np.zeros_like(kc2)
        kr = oracle.rope(k, positions, base)
        for t in range(T):
            p = int(positions[t])
            s = t if seq_ids is None else int(seq_ids[t])
            if p < 0 or p // 16 >= table.shape[1]:
                continue
            phys = int(table[s, p // 16])
            if check and not (0 <= phys < nb):
                continue
            kx[phys, :, p % 16, :] = k[t]
            assert np.allclose(kc2[phys, :, p % 16, :], kr[t])
        check_rotated(gkc_np[changed], kc2[changed], kx[changed], "stored keys")
    return gq, gkc, gvc, qr, kc2, vc2


def test_rope_decode_step_b64(dev):
    """The decode workload's step: one new token per sequence at position ctx - 1, stored into
    its own slot of the seed-1004 cache."""
    cfg = W.CONFIGS["paged_decode_b64"]
    d = W.decode_inputs_for(cfg)
    pos = d.ctx_lens.astype(np.int32) - 1
    nb = d.k_cache.shape[0]
    run_case(dev, cfg.B, cfg.Hq, cfg.Hkv, cfg.D, pos, None, d.block_table, nb, seed=61)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (128, 16, 1)])
def test_rope_prefill_chunk_one_sequence(D, Hq, Hkv, dev):
    """A 300-token chunk of one sequence (positions 500..799) through a sequence map."""
    T, nb = 300, 64
    table = np.random.default_rng(3).permutation(nb).astype(np.int32)[None, :]
    pos = np.arange(500, 500 + T, dtype=np.int32)
    run_case(dev, T, Hq, Hkv, D, pos, np.zeros(T, np.int32), table, nb, seed=62 + D)


def test_rope_skips_and_in_place(dev):
    """Negative positions, rows past the table, out-of-pool entries (checked) store nothing;
    the queries are rotated anyway, here in place; a large position and base 500000."""
    T, Hq, Hkv, D, nb = 6, 4, 2, 128, 5
    table = np.array([[0, 1], [2, 9], [3, 4], [1, 0], [4, 4], [2, 3]], dtype=np.int32)
    pos = np.array([5, 17, -3, 40, 31, 2], dtype=np.int32)     # token 3: row 2 > stride
    run_case(dev, T, Hq, Hkv, D, pos, None, table, nb, seed=63, in_place=True)
    big = np.array([1_000_003, 262_147, 7, 0, 31, 16], dtype=np.int32)
    tbl = np.repeat((np.arange(6) % nb).astype(np.int32)[:, None], 1_000_003 // 16 + 1, axis=1)
    run_case(dev, T, Hq, Hkv, D, big, None, tbl, nb, seed=64, base=500000.0)


def test_rope_then_decode_reads_the_store(dev):
    """Write the new token of every sequence with RoPE, then decode with the rotated queries:
    equals the oracle decode over the oracle's cache and rotated queries."""
    d = W.decode_inputs(B=12, Hq=32, Hkv=8, D=128, block_size=16, ctx_lo=1, ctx_hi=900,
                        seed=65)
    B = 12
    pos = d.ctx_lens.astype(np.int32) - 1
    q, k, v = W.rope_inputs(B, 32, 8, 128, seed=66)
    gq, gk, gv = bf(q, dev), bf(k, dev), bf(v, dev)
    gkc, gvc = bf(d.k_cache, dev), bf(d.v_cache, dev)
    gbt, gcl = i32(d.block_table, dev), i32(d.ctx_lens, dev)
    qr_g = A.rope_cache_write(gq, gk, gv, i32(pos, dev), gkc, gvc, gbt)
    o, lse = A.attn_decode_paged_full(qr_g, gkc, gvc, gbt, gcl)
    torch.cuda.synchronize()
    qr, kc2, vc2 = oracle.rope_cache_write(q, k, v, pos, d.k_cache, d.v_cache, d.block_table)
    # the decode's operands are bf16 tensors: the rotated queries and the stored keys are held
    # at bf16 on both sides (the oracle's own values, rounded), so the attention bar applies
    qr_b = W.bf16_round(qr.astype(np.float32))
    kc2_b = W.bf16_round(kc2.astype(np.float32))
    O, L = oracle.decode_paged(qr_b, kc2_b, vc2, d.block_table, d.ctx_lens, 16)
    check_bf16(to_np(o), O)
    check_lse(to_np(lse), L)
