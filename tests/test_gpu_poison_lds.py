"""The LDS-poisoning check build against the normal library on the GPU.

libattn_poison.so is the same sources compiled with -DATTN_POISON_LDS: every kernel first fills
the LDS arrays it uses with 0xff bytes (NaN as fp32 and as bf16). The kernels are written so
that no output depends on an LDS byte they did not write themselves: K/V stages past a context
or past Sk, stages that staged Q before their first tile or O after their last, the dummy block
before a wide loop's first, decode slots of blocks outside the pool. So both builds must give
the same bits on every output, here for every kernel family of the library: the wide forward (with key-range splits
and cross-XCD item taking), the paired-tile and the tile forwards, the fp32 forward, the paged
prefill, the paged decode, RoPE + cache store and the residual-add RMS norm. A difference
means a read of a byte no instruction of the kernel wrote (a race, or a missing clear), which
a normal build may hide whenever the stale bytes happen to be finite.
"""
import os

import numpy as np
import pytest
import torch

import exact_attention_42_amd as A
import oracle
import workloads as W
from tests.parity import check_bf16, check_lse, to_np

pytestmark = pytest.mark.gpu

POISON_LIB = os.path.join(os.path.dirname(A.__file__), "libattn_poison.so")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def libs():
    """(normal, poisoned) handles; the binding is pointed at one or the other per call."""
    assert os.path.exists(POISON_LIB), f"{POISON_LIB} is missing: run __graft_entry__.build()"
    normal = A.load_library()
    saved_path = A._LIB_PATH
    A._lib, A._LIB_PATH = None, POISON_LIB
    try:
        poisoned = A.load_library()
    finally:
        A._lib, A._LIB_PATH = normal, saved_path
    return normal, poisoned


def both(libs, fn):
    """fn() through each build; returns the two results (tensors or tuples of them), each
    copied to the host after a synchronisation."""
    out = []
    saved = A._lib
    try:
        for lib in libs:
            A._lib = lib
            r = fn()
            torch.cuda.synchronize()
            r = r if isinstance(r, tuple) else (r,)
            out.append(tuple(x.detach().cpu().clone() for x in r))
    finally:
        A._lib = saved
    return out


def assert_same_bits(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape and x.dtype == y.dtype, f"{what}[{i}]"
        xb = x.contiguous().view(torch.uint8)
        yb = y.contiguous().view(torch.uint8)
        n = int((xb != yb).sum())
        assert n == 0, f"{what}[{i}]: {n} bytes differ between the normal and poisoned builds"


def bf(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)


def i32(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)


# (mapping, B, Hq, Hkv, Sq, Sk, D, causal): ragged tails, one query, Sq above and below Sk,
# GQA, key-range splits (few tiles), and a wide case with more items than CUs (item taking)
FWD = [
    ("wide", 1, 2, 1, 300, 300, 128, True),
    ("wide", 1, 2, 2, 1, 777, 128, True),
    ("wide", 1, 2, 1, 300, 100, 128, True),
    ("wide", 1, 2, 2, 513, 2000, 128, False),
    ("wide", 1, 32, 8, 512, 4096, 128, True),      # key-range splits + combine
    ("wide", 2, 48, 8, 768, 768, 128, True),       # more items than CUs: cross-XCD taking
    ("pair", 4, 8, 4, 1000, 1000, 128, True),
    ("pair", 2, 8, 2, 900, 400, 64, True),
    ("tile", 2, 4, 2, 200, 330, 128, False),
    ("tile", 1, 8, 2, 333, 333, 64, True),
    ("tile", 1, 8, 8, 257, 3000, 128, True),       # few tiles: key-range splits
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "-".join(map(str, c)))
def test_forward_bits_match(case, dev, libs):
    mapping, B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = W.fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed=7000 + Sq + Sk + D)
    g = [bf(x, dev) for x in (q, k, v)]
    scale = float(1 / np.sqrt(D))

    def run():
        prev = A.attn_fwd_force_mapping(mapping)
        try:
            return A.attn_fwd(*g, causal=causal, scale=scale)
        finally:
            A.attn_fwd_force_mapping(prev)

    a, b = both(libs, run)
    assert_same_bits(a, b, f"attn_fwd {case}")
    if B * Hq * Sq * Sk <= 2 ** 24:   # (and the normal build against the oracle where cheap)
        O, L = oracle.attention(q, k, v, causal=causal, scale=np.float32(scale))
        check_bf16(a[0].float().numpy(), O, what=f"{case} O")
        check_lse(a[1].numpy(), L, what=f"{case} LSE")


def test_forward_f32_bits_match(dev, libs):
    q, k, v = W.fwd_inputs(1, 4, 2, 150, 290, 64, seed=7101)
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    g = [f(x) for x in (q, k, v)]
    a, b = both(libs, lambda: A.attn_fwd_f32(*g, causal=True))
    assert_same_bits(a, b, "attn_fwd_f32")


@pytest.mark.parametrize("case", [
    (8, 2, 128, (300,), (1000,), True),                  # few tiles: key-range splits
    (4, 4, 64, (1, 129, 0, 77), (1, 500, 33, 77), True),
    (32, 8, 128, (512, 384, 256, 130), (4096, 400, 1024, 130), True),
    (8, 8, 128, (100,), (40,), False),
], ids=lambda c: f"h{c[0]}-{c[1]}-d{c[2]}-q{c[3]}-k{c[4]}")
def test_paged_prefill_bits_match(case, dev, libs):
    Hq, Hkv, D, ql, kl, causal = case
    x = W.paged_prefill_inputs(Hq, Hkv, D, ql, kl, seed=7200 + sum(ql) + sum(kl), poison="nan",
                               extra_blocks=3)
    t = (bf(x.q, dev), bf(x.k_cache, dev), bf(x.v_cache, dev), i32(x.block_table, dev),
         i32(x.cu_seqlens_q, dev), i32(x.ctx_lens, dev))
    mq, mk = max(1, max(ql)), max(kl)
    a, b = both(libs, lambda: A.attn_fwd_paged(*t, mq, mk, causal=causal))
    assert_same_bits(a, b, f"attn_fwd_paged {case}")


def test_paged_prefill_wrap_bits_match(dev, libs):
    """max_q below a chunk's length: each workgroup computes several query tiles in turn, and
    the stages that held one tile's O are loaded again for the next."""
    x = W.paged_prefill_inputs(8, 2, 128, (700, 20), (900, 4000), seed=7250, poison="nan")
    t = (bf(x.q, dev), bf(x.k_cache, dev), bf(x.v_cache, dev), i32(x.block_table, dev),
         i32(x.cu_seqlens_q, dev), i32(x.ctx_lens, dev))
    for causal in (True, False):
        a, b = both(libs, lambda: A.attn_fwd_paged(*t, 128, 4000, causal=causal))
        assert_same_bits(a, b, f"attn_fwd_paged max_q=128 causal={causal}")


@pytest.mark.parametrize("workers", [0, 100])
def test_decode_bits_match(workers, dev, libs):
    """NaN in every cache slot past a context; a block-table entry outside the pool; the
    default worker count and a small one (long shares, several rounds of descriptions)."""
    d = W.decode_inputs(B=16, Hq=32, Hkv=8, D=128, block_size=16, ctx_lo=1, ctx_hi=900,
                        seed=7300 + workers, poison="nan")
    q, kc, vc, bt, cl = (bf(d.q, dev), bf(d.k_cache, dev), bf(d.v_cache, dev),
                         i32(d.block_table, dev), i32(d.ctx_lens, dev))
    bt[3, 1] = kc.shape[0] + 5   # outside the pool: its keys take no part
    a, b = both(libs, lambda: A.attn_decode_paged_full(q, kc, vc, bt, cl, num_workers=workers))
    assert_same_bits(a, b, f"attn_decode_paged_full workers={workers}")


def test_rope_cache_and_norm_bits_match(dev, libs):
    d = W.decode_inputs(B=8, Hq=32, Hkv=8, D=128, block_size=16, ctx_lo=16, ctx_hi=300,
                        seed=7400)
    q, k, v = W.rope_inputs(8, 32, 8, 128, seed=7401)
    pos = i32(d.ctx_lens.astype(np.int64) - 1, dev)
    table = i32(d.block_table, dev)

    def rope():
        kc, vc = bf(d.k_cache, dev), bf(d.v_cache, dev)
        qo = A.rope_cache_write(bf(q, dev), bf(k, dev), bf(v, dev), pos, kc, vc, table)
        return qo, kc, vc

    a, b = both(libs, rope)
    assert_same_bits(a, b, "rope_cache_write")

    x, r, w = W.norm_inputs(33, 5120, seed=7402)
    gx, gr, gw = bf(x, dev), bf(r, dev), bf(w, dev)
    a, b = both(libs, lambda: A.add_rms_norm(gx, gr, gw))
    assert_same_bits(a, b, "add_rms_norm")
