"""Paged prefill on the GPU (attn_fwd_paged): packed query chunks of several sequences against
their contexts in the paged cache, compared with the fp64 oracle (the oracle gathers each
context through the block table and applies the plain definition) on every output element.
Covers ragged chunk and context ends, NaN in every cache slot past a context, grouped heads,
both head sizes, both masks, the key-range split path and the unsplit one, chunks longer than
max_q, empty chunks and contexts, rows that see no key, a table wider than any context and a
block outside the pool; and the two workloads the bench times, in full."""
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


def upload(x, dev):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return (bf(x.q), bf(x.k_cache), bf(x.v_cache), i32(x.block_table), i32(x.cu_seqlens_q),
            i32(x.ctx_lens))


def run(x, dev, causal, scale, max_q=None, max_ctx=None, check_blocks=True, table=None,
        workspace=None):
    q, kc, vc, bt, cu, ctx = upload(x, dev)
    if table is not None:
        bt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(dev)
    ql = np.diff(x.cu_seqlens_q)
    max_q = int(ql.max()) if max_q is None else max_q
    max_ctx = int(np.max(x.ctx_lens)) if max_ctx is None else max_ctx
    o, lse = A.attn_fwd_paged(q, kc, vc, bt, cu, ctx, max_q, max_ctx, causal=causal,
                              scale=float(scale), check_blocks=check_blocks,
                              workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def check(x, o, lse, causal, scale, num_blocks=0, table=None, what=""):
    O, L = oracle.prefill_paged(x.q, x.k_cache, x.v_cache,
                                x.block_table if table is None else table, x.cu_seqlens_q,
                                x.ctx_lens, 16, causal=causal, scale=scale,
                                num_blocks=num_blocks)
    mx, mn = check_bf16(to_np(o), O, what=what)
    err = check_lse(to_np(lse), L, what=what + " LSE")
    print(f"{what}: O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}")


# (Hq, Hkv, D, chunk lengths, context lengths, causal): several tiles, ragged ends
SMALL = [
    (8, 2, 128, (300,), (1000,), True),                        # few tiles: key-range splits
    (8, 2, 128, (300,), (1000,), False),
    (4, 4, 64, (1, 129, 0, 77), (1, 500, 33, 77), True),       # whole prompts, an empty chunk
    (16, 1, 128, (64, 200), (5000, 200), False),                # 16 query heads per KV head
    (32, 8, 128, (512, 384, 256, 130), (4096, 400, 1024, 130), True),   # enough tiles: unsplit
    (32, 8, 64, (512, 384, 256, 130), (4096, 400, 1024, 130), True),
    (8, 8, 128, (100,), (40,), True),                           # 60 rows see no key
    (4, 2, 64, (10, 5), (0, 5), True),                          # a sequence with no context
    (2, 1, 128, (1000, 3), (1000, 1003), True),                 # a long whole prompt
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"h{c[0]}-{c[1]}-d{c[2]}-q{c[3]}-k{c[4]}"
                         f"-{'causal' if c[5] else 'full'}")
def test_paged_prefill_small(dev, case):
    Hq, Hkv, D, ql, kl, causal = case
    x = W.paged_prefill_inputs(Hq, Hkv, D, ql, kl, seed=3000 + sum(ql) + sum(kl), poison="nan",
                               extra_blocks=5)
    scale = np.float32(1 / np.sqrt(D))
    o, lse = run(x, dev, causal, scale)
    check(x, o, lse, causal, scale, what=f"paged {case}")


def test_paged_prefill_wraps_past_max_q(dev):
    """max_q only sizes the grid: a chunk longer than it is still computed whole."""
    x = W.paged_prefill_inputs(8, 2, 128, (700, 20), (900, 4000), seed=3101, poison="nan")
    scale = np.float32(1 / np.sqrt(128))
    o, lse = run(x, dev, True, scale, max_q=128)
    check(x, o, lse, True, scale, what="max_q 128 for a 700-token chunk")


def test_paged_prefill_wide_table_and_pool_check(dev):
    """A table preallocated wider than any context; one entry inside a context points outside
    the pool: with the pool size passed, that block's keys take no part (as in the oracle);
    entries past the contexts are never read."""
    x = W.paged_prefill_inputs(8, 4, 128, (64, 200, 33), (300, 700, 33), seed=3102,
                               poison="nan", extra_blocks=3, table_stride=97)
    pool = x.k_cache.shape[0]
    table = x.block_table.copy()
    table[1, 5] = pool + 11         # inside sequence 1's context
    table[:, 60:] = 1 << 30         # far past every context: must never be read
    scale = np.float32(1 / np.sqrt(128))
    for causal in (True, False):
        o, lse = run(x, dev, causal, scale, table=table, check_blocks=True)
        check(x, o, lse, causal, scale, num_blocks=pool, table=table,
              what=f"pool check, causal={causal}")


def test_paged_prefill_caller_workspace_and_determinism(dev):
    """The split path through a caller workspace equals the library workspace bit for bit,
    and repeated calls are bitwise identical."""
    x = W.paged_prefill_inputs(8, 2, 128, (257,), (3000,), seed=3103, poison="nan")
    scale = np.float32(1 / np.sqrt(128))
    need = A.attn_fwd_paged_workspace_bytes(1, 257, 8, 2, 128, 257, 3000, True)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o1, l1 = run(x, dev, True, scale, workspace=ws)
    o2, l2 = run(x, dev, True, scale)
    o3, l3 = run(x, dev, True, scale)
    assert torch.equal(o1, o2) and torch.equal(o2, o3)
    assert torch.equal(l1, l2) and torch.equal(l2, l3)
    check(x, o1, l1, True, scale, what="caller workspace")


def test_paged_prefill_rows_outside_sequences_untouched(dev):
    """Rows of q that belong to no sequence (past cu_seqlens_q[B]) are not written."""
    x = W.paged_prefill_inputs(4, 2, 64, (50, 70), (60, 300), seed=3104, poison="nan")
    q, kc, vc, bt, cu, ctx = upload(x, dev)
    T = q.shape[0]
    qpad = torch.zeros((T + 9, 4, 64), dtype=torch.bfloat16, device=dev)
    qpad[:T] = q
    o = torch.full_like(qpad, 7.0)
    lse = torch.full((T + 9, 4), 7.0, dtype=torch.float32, device=dev)
    A.attn_fwd_paged(qpad, kc, vc, bt, cu, ctx, 70, 300, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.all(o[T:] == 7.0)) and bool(torch.all(lse[T:] == 7.0))
    check(x, o[:T], lse[:T], True, np.float32(1 / 8), what="padded q")


def random_paged_case(seed):
    """1-6 sequences with random chunk lengths (0-700) over random contexts (the chunk's
    length up to 3000 more), random GQA group and head size, either mask."""
    rng = np.random.default_rng(4000 + seed)
    nseq = int(rng.integers(1, 7))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    ql = [int(x) for x in rng.integers(0, 700, nseq)]
    kl = [q + int(rng.integers(0, 3000)) for q in ql]
    return Hq, Hkv, D, tuple(ql), tuple(kl), bool(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(8))
def test_paged_prefill_random_batches(dev, seed):
    Hq, Hkv, D, ql, kl, causal = random_paged_case(seed)
    x = W.paged_prefill_inputs(Hq, Hkv, D, ql, kl, seed=4100 + seed, poison="nan",
                               extra_blocks=int(seed))
    scale = np.float32(1 / np.sqrt(D))
    o, lse = run(x, dev, causal, scale, max_q=max(1, max(ql)), max_ctx=max(kl))
    check(x, o, lse, causal, scale, what=f"random batch {seed}: Hq={Hq} Hkv={Hkv} D={D} "
          f"q={ql} k={kl} causal={causal}")


@pytest.mark.parametrize("name", list(W.PAGED_PREFILL_CONFIGS))
def test_paged_prefill_workloads(dev, name):
    """The bench's paged-prefill workloads at full size, every element against the oracle."""
    cfg = W.PAGED_PREFILL_CONFIGS[name]
    x = W.paged_prefill_inputs_for(cfg)
    o, lse = run(x, dev, cfg.causal, cfg.scale)
    check(x, o, lse, cfg.causal, cfg.scale, what=name)


def test_paged_chunk_equals_contiguous_chunk(dev):
    """A 512-token chunk over 4096 keys with D = 64 through the paged cache and through the
    contiguous forward (same keys gathered into [B, Hkv, S, D]): both run the tile kernel's
    arithmetic with the same key ranges, so they agree bit for bit. (With D = 128 the contiguous
    forward takes such a chunk on the wide kernel instead, which rounds in another order.)"""
    x = W.paged_prefill_inputs(32, 8, 64, (512,), (4096,), seed=1012)
    scale = np.float32(1 / np.sqrt(64))
    o, lse = run(x, dev, True, scale)
    K = oracle.gather_paged(x.k_cache, x.block_table, 4096, 0, 16)[None]
    V = oracle.gather_paged(x.v_cache, x.block_table, 4096, 0, 16)[None]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(
        torch.bfloat16)
    qd = bf(np.transpose(x.q, (1, 0, 2))[None])
    od, ld = A.attn_fwd(qd, bf(K), bf(V), causal=True, scale=float(scale))
    torch.cuda.synchronize()
    assert torch.equal(o, od[0].transpose(0, 1).contiguous())
    assert torch.equal(lse, ld[0].transpose(0, 1).contiguous())
    check(x, o, lse, True, scale, what="paged D=64 chunk")
