"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This module draws and lays out input data only: random normals, their rounding to
bfloat16, and the paged KV-cache layout with its block table. It contains none of the
attention arithmetic, so the CPU oracle and the HIP path stay independent of each other
while still seeing bit-identical inputs.

Workload shapes follow the pages:
  * the Llama-3-8B-shaped prefill (32 query heads, 8 KV heads, head size 128) matches the
    projection widths given in "Kernel and Operator Fusion -- Inference Optimization", §5
    (the horizontal QKV fusion example: 4096 -> 4096 for Q, 4096 -> 1024 for K and V);
  * the batched B=8, H=32, S=4096 case is the score tensor of more than four billion elements
    in "Kernel Fusion, Softmax, and Attention", third paragraph;
  * the 32K-token case is the T x T score matrix of more than a billion entries in
    "Optimizing Large Language Model Inference Through Kernel Fusion and Advanced Memory
    Management", §FlashAttention and the Memory-Efficiency Revolution;
  * the chunked prefill (the §8(f) N3 step) splits a prompt into chunks that each attend to
    everything before them; prefill and decode as different schedules of one equation are in
    "Kernel Fusion, Softmax, and Attention", fifth paragraph;
  * the paged decode layout (fixed-size blocks, a block table mapping a sequence's logical
    blocks to physical ones) is the one in §Paged Attention and Dynamic KV Cache Management
    of that same article;
  * the residual-add RMS norm is measured on a (64, 8192) bfloat16 tensor in "Kernel and
    Operator Fusion -- Inference Optimization", §4; the other two shapes are the Llama-3-8B
    hidden width (4096, the projection input width of §5) over a 2048-token prefill, and an
    8192-wide hidden state over 16384 tokens for a bandwidth-bound size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "FwdConfig", "DecodeConfig", "CONFIGS", "bf16_round", "bf16_bits", "bits_to_f32",
    "fwd_inputs", "decode_inputs", "DecodeInputs", "sample_rows", "PagedPrefillInputs",
    "paged_prefill_inputs", "PagedPrefillConfig", "PAGED_PREFILL_CONFIGS",
    "paged_prefill_inputs_for", "NormConfig", "NORM_CONFIGS",
    "norm_inputs", "norm_inputs_for", "rope_inputs",
]


# ----------------------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even) done with integer bit operations.
# ----------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Return the uint16 bfloat16 bit patterns of float32 ``x`` under round-to-nearest-even.

    NaN inputs map to a quiet NaN. Infinities and values that round past the largest finite
    bfloat16 become infinities, as IEEE rounding requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb, in place in 32 bits: it cannot wrap for a finite value (the largest
    # magnitude pattern 0xFF7FFFFF plus 0x8000 stays below 2^32); NaN patterns are redone below
    r = (u >> 16) & 1
    r += u
    r += 0x7FFF
    r >>= 16
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 and return them as (exact) float32."""
    return bits_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------------------
@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    dtype: str          # "bf16" or "f32": the type of Q, K, V and O
    causal: bool
    seed: int
    input_scale: float = 1.0   # N(0,1) draws are multiplied by this before rounding
    kind: str = field(default="fwd")

    @property
    def scale(self) -> np.float32:
        """Softmax scale 1/sqrt(D) as the float32 value handed to the library."""
        return np.float32(1.0 / math.sqrt(self.D))


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    ctx_lo: int
    ctx_hi: int
    seed: int
    dtype: str = "bf16"
    kind: str = field(default="decode")

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.D))


CONFIGS = {
    "tiny_f32": FwdConfig("tiny_f32", B=1, Hq=1, Hkv=1, Sq=128, Sk=128, D=64,
                          dtype="f32", causal=False, seed=1001),
    "llama3_8b_prefill": FwdConfig("llama3_8b_prefill", B=1, Hq=32, Hkv=8, Sq=2048, Sk=2048,
                                   D=128, dtype="bf16", causal=True, seed=1002),
    "batched_b8_s4096": FwdConfig("batched_b8_s4096", B=8, Hq=32, Hkv=32, Sq=4096, Sk=4096,
                                  D=128, dtype="bf16", causal=True, seed=1003),
    "paged_decode_b64": DecodeConfig("paged_decode_b64", B=64, Hq=32, Hkv=8, D=128,
                                     block_size=16, ctx_lo=512, ctx_hi=4096, seed=1004),
    "long_s32768": FwdConfig("long_s32768", B=1, Hq=32, Hkv=8, Sq=32768, Sk=32768, D=128,
                             dtype="bf16", causal=True, seed=1005, input_scale=0.5),
    # a prefill chunk: the last 512 tokens of a 4096-token prompt attend to the whole prefix
    # (bottom-right causal), as a chunked prefill step does
    "chunked_prefill_512_of_4096": FwdConfig("chunked_prefill_512_of_4096", B=1, Hq=32, Hkv=8,
                                             Sq=512, Sk=4096, D=128, dtype="bf16",
                                             causal=True, seed=1009),
}


# ----------------------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, dtype: str, input_scale: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if input_scale != 1.0:
        x *= np.float32(input_scale)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def fwd_inputs(B, Hq, Hkv, Sq, Sk, D, seed, dtype="bf16", input_scale=1.0):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Sk,D] as float32 arrays, drawn in the order Q, K, V.

    For ``dtype="bf16"`` every value is already rounded to bfloat16 (RNE), so handing the
    arrays to either side is exact.
    """
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, Hq, Sq, D), dtype, input_scale)
    k = _normal(rng, (B, Hkv, Sk, D), dtype, input_scale)
    v = _normal(rng, (B, Hkv, Sk, D), dtype, input_scale)
    return q, k, v


def fwd_inputs_for(cfg: FwdConfig):
    return fwd_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Sq, cfg.Sk, cfg.D, cfg.seed,
                      cfg.dtype, cfg.input_scale)


@dataclass
class DecodeInputs:
    q: np.ndarray            # [B, Hq, D] float32 (bf16-exact)
    k_cache: np.ndarray      # [num_blocks, Hkv, block_size, D] float32 (bf16-exact)
    v_cache: np.ndarray      # same shape as k_cache
    block_table: np.ndarray  # [B, max_blocks] int32, -1 past a sequence's last block
    ctx_lens: np.ndarray     # [B] int32
    block_size: int


POISON_FINITE = np.float32(1.0e4)


def decode_inputs(B, Hq, Hkv, D, block_size, ctx_lo, ctx_hi, seed, ctx_lens=None,
                  poison="finite", dtype="bf16", extra_blocks=0):
    """Paged KV cache for one-token decode.

    Draw order: context lengths (uniform integers in [ctx_lo, ctx_hi], unless ``ctx_lens``
    is given), a permutation of the physical block pool, then q, k_cache and v_cache from
    N(0,1). Sequence b owns ceil(ctx_b / block_size) blocks; its logical block j lives in
    physical block ``perm[offset_b + j]``. Slots past the end of a sequence's last block are
    overwritten with ``poison`` ("finite" = 1e4, "nan" = NaN, None = left as drawn), so a
    kernel that reads them shows it. ``extra_blocks`` adds unused physical blocks to the pool.
    """
    rng = np.random.default_rng(seed)
    if ctx_lens is None:
        ctx = rng.integers(ctx_lo, ctx_hi, size=B, endpoint=True).astype(np.int32)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int32).copy()
        assert ctx.shape == (B,)
    nblk = (ctx.astype(np.int64) + block_size - 1) // block_size
    pool = int(nblk.sum()) + int(extra_blocks)
    perm = rng.permutation(pool).astype(np.int32)
    max_blocks = max(1, int(nblk.max()) if B else 1)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = perm[off:off + n]
        off += n
    q = _normal(rng, (B, Hq, D), dtype, 1.0)
    kc = _normal(rng, (pool, Hkv, block_size, D), dtype, 1.0)
    vc = _normal(rng, (pool, Hkv, block_size, D), dtype, 1.0)
    if poison is not None:
        val = POISON_FINITE if poison == "finite" else np.float32(np.nan)
        for b in range(B):
            n = int(nblk[b])
            tail = int(ctx[b]) - (n - 1) * block_size   # valid slots in the last block
            if n > 0 and tail < block_size:
                pb = table[b, n - 1]
                kc[pb, :, tail:, :] = val
                vc[pb, :, tail:, :] = val
    return DecodeInputs(q, kc, vc, table, ctx, block_size)


def decode_inputs_for(cfg: DecodeConfig, **kw):
    return decode_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.block_size, cfg.ctx_lo,
                         cfg.ctx_hi, cfg.seed, **kw)


@dataclass
class PagedPrefillInputs:
    q: np.ndarray            # [T, Hq, D] float32 (bf16-exact), sequences packed token-major
    k_cache: np.ndarray      # [num_blocks, Hkv, 16, D] float32 (bf16-exact)
    v_cache: np.ndarray
    block_table: np.ndarray  # [B, stride] int32, -1 past a sequence's last block
    cu_seqlens_q: np.ndarray # [B + 1] int32
    ctx_lens: np.ndarray     # [B] int32, keys per sequence (its new tokens included)
    block_size: int


def paged_prefill_inputs(Hq, Hkv, D, q_lens, ctx_lens, seed, poison="finite", extra_blocks=0,
                         table_stride=None):
    """A chunked-prefill step over a paged cache: sequence b has ctx_lens[b] keys in the cache,
    of which its last q_lens[b] are the new tokens whose queries are packed into q.

    The cache, block table and poisoned tails are drawn exactly as decode_inputs draws them
    (same seed); q comes from a second generator seeded with seed + 7919, N(0,1) rounded to
    bf16. ``table_stride`` widens the table (extra entries -1), as a serving stack that sizes
    its tables for the longest context does."""
    B = len(ctx_lens)
    d = decode_inputs(B, Hq, Hkv, D, 16, 0, 0, seed, ctx_lens=ctx_lens, poison=poison,
                      extra_blocks=extra_blocks)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    assert q_lens.shape == (B,)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    rng = np.random.default_rng(seed + 7919)
    q = _normal(rng, (int(cu[-1]), Hq, D), "bf16", 1.0)
    table = d.block_table
    if table_stride is not None and table_stride > table.shape[1]:
        wide = np.full((B, table_stride), -1, dtype=np.int32)
        wide[:, :table.shape[1]] = table
        table = wide
    return PagedPrefillInputs(q, d.k_cache, d.v_cache, table, cu, d.ctx_lens, 16)


@dataclass(frozen=True)
class PagedPrefillConfig:
    name: str
    Hq: int
    Hkv: int
    D: int
    q_lens: tuple
    ctx_lens: tuple
    seed: int
    causal: bool = True
    kind: str = field(default="paged_prefill")

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.D))


PAGED_PREFILL_CONFIGS = {
    # the chunked-prefill step through the paged cache: the last 512 tokens of a 4096-token
    # prompt, whose keys and values (the chunk's included) sit in 16-token blocks of the pool
    "paged_prefill_512_of_4096": PagedPrefillConfig(
        "paged_prefill_512_of_4096", Hq=32, Hkv=8, D=128, q_lens=(512,), ctx_lens=(4096,),
        seed=1010),
    # a mixed batch of chunks of eight sequences, as a scheduler that batches the prefill
    # chunks of several requests forms it: chunk lengths and contexts of all sizes, ragged ends
    "paged_prefill_varlen_b8": PagedPrefillConfig(
        "paged_prefill_varlen_b8", Hq=32, Hkv=8, D=128,
        q_lens=(512, 64, 1024, 300, 128, 2048, 17, 707),
        ctx_lens=(4096, 8192, 1024, 2000, 3000, 2048, 6000, 5000), seed=1011),
}


def paged_prefill_inputs_for(cfg: PagedPrefillConfig, **kw):
    return paged_prefill_inputs(cfg.Hq, cfg.Hkv, cfg.D, cfg.q_lens, cfg.ctx_lens, cfg.seed, **kw)


def sample_rows(B, Hq, Sq, n, seed, must=()):
    """Pick ``n`` distinct (b, h, i) query rows to check one by one at full size.

    Always includes the first and last rows of every tile edge listed in ``must`` (pairs of
    row indices) and the global first and last rows; the rest are uniform random.
    """
    rng = np.random.default_rng(seed)
    picks = {(0, 0, 0), (B - 1, Hq - 1, Sq - 1)}
    for i in must:
        if 0 <= i < Sq:
            picks.add((int(rng.integers(B)), int(rng.integers(Hq)), int(i)))
    while len(picks) < n:
        picks.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Sq))))
    return sorted(picks)


# ----------------------------------------------------------------------------------------
# Residual-add RMS norm inputs
# ----------------------------------------------------------------------------------------
@dataclass(frozen=True)
class NormConfig:
    name: str
    M: int          # rows (tokens)
    d: int          # row length (hidden size)
    seed: int
    eps: float = 1e-6
    kind: str = "norm"


NORM_CONFIGS = {
    "add_rms_norm_64x8192": NormConfig("add_rms_norm_64x8192", M=64, d=8192, seed=1006),
    "add_rms_norm_2048x4096": NormConfig("add_rms_norm_2048x4096", M=2048, d=4096, seed=1007),
    "add_rms_norm_16384x8192": NormConfig("add_rms_norm_16384x8192", M=16384, d=8192,
                                          seed=1008),
}


def norm_inputs(M, d, seed):
    """x and residual [M, d] ~ N(0, 1) and weight [d] ~ 1 + 0.1 N(0, 1), drawn in that order
    and rounded to bfloat16 (returned as exact float32 arrays)."""
    rng = np.random.default_rng(seed)
    x = bf16_round(rng.standard_normal(size=(M, d), dtype=np.float32))
    r = bf16_round(rng.standard_normal(size=(M, d), dtype=np.float32))
    w = bf16_round(np.float32(1.0) + np.float32(0.1) * rng.standard_normal(size=d,
                                                                          dtype=np.float32))
    return x, r, w


def norm_inputs_for(cfg: NormConfig):
    return norm_inputs(cfg.M, cfg.d, cfg.seed)


# ----------------------------------------------------------------------------------------
# RoPE + cache-write inputs
# ----------------------------------------------------------------------------------------
def rope_inputs(T, Hq, Hkv, D, seed):
    """Per-token projections q [T, Hq, D], k and v [T, Hkv, D] ~ N(0, 1), drawn in that order
    and rounded to bfloat16 (returned as exact float32 arrays)."""
    rng = np.random.default_rng(seed)
    q = bf16_round(rng.standard_normal(size=(T, Hq, D), dtype=np.float32))
    k = bf16_round(rng.standard_normal(size=(T, Hkv, D), dtype=np.float32))
    v = bf16_round(rng.standard_normal(size=(T, Hkv, D), dtype=np.float32))
    return q, k, v
