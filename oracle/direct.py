"""Plain, slow, fp64 CPU attention -- the oracle. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
this module; the HIP library never does. It shares no code with the HIP path: the only thing
both sides import is the seeded input generator in ``workloads/``.

What it computes
----------------
The attention equation of "Fused Kernel Compiler" (Candle paper), §FlashAttention
Integration, displayed equation: for each head, softmax(Q K^T / sqrt(d_k)) V. The scale is
taken as an argument (the float32 value handed to the GPU, 1/sqrt(d_k) in every workload) and
an optional causal mask is added to the scaled scores before the softmax (the "scale, mask,
softmax" pattern in that page's Table "Kernel fusion opportunities").

The fused kernel is exact (it reaches this same result up to floating-point rounding order:
"Kernel Fusion, Softmax, and Attention", fifth paragraph; "Optimizing Large Language Model
Inference ...", §The Shift Toward Efficient Inference Architectures). So the oracle is the
plain definition, evaluated the direct way that "Kernel Fusion, Softmax, and Attention"
describes in its third paragraph: the full score row is formed, a softmax is taken over it,
and the probabilities weight the value vectors. Everything is done in float64 on values
that arrive as float32 (bfloat16-exact for the bf16 workloads), so the only rounding is fp64's.

Readings where the pages are silent:
  * mask: none, or causal aligned to the bottom-right corner -- key j is visible to query i
    iff j <= i + (Sk - Sq); identical to the usual top-left rule when Sq == Sk;
  * a row with no visible key has O = 0 and LSE = -inf;
  * LSE (the per-row log-sum-exp) is the natural log of the sum of exp(scaled, masked score);
  * grouped-query heads: query head h reads KV head h // (Hq // Hkv);
  * decode attends the one new query to all ctx_lens[b] cached tokens (no mask inside the
    context); the paged cache holds token t of sequence b in physical block
    block_table[b, t // block_size], slot t % block_size ("Optimizing Large Language Model
    Inference ...", §Paged Attention and Dynamic KV Cache Management).

Memory: the score matrix of one head is built in slabs of complete rows (each row is still
a full, two-pass softmax), so the 32K-token workload fits in host memory. This is memory
chunking only; no row is ever split.
"""
from __future__ import annotations

import numpy as np

_SLAB_BYTES = 128 << 20   # at most this many bytes of fp64 scores per slab


def _rows(qrows, rows_idx, K, V, causal, offset, scale):
    """Attention for a set of query rows of one head, straight from the definition.

    qrows [n, D] fp64, rows_idx [n] (query positions, for the causal mask), K [Sk, D],
    V [Sk, Dv] fp64. Returns O [n, Dv] and LSE [n] in fp64.
    """
    Sk = K.shape[0]
    S = scale * (qrows @ K.T)                           # [n, Sk] raw scores, scaled
    if causal:
        keys = np.arange(Sk)[None, :]
        visible = keys <= (rows_idx[:, None] + offset)  # bottom-right aligned causal mask
        S = np.where(visible, S, -np.inf)
    m = S.max(axis=1) if Sk else np.full(S.shape[0], -np.inf)
    empty = ~np.isfinite(m)                             # rows with no visible key
    m_safe = np.where(empty, 0.0, m)
    P = np.exp(S - m_safe[:, None])                     # exp(-inf) = 0 for masked keys
    l = P.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = (P @ V) / l[:, None]
        lse = m_safe + np.log(l)
    O[empty] = 0.0
    lse[empty] = -np.inf
    return O, lse


def attention(q, k, v, causal=False, scale=None):
    """O = softmax(scale * Q K^T + mask) V and LSE for every row, in float64.

    q [B, Hq, Sq, D]; k [B, Hkv, Sk, D]; v [B, Hkv, Sk, Dv]; Hq a multiple of Hkv.
    ``scale`` defaults to 1/sqrt(D) rounded to float32 (the value the GPU receives).
    Returns O [B, Hq, Sq, Dv] float64 and LSE [B, Hq, Sq] float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    assert Bk == B and Dk == D and v.shape[:3] == (B, Hkv, Sk) and Hq % Hkv == 0
    Dv = v.shape[3]
    if scale is None:
        scale = np.float32(1.0 / np.sqrt(D))
    s = float(np.float64(np.float32(scale)))
    g = Hq // Hkv
    O = np.zeros((B, Hq, Sq, Dv), dtype=np.float64)
    L = np.zeros((B, Hq, Sq), dtype=np.float64)
    slab = max(1, _SLAB_BYTES // max(1, 8 * Sk))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            K = k[b, hk].astype(np.float64)
            V = v[b, hk].astype(np.float64)
            for r0 in range(0, Sq, slab):
                r1 = min(Sq, r0 + slab)
                idx = np.arange(r0, r1)
                o, lse = _rows(q[b, h, r0:r1].astype(np.float64), idx, K, V, causal,
                               Sk - Sq, s)
                O[b, h, r0:r1] = o
                L[b, h, r0:r1] = lse
    return O, L


def attention_rows(q, k, v, rows, causal=False, scale=None):
    """The same definition evaluated only at the listed (b, h, i) query rows.

    Used to check full-size workloads whose complete output the CPU cannot afford. The rows
    of one head are evaluated together (complete score rows, in slabs, exactly as in
    ``attention``), so K and V of a head are widened to float64 once.
    Returns O [n, Dv] and LSE [n] in float64, in the order of ``rows``.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = np.float32(1.0 / np.sqrt(D))
    s = float(np.float64(np.float32(scale)))
    g = Hq // Hkv
    outO = np.zeros((len(rows), v.shape[3]), dtype=np.float64)
    outL = np.zeros(len(rows), dtype=np.float64)
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((int(b), int(h)), []).append((n, int(i)))
    slab = max(1, _SLAB_BYTES // max(1, 8 * Sk))
    for (b, h), items in by_head.items():
        hk = h // g
        K = k[b, hk].astype(np.float64)
        V = v[b, hk].astype(np.float64)
        pos = np.array([n for n, _ in items])
        idx = np.array([i for _, i in items])
        for r0 in range(0, len(idx), slab):
            r1 = min(len(idx), r0 + slab)
            o, lse = _rows(q[b, h, idx[r0:r1]].astype(np.float64), idx[r0:r1], K, V, causal,
                           Sk - Sq, s)
            outO[pos[r0:r1]] = o
            outL[pos[r0:r1]] = lse
    return outO, outL


def gather_paged(cache, block_table, ctx_len, b, block_size):
    """Logical [Hkv, ctx_len, D] view of sequence b, read through its block-table row."""
    t = np.arange(ctx_len)
    phys = block_table[b, t // block_size]
    slot = t % block_size
    return np.transpose(cache[phys, :, slot, :], (1, 0, 2))   # [Hkv, ctx, D]


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, block_size, scale=None):
    """One-token decode over a paged KV cache, in float64.

    q [B, Hq, D]; k_cache, v_cache [num_blocks, Hkv, block_size, D]; block_table [B, *]
    int32; ctx_lens [B]. Each sequence's cached tokens are gathered through the block table
    (logical block -> physical block) and attended with no mask. Returns O [B, Hq, D] and
    LSE [B, Hq] in float64. A sequence with ctx_len == 0 gets O = 0, LSE = -inf.
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    O = np.zeros((B, Hq, v_cache.shape[3]), dtype=np.float64)
    L = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(ctx_lens[b])
        if n == 0:
            continue
        Kb = gather_paged(k_cache, block_table, n, b, block_size)[None]
        Vb = gather_paged(v_cache, block_table, n, b, block_size)[None]
        o, lse = attention(q[b][None, :, None, :], Kb, Vb, causal=False, scale=scale)
        O[b] = o[0, :, 0, :]
        L[b] = lse[0, :, 0]
    return O, L


def prefill_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, block_size,
                  causal=True, scale=None, num_blocks=0):
    """Prefill of packed query tokens against a paged KV cache, in float64.

    Prefill and decode are two schedules of one attention ("Kernel Fusion, Softmax, and
    Attention", fifth paragraph); here the new tokens of each sequence attend to its cached
    context, read through its block table ("Optimizing Large Language Model Inference ...",
    §Paged Attention and Dynamic KV Cache Management).

    q [T, Hq, D], sequence b owning rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; caches
    [num_blocks, Hkv, block_size, D]; block_table [B, *]; ctx_lens [B] keys per sequence, its
    own query tokens being the last of them. Each sequence's context is gathered through the
    table and its queries attend to it with the plain definition (``attention``), the causal
    mask aligned to the bottom right (query i of n sits at position ctx - n + i). With
    num_blocks > 0, the keys of a block whose table entry lies outside [0, num_blocks), or
    that has no entry in the table's row, take no part. Returns O [T, Hq, D] and LSE [T, Hq];
    rows that belong to no sequence stay O = 0, LSE = -inf.
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    O = np.zeros((T, Hq, v_cache.shape[3]), dtype=np.float64)
    L = np.full((T, Hq), -np.inf, dtype=np.float64)
    for b in range(len(ctx_lens)):
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n, ctx = r1 - r0, int(ctx_lens[b])
        if n <= 0:
            continue
        qb = np.transpose(q[r0:r1], (1, 0, 2))[None]           # [1, Hq, n, D]
        if ctx <= 0:
            continue                                            # no keys: O = 0, LSE = -inf
        keep = np.ones(ctx, dtype=bool)
        if num_blocks > 0:
            t = np.arange(ctx)
            lb = t // block_size
            has = lb < block_table.shape[1]
            phys = np.where(has, block_table[b, np.minimum(lb, block_table.shape[1] - 1)], -1)
            keep = has & (phys >= 0) & (phys < num_blocks)
        idx = np.nonzero(keep)[0]
        if num_blocks > 0 and len(idx) < ctx:
            # some keys take no part: attend each row over the kept keys it can see
            t = np.arange(ctx)
            safe = np.where(keep, t, 0)
            Kb = np.transpose(k_cache[block_table[b, safe // block_size], :, safe % block_size, :],
                              (1, 0, 2))
            Vb = np.transpose(v_cache[block_table[b, safe // block_size], :, safe % block_size, :],
                              (1, 0, 2))
            for i in range(n):
                pos = ctx - n + i
                vis = keep & ((t <= pos) if causal else True)
                sel = np.nonzero(vis)[0]
                o, lse = attention(qb[:, :, i:i + 1, :], Kb[None][:, :, sel, :],
                                   Vb[None][:, :, sel, :], causal=False, scale=scale)
                O[r0 + i] = o[0, :, 0, :]
                L[r0 + i] = lse[0, :, 0]
            continue
        Kb = gather_paged(k_cache, block_table, ctx, b, block_size)[None]
        Vb = gather_paged(v_cache, block_table, ctx, b, block_size)[None]
        o, lse = attention(qb, Kb, Vb, causal=causal, scale=scale)
        O[r0:r1] = np.transpose(o[0], (1, 0, 2))
        L[r0:r1] = lse[0].T
    return O, L

