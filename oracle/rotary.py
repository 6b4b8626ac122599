"""Plain fp64 CPU rotary position embedding and paged KV-cache write -- the oracle.
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
this module; the HIP library never does. It shares no code with the HIP path.

What it computes: the step that precedes decode attention, "RoPE then KV store" fused into one
pass ("Kernel and Operator Fusion -- Inference Optimization", §2, item 6; the table of kernel
fusion opportunities in "Fused Kernel Compiler" (Candle paper) lists RoPE as sin, cos,
rotate). The pages name the operation but print no formula, so the reading taken is the usual
rotary embedding in its rotate-half form: for a head vector x of length D and position p,
  theta_i = base^(-2 i / D),  a_i = p * theta_i,         i = 0 .. D/2 - 1
  y_i         = x_i cos a_i - x_{i+D/2} sin a_i
  y_{i+D/2}   = x_{i+D/2} cos a_i + x_i sin a_i
applied to every query head and every key head of the token; values are not rotated. The
rotated key and the value of token t of sequence s at position p are then stored into the
paged cache [num_blocks, Hkv, block_size, D] at physical block block_table[s, p // block_size],
slot p % block_size ("Optimizing Large Language Model Inference ...", §Paged Attention and
Dynamic KV Cache Management) -- the layout the paged decode reads.
"""
from __future__ import annotations

import numpy as np


def rope(x, positions, base=10000.0):
    """x [T, H, D] (any float dtype), positions [T] ints. Returns the rotated x in float64."""
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / D)                     # [D/2]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]   # [T, D/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_cache_write(q, k, v, positions, k_cache, v_cache, block_table, seq_ids=None,
                     base=10000.0, block_size=16, num_blocks=0):
    """Rotates q [T, Hq, D] and k [T, Hkv, D] by their token's position, then stores the
    rotated k and the unrotated v of token t into the caches (copies, float64) at the slot
    its sequence's block table gives. Tokens whose position is negative or lies past the end
    of the table row, or whose table entry falls outside [0, num_blocks) when num_blocks > 0,
    leave the caches untouched.
    Returns (q_rot, k_cache_out, v_cache_out)."""
    q_rot = rope(q, positions, base)
    k_rot = rope(k, positions, base)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    v = np.asarray(v, dtype=np.float64)
    for t in range(q_rot.shape[0]):
        s = t if seq_ids is None else int(seq_ids[t])
        p = int(positions[t])
        if p < 0 or p // block_size >= block_table.shape[1]:
            continue
        phys = int(block_table[s, p // block_size])
        if num_blocks > 0 and not (0 <= phys < num_blocks):
            continue
        kc[phys, :, p % block_size, :] = k_rot[t]
        vc[phys, :, p % block_size, :] = v[t]
    return q_rot, kc, vc
