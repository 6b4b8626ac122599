"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check that
at least one pin fails. This is what makes the pins a check of the oracle rather than a
restatement of it: a dropped term, a wrong sign or index, a transposed operand, a wrong log
base or mask offset each has to trip something.
"""
import numpy as np
import pytest

import oracle.direct as OA
import oracle.rmsnorm as ON
import oracle.rotary as OR
from tests import pins


def _rows_mutant(kind):
    def rows(qrows, rows_idx, K, V, causal, offset, scale):
        Sk = K.shape[0]
        s = scale
        if kind == "no_scale":
            s = 1.0
        if kind == "scale_sqrt":
            s = np.sqrt(scale)
        S = s * (qrows @ K.T)
        if kind == "wrong_sign":
            S = -S
        if causal:
            keys = np.arange(Sk)[None, :]
            if kind == "causal_strict":
                visible = keys < (rows_idx[:, None] + offset)
            elif kind == "causal_topleft":
                visible = keys <= rows_idx[:, None]
            elif kind == "causal_transposed":
                visible = keys >= (rows_idx[:, None] + offset)
            else:
                visible = keys <= (rows_idx[:, None] + offset)
            if kind != "mask_after_softmax":
                S = np.where(visible, S, -np.inf)
        m = S.max(axis=1) if Sk else np.full(S.shape[0], -np.inf)
        empty = ~np.isfinite(m)
        m_safe = np.where(empty, 0.0, m)
        if kind == "no_max_sub":
            with np.errstate(over="ignore"):
                P = np.exp(S)
        elif kind == "exp2":
            P = np.exp2(S - m_safe[:, None])
        else:
            P = np.exp(S - m_safe[:, None])
        l = P.sum(axis=1)
        if kind == "mask_after_softmax" and causal:
            P = np.where(visible, P, 0.0)
        with np.errstate(invalid="ignore", divide="ignore"):
            if kind == "no_normalize":
                O = P @ V
            elif kind == "values_from_keys":
                O = (P @ K[:, :V.shape[1]]) / l[:, None] if K.shape[1] >= V.shape[1] else (P @ V) / l[:, None] * 0
            else:
                O = (P @ V) / l[:, None]
            if kind == "lse_log2":
                lse = m_safe + np.log2(l)
            elif kind == "lse_no_max":
                lse = np.log(l)
            elif kind == "lse_no_log":
                lse = m_safe + l
            else:
                lse = m_safe + np.log(l)
        O[empty] = 0.0
        if kind != "empty_lse_zero":
            lse[empty] = -np.inf
        else:
            lse[empty] = 0.0
        return O, lse
    return rows


ROW_MUTANTS = ["no_scale", "scale_sqrt", "wrong_sign", "causal_strict", "causal_topleft",
               "causal_transposed", "mask_after_softmax", "no_max_sub", "exp2", "no_normalize",
               "values_from_keys", "lse_log2", "lse_no_max", "lse_no_log", "empty_lse_zero"]


def _gqa_mutant(q, k, v, causal=False, scale=None):
    """attention() with query head h reading KV head h % Hkv (interleaved, not grouped)."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    s = float(np.float32(scale if scale is not None else 1 / np.sqrt(D)))
    O = np.zeros((B, Hq, Sq, v.shape[3]))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            o, lse = OA._rows(q[b, h].astype(np.float64), np.arange(Sq), k[b, h % Hkv],
                              v[b, h % Hkv], causal, Sk - Sq, s)
            O[b, h], L[b, h] = o, lse
    return O, L


def _gather_mutant(kind):
    def gather(cache, block_table, ctx_len, b, block_size):
        n = ctx_len + 1 if kind == "one_past_end" else ctx_len
        t = np.arange(n)
        if kind == "swap_block_slot":
            phys = block_table[b, t % block_size]
            slot = t // block_size % block_size
        elif kind == "table_row_by_slot":
            phys = block_table[b, np.minimum(t // block_size + (t % block_size == block_size - 1), block_table.shape[1] - 1)]
            slot = t % block_size
        elif kind == "physical_is_logical":
            phys = t // block_size
            slot = t % block_size
        else:
            phys = block_table[b, t // block_size]
            slot = t % block_size
        return np.transpose(cache[phys, :, slot, :], (1, 0, 2))
    return gather


def _prefill_mutant(kind):
    """prefill_paged with one planted mistake (the pool check is left out of every mutant but
    the one that ignores it, which is what the pins exercise it with)."""
    real = OA.prefill_paged

    def prefill(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, block_size,
                causal=True, scale=None, num_blocks=0):
        if kind == "pool_check_ignored":
            return real(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, block_size,
                        causal=causal, scale=scale, num_blocks=0)
        if num_blocks > 0:
            return real(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, block_size,
                        causal=causal, scale=scale, num_blocks=num_blocks)
        T, Hq, D = q.shape
        O = np.zeros((T, Hq, v_cache.shape[3]))
        L = np.full((T, Hq), -np.inf)
        for b in range(len(ctx_lens)):
            r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            if kind == "rows_shifted":
                r0, r1 = min(r0 + 1, T), min(r1 + 1, T)
            n, ctx = r1 - r0, int(ctx_lens[b])
            if kind == "context_excludes_chunk":
                ctx -= n
            if n <= 0 or ctx <= 0:
                continue
            qb = np.transpose(q[r0:r1], (1, 0, 2))[None]
            Kb = OA.gather_paged(k_cache, block_table, ctx, b, block_size)[None]
            Vb = OA.gather_paged(v_cache, block_table, ctx, b, block_size)[None]
            if kind == "mask_top_left" and causal:
                # queries placed at positions 0 .. n-1 instead of the context's last ones
                Sq = qb.shape[2]
                pad = np.zeros((1, Hq, ctx - Sq, D)) if ctx > Sq else np.zeros((1, Hq, 0, D))
                o, lse = OA.attention(np.concatenate([qb, pad], axis=2)[:, :, :max(ctx, Sq)],
                                      Kb, Vb, causal=True, scale=scale)
                o, lse = o[:, :, :Sq], lse[:, :, :Sq]
            else:
                o, lse = OA.attention(qb, Kb, Vb, causal=causal and kind != "mask_ignored",
                                      scale=scale)
            O[r0:r1] = np.transpose(o[0], (1, 0, 2))
            L[r0:r1] = lse[0].T
        return O, L
    return prefill


PREFILL_MUTANTS = ["pool_check_ignored", "rows_shifted", "context_excludes_chunk",
                   "mask_top_left", "mask_ignored"]


@pytest.mark.parametrize("kind", PREFILL_MUTANTS)
def test_prefill_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(OA, "prefill_paged", _prefill_mutant(kind))
    assert "pin_prefill_paged" in _some_pin_fails()


def test_unmutated_prefill_copy_passes(monkeypatch):
    monkeypatch.setattr(OA, "prefill_paged", _prefill_mutant("none"))
    assert _some_pin_fails() == []


def _some_pin_fails():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("kind", ROW_MUTANTS)
def test_row_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(OA, "_rows", _rows_mutant(kind))
    assert _some_pin_fails(), f"no pin catches mutant {kind}"


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(OA, "_rows", _rows_mutant("none"))
    assert _some_pin_fails() == []


def test_gqa_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(OA, "attention", _gqa_mutant)
    assert "pin_gqa" in _some_pin_fails()


@pytest.mark.parametrize("kind", ["one_past_end", "swap_block_slot", "table_row_by_slot",
                                  "physical_is_logical"])
def test_gather_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(OA, "gather_paged", _gather_mutant(kind))
    assert "pin_decode_paged" in _some_pin_fails()


def _norm_mutant(kind):
    def add_rms_norm(x, residual, weight, eps=1e-6):
        x = np.asarray(x, dtype=np.float64)
        r = np.asarray(residual, dtype=np.float64)
        w = np.asarray(weight, dtype=np.float64)
        t = x - r if kind == "residual_sub" else x + r
        d = t.shape[-1]
        if kind == "sum_not_mean":
            ms = np.sum(t * t, axis=-1, keepdims=True)
        elif kind == "d_minus_1":
            ms = np.sum(t * t, axis=-1, keepdims=True) / (d - 1)
        elif kind == "centred":
            ms = np.var(t, axis=-1, keepdims=True)
        else:
            ms = np.mean(t * t, axis=-1, keepdims=True)
        if kind == "no_eps":
            inv = 1.0 / np.sqrt(ms)
        elif kind == "eps_outside":
            inv = 1.0 / np.sqrt(ms) + eps
        elif kind == "no_sqrt":
            inv = 1.0 / (ms + eps)
        else:
            inv = 1.0 / np.sqrt(ms + eps)
        out = t * inv
        if kind == "weight_added":
            out = out + w
        elif kind != "no_weight":
            out = out * w
        if kind == "returns_input":
            return out, x
        return out, t
    return add_rms_norm


NORM_MUTANTS = ["residual_sub", "sum_not_mean", "d_minus_1", "centred", "no_eps",
                "eps_outside", "no_sqrt", "weight_added", "no_weight", "returns_input"]


@pytest.mark.parametrize("kind", NORM_MUTANTS)
def test_norm_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ON, "add_rms_norm", _norm_mutant(kind))
    failed = [f for f in _some_pin_fails() if f.startswith("pin_norm")]
    assert failed, f"no pin catches mutant {kind}"


def test_unmutated_norm_copy_passes(monkeypatch):
    monkeypatch.setattr(ON, "add_rms_norm", _norm_mutant("none"))
    assert _some_pin_fails() == []


def _rope_mutant(kind):
    def rope(x, positions, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        T, H, D = x.shape
        half = D // 2
        i = np.arange(half, dtype=np.float64)
        if kind == "theta_half_exponent":
            theta = np.power(float(base), -1.0 * i / D)
        elif kind == "theta_positive":
            theta = np.power(float(base), 2.0 * i / D)
        else:
            theta = np.power(float(base), -2.0 * i / D)
        p = np.asarray(positions, dtype=np.float64) + (1 if kind == "position_plus_one" else 0)
        ang = p[:, None] * theta[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        if kind == "sin_sign":
            s = -s
        if kind == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            y = np.empty_like(x)
            y[..., 0::2] = x1 * c - x2 * s
            y[..., 1::2] = x2 * c + x1 * s
            return y
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return rope


ROPE_MUTANTS = ["theta_half_exponent", "theta_positive", "position_plus_one", "sin_sign",
                "interleaved"]


@pytest.mark.parametrize("kind", ROPE_MUTANTS)
def test_rope_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(OR, "rope", _rope_mutant(kind))
    failed = [f for f in _some_pin_fails() if f.startswith("pin_rope")]
    assert failed, f"no pin catches mutant {kind}"


def _rope_write_mutant(kind):
    def write(q, k, v, positions, k_cache, v_cache, block_table, seq_ids=None, base=10000.0,
              block_size=16, num_blocks=0):
        q_rot = OR.rope(q, positions, base)
        k_rot = OR.rope(k, positions, base) if kind != "key_unrotated" else np.asarray(k, float)
        kc = np.array(k_cache, dtype=np.float64, copy=True)
        vc = np.array(v_cache, dtype=np.float64, copy=True)
        vv = OR.rope(v, positions, base) if kind == "value_rotated" else np.asarray(v, float)
        for t in range(q_rot.shape[0]):
            s = t if seq_ids is None else int(seq_ids[t])
            p = int(positions[t])
            if p < 0 and kind != "negative_written":
                continue
            if p // block_size >= block_table.shape[1] and kind != "past_row_written":
                continue
            if kind == "block_slot_swapped":
                blk, slot = p % block_size, p // block_size
            else:
                blk, slot = p // block_size, p % block_size
            if kind == "seq_map_ignored":
                s = t
            phys = int(block_table[s, min(blk, block_table.shape[1] - 1)])
            if num_blocks > 0 and not (0 <= phys < num_blocks) and kind != "no_range_check":
                continue
            if kind == "no_range_check":
                phys %= k_cache.shape[0]
            kc[phys, :, slot, :] = k_rot[t]
            vc[phys, :, slot, :] = vv[t]
        return q_rot, kc, vc
    return write


ROPE_WRITE_MUTANTS = ["key_unrotated", "value_rotated", "negative_written",
                      "block_slot_swapped", "seq_map_ignored", "no_range_check",
                      "past_row_written"]


@pytest.mark.parametrize("kind", ROPE_WRITE_MUTANTS)
def test_rope_write_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(OR, "rope_cache_write", _rope_write_mutant(kind))
    failed = [f for f in _some_pin_fails() if f.startswith("pin_rope")]
    assert failed, f"no pin catches mutant {kind}"


def test_unmutated_rope_copies_pass(monkeypatch):
    monkeypatch.setattr(OR, "rope", _rope_mutant("none"))
    monkeypatch.setattr(OR, "rope_cache_write", _rope_write_mutant("none"))
    assert _some_pin_fails() == []
