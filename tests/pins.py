"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, not by the oracle.

Each ``pin_*`` function raises AssertionError when the oracle breaks the fact it checks.
They look the oracle up through its module at call time, so ``test_oracle_mutants.py`` can
swap in a copy with one planted mistake and confirm that some pin catches it.

Sources of the facts:
  * the attention equation: "Fused Kernel Compiler" (Candle paper), §FlashAttention
    Integration, displayed equation; softmax rows are probability distributions;
  * the running (online) softmax and its merge algebra: the same section (online softmax
    avoids the full attention matrix) and "Kernel Fusion, Softmax, and Attention", fifth
    paragraph (a stable running softmax derived on small rows that can be checked by hand --
    the extract does not carry those rows, so the worked rows here are our own, evaluated in
    closed form and printed to ten digits);
  * exactness up to rounding order: "Kernel Fusion, Softmax, and Attention", fifth paragraph;
  * the paged cache with a block table: "Optimizing Large Language Model Inference ...",
    §Paged Attention and Dynamic KV Cache Management;
  * the residual add + RMS norm and its two outputs: "Kernel and Operator Fusion -- Inference
    Optimization", §4 (the unfused listing: add, mean of squares, reciprocal square root of
    that plus eps, times the weight) and §5 (the new residual is returned too);
  * RoPE then the KV store, fused ("Kernel and Operator Fusion -- Inference Optimization",
    §2 item 6): the pages give no formula, so the pins fix the reading taken (rotate-half
    pairs, theta_i = base^(-2i/D)) by a hand-worked vector, and the properties any rotary
    embedding has (norm kept, positions compose, scores depend only on relative position).
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np

import oracle.direct as OA
import oracle.rmsnorm as ON
import oracle.rotary as OR


def _fwd(*a, **kw):
    return OA.attention(*a, **kw)


def _dec(*a, **kw):
    return OA.decode_paged(*a, **kw)


def _prefill(*a, **kw):
    return OA.prefill_paged(*a, **kw)


def _norm(*a, **kw):
    return ON.add_rms_norm(*a, **kw)


def _rope(*a, **kw):
    return OR.rope(*a, **kw)


def _rope_write(*a, **kw):
    return OR.rope_cache_write(*a, **kw)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), f"{what}: finite pattern differs"
    assert np.array_equal(a[~fa], b[~fb]), f"{what}: non-finite values differ"
    err = np.max(np.abs(a[fa] - b[fb])) if fa.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --- P1: softmax rows are probability distributions ------------------------------------
def pin_rows_sum_to_one():
    """With V = identity the output row *is* the probability row: non-negative, summing to
    one, and zero exactly where the causal mask hides a key."""
    r = _rng(11)
    for causal in (False, True):
        S = 7
        q = r.standard_normal((1, 2, S, 5))
        k = r.standard_normal((1, 2, S, 5))
        v = np.broadcast_to(np.eye(S), (1, 2, S, S)).copy()
        O, _ = _fwd(q, k, v, causal=causal, scale=0.7)
        assert np.all(O >= 0.0), "probabilities must be non-negative"
        _close(O.sum(axis=-1), np.ones((1, 2, S)), 1e-12, "row sums")
        if causal:
            upper = np.triu(np.ones((S, S), dtype=bool), 1)
            assert np.all(O[0, :, upper] == 0.0), "masked keys must get probability 0"


# --- P2: worked rows, online vs two-pass, merge, stability, masked row --------------------
WORKED = dict(
    # scores x = [1, 2, 3], values [[1,0],[0,1],[1,1]]:
    #   l = 1 + e^-1 + e^-2 (after subtracting the max 3),
    #   p = [e^-2, e^-1, 1] / l,  o = [p0 + p2, p1 + p2],  LSE = 3 + ln l.
    p=[0.0900305732, 0.2447284711, 0.6652409558],
    o=[0.7552715290, 0.9099694269],
    lse=3.4076059644,
    # masked row: scores [0.5, 1.5] visible, third key hidden: p = [e^-1, 1] / (1 + e^-1)
    p_masked=[0.2689414214, 0.7310585786],
    lse_masked=1.8132616875,
)


def _worked_inputs():
    q = np.array([[[[1.0]]]])                      # B=H=Sq=D=1
    k = np.array([[[[1.0], [2.0], [3.0]]]])        # scores 1, 2, 3 at scale 1
    v = np.array([[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]]])
    return q, k, v


def pin_worked_row():
    q, k, v = _worked_inputs()
    O, L = _fwd(q, k, v, causal=False, scale=1.0)
    _close(O[0, 0, 0], WORKED["o"], 1e-9, "worked row O (10-digit table)")
    _close(L[0, 0, 0], WORKED["lse"], 1e-9, "worked row LSE (10-digit table)")
    l = 1.0 + math.exp(-1.0) + math.exp(-2.0)
    p = [math.exp(-2.0) / l, math.exp(-1.0) / l, 1.0 / l]
    _close(O[0, 0, 0], [p[0] + p[2], p[1] + p[2]], 1e-15, "worked row O (closed form)")
    _close(L[0, 0, 0], 3.0 + math.log(l), 1e-15, "worked row LSE (closed form)")
    # probabilities through V = I
    O2, _ = _fwd(q, k, np.eye(3)[None, None], causal=False, scale=1.0)
    _close(O2[0, 0, 0], WORKED["p"], 1e-9, "worked row p")


def pin_online_equals_two_pass():
    """Running max/sum over chunks [1, 2] then [3], carried out by hand in scalars,
    gives the oracle's two-pass result."""
    q, k, v = _worked_inputs()
    O, L = _fwd(q, k, v, causal=False, scale=1.0)
    # chunk 1: scores 1, 2
    m1 = 2.0
    l1 = math.exp(1.0 - m1) + math.exp(2.0 - m1)
    acc1 = [math.exp(1.0 - m1) * 1.0 + math.exp(2.0 - m1) * 0.0,
            math.exp(1.0 - m1) * 0.0 + math.exp(2.0 - m1) * 1.0]
    _close(l1, 1.3678794412, 1e-9, "online l1")
    # chunk 2: score 3 -> new max, rescale by alpha = e^(m1 - m2)
    m2 = max(m1, 3.0)
    alpha = math.exp(m1 - m2)
    l2 = alpha * l1 + math.exp(3.0 - m2)
    acc2 = [alpha * acc1[0] + 1.0, alpha * acc1[1] + 1.0]
    _close(acc2, [1.1353352832, 1.3678794412], 1e-9, "online acc2")
    _close(O[0, 0, 0], [acc2[0] / l2, acc2[1] / l2], 1e-15, "online vs two-pass O")
    _close(L[0, 0, 0], m2 + math.log(l2), 1e-15, "online vs two-pass LSE")


def _merge(parts):
    """Combine (O_s, LSE_s) computed over disjoint key sets into the full result."""
    lses = np.stack([p[1] for p in parts])             # [S, ...]
    Ltot = np.logaddexp.reduce(lses, axis=0)
    w = np.exp(lses - Ltot)
    O = sum(w[i][..., None] * parts[i][0] for i in range(len(parts)))
    return O, Ltot


def pin_split_merge():
    """Attention over keys A and keys B separately, merged through their LSEs, equals
    attention over A and B together (split-KV algebra). Checks the worked row first."""
    q, k, v = _worked_inputs()
    OA_, LA = _fwd(q, k[:, :, :2], v[:, :, :2], scale=1.0)
    OB_, LB = _fwd(q, k[:, :, 2:], v[:, :, 2:], scale=1.0)
    _close(LA[0, 0, 0], 2.3132616875, 1e-9, "lse over chunk A")
    _close(LB[0, 0, 0], 3.0, 1e-15, "lse over chunk B")
    O, L = _merge([(OA_, LA), (OB_, LB)])
    Of, Lf = _fwd(q, k, v, scale=1.0)
    _close(O, Of, 1e-15, "merged O")
    _close(L, Lf, 1e-14, "merged LSE")
    r = _rng(12)
    qq = r.standard_normal((2, 3, 5, 8))
    kk = r.standard_normal((2, 3, 37, 8))
    vv = r.standard_normal((2, 3, 37, 6))
    Of, Lf = _fwd(qq, kk, vv, scale=0.35)
    for cuts in ([16], [1, 36], [5, 17, 30], list(range(1, 37))):
        edges = [0] + cuts + [37]
        parts = [_fwd(qq, kk[:, :, a:b], vv[:, :, a:b], scale=0.35)
                 for a, b in zip(edges[:-1], edges[1:])]
        O, L = _merge(parts)
        _close(O, Of, 1e-12, f"split {cuts} O")
        _close(L, Lf, 1e-12, f"split {cuts} LSE")


def pin_stability():
    """Scores 1000, 1001, 1002 give the softmax of 0, 1, 2 (exp(1000) overflows fp64, so an
    implementation without max subtraction fails), and LSE shifts by exactly 1000."""
    v = np.array([[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]]])
    q = np.array([[[[1.0]]]])
    Ob, Lb = _fwd(q, np.array([[[[1000.0], [1001.0], [1002.0]]]]), v, scale=1.0)
    Os, Ls = _fwd(q, np.array([[[[0.0], [1.0], [2.0]]]]), v, scale=1.0)
    assert np.all(np.isfinite(Ob)) and np.all(np.isfinite(Lb)), "large scores overflowed"
    _close(Ob, Os, 1e-15, "shifted O")
    _close(Lb, Ls + 1000.0, 1e-12, "shifted LSE")


def pin_masked_row():
    """Causal row 1 of a 3x3 problem sees keys 0 and 1 only (scores 0.5 and 1.5)."""
    q = np.array([[[[0.3], [1.0], [2.0]]]])
    k = np.array([[[[0.5], [1.5], [7.0]]]])
    v = np.eye(3)[None, None]
    O, L = _fwd(q, k, v, causal=True, scale=1.0)
    _close(O[0, 0, 1], WORKED["p_masked"] + [0.0], 1e-9, "masked row p")
    _close(L[0, 0, 1], WORKED["lse_masked"], 1e-9, "masked row LSE")


# --- P3/P4/P6: closed forms ----------------------------------------------------------------
def pin_identical_keys():
    """All keys equal: every visible key gets the same weight, so O_i is the mean of the
    visible values and LSE_i = s * q_i . k + ln(#visible)."""
    r = _rng(13)
    S, D = 9, 4
    q = r.standard_normal((1, 1, S, D))
    kv = r.standard_normal(D)
    k = np.broadcast_to(kv, (1, 1, S, D)).copy()
    v = r.standard_normal((1, 1, S, 3))
    s = 0.5
    O, L = _fwd(q, k, v, causal=False, scale=s)
    _close(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (S, 3)), 1e-13, "mean of V")
    _close(L[0, 0], s * (q[0, 0] @ kv) + math.log(S), 1e-13, "LSE equal keys")
    O, L = _fwd(q, k, v, causal=True, scale=s)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    _close(O[0, 0], prefix, 1e-13, "prefix means of V")
    _close(L[0, 0], s * (q[0, 0] @ kv) + np.log(np.arange(1, S + 1)), 1e-13,
           "LSE equal keys causal")


def pin_causal_row0():
    """With Sq == Sk, causal row 0 sees only key 0: O_0 = V_0 exactly, LSE_0 = s q_0.k_0."""
    r = _rng(14)
    q = r.standard_normal((2, 2, 6, 4))
    k = r.standard_normal((2, 2, 6, 4))
    v = r.standard_normal((2, 2, 6, 4))
    O, L = _fwd(q, k, v, causal=True, scale=0.8125)
    assert np.array_equal(O[:, :, 0], v[:, :, 0]), "causal row 0 must equal V_0"
    _close(L[:, :, 0], 0.8125 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14,
           "causal row 0 LSE")


def pin_degenerate():
    """scale = 0 gives uniform weights; one key gives that key's value."""
    r = _rng(15)
    q = r.standard_normal((1, 2, 5, 4))
    k = r.standard_normal((1, 2, 5, 4))
    v = r.standard_normal((1, 2, 5, 3))
    O, L = _fwd(q, k, v, causal=False, scale=0.0)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-14, "scale 0")
    _close(L, np.full(L.shape, math.log(5)), 1e-14, "scale 0 LSE")
    O, L = _fwd(q, k, v, causal=True, scale=0.0)
    cnt = np.arange(1, 6)
    _close(O[0, 0], np.cumsum(v[0, 0], axis=0) / cnt[:, None], 1e-14, "scale 0 causal")
    _close(L[0, 0], np.log(cnt), 1e-14, "scale 0 causal LSE")
    O, L = _fwd(q, k[:, :, :1], v[:, :, :1], causal=False, scale=0.875)
    _close(O, np.broadcast_to(v[:, :, :1], O.shape), 1e-15, "single key")
    _close(L, 0.875 * np.einsum("bhsd,bhd->bhs", q, k[:, :, 0]), 1e-14, "single key LSE")


# --- P5: brute force in 40-digit decimal --------------------------------------------------
def _decimal_attention(q, k, v, causal, scale):
    getcontext().prec = 40
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    g = Hq // Hkv
    sc = Decimal(float(np.float32(scale)))
    O = np.zeros((B, Hq, Sq, Dv))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Sq):
                scores = []
                for j in range(Sk):
                    if causal and j > i + (Sk - Sq):
                        continue
                    dot = sum(Decimal(float(q[b, h, i, d])) * Decimal(float(k[b, hk, j, d]))
                              for d in range(D))
                    scores.append((j, sc * dot))
                if not scores:
                    L[b, h, i] = -np.inf
                    continue
                m = max(s for _, s in scores)
                w = [(j, (s - m).exp()) for j, s in scores]
                tot = sum(x for _, x in w)
                for d in range(Dv):
                    O[b, h, i, d] = float(sum(x * Decimal(float(v[b, hk, j, d]))
                                              for j, x in w) / tot)
                L[b, h, i] = float(m + tot.ln())
    return O, L


def pin_brute_force():
    """Whole oracle against scalar 40-digit arithmetic on tiny inputs, including GQA,
    Sq < Sk, Sq > Sk (rows with no visible key) and a non-square value width."""
    r = _rng(16)
    for (Hq, Hkv, Sq, Sk, D, Dv, causal) in [
        (2, 1, 5, 5, 3, 3, False), (2, 1, 5, 5, 3, 2, True),
        (2, 2, 3, 6, 4, 4, True), (3, 1, 6, 4, 2, 3, True), (1, 1, 1, 6, 4, 4, False),
    ]:
        q = r.standard_normal((1, Hq, Sq, D))
        k = r.standard_normal((1, Hkv, Sk, D))
        v = r.standard_normal((1, Hkv, Sk, Dv))
        O, L = _fwd(q, k, v, causal=causal, scale=0.6)
        Od, Ld = _decimal_attention(q, k, v, causal, 0.6)
        _close(O, Od, 1e-13, f"brute force O {Hq, Hkv, Sq, Sk, causal}")
        _close(L, Ld, 1e-13, f"brute force LSE {Hq, Hkv, Sq, Sk, causal}")
        rows = [(0, h, i) for h in range(Hq) for i in (0, Sq // 2, Sq - 1)]
        Or, Lr = OA.attention_rows(q, k, v, rows, causal=causal, scale=0.6)
        idx = tuple(np.array(rows).T)
        _close(Or, Od[idx], 1e-13, f"brute force sampled rows O {Hq, Hkv, Sq, Sk, causal}")
        _close(Lr, Ld[idx], 1e-13, f"brute force sampled rows LSE {Hq, Hkv, Sq, Sk, causal}")


# --- P7/P8/P9/P10: invariances ----------------------------------------------------------
def pin_shift_invariance():
    """Adding one vector u to every key leaves O unchanged and shifts LSE by s * q . u."""
    r = _rng(17)
    q = r.standard_normal((1, 2, 6, 5))
    k = r.standard_normal((1, 2, 8, 5))
    v = r.standard_normal((1, 2, 8, 5))
    u = r.standard_normal(5)
    for causal in (False, True):
        O, L = _fwd(q, k, v, causal=causal, scale=0.375)
        O2, L2 = _fwd(q, k + u, v, causal=causal, scale=0.375)
        _close(O2, O, 1e-13, "shift O")
        _close(L2, L + 0.375 * (q @ u), 1e-13, "shift LSE")


def pin_v_affine():
    """O(V W + 1 c^T) = O(V) W + 1 c^T, because each row of weights sums to one."""
    r = _rng(18)
    q = r.standard_normal((1, 1, 5, 4))
    k = r.standard_normal((1, 1, 7, 4))
    v = r.standard_normal((1, 1, 7, 3))
    W = r.standard_normal((3, 2))
    c = r.standard_normal(2)
    for causal in (False, True):
        O, _ = _fwd(q, k, v, causal=causal, scale=0.9)
        O2, _ = _fwd(q, k, v @ W + c, causal=causal, scale=0.9)
        _close(O2, O @ W + c, 1e-13, "V affine")


def pin_gqa():
    """Grouped heads equal full multi-head attention with each KV head repeated for its
    contiguous group of Hq/Hkv query heads."""
    r = _rng(19)
    q = r.standard_normal((2, 6, 5, 4))
    k = r.standard_normal((2, 2, 5, 4))
    v = r.standard_normal((2, 2, 5, 4))
    for causal in (False, True):
        O, L = _fwd(q, k, v, causal=causal, scale=0.5)
        O2, L2 = _fwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal=causal,
                      scale=0.5)
        _close(O, O2, 1e-15, "GQA O")
        _close(L, L2, 1e-15, "GQA LSE")


def pin_permutations():
    """Non-causal attention ignores key order (K and V permuted together); permuting the
    queries permutes the output rows."""
    r = _rng(20)
    q = r.standard_normal((1, 2, 6, 4))
    k = r.standard_normal((1, 2, 9, 4))
    v = r.standard_normal((1, 2, 9, 3))
    O, L = _fwd(q, k, v, scale=0.7)
    pk = r.permutation(9)
    O2, L2 = _fwd(q, k[:, :, pk], v[:, :, pk], scale=0.7)
    _close(O2, O, 1e-14, "key permutation O")
    _close(L2, L, 1e-14, "key permutation LSE")
    pq = r.permutation(6)
    O3, L3 = _fwd(q[:, :, pq], k, v, scale=0.7)
    _close(O3, O[:, :, pq], 0.0, "query permutation O")
    _close(L3, L[:, :, pq], 0.0, "query permutation LSE")


# --- P11: paged decode ---------------------------------------------------------------------
def _scatter_paged(K, V, block_size, rng, extra=3):
    """Put logical per-sequence K/V ([Hkv, n_b, D] each) into a shuffled physical pool.
    Written independently of the oracle's gather: loops over tokens one at a time."""
    B = len(K)
    Hkv, D = K[0].shape[0], K[0].shape[2]
    nblk = [(kb.shape[1] + block_size - 1) // block_size for kb in K]
    pool = sum(nblk) + extra
    perm = rng.permutation(pool)
    table = np.full((B, max(nblk)), -1, dtype=np.int32)
    kc = rng.standard_normal((pool, Hkv, block_size, D)) * 1e3   # junk everywhere else
    vc = rng.standard_normal((pool, Hkv, block_size, D)) * 1e3
    off = 0
    for b in range(B):
        for j in range(nblk[b]):
            table[b, j] = perm[off + j]
        off += nblk[b]
        for t in range(K[b].shape[1]):
            phys = table[b, t // block_size]
            kc[phys, :, t % block_size, :] = K[b][:, t, :]
            vc[phys, :, t % block_size, :] = V[b][:, t, :]
    return kc, vc, table


def pin_decode_paged():
    """Decode of the newest token over a paged cache equals the last row of causal prefill
    over the same sequence, for several block sizes and lengths that end mid-block; it does
    not depend on where the blocks sit in the pool, and never reads slots past ctx_len."""
    r = _rng(21)
    Hq, Hkv, D = 4, 2, 8
    for bs in (1, 4, 16):
        lens = [1, bs, bs + 1, 3 * bs - 1, 37]
        Ks = [r.standard_normal((Hkv, n, D)) for n in lens]
        Vs = [r.standard_normal((Hkv, n, D)) for n in lens]
        Qs = [r.standard_normal((Hq, n, D)) for n in lens]
        kc, vc, table = _scatter_paged(Ks, Vs, bs, r)
        q = np.stack([Qs[b][:, -1, :] for b in range(len(lens))])
        ctx = np.array(lens, dtype=np.int32)
        O, L = _dec(q, kc, vc, table, ctx, bs, scale=0.3)
        for b, n in enumerate(lens):
            Of, Lf = _fwd(Qs[b][None], Ks[b][None], Vs[b][None], causal=True, scale=0.3)
            _close(O[b], Of[0, :, -1], 1e-13, f"decode vs causal last row bs={bs} n={n}")
            _close(L[b], Lf[0, :, -1], 1e-13, f"decode LSE bs={bs} n={n}")
        # moving every physical block elsewhere changes nothing
        pool = kc.shape[0]
        p = r.permutation(pool)
        inv = np.empty_like(p)
        inv[p] = np.arange(pool)
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[inv] = kc
        vc2[inv] = vc
        table2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1).astype(np.int32)
        O2, L2 = _dec(q, kc2, vc2, table2, ctx, bs, scale=0.3)
        _close(O2, O, 0.0, "block permutation O")
        _close(L2, L, 0.0, "block permutation LSE")
        # NaN in every slot past the end of each sequence is never touched
        kc3, vc3 = kc.copy(), vc.copy()
        for b, n in enumerate(lens):
            last = table[b, (n - 1) // bs]
            kc3[last, :, (n - 1) % bs + 1:, :] = np.nan
            vc3[last, :, (n - 1) % bs + 1:, :] = np.nan
        O3, L3 = _dec(q, kc3, vc3, table, ctx, bs, scale=0.3)
        _close(O3, O, 0.0, "poisoned tail O")
        _close(L3, L, 0.0, "poisoned tail LSE")


# --- N3: prefill over a paged cache -----------------------------------------------------
def pin_prefill_paged():
    """A chunk of new tokens of each sequence, packed together with other sequences' chunks,
    gets exactly the last rows of a full causal prefill over its whole sequence (the chunk's
    tokens are the sequence's last positions); the last row of each chunk is the paged decode
    of that token; without the mask every row is plain attention over the whole context;
    slots past a context (NaN-poisoned) are never read; and with the pool size given, a block
    whose table entry is outside the pool drops out as if its keys were not there."""
    r = _rng(23)
    Hq, Hkv, D, s = 4, 2, 8, 0.3
    for bs in (4, 16):
        lens = [5, bs, 2 * bs + 3, 37, 9, 6]       # keys of each sequence
        qlens = [5, 1, bs + 2, 0, 3, 6]           # its new tokens: the last qlens positions
        Ks = [r.standard_normal((Hkv, n, D)) for n in lens]
        Vs = [r.standard_normal((Hkv, n, D)) for n in lens]
        Qs = [r.standard_normal((Hq, n, D)) for n in lens]
        kc, vc, table = _scatter_paged(Ks, Vs, bs, r)
        for b, n in enumerate(lens):
            last = table[b, (n - 1) // bs]
            kc[last, :, (n - 1) % bs + 1:, :] = np.nan
            vc[last, :, (n - 1) % bs + 1:, :] = np.nan
        cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        q = np.concatenate([np.transpose(Qs[b][:, n - m:, :], (1, 0, 2))
                            for b, (n, m) in enumerate(zip(lens, qlens))])
        ctx = np.array(lens, dtype=np.int32)
        O, L = _prefill(q, kc, vc, table, cu, ctx, bs, causal=True, scale=s)
        On, Ln = _prefill(q, kc, vc, table, cu, ctx, bs, causal=False, scale=s)
        for b, (n, m) in enumerate(zip(lens, qlens)):
            if m == 0:
                continue
            Of, Lf = _fwd(Qs[b][None], Ks[b][None], Vs[b][None], causal=True, scale=s)
            _close(O[cu[b]:cu[b + 1]], np.transpose(Of[0][:, n - m:, :], (1, 0, 2)), 1e-13,
                   f"chunk vs full prefill bs={bs} b={b}")
            _close(L[cu[b]:cu[b + 1]], Lf[0][:, n - m:].T, 1e-13, f"chunk LSE bs={bs} b={b}")
            Od, Ld = _dec(Qs[b][:, -1, :][None], kc, vc, table[b:b + 1], ctx[b:b + 1], bs,
                          scale=s)
            _close(O[cu[b + 1] - 1], Od[0], 1e-13, f"last chunk row vs decode bs={bs} b={b}")
            _close(L[cu[b + 1] - 1], Ld[0], 1e-13, f"last chunk LSE vs decode bs={bs} b={b}")
            Ou, Lu = _fwd(Qs[b][None][:, :, n - m:, :], Ks[b][None], Vs[b][None], causal=False,
                          scale=s)
            _close(On[cu[b]:cu[b + 1]], np.transpose(Ou[0], (1, 0, 2)), 1e-13,
                   f"unmasked chunk bs={bs} b={b}")
            _close(Ln[cu[b]:cu[b + 1]], Lu[0].T, 1e-13, f"unmasked LSE bs={bs} b={b}")
        # a block outside the pool (sequence 3's third block) drops out when the pool is given
        pool = kc.shape[0]
        b, drop = 3, 2
        table2 = table.copy()
        table2[b, drop] = pool + 5
        cu2 = np.array([0, 0, 0, 0, 4, 4, 4], dtype=np.int32)     # four new tokens of seq 3
        n = lens[b]
        q2 = np.transpose(Qs[b][:, n - 4:, :], (1, 0, 2))
        keep = np.ones(n, dtype=bool)
        keep[drop * bs:(drop + 1) * bs] = False
        Ok, Lk = _prefill(q2, kc, vc, table2, cu2, ctx, bs, causal=False, scale=s,
                          num_blocks=pool)
        Oe, Le = _fwd(Qs[b][None][:, :, n - 4:, :], Ks[b][None][:, :, keep, :],
                      Vs[b][None][:, :, keep, :], causal=False, scale=s)
        _close(Ok, np.transpose(Oe[0], (1, 0, 2)), 1e-13, f"dropped block bs={bs}")
        _close(Lk, Le[0].T, 1e-13, f"dropped block LSE bs={bs}")
        Okc, Lkc = _prefill(q2, kc, vc, table2, cu2, ctx, bs, causal=True, scale=s,
                            num_blocks=pool)
        _close(Okc[-1], Ok[-1], 1e-13, f"dropped block, causal last row bs={bs}")
        _close(Lkc[-1], Lk[-1], 1e-13, f"dropped block, causal last LSE bs={bs}")


# --- N4: residual add + RMS norm ---------------------------------------------------------
def _norm_rows(seed, M=4, d=37):
    rng = _rng(seed)
    x = rng.standard_normal((M, d)).astype(np.float32)
    r = rng.standard_normal((M, d)).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return x, r, w


def pin_norm_residual_is_sum():
    """The second output is the sum x + residual itself (the page returns it for the next
    layer's add), exactly: the sum of two float32 values is exact in float64."""
    x, r, w = _norm_rows(40)
    _, t = _norm(x, r, w)
    assert np.array_equal(t, x.astype(np.float64) + r.astype(np.float64))
    assert np.array_equal(_norm(r, x, w)[1], t)           # the add is symmetric


def pin_norm_unit_rms():
    """With eps = 0 and unit weight, every output row has mean square exactly 1: the row is
    divided by the root of its mean square (the mean over d, not the sum or d - 1)."""
    x, r, _ = _norm_rows(41, M=6, d=29)
    out, _ = _norm(x, r, np.ones(29, np.float32), eps=0.0)
    ms = np.mean(out * out, axis=1)
    _close(ms, np.ones(6), 1e-13, "mean square of the normalised rows")


def pin_norm_scale_invariance():
    """eps = 0: scaling x and the residual by the same a > 0 leaves the output unchanged (the
    normalisation divides the scale out); scaling the weight scales the output."""
    x, r, w = _norm_rows(42)
    o1, _ = _norm(x, r, w, eps=0.0)
    o2, _ = _norm(3.75 * x.astype(np.float64), 3.75 * r.astype(np.float64), w, eps=0.0)
    _close(o2, o1, 1e-13, "scale invariance")
    o3, _ = _norm(x, r, 2.0 * w.astype(np.float64), eps=0.0)
    _close(o3, 2.0 * o1, 1e-13, "linear in the weight")
    o4, _ = _norm(-x.astype(np.float64), -r.astype(np.float64), w, eps=0.0)
    _close(o4, -o1, 1e-13, "odd in the input")


def pin_norm_constant_and_eps():
    """Closed forms that fix where eps enters: a row whose sum is the constant c gives
    c / sqrt(c^2 + eps) * w. With c^2 = eps the result is w / sqrt(2) exactly; with eps = 0
    it is sign(c) * w."""
    d = 8
    w = np.linspace(0.5, 1.5, d)
    c = 1e-3                                   # c^2 = 1e-6 = eps
    x = np.full((1, d), c / 4)
    r = np.full((1, d), 3 * c / 4)
    out, _ = _norm(x, r, w, eps=1e-6)
    _close(out[0], w / math.sqrt(2.0), 1e-12, "constant row with c^2 = eps")
    out0, _ = _norm(-x, -r, w, eps=0.0)
    _close(out0[0], -w, 1e-12, "constant row, eps = 0")
    big, _ = _norm(1e3 * x, 1e3 * r, w, eps=1e-6)      # c = 1: eps nearly negligible
    _close(big[0], w / math.sqrt(1.0 + 1e-6), 1e-12, "constant row with c = 1")


def pin_norm_brute_force():
    """Scalar Decimal arithmetic (40 digits) straight from the page's unfused listing, on
    small rows, independent of numpy."""
    getcontext().prec = 40
    x, r, w = _norm_rows(43, M=2, d=5)
    out, t = _norm(x, r, w, eps=1e-6)
    for i in range(2):
        ti = [Decimal(float(x[i, j])) + Decimal(float(r[i, j])) for j in range(5)]
        var = sum(v * v for v in ti) / Decimal(5)
        inv = Decimal(1) / (var + Decimal("0.000001")).sqrt()
        for j in range(5):
            ref = ti[j] * inv * Decimal(float(w[j]))
            assert abs(Decimal(float(out[i, j])) - ref) <= Decimal("1e-13"), (i, j)
            assert Decimal(float(t[i, j])) == ti[j]


# --- N1: rotary embedding + paged cache write ---------------------------------------------
def pin_rope_worked():
    """D = 4, base 10000, position 1: pairs (0, 2) turn by 1 rad and (1, 3) by 10000^-1/2 =
    0.01 rad; written out with scalar math.cos / math.sin."""
    y = _rope(np.array([[[1.0, 2.0, 3.0, 4.0]]]), [1], base=10000.0)[0, 0]
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    ref = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    _close(y, ref, 1e-14, "worked rotary vector")
    # position 0 is the identity; D = 2 turns the single pair by p radians
    x = _rng(50).standard_normal((3, 2, 8))
    _close(_rope(x, [0, 0, 0]), x, 0.0, "position 0")
    y2 = _rope(np.array([[[0.6, -0.8]]]), [3])[0, 0]
    _close(y2, [0.6 * math.cos(3) + 0.8 * math.sin(3), -0.8 * math.cos(3) + 0.6 * math.sin(3)],
           1e-14, "D = 2")


def pin_rope_rotation_properties():
    """Each pair is rotated: head-vector norms are kept, rotations by a and b compose to a + b,
    and a query-key score depends only on the distance between the positions."""
    rng = _rng(51)
    x = rng.standard_normal((5, 3, 16))
    pos = np.array([0, 1, 7, 100, 4095])
    y = _rope(x, pos)
    _close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), 1e-12, "norm kept")
    _close(_rope(_rope(x, pos, base=500.0), 2 * pos + 3, base=500.0), _rope(x, 3 * pos + 3,
           base=500.0), 1e-10, "composition")
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    for m, n, sh in ((5, 2, 40), (0, 9, 1000), (300, 300, 7)):
        a = float(np.sum(_rope(q, [m]) * _rope(k, [n])))
        b = float(np.sum(_rope(q, [m + sh]) * _rope(k, [n + sh])))
        assert abs(a - b) <= 1e-10, (m, n, sh, a, b)


def pin_rope_cache_write():
    """The store: token t's rotated key and (unrotated) value land in block
    table[seq, p // 16], slot p % 16, of every KV head; nothing else changes; a negative
    position, a position past the table row, or an entry outside the pool (when the pool size
    is given) writes nothing."""
    rng = _rng(52)
    T, Hq, Hkv, D, nb = 5, 4, 2, 8, 6
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    kc = rng.standard_normal((nb, Hkv, 16, D))
    vc = rng.standard_normal((nb, Hkv, 16, D))
    table = np.array([[3, 1, -1], [0, 5, 2], [4, 9, -1], [2, 2, 2], [1, 1, 1]], dtype=np.int32)
    pos = np.array([17, 40, 20, -1, 48])
    qr, kc2, vc2 = _rope_write(q, k, v, pos, kc, vc, table, base=10000.0, num_blocks=nb)
    _close(qr, _rope(q, pos), 0.0, "rotated queries")
    expect_k, expect_v = kc.copy(), vc.copy()
    kr = _rope(k, pos)
    for t, (blk, slot) in enumerate([(1, 1), (2, 8)]):   # tokens 0 and 1
        expect_k[blk, :, slot, :] = kr[t]
        expect_v[blk, :, slot, :] = v[t]
    # token 2: table[2, 1] = 9 is outside the pool of 6; token 3: negative position;
    # token 4: position 48 is block 3, past its table row of 3 entries
    _close(kc2, expect_k, 0.0, "key cache")
    _close(vc2, expect_v, 0.0, "value cache")
    # an explicit sequence map: tokens 0 and 1 both belong to sequence 1
    _, kc3, _ = _rope_write(q[:2], k[:2], v[:2], np.array([0, 33]), kc, vc, table,
                            seq_ids=np.array([1, 1]))
    _close(kc3[0, :, 0, :], _rope(k[:1], [0])[0], 0.0, "sequence map, token 0")
    _close(kc3[2, :, 1, :], _rope(k[1:2], [33])[0], 0.0, "sequence map, token 1")


ALL_PINS = [
    pin_rows_sum_to_one, pin_worked_row, pin_online_equals_two_pass, pin_split_merge,
    pin_stability, pin_masked_row, pin_identical_keys, pin_causal_row0, pin_degenerate,
    pin_brute_force, pin_shift_invariance, pin_v_affine, pin_gqa, pin_permutations,
    pin_decode_paged, pin_prefill_paged, pin_norm_residual_is_sum, pin_norm_unit_rms, pin_norm_scale_invariance,
    pin_norm_constant_and_eps, pin_norm_brute_force, pin_rope_worked,
    pin_rope_rotation_properties, pin_rope_cache_write,
]
