"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, a library routine, a brute-force enumeration or an invariant that
the pages and the mathematics fix. ``test_oracle_pins.py`` runs them all;
``test_oracle_mutants.py`` plants mistakes in the oracle and checks that some
pin fails for each.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import scipy.special

import synth
import oracle
from oracle import REPEAT, CAUSAL


def _bits(x):
    return synth.f32_to_bf16(np.asarray(x, dtype=np.float32))


def _tiny(seed, Hq, Hkv, D, n_ctx, n_q, mask, chunk, qstd=0.5):
    r = synth.Recipe(Hq=Hq, Hkv=Hkv, D=D, n_ctx=n_ctx, n_q=n_q, mask=mask, chunk=chunk,
                     scale=1.0, q_prescale=qstd)
    return synth.draw(r, seed)


# ---------------------------------------------------------------- LSE pins

def pin_softmax_rows_sum_to_one():
    """Every row of the softmax built from the oracle's LSE sums to 1."""
    for mask, chunk in [(REPEAT, 5), (REPEAT, 0), (CAUSAL, 0)]:
        n_ctx = 13 if mask == REPEAT else 11
        d = _tiny(7, 6, 2, 64, n_ctx, 11, mask, chunk, qstd=1.0)
        L = oracle.lse(d["Q"], d["Kctx"], d.get("Kself"), 1.0, mask, chunk)
        c = chunk if chunk else 11
        for g in range(6):
            for j0 in range(0, 11, c):
                j1 = min(j0 + c, 11)
                a = oracle.attention_weights(d["Q"], d["Kctx"], d.get("Kself"), 1.0, mask, chunk,
                                             g, j0, j1, L[g, j0:j1])
                assert np.allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-12), (mask, g, j0)


def pin_lse_zero_queries():
    """Q = 0: every visible logit is 0, so LSE_j = ln |V(j)| with
    |V(j)| = n_ctx + (j mod C) + 1 (repeat) or j + 1 (causal)."""
    Hq, Hkv, D, n_ctx, n_q, C = 4, 2, 64, 9, 10, 4
    Q = np.zeros((Hq, n_q, D), dtype=np.uint16)
    d = _tiny(3, Hq, Hkv, D, n_ctx, n_q, REPEAT, C)
    L = oracle.lse(Q, d["Kctx"], d["Kself"], 0.125, REPEAT, C)
    want = np.log(n_ctx + (np.arange(n_q) % C) + 1.0)
    assert np.allclose(L, want[None, :], rtol=0, atol=1e-13)
    dc = _tiny(3, Hq, Hkv, D, n_q, n_q, CAUSAL, 0)
    Lc = oracle.lse(Q, dc["Kctx"], None, 0.125, CAUSAL, 0)
    assert np.allclose(Lc, np.log(np.arange(n_q) + 1.0)[None, :], rtol=0, atol=1e-13)


def _brute_visible(Qf, Kc, Ks, g, h, j, scale, mask, chunk, n_q):
    """Visible logits of (g, j), enumerated key by key with exact sums."""
    out = []
    if mask == REPEAT:
        c = chunk if chunk else n_q
        c0 = (j // c) * c
        keys = [Kc[h, i] for i in range(Kc.shape[1])] + [Ks[h, p] for p in range(c0, j + 1)]
    else:
        keys = [Kc[h, i] for i in range(j + 1)]
    for k in keys:
        out.append(scale * math.fsum(float(a) * float(b) for a, b in zip(Qf[g, j], k)))
    return out


def pin_lse_brute_force_logsumexp():
    """LSE against scipy's logsumexp over brute-force enumerated logits."""
    for mask, chunk, n_ctx, n_q in [(REPEAT, 3, 5, 7), (CAUSAL, 0, 6, 6)]:
        d = _tiny(11, 4, 2, 64, n_ctx, n_q, mask, chunk, qstd=1.0)
        Qf = synth.bf16_to_f32(d["Q"]).astype(np.float64)
        Kc = synth.bf16_to_f32(d["Kctx"]).astype(np.float64)
        Ks = synth.bf16_to_f32(d["Kself"]).astype(np.float64) if "Kself" in d else None
        L = oracle.lse(d["Q"], d["Kctx"], d.get("Kself"), 0.5, mask, chunk)
        for g, j in itertools.product(range(4), range(n_q)):
            h = g // 2
            want = scipy.special.logsumexp(_brute_visible(Qf, Kc, Ks, g, h, j, 0.5, mask, chunk, n_q))
            assert abs(L[g, j] - want) < 1e-12, (mask, g, j)


# ---------------------------------------------------------------- attention-output pins

def _brute_visible_values(Vc, Vs, h, j, mask, chunk, n_q):
    """The value rows query j sees, in the order of ``_brute_visible``'s keys."""
    if mask == REPEAT:
        c = chunk if chunk else n_q
        c0 = (j // c) * c
        return [Vc[h, i] for i in range(Vc.shape[1])] + [Vs[h, p] for p in range(c0, j + 1)]
    return [Vc[h, i] for i in range(j + 1)]


def _f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def pin_attn_brute_force():
    """O_j = sum_i exp(l_ji) v_i / sum_i exp(l_ji) and LSE_j, every visible key
    enumerated one by one with exact sums."""
    for mask, chunk, n_ctx, n_q in [(REPEAT, 3, 5, 7), (CAUSAL, 0, 6, 6)]:
        d = _tiny(13, 4, 2, 64, n_ctx, n_q, mask, chunk, qstd=1.0)
        Qf, Kc, Vc = _f64(d["Q"]), _f64(d["Kctx"]), _f64(d["V"])
        Ks = _f64(d["Kself"]) if "Kself" in d else None
        Vs = _f64(d["Vself"]) if "Vself" in d else None
        O, L = oracle.attention(d["Q"], d["Kctx"], d.get("Kself"), d["V"], d.get("Vself"), 0.5, mask, chunk)
        for g, j in itertools.product(range(4), range(n_q)):
            h = g // 2
            logits = _brute_visible(Qf, Kc, Ks, g, h, j, 0.5, mask, chunk, n_q)
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            tot = math.fsum(w)
            assert abs(L[g, j] - (m + math.log(tot))) < 1e-12, (mask, g, j)
            vals = _brute_visible_values(Vc, Vs, h, j, mask, chunk, n_q)
            for dd in range(Qf.shape[2]):
                want = math.fsum(wi * float(v[dd]) for wi, v in zip(w, vals)) / tot
                assert abs(O[g, j, dd] - want) < 1e-12, (mask, g, j, dd)


def pin_attn_constant_values():
    """Every value row equal to c: the weights sum to 1, so O_j = c."""
    for mask, chunk in [(REPEAT, 4), (CAUSAL, 0)]:
        d = _tiny(17, 6, 3, 64, 9 if mask == REPEAT else 10, 10, mask, chunk, qstd=1.0)
        c = d["V"][0, 0].copy()
        V = np.broadcast_to(c, d["V"].shape).copy()
        Vs = np.broadcast_to(c, d["Vself"].shape).copy() if "Vself" in d else None
        O, _ = oracle.attention(d["Q"], d["Kctx"], d.get("Kself"), V, Vs, 0.125, mask, chunk)
        assert np.allclose(O, _f64(c)[None, None, :], rtol=1e-13, atol=1e-13), mask


def pin_attn_zero_queries():
    """Q = 0: all visible logits are equal, so O_j is the plain mean of the
    value rows j sees (context rows plus its chunk's self rows up to j;
    causal: rows 0..j)."""
    Hq, Hkv, D, n_ctx, n_q, C = 4, 2, 64, 7, 9, 4
    d = _tiny(19, Hq, Hkv, D, n_ctx, n_q, REPEAT, C)
    Q = np.zeros_like(d["Q"])
    O, _ = oracle.attention(Q, d["Kctx"], d["Kself"], d["V"], d["Vself"], 0.125, REPEAT, C)
    Vc, Vs = _f64(d["V"]), _f64(d["Vself"])
    for g, j in itertools.product(range(Hq), range(n_q)):
        h, c0 = g // 2, (j // C) * C
        want = (Vc[h].sum(axis=0) + Vs[h, c0:j + 1].sum(axis=0)) / (n_ctx + j - c0 + 1)
        assert np.allclose(O[g, j], want, rtol=0, atol=1e-13), (g, j)
    dc = _tiny(19, Hq, Hkv, D, n_q, n_q, CAUSAL, 0)
    Oc, _ = oracle.attention(Q, dc["Kctx"], None, dc["V"], None, 0.125, CAUSAL, 0)
    Vc = _f64(dc["V"])
    for g, j in itertools.product(range(Hq), range(n_q)):
        assert np.allclose(Oc[g, j], Vc[g // 2, :j + 1].mean(axis=0), rtol=0, atol=1e-13), (g, j)


def pin_attn_linear_in_values():
    """O is linear in V: O(V1 + V2) = O(V1) + O(V2) (small integers, so the
    bf16 sums are exact)."""
    d = _tiny(23, 4, 2, 64, 6, 8, REPEAT, 3, qstd=1.0)
    rng = np.random.default_rng(5)
    V1 = rng.integers(-8, 9, size=d["V"].shape).astype(np.float32)
    V2 = rng.integers(-8, 9, size=d["V"].shape).astype(np.float32)
    S1 = rng.integers(-8, 9, size=d["Vself"].shape).astype(np.float32)
    S2 = rng.integers(-8, 9, size=d["Vself"].shape).astype(np.float32)
    run = lambda V, S: oracle.attention(d["Q"], d["Kctx"], d["Kself"], _bits(V), _bits(S), 0.25, REPEAT, 3)[0]
    assert np.allclose(run(V1 + V2, S1 + S2), run(V1, S1) + run(V2, S2), rtol=0, atol=1e-11)


# ---------------------------------------------------------------- decode-over-cache pins

def _decode_inputs(seed, Hq, Hkv, D, counts, n_q=1):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Q = synth.normal_bf16(seed, 1, (Hq, n_q, D))
    Kc = synth.normal_bf16(seed, 2, (int(offs[-1]), D))
    Vc = synth.normal_bf16(seed, 3, (int(offs[-1]), D))
    return Q, Kc, Vc, offs


def pin_decode_brute_force():
    """Every kept row of the query's head enumerated one by one with exact sums;
    a head with no rows gives O = 0, LSE = -inf."""
    Hq, Hkv, D = 6, 3, 64
    Q, Kc, Vc, offs = _decode_inputs(47, Hq, Hkv, D, [5, 0, 7], n_q=2)
    O, L = oracle.decode_attention(Q, Kc, Vc, offs, 0.25)
    Qf, Kf, Vf = _f64(Q), _f64(Kc), _f64(Vc)
    for g, t in itertools.product(range(Hq), range(2)):
        h = g // 2
        rows = range(int(offs[h]), int(offs[h + 1]))
        if not rows:
            assert L[g, t] == -np.inf and np.all(O[g, t] == 0), (g, t)
            continue
        logits = [0.25 * math.fsum(float(a) * float(b) for a, b in zip(Qf[g, t], Kf[r])) for r in rows]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        tot = math.fsum(w)
        assert abs(L[g, t] - (m + math.log(tot))) < 1e-12, (g, t)
        for dd in range(D):
            want = math.fsum(wi * float(Vf[r, dd]) for wi, r in zip(w, rows)) / tot
            assert abs(O[g, t, dd] - want) < 1e-12, (g, t, dd)


def pin_decode_single_row_and_constant_values():
    """One kept row per head: O = that row's value, LSE = its logit. Every row
    equal to c: O = c."""
    Hq, Hkv, D = 4, 2, 64
    Q, Kc, Vc, offs = _decode_inputs(53, Hq, Hkv, D, [1, 1])
    O, L = oracle.decode_attention(Q, Kc, Vc, offs, 0.5)
    Qf, Kf, Vf = _f64(Q), _f64(Kc), _f64(Vc)
    for g in range(Hq):
        h = g // 2
        assert np.array_equal(O[g, 0], Vf[h])
        assert abs(L[g, 0] - 0.5 * math.fsum(float(a) * float(b) for a, b in zip(Qf[g, 0], Kf[h]))) < 1e-12
    Q, Kc, Vc, offs = _decode_inputs(59, Hq, Hkv, D, [9, 4])
    c = Vc[3].copy()
    Vconst = np.broadcast_to(c, Vc.shape).copy()
    O, _ = oracle.decode_attention(Q, Kc, Vconst, offs, 0.5)
    assert np.allclose(O, _f64(c)[None, None, :], rtol=1e-13, atol=1e-13)


def pin_decode_over_compacted_equals_masked_layer():
    """Decoding over select + compact equals attending, in the uncompacted
    layer, to exactly the kept positions (brute force on the kept set)."""
    Hkv, n, D, G = 2, 40, 64, 2
    K = synth.normal_bf16(61, 1, (Hkv, n, D))
    V = synth.normal_bf16(61, 2, (Hkv, n, D))
    Q = synth.normal_bf16(61, 3, (Hkv * G, 1, D))
    scores = synth.evict_scores(61, Hkv, n)
    kept = oracle.select(scores, 6, k=9)
    Kc, Vc, offs = oracle.compact(K, V, kept)
    O, _ = oracle.decode_attention(Q, Kc, Vc, offs, 0.125)
    Qf, Kf, Vf = _f64(Q), _f64(K), _f64(V)
    for g in range(Hkv * G):
        h = g // G
        logits = [0.125 * math.fsum(float(a) * float(b) for a, b in zip(Qf[g, 0], Kf[h, i])) for i in kept[h]]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        tot = math.fsum(w)
        want = np.array([math.fsum(wi * float(Vf[h, i, dd]) for wi, i in zip(w, kept[h])) / tot for dd in range(D)])
        assert np.allclose(O[g, 0], want, rtol=0, atol=1e-12), g


# ---------------------------------------------------------------- value-norm pins

def _vn_inputs(seed, Hkv, n, D, d_model):
    V = synth.normal_bf16(seed, 1, (Hkv, n, D))
    W = synth.normal_bf16(seed, 2, (d_model, Hkv * D), std=0.05)
    return V, W


def pin_vnorm_orthogonal_columns():
    """Row f of W_h holds one entry +-c at column f mod D: W_h^T W_h = c^2 (d_model/D) I,
    so ||W_h v|| = c sqrt(d_model/D) ||v||."""
    Hkv, n, D, d_model, c = 2, 9, 64, 256, 0.25
    V, _ = _vn_inputs(31, Hkv, n, D, d_model)
    W = np.zeros((d_model, Hkv * D), dtype=np.float32)
    sign = np.where(np.arange(d_model) % 3 == 0, -1.0, 1.0)
    for h in range(Hkv):
        W[np.arange(d_model), h * D + np.arange(d_model) % D] = c * sign
    got = oracle.value_norms(V, _bits(W), Hkv)
    Vf = _f64(V)
    want = c * math.sqrt(d_model / D) * np.sqrt((Vf * Vf).sum(axis=2))
    assert np.allclose(got, want, rtol=1e-13, atol=0)


def pin_vnorm_gram_form():
    """||W_h v||^2 = v^T (W_h^T W_h) v, evaluated through the D x D Gram matrix."""
    Hkv, n, D, d_model = 3, 11, 64, 160
    V, W = _vn_inputs(37, Hkv, n, D, d_model)
    got = oracle.value_norms(V, W, Hkv)
    Vf, Wf = _f64(V), _f64(W)
    for h in range(Hkv):
        Wh = Wf[:, h * D:(h + 1) * D]
        G = Wh.T @ Wh
        want = np.sqrt(np.einsum("nd,de,ne->n", Vf[h], G, Vf[h]))
        assert np.allclose(got[h], want, rtol=1e-11, atol=0), h


def pin_vnorm_single_row_brute_force():
    """One nonzero row w in each head's block: ||W_h v|| = |w . v| (exact sum)."""
    Hkv, n, D, d_model = 2, 5, 64, 96
    V, W = _vn_inputs(41, Hkv, n, D, d_model)
    Wz = np.zeros_like(W)
    Wz[17] = W[17]
    got = oracle.value_norms(V, Wz, Hkv)
    Vf, wf = _f64(V), _f64(W[17])
    for h, i in itertools.product(range(Hkv), range(n)):
        want = abs(math.fsum(float(a) * float(b) for a, b in zip(wf[h * D:(h + 1) * D], Vf[h, i])))
        assert abs(got[h, i] - want) <= 1e-12 * max(want, 1e-300), (h, i)


def pin_vnorm_head_block_isolation():
    """Only head h's column block of W_O acts on head h's values."""
    Hkv, n, D, d_model = 3, 6, 64, 128
    V, W = _vn_inputs(43, Hkv, n, D, d_model)
    Wb = np.zeros_like(W)
    Wb[:, D:2 * D] = W[:, D:2 * D]
    got = oracle.value_norms(V, Wb, Hkv)
    assert np.all(got[0] == 0) and np.all(got[2] == 0) and np.all(got[1] > 0)


# ---------------------------------------------------------------- max-mode pins

def pin_max_zero_queries():
    """Q = 0: a_ji = 1/|V(j)|, so the unweighted score is 1/(n_ctx + 1) (the
    first query of a chunk sees the fewest keys) and the weighted score is
    vnorm_i * max_j 1 / ((n_ctx + (j mod C) + 1) * hnorm_j)."""
    Hq, Hkv, D, n_ctx, n_q, C = 6, 2, 64, 8, 9, 4
    d = _tiny(5, Hq, Hkv, D, n_ctx, n_q, REPEAT, C)
    Q = np.zeros((Hq, n_q, D), dtype=np.uint16)
    L = oracle.lse(Q, d["Kctx"], d["Kself"], 0.125, REPEAT, C)
    s = oracle.max_scores(Q, d["Kctx"], L, 0.125, Hkv)
    assert np.allclose(s, 1.0 / (n_ctx + 1), rtol=1e-13, atol=0)
    vn = np.linspace(0.5, 3.0, Hkv * n_ctx).reshape(Hkv, n_ctx)
    hn = np.linspace(2.0, 0.25, n_q)
    sw = oracle.max_scores(Q, d["Kctx"], L, 0.125, Hkv, vnorm=vn, hnorm=hn)
    nv = n_ctx + (np.arange(n_q) % C) + 1.0
    want = vn * np.max(1.0 / (nv * hn))
    assert np.allclose(sw, want, rtol=1e-13, atol=0)


def pin_max_orthogonal_keys():
    """Orthogonal keys k_i = e_i (D = 64, 16 context keys, zero self keys) and
    queries 64 * e_j on query head 1 only (other heads zero), scale 1. Head 1
    belongs to KV head 0 when G = 2, so on KV head 0 key i is hit once, by
    j = i: s_i = e^64 / (e^64 + 16 + i); KV head 1 only sees zero queries:
    s_i = 1/17."""
    D, T = 64, 16
    Hq, Hkv = 4, 2
    K = np.zeros((Hkv, T, D), dtype=np.float32)
    for h in range(Hkv):
        K[h, np.arange(T), np.arange(T)] = 1.0
    Q = np.zeros((Hq, T, D), dtype=np.float32)
    Q[1, np.arange(T), np.arange(T)] = 64.0
    Qb, Kb = _bits(Q), _bits(K)
    Ks = np.zeros((Hkv, T, D), dtype=np.uint16)
    L = oracle.lse(Qb, Kb, Ks, 1.0, REPEAT, T)
    s = oracle.max_scores(Qb, Kb, L, 1.0, Hkv)
    i = np.arange(T)
    want0 = 1.0 / (1.0 + (16.0 + i) * math.exp(-64.0))
    assert np.allclose(s[0], want0, rtol=1e-15, atol=0)
    assert np.all(s[0] >= 1 - 32 * math.exp(-64.0))
    assert np.allclose(s[1], 1.0 / 17.0, rtol=1e-13, atol=0)


def pin_max_brute_force():
    """Scores against brute force: scipy softmax over each (g, j)'s visible
    logits, then a plain max over queries and the group's heads."""
    Hq, Hkv, D, n_ctx, n_q, C = 4, 2, 64, 6, 7, 3
    d = _tiny(13, Hq, Hkv, D, n_ctx, n_q, REPEAT, C, qstd=1.5)
    vn = np.linspace(1.0, 2.0, Hkv * n_ctx).reshape(Hkv, n_ctx)
    hn = np.linspace(1.5, 0.5, n_q)
    Qf = synth.bf16_to_f32(d["Q"]).astype(np.float64)
    Kc = synth.bf16_to_f32(d["Kctx"]).astype(np.float64)
    Ks = synth.bf16_to_f32(d["Kself"]).astype(np.float64)
    L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], 0.25, REPEAT, C)
    s = oracle.max_scores(d["Q"], d["Kctx"], L, 0.25, Hkv, vnorm=vn, hnorm=hn)
    for h in range(Hkv):
        for i in range(n_ctx):
            best = 0.0
            for g in range(h * 2, h * 2 + 2):
                for j in range(n_q):
                    a = scipy.special.softmax(_brute_visible(Qf, Kc, Ks, g, h, j, 0.25, REPEAT, C, n_q))
                    best = max(best, a[i] * vn[h, i] / hn[j])
            assert abs(s[h, i] - best) <= 1e-12 * best, (h, i)


def pin_max_weight_scaling():
    """Eq. 3's weights act linearly: doubling vnorm doubles the score, and a
    constant hnorm c divides it by c."""
    d = _tiny(17, 4, 2, 64, 10, 8, REPEAT, 4, qstd=1.0)
    L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], 0.5, REPEAT, 4)
    s = oracle.max_scores(d["Q"], d["Kctx"], L, 0.5, 2)
    s2 = oracle.max_scores(d["Q"], d["Kctx"], L, 0.5, 2, vnorm=np.full((2, 10), 2.0),
                           hnorm=np.full(8, 4.0))
    assert np.allclose(s2, s * 0.5, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- sum-mode pins

def _causal_lse(d, scale):
    return oracle.lse(d["Q"], d["Kctx"], None, scale, CAUSAL, 0)


def pin_sum_zero_queries():
    """Q = 0: a_ji = 1/(j+1) under the causal mask, so
    t_i = G * sum_{j=i+w}^{T-1} 1/(j+1) (a harmonic tail)."""
    Hq, Hkv, D, T = 6, 2, 64, 12
    d = _tiny(19, Hq, Hkv, D, T, T, CAUSAL, 0)
    Q = np.zeros((Hq, T, D), dtype=np.uint16)
    L = oracle.lse(Q, d["Kctx"], None, 0.125, CAUSAL, 0)
    for w in (0, 1, 3, 11, 12, 40):
        t = oracle.future_mass(Q, d["Kctx"], L, 0.125, w, Hkv)
        want = np.array([3 * sum(1.0 / (j + 1) for j in range(i + w, T)) for i in range(T)])
        assert np.allclose(t, want[None, :], rtol=1e-13, atol=1e-15), w


def pin_sum_mass_conservation():
    """w = 0: every query row's softmax sums to 1 and every visible key is
    counted, so the targets of a KV head add up to G * T."""
    Hq, Hkv, D, T = 8, 2, 64, 23
    d = _tiny(23, Hq, Hkv, D, T, T, CAUSAL, 0, qstd=2.0)
    L = _causal_lse(d, 0.5)
    t = oracle.future_mass(d["Q"], d["Kctx"], L, 0.5, 0, Hkv)
    assert np.allclose(t.sum(axis=1), 4 * T, rtol=1e-13, atol=0)
    t_big = oracle.future_mass(d["Q"], d["Kctx"], L, 0.5, T, Hkv)
    assert np.all(t_big == 0.0)


def pin_sum_brute_force():
    """Future mass against brute force with scipy softmax rows."""
    Hq, Hkv, D, T, w = 4, 2, 64, 9, 2
    d = _tiny(29, Hq, Hkv, D, T, T, CAUSAL, 0, qstd=1.5)
    Qf = synth.bf16_to_f32(d["Q"]).astype(np.float64)
    Kc = synth.bf16_to_f32(d["Kctx"]).astype(np.float64)
    vn = np.linspace(0.5, 1.5, Hkv * T).reshape(Hkv, T)
    hn = np.linspace(1.0, 3.0, T)
    L = _causal_lse(d, 0.25)
    t = oracle.future_mass(d["Q"], d["Kctx"], L, 0.25, w, Hkv, vnorm=vn, hnorm=hn)
    for h in range(Hkv):
        for i in range(T):
            acc = []
            for g in range(h * 2, h * 2 + 2):
                for j in range(i + w, T):
                    a = scipy.special.softmax(_brute_visible(Qf, Kc, None, g, h, j, 0.25, CAUSAL, 0, T))
                    acc.append(a[i] * vn[h, i] / hn[j])
            want = math.fsum(acc)
            assert abs(t[h, i] - want) <= 1e-12 * max(want, 1e-300), (h, i)


# ---------------------------------------------------------------- selection pins

def _sel_scores():
    s = synth.evict_scores(31, 3, 200, tie_frac=0.2, zero_frac=0.05)
    s[1, 5] = np.float32(-0.0)
    s[1, 6] = np.float32(0.0)
    s[2, 7] = np.nan
    s[2, 8] = np.inf
    s[2, 9] = -np.inf
    s[0, 3] = np.nan
    return s


def pin_select_topk_library_order():
    """Top-k equals the first k of Python's sort on (NaN last, -score,
    position) over the non-window keys, plus the window."""
    s = _sel_scores()
    for k, w in [(0, 0), (17, 10), (50, 0), (190, 10), (500, 30), (5, 200), (5, 250)]:
        kept = oracle.select(s, w, k=k)
        for h in range(s.shape[0]):
            n = s.shape[1]
            ww = min(w, n)
            cand = s[h, : n - ww].astype(np.float64).tolist()
            order = sorted(range(len(cand)),
                           key=lambda i: (math.isnan(cand[i]), 0.0 if math.isnan(cand[i]) else -cand[i], i))
            order = np.asarray(order, dtype=np.int64)
            want = np.union1d(order[: min(k, n - ww)], np.arange(n - ww, n))
            assert np.array_equal(kept[h], want), (k, w, h)


def pin_select_invariants():
    """Exactly k' + |W| kept; W kept; ascending; top-k sets nest in k;
    tau = 0 keeps every non-negative score; tau = inf keeps only the window."""
    s = _sel_scores()
    n, w = s.shape[1], 16
    prev = None
    for k in range(0, n - w + 3, 7):
        kept = oracle.select(s, w, k=k)
        for h in range(s.shape[0]):
            assert kept[h].size == min(k, n - w) + w
            assert np.all(np.diff(kept[h]) > 0)
            assert set(range(n - w, n)) <= set(kept[h].tolist())
            if prev is not None:
                assert set(prev[h].tolist()) <= set(kept[h].tolist())
        prev = kept
    kept0 = oracle.select(s, w, tau=0.0)
    for h in range(s.shape[0]):
        want = np.union1d(np.nonzero(s[h, : n - w] >= 0)[0], np.arange(n - w, n))
        assert np.array_equal(kept0[h], want)
    kinf = oracle.select(s, w, tau=np.inf)
    for h in range(s.shape[0]):
        want = np.union1d(np.nonzero(s[h, : n - w] == np.inf)[0], np.arange(n - w, n))
        assert np.array_equal(kinf[h], want)


def pin_select_ties_lower_index_first():
    """Equal scores at the cut are taken lowest position first; -0 == +0."""
    s = np.array([[1.0, 2.0, 2.0, 2.0, 0.5, 2.0, 3.0, 0.0]], dtype=np.float32)
    assert oracle.select(s, 1, k=3)[0].tolist() == [1, 2, 6, 7]
    z = np.array([[-0.0, 0.0, -0.0, 1.0]], dtype=np.float32)
    assert oracle.select(z, 0, k=2)[0].tolist() == [0, 3]
    assert oracle.select(z, 0, tau=0.0)[0].tolist() == [0, 1, 2, 3]


def pin_select_layer_scope_library_order():
    """Layer scope: Python's sort of (-score, head, position) over every head's
    candidates, first k, plus each head's window."""
    s = _sel_scores()
    Hkv, n = s.shape
    for k, w in [(0, 3), (7, 0), (25, 5), (10 ** 6, 4)]:
        got = oracle.select(s, w, k=k, scope="layer")
        cand = [(h, i) for h in range(Hkv) for i in range(n - w)]
        rank = sorted(cand, key=lambda hi: (math.isnan(s[hi]), 0.0 if math.isnan(s[hi]) else -float(s[hi]),
                                            hi[0], hi[1]))
        want = [set(range(n - w, n)) for _ in range(Hkv)]
        for h, i in rank[:min(k, len(cand))]:
            want[h].add(i)
        for h in range(Hkv):
            assert list(got[h]) == sorted(want[h]), (k, w, h)


def pin_select_layer_scope_budget_follows_scores():
    """Head h's candidates all outscore head h+1's: a layer budget of k fills
    the heads in order (head 0 first), whatever the per-head share."""
    Hkv, n, w = 3, 20, 2
    s = np.stack([np.linspace(1.0, 0.9, n) + (Hkv - h) for h in range(Hkv)]).astype(np.float32)
    got = oracle.select(s, w, k=25, scope="layer")
    assert [g.size for g in got] == [18 + w, 7 + w, w]
    # equal scores in every head: ties go to the lower head, then the lower position
    t = np.tile(np.array([5, 9, 9, 1, 7, 3], dtype=np.float32), (3, 1))
    got = oracle.select(t, 0, k=4, scope="layer")
    assert [list(g) for g in got] == [[1, 2], [1, 2], []]
    same = oracle.select(s, w, tau=2.5, scope="layer")  # scope plays no part under a threshold
    assert all(np.array_equal(a, b) for a, b in zip(same, oracle.select(s, w, tau=2.5)))


def pin_select_threshold_is_ge():
    """Keep iff score >= tau (Algorithm 1's comparison), window always kept."""
    s = np.array([[0.1, 0.2, 0.3, 0.2, 0.05, 0.0]], dtype=np.float32)
    assert oracle.select(s, 2, tau=np.float32(0.2))[0].tolist() == [1, 2, 3, 4, 5]
    assert oracle.select(s, 0, tau=np.float32(0.2))[0].tolist() == [1, 2, 3]


# ---------------------------------------------------------------- compaction pins

def pin_compact_rows_bitwise():
    """Compacted rows are the kept rows, bit for bit, head after head."""
    K = synth.normal_bf16(41, 1, (3, 50, 64))
    V = synth.normal_bf16(41, 2, (3, 50, 64))
    kept = [np.array([0, 7, 49]), np.array([], dtype=np.int64), np.arange(10, 50, 3)]
    Ko, Vo, off = oracle.compact(K, V, kept)
    assert off.tolist() == [0, 3, 3, 3 + len(range(10, 50, 3))]
    r = 0
    for h, idx in enumerate(kept):
        for i in idx:
            assert np.array_equal(Ko[r], K[h, i]) and np.array_equal(Vo[r], V[h, i])
            r += 1


# ---------------------------------------------------------------- streaming threshold

def pin_stream_hand_example():
    """Worked by hand from the keep rule (w = 2, tau = 3, one head), scores
    5, 1, 7, 2, 9, 0 arriving in calls of 2, 1 and 3 tokens: position 0
    (score 5) stays when it leaves at length 3, position 1 (score 1) goes at
    length 4, position 2 (7) stays at length 5, position 3 (2) goes at 6."""
    st = oracle.stream_states(np.array([[5, 1, 7, 2, 9, 0]], dtype=np.float32), 2, 3.0, [2, 1, 3])
    (n1, sl1, k1), (n2, sl2, k2), (n3, sl3, k3) = st
    assert (n1, sl1.tolist(), k1[0].tolist()) == (2, [[0, 1]], [])
    assert (n2, sl2.tolist(), k2[0].tolist()) == (3, [[2, 1]], [0])
    assert (n3, sl3.tolist(), k3[0].tolist()) == (6, [[4, 5]], [0, 2])


def _stream_scores(seed, Hkv, T):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(Hkv, T)).astype(np.float32)
    s[0, 2] = np.nan
    s[-1, 4] = np.inf
    s[0, 6] = 0.25  # equal to tau below
    s[-1, 9] = 0.25
    return s


def pin_stream_equals_rule_at_every_length():
    """After every call, the window slots plus the kept tokens are exactly
    what the keep rule gives for the tokens seen so far (the batch selection
    with the same window and threshold)."""
    for w, steps in ((0, [1, 4, 1, 20]), (1, [1, 1, 7, 3]), (3, [2, 1, 1, 9, 1]), (7, [1, 30, 2])):
        s = _stream_scores(100 + w, 3, sum(steps))
        for n, slots, kept in oracle.stream_states(s, w, 0.25, steps):
            ref = oracle.select(s[:, :n], w, tau=0.25)
            for h in range(3):
                live = np.sort(np.concatenate([slots[h][slots[h] >= 0], kept[h]]))
                assert np.array_equal(live, ref[h]), (w, n, h)


def pin_stream_slots_and_order():
    """Slot s holds the window token p with p mod w = s, the window is the
    last min(n, w) positions, and kept tokens are ascending and older."""
    w, steps = 5, [3, 1, 1, 11, 2]
    s = _stream_scores(7, 2, sum(steps))
    for n, slots, kept in oracle.stream_states(s, w, 0.25, steps):
        for h in range(2):
            win = sorted(int(p) for p in slots[h] if p >= 0)
            assert win == list(range(max(0, n - w), n))
            for sl, p in enumerate(slots[h]):
                assert p < 0 or p % w == sl
            k = kept[h].tolist()
            assert k == sorted(k) and all(p < n - w for p in k)


def pin_stream_window_zero():
    """w = 0: every token is decided on arrival; the kept tokens are those
    whose score passes, in order."""
    s = _stream_scores(9, 2, 12)
    n, slots, kept = oracle.stream_states(s, 0, 0.25, [5, 7])[-1]
    assert n == 12 and slots.shape == (2, 0)
    for h in range(2):
        assert kept[h].tolist() == [p for p in range(12) if s[h, p] >= np.float32(0.25)]


# ---------------------------------------------------------------- sampling

def pin_sampled_rows_and_keys_match_full():
    """Restricting the oracle to sampled query rows or keys returns exactly the
    matching entries of the full computation (used for full-size sampling)."""
    d = _tiny(37, 6, 2, 64, 40, 29, REPEAT, 10, qstd=1.0)
    L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], 0.5, REPEAT, 10)
    rows = np.array([0, 3, 9, 10, 19, 28])
    Ls = oracle.lse(d["Q"], d["Kctx"], d["Kself"], 0.5, REPEAT, 10, rows=rows)
    assert np.array_equal(Ls, L[:, rows])
    s = oracle.max_scores(d["Q"], d["Kctx"], L, 0.5, 2)
    keys = np.array([1, 5, 39])
    assert np.array_equal(oracle.max_scores(d["Q"], d["Kctx"], L, 0.5, 2, keys=keys), s[:, keys])
    dc = _tiny(41, 4, 2, 64, 30, 30, CAUSAL, 0, qstd=1.0)
    Lc = _causal_lse(dc, 0.5)
    t = oracle.future_mass(dc["Q"], dc["Kctx"], Lc, 0.5, 3, 2)
    keys = np.array([0, 7, 26, 29])
    assert np.allclose(oracle.future_mass(dc["Q"], dc["Kctx"], Lc, 0.5, 3, 2, keys=keys), t[:, keys],
                       rtol=1e-14, atol=0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
