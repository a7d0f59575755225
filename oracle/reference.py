"""fp64 reference for the scoring and eviction path (test infrastructure only).

Pages cited (by title; section, equation or algorithm on that page):

* [KVzap]  "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning"
  (Jump2Paper archive page): §3.1 (KVzip score, Eq. 1, the repeat prompt and
  the GQA note in its variable table), §3.2 (Eq. 2 residual update, Eq. 3
  KVzip+ score), the thresholding + sliding-window rule, Algorithm 1.
* [KVpop]  "[논문리뷰] KVpop -- Key-Value Cache Compression with Predictive
  Online Pruning": §1 Key Terms (future-attention target, transposed-attention
  pass from LSE normalisers), §3 Method (per-head top-k).
* [KVzip]  KVzip review blog: "Methods" (teacher-forced, parallel repeat of
  the context), "Methods: technical-details" (the repeat runs chunk by chunk).

Conventions (readings where the pages are silent; each is listed in the
design notes):

* The logit of query j (query head g) against key i is l_ji = scale * q_j.k_i.
* Query head g belongs to KV head h = g // G, G = Hq / Hkv (consecutive groups).
* REPEAT visibility: repeat query j of chunk c sees every context key plus the
  self keys of chunk c whose position is <= j. CAUSAL visibility: key i <= j.
* Inputs are bf16 bit patterns (uint16); they are widened exactly to fp64.

No blocking here changes any arithmetic: query rows are independent, and rows
are visited in blocks only to bound memory.
"""
from __future__ import annotations

import numpy as np

REPEAT = "repeat"
CAUSAL = "causal"

_ROWS = 256  # query rows per block (memory bound only)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _row_blocks(n_q: int, mask: str, chunk: int, rows=None):
    """Blocks of query positions (int arrays); under REPEAT a block stays inside
    one chunk [c0, c1). ``rows`` restricts the positions visited."""
    c = chunk if (mask == REPEAT and chunk > 0) else max(n_q, 1)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    for c0 in range(0, n_q, c):
        c1 = min(c0 + c, n_q)
        in_chunk = rows[(rows >= c0) & (rows < c1)]
        for b0 in range(0, in_chunk.size, _ROWS):
            yield in_chunk[b0:b0 + _ROWS], c0, c1


def visible_logits(q_rows, rows, Kctx_h, Kself_h, scale, mask, c0=0, c1=0):
    """Logits of the queries at positions ``rows`` against the keys they can
    see; -inf elsewhere.

    REPEAT ([KVzap] §3.1 repeat prompt; [KVzip] Methods and technical
    details): columns are the n_ctx context keys followed by the self keys of
    the chunk [c0, c1) that holds the rows; self key p is visible to query j
    iff p <= j (teacher-forced, causal inside the repeat).
    CAUSAL: columns are the keys 0..n_ctx-1; key i is visible iff i <= j.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if mask == REPEAT:
        l_ctx = scale * (q_rows @ Kctx_h.T)
        self_pos = np.arange(c0, c1)
        l_self = scale * (q_rows @ Kself_h[c0:c1].T)
        l_self = np.where(self_pos[None, :] <= rows[:, None], l_self, -np.inf)
        return np.concatenate([l_ctx, l_self], axis=1)
    if mask == CAUSAL:
        l = scale * (q_rows @ Kctx_h.T)
        keys = np.arange(Kctx_h.shape[0])
        return np.where(keys[None, :] <= rows[:, None], l, -np.inf)
    raise ValueError(mask)


def kv_head_of(g: int, G: int) -> int:
    """GQA: query head g reads KV head g // G (consecutive groups of G)."""
    return g // G


def outside_window(keys, rows, window):
    """True where key i has left the window of the last `window` tokens at
    query j, i.e. j >= i + window ([KVpop] §1 future-attention target)."""
    return keys[None, :] + window <= rows[:, None]


def _dims(Q, Kctx):
    Hq, n_q, D = Q.shape
    Hkv = Kctx.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq, n_q, D, Hkv, Hq // Hkv


def lse(Q, Kctx, Kself, scale, mask=REPEAT, chunk=0, rows=None):
    """Per-query log-sum-exp normaliser, natural log, fp64 [Hq, n_q].

    LSE_j = ln sum_{i visible to j} exp(l_ji), the normaliser an attention
    kernel returns alongside its output ([KVpop] §1, transposed-attention
    pass), evaluated as M + ln sum exp(l - M) with M the row maximum.
    ``rows`` (positions) restricts the output to those queries: [Hq, len(rows)].
    """
    Hq, n_q, D, Hkv, G = _dims(Q, Kctx)
    Qf, Kc = bf16_bits_to_f64(Q), bf16_bits_to_f64(Kctx)
    Ks = bf16_bits_to_f64(Kself) if Kself is not None else None
    scale = float(np.float32(scale))
    want = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    col_of = {int(j): c for c, j in enumerate(want)}
    out = np.empty((Hq, want.size))
    for g in range(Hq):
        h = kv_head_of(g, G)
        for blk, c0, c1 in _row_blocks(n_q, mask, chunk, want):
            L = visible_logits(Qf[g, blk], blk, Kc[h], Ks[h] if Ks is not None else None,
                               scale, mask, c0, c1)
            M = L.max(axis=1, keepdims=True)
            out[g, [col_of[int(j)] for j in blk]] = M[:, 0] + np.log(np.exp(L - M).sum(axis=1))
    return out


def attention(Q, Kctx, Kself, Vctx, Vself, scale, mask=REPEAT, chunk=0, rows=None):
    """Attention output and normaliser, fp64: (O [Hq, m, D], LSE [Hq, m]) for
    the m query positions in ``rows`` (all when None).

    o_j = sum_i a_ji v_i over the keys visible to j, a_ji = exp(l_ji - LSE_j):
    the per-head sum that [KVzap] §3.2 Eq. 2 adds to the residual stream
    (there after W_O), and the output an attention kernel returns together
    with LSE_j ([KVpop] §1). Values follow the columns of ``visible_logits``:
    REPEAT sees the context values, then the self values of the query's
    chunk; CAUSAL sees the values 0..n_ctx-1. Values share the key layout
    ([Hkv, n, D], bf16 bits).
    """
    Hq, n_q, D, Hkv, G = _dims(Q, Kctx)
    Qf, Kc, Vc = bf16_bits_to_f64(Q), bf16_bits_to_f64(Kctx), bf16_bits_to_f64(Vctx)
    Ks = bf16_bits_to_f64(Kself) if Kself is not None else None
    Vs = bf16_bits_to_f64(Vself) if Vself is not None else None
    scale = float(np.float32(scale))
    want = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    col_of = {int(j): c for c, j in enumerate(want)}
    O = np.empty((Hq, want.size, D))
    L_out = np.empty((Hq, want.size))
    for g in range(Hq):
        h = kv_head_of(g, G)
        for blk, c0, c1 in _row_blocks(n_q, mask, chunk, want):
            L = visible_logits(Qf[g, blk], blk, Kc[h], Ks[h] if Ks is not None else None,
                               scale, mask, c0, c1)
            vals = np.concatenate([Vc[h], Vs[h][c0:c1]], axis=0) if mask == REPEAT else Vc[h]
            M = L.max(axis=1, keepdims=True)
            E = np.exp(L - M)
            tot = E.sum(axis=1, keepdims=True)
            cols = [col_of[int(j)] for j in blk]
            L_out[g, cols] = M[:, 0] + np.log(tot[:, 0])
            O[g, cols] = (E / tot) @ vals
    return O, L_out


def attention_weights(Q, Kctx, Kself, scale, mask, chunk, g, j0, j1, lse_rows):
    """Softmax rows a_ji = exp(l_ji - LSE_j) for query head g, rows [j0, j1)
    (one chunk at most), over the same columns as ``visible_logits``."""
    Hq, n_q, D, Hkv, G = _dims(Q, Kctx)
    Qf, Kc = bf16_bits_to_f64(Q), bf16_bits_to_f64(Kctx)
    Ks = bf16_bits_to_f64(Kself) if Kself is not None else None
    c = chunk if (mask == REPEAT and chunk > 0) else max(n_q, 1)
    c0 = (j0 // c) * c
    c1 = min(c0 + c, n_q)
    h = kv_head_of(g, G)
    L = visible_logits(Qf[g, j0:j1], np.arange(j0, j1), Kc[h], Ks[h] if Ks is not None else None,
                       float(np.float32(scale)), mask, c0, c1)
    return np.exp(L - np.asarray(lse_rows, dtype=np.float64)[:, None])


def max_scores(Q, Kctx, lse_in, scale, n_kvheads, vnorm=None, hnorm=None, keys=None):
    """KVzip / KVzip+ score of every context key, fp64 [Hkv, n_ctx].

    [KVzap] §3.1 Eq. 1: s_i = max over repeat queries j of a_ji, with every
    query head of the key's GQA group taking part. [KVzap] §3.2 Eq. 3: the
    KVzip+ score multiplies a_ji by ||W_O v_i|| / ||h_j|| inside the max
    (``vnorm[h, i]`` and ``hnorm[j]``; either may be omitted, meaning 1).
    a_ji = exp(l_ji - LSE_j), with LSE_j taken as given (``lse_in`` [Hq, n_q]).
    Context keys are visible to every repeat query. With no queries the
    score is 0. ``keys`` (positions) restricts the output to those keys.
    """
    Hq, n_q, D, Hkv, G = _dims(Q, Kctx)
    assert Hkv == n_kvheads
    Qf, Kc = bf16_bits_to_f64(Q), bf16_bits_to_f64(Kctx)
    lse_in = np.asarray(lse_in, dtype=np.float64)
    scale = float(np.float32(scale))
    n_ctx = Kc.shape[1]
    vn = np.ones((Hkv, n_ctx)) if vnorm is None else np.asarray(vnorm, dtype=np.float64)
    hn = np.ones(n_q) if hnorm is None else np.asarray(hnorm, dtype=np.float64)
    if keys is not None:
        keys = np.asarray(keys, dtype=np.int64)
        Kc, vn = Kc[:, keys], vn[:, keys]
        n_ctx = keys.size
    s = np.zeros((Hkv, n_ctx))
    for g in range(Hq):
        h = kv_head_of(g, G)
        for j0 in range(0, n_q, _ROWS):
            j1 = min(j0 + _ROWS, n_q)
            a = np.exp(scale * (Qf[g, j0:j1] @ Kc[h].T) - lse_in[g, j0:j1, None])
            w = a * vn[h][None, :] / hn[j0:j1, None]
            s[h] = np.maximum(s[h], w.max(axis=0))
    return s


def future_mass(Q, K, lse_in, scale, window, n_kvheads, vnorm=None, hnorm=None, keys=None):
    """KVpop future-attention target, fp64 [Hkv, T].

    [KVpop] §1: the attention mass token i receives after it has left the
    protected window of the last w tokens, computed from the LSE normalisers
    rather than a stored attention map. Token i is outside the window of query
    j exactly when j >= i + w, so t_i = sum_{g in group} sum_{i+w <= j < T} a_ji,
    a_ji = exp(l_ji - LSE_j) with LSE_j given (``lse_in`` [Hq, T]). Query heads
    of a group are summed. Optional ``vnorm[h, i]`` / ``hnorm[j]`` weight each
    term as in [KVzap] §3.2 Eq. 3. ``keys`` (positions) restricts the output
    to those keys.
    """
    Hq, T, D, Hkv, G = _dims(Q, K)
    assert Hkv == n_kvheads and K.shape[1] == T
    Qf, Kf = bf16_bits_to_f64(Q), bf16_bits_to_f64(K)
    lse_in = np.asarray(lse_in, dtype=np.float64)
    scale = float(np.float32(scale))
    vn = np.ones((Hkv, T)) if vnorm is None else np.asarray(vnorm, dtype=np.float64)
    hn = np.ones(T) if hnorm is None else np.asarray(hnorm, dtype=np.float64)
    keys = np.arange(T) if keys is None else np.asarray(keys, dtype=np.int64)
    Kf, vn = Kf[:, keys], vn[:, keys]
    t = np.zeros((Hkv, keys.size))
    for g in range(Hq):
        h = kv_head_of(g, G)
        for j0 in range(0, T, _ROWS):
            j1 = min(j0 + _ROWS, T)
            rows = np.arange(j0, j1)
            a = np.exp(scale * (Qf[g, j0:j1] @ Kf[h].T) - lse_in[g, j0:j1, None])
            after_window = outside_window(keys, rows, window)
            w = np.where(after_window, a * vn[h][None, :] / hn[j0:j1, None], 0.0)
            t[h] += w.sum(axis=0)
    return t


def decode_attention(Q, K_cache, V_cache, head_offsets, scale):
    """Decode queries attending to the compacted per-head cache, fp64:
    (O [Hq, n_q, D], LSE [Hq, n_q]).

    Eviction leaves each KV head its own number of rows, written head after
    head ([KVzap] Algorithm 1: keys[indices], values[indices]); the pages name
    that non-uniform cache as what a variable-length kernel must serve before
    pruning pays off ([KVzap] "Limitation 3" and FAQ "Q4"). Query head g
    (KV head h = g // G) sees rows head_offsets[h] .. head_offsets[h+1]-1 of
    K_cache / V_cache ([rows, D] bf16 bits), every decode query all of them:
    o_j = sum_r a_jr v_r, a_jr = exp(l_jr - LSE_j), l_jr = scale * q_j . k_r
    (the per-head sum of [KVzap] §3.2 Eq. 2). A head that kept no rows gives
    O = 0 and LSE = -inf.
    """
    Qf, Kf, Vf = bf16_bits_to_f64(Q), bf16_bits_to_f64(K_cache), bf16_bits_to_f64(V_cache)
    Hq, n_q, D = Qf.shape
    offs = np.asarray(head_offsets, dtype=np.int64)
    Hkv = offs.size - 1
    G = Hq // Hkv
    scale = float(np.float32(scale))
    O = np.zeros((Hq, n_q, D))
    L_out = np.full((Hq, n_q), -np.inf)
    for g in range(Hq):
        h = kv_head_of(g, G)
        r0, r1 = int(offs[h]), int(offs[h + 1])
        if r1 == r0:
            continue
        L = scale * (Qf[g] @ Kf[r0:r1].T)          # [n_q, rows]
        M = L.max(axis=1, keepdims=True)
        E = np.exp(L - M)
        tot = E.sum(axis=1, keepdims=True)
        L_out[g] = M[:, 0] + np.log(tot[:, 0])
        O[g] = (E / tot) @ Vf[r0:r1]
    return O, L_out


def value_norms(V, W_O, n_kvheads):
    """||W_O v_i|| per KV head and key, fp64 [Hkv, n].

    [KVzap] §3.2, Eq. 3 and its variable table: the L2 norm of value vector
    v_i after the attention output projection W_O, the weight KVzip+ puts on
    a_ji. W_O is [d_model, Hkv * D] (bf16 bits); KV head h's values meet the
    column block [h*D, (h+1)*D). Computed as the plain matrix-vector product
    y = W_h v_i and its Euclidean norm.
    """
    Vf, Wf = bf16_bits_to_f64(V), bf16_bits_to_f64(W_O)
    Hkv, n, D = Vf.shape
    assert Hkv == n_kvheads and Wf.shape[1] == Hkv * D
    out = np.empty((Hkv, n))
    for h in range(Hkv):
        W_h = Wf[:, h * D:(h + 1) * D]
        for i0 in range(0, n, _ROWS):
            i1 = min(i0 + _ROWS, n)
            Y = Vf[h, i0:i1] @ W_h.T          # [rows, d_model]
            out[h, i0:i1] = np.sqrt((Y * Y).sum(axis=1))
    return out


def select(scores, window, k=None, tau=None, scope="head"):
    """Kept positions per KV head, ascending, as a list of int64 arrays.

    The last ``window`` positions are always kept ([KVzap] thresholding rule and
    Algorithm 1: the window's scores are forced to +inf). Among the rest:
    * top-k ([KVpop] §3 per-head top-k; KVzip's fixed keep ratio in [KVzap]
      "Thresholding"): the min(k, candidates) best by (score descending,
      position ascending);
    * threshold: keep iff score >= tau ([KVzap] thresholding rule, Algorithm 1).
    ``scope="layer"`` (top-k only) ranks the candidates of all heads together,
    the layer-wise top-k that [KVzap] §4.6 "threshold vs fixed ratio"
    compares against: the min(k, all candidates) best by (score descending,
    head ascending, position ascending), so each head keeps its own share.
    NaN scores rank below every number and never pass the threshold; -0 and +0
    are equal. Output order is ascending position, as a where() over the mask.
    """
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k, tau")
    if scope not in ("head", "layer"):
        raise ValueError(scope)
    s_all = np.asarray(scores, dtype=np.float64)
    if scope == "layer" and k is not None:
        Hkv, n = s_all.shape
        w = min(max(int(window), 0), n)
        heads = np.repeat(np.arange(Hkv), n - w)
        pos = np.tile(np.arange(n - w), Hkv)
        vals = s_all[:, : n - w].reshape(-1)
        is_nan = np.isnan(vals)
        neg = np.where(is_nan, 0.0, -vals)
        kk = min(max(int(k), 0), vals.size)
        order = np.lexsort((pos, heads, neg, is_nan))  # NaN last, then -score, head, position
        keep = np.zeros((Hkv, n), dtype=bool)
        keep[:, n - w:] = True
        keep[heads[order[:kk]], pos[order[:kk]]] = True
        return [np.nonzero(keep[h])[0].astype(np.int64) for h in range(Hkv)]
    out = []
    for h in range(s_all.shape[0]):
        s = s_all[h]
        n = s.shape[0]
        w = min(max(int(window), 0), n)
        cand = np.arange(n - w)
        keep = np.zeros(n, dtype=bool)
        keep[n - w:] = True
        if k is not None:
            kk = min(max(int(k), 0), cand.size)
            is_nan = np.isnan(s[cand])
            neg = np.where(is_nan, 0.0, -s[cand])
            order = np.lexsort((cand, neg, is_nan))  # NaN last, then -score, then position
            keep[cand[order[:kk]]] = True
        else:
            keep[cand] |= s[cand] >= float(np.float32(tau))
        out.append(np.nonzero(keep)[0].astype(np.int64))
    return out


def stream_states(scores, window, tau, steps):
    """Threshold pruning applied as tokens arrive, simulated token by token.

    [KVzap] thresholding rule: at sequence length T, token t is kept iff
    score_t >= tau or t >= T - w. The page asks for a criterion that also
    works while decoding (its phase-agnostic criterion), so the rule is
    re-applied at every length T: when the token at position p arrives
    (T = p + 1), the token at p - w leaves the window and stays only if its
    score passes; a token once dropped never returns. With w = 0 the arriving
    token is decided at once.

    Storage this returns, per KV head (the layout the cache keeps): a ring of
    w window slots, slot p mod w holding the window token at position p
    (-1 while empty), and the kept tokens that left the window, ascending.
    ``scores`` is [Hkv, T_total]; ``steps`` lists the tokens appended by each
    call. Returns one (n_seen, slot_pos [Hkv, w], kept list) per call.
    """
    s = np.asarray(scores, dtype=np.float64)
    Hkv = s.shape[0]
    w = max(int(window), 0)
    tau32 = float(np.float32(tau))
    slot_pos = np.full((Hkv, w), -1, dtype=np.int64)
    kept = [[] for _ in range(Hkv)]
    n = 0
    out = []
    for m in steps:
        for _ in range(int(m)):
            p = n  # the arriving token; the sequence length becomes p + 1
            for h in range(Hkv):
                q = p - w  # the token that has just left the last w positions
                if q >= 0 and s[h, q] >= tau32:
                    kept[h].append(q)
                if w > 0:
                    slot_pos[h, p % w] = p
            n += 1
        out.append((n, slot_pos.copy(), [np.array(k, dtype=np.int64) for k in kept]))
    return out


def compact(K, V, kept):
    """Copy the kept rows of K and V per head into one dense cache.

    Algorithm 1 of [KVzap] returns keys[indices], values[indices]. Heads are
    laid out one after another; ``head_offsets[h]`` is the first row of head h
    and ``head_offsets[Hkv]`` the total. Rows are copied bit for bit.
    """
    counts = np.array([idx.size for idx in kept], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    D = K.shape[2]
    K_out = np.empty((offsets[-1], D), dtype=K.dtype)
    V_out = np.empty((offsets[-1], D), dtype=V.dtype)
    for h, idx in enumerate(kept):
        K_out[offsets[h]:offsets[h + 1]] = K[h, idx]
        V_out[offsets[h]:offsets[h + 1]] = V[h, idx]
    return K_out, V_out, offsets
