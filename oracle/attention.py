"""fp64 reference attention: materialised scores, two-pass softmax, P V, LSE.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP path.  Every array is converted to float64 on entry; bf16 and fp32 inputs
upcast exactly, so the oracle sees exactly the stored input values.

Readings of the pages that this file fixes (page titles abbreviated):

* Scale is a multiplier applied to Q K^T ("Attention三算子融合实战" 3.2 writes
  the score as qk * scale with scale usually 1/sqrt(D); section 1.1's "divide
  by the scaling factor" is the same thing with the reciprocal).
* Causal: query i sees key j iff j <= i, diagonal included (same page, 4.3:
  keys j > row get -inf).  Prefill has as many queries as keys.
* GQA: query head h reads KV head g = h // (Hq / Hkv), i.e. contiguous groups
  ("手写Triton kernel重构Qwen3.5-0.8B" 2.1 broadcasts 2 KV heads to 8 query
  heads).
* Layout [B, H, S, D], contiguous ("Attention三算子融合实战" 3.2 addresses a
  row as head * S * D + row * D + d).
* Decode cache is packed per sequence: sequence b is a [Hkv, L_b, D] block at
  element offset Hkv * D * sum(L_0 .. L_{b-1}).  The single query of sequence b
  attends to all L_b cached keys (it is the newest token; section 1.3 of the
  same page: Q has one row while K and V grow with the history).
* LSE is the natural-log log-sum-exp of the scaled, masked score row
  ("triton-optimization" 3.5: m + log(d)).
* A row with no visible key (L_b = 0) gives o = 0 and lse = -inf; the pages
  never produce one.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _kv_head(h, Hq, Hkv):
    """KV head read by query head h: contiguous groups of Hq // Hkv heads."""
    return h // (Hq // Hkv)


def _check_heads(Hq, Hkv):
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")


def _visible(query_pos, n_keys, causal):
    """Boolean [len(query_pos), n_keys]: may query at position i see key j?"""
    j = np.arange(n_keys)[None, :]
    if causal:
        return j <= np.asarray(query_pos)[:, None]
    return np.ones((len(query_pos), n_keys), dtype=bool)


def _two_pass_softmax(s, visible):
    """Row softmax of the scores s over the visible entries, in two passes.

    Pass 1 takes the row max m over visible scores; pass 2 exponentiates
    s - m, sums to l and divides.  Returns (P, lse) with lse = m + ln(l).
    Invisible entries get probability 0 (a -inf score).  Rows with no visible
    entry return P = 0 and lse = -inf.
    """
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=-1, initial=-np.inf)                  # pass 1
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.where(visible, np.exp(s - m_safe[..., None]), 0.0)   # pass 2
    l = p.sum(axis=-1)
    l_safe = np.where(empty, 1.0, l)
    P = p / l_safe[..., None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return P, lse


def softmax_probabilities(q, k, scale, causal):
    """The probability matrix P [B, Hq, S, S] of prefill attention."""
    q, k = _f64(q), _f64(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _check_heads(Hq, Hkv)
    P = np.zeros((B, Hq, S, S))
    vis = _visible(np.arange(S), S, causal)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (q[b, h] @ k[b, g].T)
            P[b, h], _ = _two_pass_softmax(s, vis)
    return P


def prefill(q, k, v, scale, causal):
    """Prefill attention.  q [B,Hq,S,D]; k, v [B,Hkv,S,D].

    Returns (o [B,Hq,S,D], lse [B,Hq,S]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _check_heads(Hq, Hkv)
    if k.shape != (B, Hkv, S, D) or v.shape != (B, Hkv, S, D):
        raise ValueError("k and v must be [B, Hkv, S, D] matching q")
    o = np.zeros((B, Hq, S, D))
    lse = np.zeros((B, Hq, S))
    vis = _visible(np.arange(S), S, causal)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (q[b, h] @ k[b, g].T)            # materialised S
            P, lse[b, h] = _two_pass_softmax(s, vis)
            o[b, h] = P @ v[b, g]
    return o, lse


def prefill_rows(q, k, v, scale, causal, rows):
    """Prefill attention evaluated only at selected query rows.

    rows: int array [Hq, R]; head h is evaluated at rows[h] (the same rows for
    every batch entry).  Returns (o [B,Hq,R,D], lse [B,Hq,R]).  Each selected
    row is the same computation as in ``prefill``; only the score rows that
    are needed are materialised.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _check_heads(Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.shape[1]
    o = np.zeros((B, Hq, R, D))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            r = rows[h]
            s = scale * (q[b, h, r] @ k[b, g].T)
            P, lse[b, h] = _two_pass_softmax(s, _visible(r, S, causal))
            o[b, h] = P @ v[b, g]
    return o, lse


def prefill_varlen(q, k, v, cu_seqlens, Hq, Hkv, scale, causal):
    """Prefill of a ragged batch: each sequence is attended on its own.

    Sequence b has S_b = cu[b+1] - cu[b] tokens; q (and the returned o) is a
    flat array of [Hq, S_b, D] blocks at element offset Hq*D*cu[b], k and v of
    [Hkv, S_b, D] blocks at Hkv*D*cu[b] (the packed layout of the decode
    cache, with the query rows packed the same way).  The returned lse holds
    [Hq, S_b] blocks at offset Hq*cu[b].  Padding never enters a score: this
    is the padding mask of "Attention三算子融合实战" 4.3 written as separate
    sequences.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    q, k, v = _f64(q).reshape(-1), _f64(k).reshape(-1), _f64(v).reshape(-1)
    B = len(cu) - 1
    N = int(cu[-1])
    if N and q.size % (Hq * N):
        raise ValueError("q does not match cu_seqlens")
    D = q.size // (Hq * N) if N else 0
    if k.size != Hkv * N * D or v.size != k.size:
        raise ValueError("k, v do not match cu_seqlens")
    o = np.zeros(Hq * N * D)
    lse = np.zeros(Hq * N)
    for b in range(B):
        S = int(cu[b + 1] - cu[b])
        if S <= 0:
            continue
        qb = q[Hq * D * cu[b]: Hq * D * cu[b + 1]].reshape(1, Hq, S, D)
        kb = k[Hkv * D * cu[b]: Hkv * D * cu[b + 1]].reshape(1, Hkv, S, D)
        vb = v[Hkv * D * cu[b]: Hkv * D * cu[b + 1]].reshape(1, Hkv, S, D)
        ob, lb = prefill(qb, kb, vb, scale, causal)
        o[Hq * D * cu[b]: Hq * D * cu[b + 1]] = ob.reshape(-1)
        lse[Hq * cu[b]: Hq * cu[b + 1]] = lb.reshape(-1)
    return o, lse


def prefill_padded(q, k, v, seqlens, scale, causal):
    """Prefill of a padded batch: q [B,Hq,S,D], k, v [B,Hkv,S,D], sequence b
    valid in its first L_b = clamp(seqlens[b], 0, S) rows.

    Valid rows attend the valid keys only (the padding mask of
    "Attention三算子融合实战" 4.3: keys past the valid length are -inf), i.e.
    sequence b is attended as the dense prefill of its first L_b rows; the
    padding rows get o = 0 and lse = -inf (the empty-row reading also used
    by decode for an empty cache).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    o = np.zeros((B, Hq, S, D))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        L = min(max(int(seqlens[b]), 0), S)
        if L == 0:
            continue
        ob, lb = prefill(q[b:b + 1, :, :L], k[b:b + 1, :, :L],
                         v[b:b + 1, :, :L], scale, causal)
        o[b, :, :L] = ob[0]
        lse[b, :, :L] = lb[0]
    return o, lse


def decode(q, kcache, vcache, seqlens, scale, Hkv):
    """Decode attention: one query row per sequence against its whole cache.

    q [B,Hq,D]; kcache, vcache: flat packed caches (sequence b is a
    [Hkv, L_b, D] block at element offset Hkv*D*sum(L[:b])); seqlens [B].
    Returns (o [B,Hq,D], lse [B,Hq]).
    """
    q = _f64(q)
    kc, vc = _f64(kcache).reshape(-1), _f64(vcache).reshape(-1)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    B, Hq, D = q.shape
    _check_heads(Hq, Hkv)
    if kc.size != Hkv * D * int(seqlens.sum()) or vc.size != kc.size:
        raise ValueError("packed caches do not match seqlens")
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    off = 0
    for b in range(B):
        L = int(seqlens[b])
        kb = kc[off: off + Hkv * L * D].reshape(Hkv, L, D)
        vb = vc[off: off + Hkv * L * D].reshape(Hkv, L, D)
        off += Hkv * L * D
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (kb[g] @ q[b, h])                 # [L]
            P, row_lse = _two_pass_softmax(s[None, :],
                                           np.ones((1, L), dtype=bool))
            lse[b, h] = row_lse[0]
            o[b, h] = (P @ vb[g])[0]
    return o, lse


def lse_combine(o_parts, lse_parts):
    """Merge attention results computed over disjoint key chunks.

    o_parts [n, ..., D]: each chunk's normalised output; lse_parts [n, ...]:
    each chunk's LSE (-inf for an empty chunk).  With M = max_s lse_s and
    w_s = exp(lse_s - M): o = sum_s w_s o_s / sum_s w_s and
    lse = M + ln(sum_s w_s).  This is the cross-chunk merge of the online
    softmax state ("Attention三算子融合实战" 2.2: the merge order does not
    matter as long as m and l are kept; 4.4: key chunks processed by separate
    blocks are merged afterwards).  All chunks empty gives o = 0, lse = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=0)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_parts - M_safe[None])
    w = np.where(np.isfinite(lse_parts), w, 0.0)
    W = w.sum(axis=0)
    W_safe = np.where(empty, 1.0, W)
    o = (w[..., None] * o_parts).sum(axis=0) / W_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, M_safe + np.log(W_safe))
    return o, lse


def prefix_softmax_state(q, k, scale, causal, b, h, row, key_counts):
    """The softmax state of one query row after its first n keys.

    This is the intermediate state that the online softmax of
    "Attention三算子融合实战" section 2.2 carries from block to block: after the
    keys 0 .. n-1 have been seen, the row max m_n of the visible scores among
    them and their log-sum-exp lse_n = m_n + ln(sum_j exp(s_j - m_n)).  Section
    6.3 of the same page compares a kernel's per-iteration m_i and l_i with
    the reference's values at the same positions; this gives those values.
    q [B,Hq,S,D], k [B,Hkv,S,D]; key_counts: iterable of n (0 <= n <= S).
    Returns (m [len], lse [len]) in float64; -inf where no key is visible.
    """
    q, k = _f64(q), _f64(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _check_heads(Hq, Hkv)
    g = _kv_head(h, Hq, Hkv)
    s = scale * (k[b, g] @ q[b, h, row])                 # the score row [S]
    vis_row = _visible(np.array([row]), S, causal)[0]
    ms, lses = [], []
    for n in key_counts:
        vis = vis_row & (np.arange(S) < n)
        _, lse = _two_pass_softmax(s[None, :], vis[None, :])
        ms.append(np.where(vis, s, -np.inf).max(initial=-np.inf))
        lses.append(lse[0])
    return np.array(ms), np.array(lses)
