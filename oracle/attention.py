"""Plain fp64 NumPy oracle for exact attention (test infrastructure only).

Nothing here is blocked, fused or reordered beyond what the pages state: the
main entry points materialise the full score matrix exactly as the standard
algorithm in "Fast Inference and Training at Scale", section 6.21
FlashAttention, does; the two online-softmax twins follow the update
equations of "Hardware Co-Design" (normalised form) and the deferred form of
"FlashAttention scaling, multi-GPU training and weight quantization",
section 1, and exist only to be compared with the definition on small inputs.

Conventions (readings of points the pages leave open):

* Scores are ``scale * q . k`` with the caller's scale (the pages use
  1/sqrt(d_k)); the value dimension equals the key dimension.
* Causal masking is bottom-right aligned: key j is visible to query i iff
  ``j <= i + (Sk - Sq)``.  For Sq == Sk this is the usual ``j <= i``, and it
  lets the last query of a decode step see the whole cache.
* Query head ``hq`` reads K/V head ``hq // (Hq // Hkv)`` (contiguous groups).
* ``lse`` is the natural-log log-sum-exp of the visible scaled scores of a
  row.  A row with no visible key has O = 0 and lse = -inf, never NaN (the
  guard the "Common mistakes" list of "Week 13. GPUs and FlashAttention"
  asks for).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head_of",
    "sdpa",
    "sdpa_rows",
    "online_softmax_normalised",
    "online_softmax_deferred",
    "gather_pages",
    "paged_decode",
    "paged_multi_query",
    "mla_decode",
    "split_partials",
    "merge_partials",
    "sdpa_backward",
]


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head ``hq`` under grouped-query attention.

    "Fast Inference and Training at Scale", section 6.2 GQA: the h query heads
    form G groups and each group shares one key head and one value head
    (G = h is MHA, G = 1 is MQA).  Groups are taken to be contiguous.
    """
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return hq // (Hq // Hkv)


def _visible(rows: np.ndarray, Sq: int, Sk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Sk] mask of the keys each listed query row sees."""
    j = np.arange(Sk)[None, :]
    if not causal:
        return np.ones((len(rows), Sk), dtype=bool)
    return j <= (np.asarray(rows)[:, None] + (Sk - Sq))


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray, scale: float):
    """One head of standard attention in fp64, one step per line.

    "Fast Inference and Training at Scale", section 6.21: S = Q K^T / sqrt(d_k)
    is materialised, P = softmax(S) row by row, O = P V.  The row maximum is
    subtracted before exponentiating (it cancels in the ratio), and the
    log-sum-exp of each row is kept ("Week 13. GPUs and FlashAttention",
    Step 2: backward needs only O and the logsumexp of each row).

    Returns (O [R,d], lse [R], P [R,Sk]) with P the normalised probabilities.
    """
    S = scale * (q @ k.T)                      # [R, Sk] score matrix
    S = np.where(vis, S, -np.inf)              # masked pairs carry no weight
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    E = np.exp(S - m_safe[:, None])            # exp(-inf) = 0 on masked pairs
    l = E.sum(axis=1)
    O = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    P = np.zeros_like(E)
    lse = np.full(q.shape[0], -np.inf)
    if has_key.any():
        P[has_key] = E[has_key] / l[has_key, None]
        O[has_key] = P[has_key] @ v
        lse[has_key] = m_safe[has_key] + np.log(l[has_key])
    return O, lse, P


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch q={q.shape} k={k.shape} v={v.shape}")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Sq, k.shape[2], d


def sdpa(q, k, v, causal: bool, scale: float, return_probs: bool = False):
    """Exact attention ``O = softmax(scale Q K^T) V`` for every (batch, head).

    q: [B, Hq, Sq, d]; k, v: [B, Hkv, Sk, d] (any real dtype; values are taken
    exactly and computed on in fp64).  Returns ``(O [B,Hq,Sq,d], lse [B,Hq,Sq])``
    and, with ``return_probs``, the probabilities ``P [B,Hq,Sq,Sk]``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Hkv, Sq, Sk, d = _check_shapes(q, k, v)
    O = np.zeros((B, Hq, Sq, d))
    lse = np.zeros((B, Hq, Sq))
    P = np.zeros((B, Hq, Sq, Sk)) if return_probs else None
    vis = _visible(np.arange(Sq), Sq, Sk, causal)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            o, l, p = _attend(q[b, hq], k[b, kv], v[b, kv], vis, scale)
            O[b, hq], lse[b, hq] = o, l
            if return_probs:
                P[b, hq] = p
    return (O, lse, P) if return_probs else (O, lse)


def sdpa_rows(q, k, v, rows, causal: bool, scale: float):
    """The same definition as :func:`sdpa`, evaluated only for chosen query rows.

    ``rows`` is an int array [B, Hq, R] (or [R], shared by every head) of query
    indices.  Returns ``(O [B,Hq,R,d], lse [B,Hq,R])``.  Each row is the plain
    definition on that row alone, so a subset can be checked at sizes where
    the whole score matrix would not fit.
    """
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    rows = np.asarray(rows)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (B, Hq, rows.shape[0]))
    R = rows.shape[2]
    O = np.zeros((B, Hq, R, d))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            r = rows[b, hq]
            vis = _visible(r, Sq, Sk, causal)
            o, l, _ = _attend(_as64(q[b, hq, r]), _as64(k[b, kv]), _as64(v[b, kv]), vis, scale)
            O[b, hq], lse[b, hq] = o, l
    return O, lse


def _blocks(Sk: int, block: int):
    return [(j0, min(j0 + block, Sk)) for j0 in range(0, Sk, block)]


def online_softmax_normalised(q, k, v, block: int, causal: bool, scale: float):
    """One head, keys visited in blocks, with the normalised online update.

    "Hardware Co-Design" (mbrenndoerfer): per query keep the running maximum
    m_i, the running sum l_i and the partial output O_i; for a new block of
    scores s,
        m_new = max(m_old, max(s))
        l_new = e^(m_old - m_new) l_old + sum_j e^(s_j - m_new)
        O_new = (e^(m_old - m_new) l_old O_old + sum_j e^(s_j - m_new) V_j) / l_new.
    A row whose keys so far are all masked keeps m = -inf, l = 0, O = 0 (the
    -inf guard of "Week 13", "Common mistakes").

    q: [Sq, d]; k, v: [Sk, d].  Returns (O [Sq,d], lse [Sq]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Sq, Sk = q.shape[0], k.shape[0]
    m = np.full(Sq, -np.inf)
    l = np.zeros(Sq)
    O = np.zeros((Sq, v.shape[1]))
    vis_all = _visible(np.arange(Sq), Sq, Sk, causal)
    for j0, j1 in _blocks(Sk, block):
        s = np.where(vis_all[:, j0:j1], scale * (q @ k[j0:j1].T), -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)
        m_ref = np.where(live, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        e = np.exp(s - m_ref[:, None])
        l_new = alpha * l + e.sum(axis=1)
        num = (alpha * l)[:, None] * O + e @ v[j0:j1]
        O = np.where(live[:, None], num / np.where(l_new > 0, l_new, 1.0)[:, None], 0.0)
        m, l = m_new, l_new
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse


def online_softmax_deferred(q, k, v, block: int, causal: bool, scale: float):
    """One head, keys visited in blocks, rescaling the unnormalised output only.

    "Week 13. GPUs and FlashAttention", Step 2: per query block keep m, the
    running denominator and the unnormalised output; on a new maximum both
    are multiplied by e^(m_old - m_new).  "FlashAttention scaling, multi-GPU
    training and weight quantization", section 1: the division by the
    denominator is postponed to the very end of the loop.

    q: [Sq, d]; k, v: [Sk, d].  Returns (O [Sq,d], lse [Sq]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Sq, Sk = q.shape[0], k.shape[0]
    m = np.full(Sq, -np.inf)
    l = np.zeros(Sq)
    acc = np.zeros((Sq, v.shape[1]))
    vis_all = _visible(np.arange(Sq), Sq, Sk, causal)
    for j0, j1 in _blocks(Sk, block):
        s = np.where(vis_all[:, j0:j1], scale * (q @ k[j0:j1].T), -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        p = np.exp(s - m_ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    O = np.zeros_like(acc)
    nz = l > 0
    O[nz] = acc[nz] / l[nz, None]
    lse = np.full(Sq, -np.inf)
    lse[nz] = m[nz] + np.log(l[nz])
    return O, lse


def gather_pages(cache, block_table_row, seqlen: int, kv_head: int, block_size: int):
    """Logical [seqlen, d] K (or V) of one sequence and one K/V head.

    "Fast Inference and Training at Scale", section 6.3 PagedAttention: the
    cache is split into fixed-size blocks that need not be contiguous; a page
    table maps a sequence's logical block p to a physical block.  ``cache`` is
    [num_blocks, Hkv, block_size, d]; logical token t lives in physical block
    ``block_table_row[t // block_size]`` at slot ``t % block_size``.
    """
    n_pages = -(-seqlen // block_size)
    ids = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    pages = np.asarray(cache)[ids, kv_head]            # [n_pages, block_size, d]
    return pages.reshape(n_pages * block_size, pages.shape[-1])[:seqlen]


def paged_decode(q, kcache, vcache, block_table, seqlens, scale: float):
    """One new query token per sequence attending to its whole paged cache.

    "Fast Inference and Training at Scale", section 6.1 KV Caching: at a step
    only the new token's query is formed and it attends over the full cache
    (which already holds the new token's K, V).  Every cached token is
    visible; the result is :func:`sdpa` on the gathered sequence with Sq = 1.

    q: [nseq, Hq, d]; kcache, vcache: [num_blocks, Hkv, block_size, d];
    block_table: [nseq, max_blocks] int; seqlens: [nseq] int.
    Returns (o [nseq, Hq, d], lse [nseq, Hq]).
    """
    q = _as64(q)
    nseq, Hq, d = q.shape
    Hkv, bs = kcache.shape[1], kcache.shape[2]
    o = np.zeros((nseq, Hq, d))
    lse = np.full((nseq, Hq), -np.inf)
    for s in range(nseq):
        n = int(seqlens[s])
        for kv in range(Hkv):
            K = _as64(gather_pages(kcache, block_table[s], n, kv, bs))
            V = _as64(gather_pages(vcache, block_table[s], n, kv, bs))
            heads = [hq for hq in range(Hq) if kv_head_of(hq, Hq, Hkv) == kv]
            vis = np.ones((len(heads), n), dtype=bool)
            oo, ll, _ = _attend(q[s, heads], K, V, vis, scale)
            o[s, heads], lse[s, heads] = oo, ll
    return o, lse


def paged_multi_query(q, kcache, vcache, block_table, seqlens, scale: float):
    """Sq new query tokens per sequence attending to the paged cache.

    "Fast Inference and Training at Scale", section 6.5 Speculative Decoding
    (the target model verifies the draft tokens in one forward pass, all of
    their queries at once) with the cache of sections 6.1 and 6.3; "Week 13.
    GPUs and FlashAttention", Step 1 (a verify pass carries B (gamma + 1)
    tokens).  The cache already holds the Sq new tokens' K and V as the last
    Sq of the sequence's ``seqlens[s]`` tokens; new token t sits at position
    seqlens[s] - Sq + t and sees the keys up to and including its own
    position (causal, bottom-right aligned).  A token whose position is
    negative (seqlens[s] < Sq) sees no key: O = 0, lse = -inf.  This is
    :func:`sdpa` with causal masking on the gathered sequence.

    q: [nseq, Sq, Hq, d]; kcache, vcache: [num_blocks, Hkv, block_size, d];
    block_table: [nseq, max_blocks] int; seqlens: [nseq] int.
    Returns (o [nseq, Sq, Hq, d], lse [nseq, Sq, Hq]).
    """
    q = _as64(q)
    nseq, Sq, Hq, d = q.shape
    Hkv, bs = kcache.shape[1], kcache.shape[2]
    o = np.zeros((nseq, Sq, Hq, d))
    lse = np.full((nseq, Sq, Hq), -np.inf)
    for s in range(nseq):
        n = int(seqlens[s])
        if n <= 0:
            continue
        K = np.stack([_as64(gather_pages(kcache, block_table[s], n, kv, bs)) for kv in range(Hkv)])[None]
        V = np.stack([_as64(gather_pages(vcache, block_table[s], n, kv, bs)) for kv in range(Hkv)])[None]
        oo, ll = sdpa(q[s].transpose(1, 0, 2)[None], K, V, True, scale)      # [1, Hq, Sq, d]
        o[s] = oo[0].transpose(1, 0, 2)
        lse[s] = ll[0].T
    return o, lse


def mla_decode(q, w_uk, w_uv_t, ccache, block_table, seqlens, scale: float):
    """Decode over a latent cache (multi-head latent attention).

    "Fast Inference and Training at Scale", section 6.4 MLA: the cache keeps
    only the compressed latent c (d_c values per token); each time a cached
    token is attended to, its keys and values are reconstructed with learned
    up-projections, K = c W_K and V = c W_V, then attention proceeds as usual
    (one new query token per sequence, section 6.1; the paged cache of
    section 6.3).  Written out as the pages state it: per head h the full
    K_h = C W_K[h] and V_h = C W_V[h] are materialised.

    q: [nseq, H, d_h]; w_uk: [H, d_c, d_h] (W_K per head); w_uv_t: [H, d_h,
    d_c] (W_V per head, transposed); ccache: [num_blocks, block_size, d_c];
    block_table [nseq, max_blocks]; seqlens [nseq].
    Returns (o [nseq, H, d_h], lse [nseq, H]).
    """
    q = _as64(q)
    nseq, H, dh = q.shape
    wk, wv = _as64(w_uk), _as64(w_uv_t)
    bs = ccache.shape[1]
    cc = np.asarray(ccache)[:, None]                     # one latent "head"
    o = np.zeros((nseq, H, dh))
    lse = np.full((nseq, H), -np.inf)
    for s in range(nseq):
        n = int(seqlens[s])
        if n <= 0:
            continue
        C = _as64(gather_pages(cc, block_table[s], n, 0, bs))       # [n, d_c]
        for h in range(H):
            K = C @ wk[h]                                           # [n, d_h]
            V = C @ wv[h].T
            vis = np.ones((1, n), dtype=bool)
            oo, ll, _ = _attend(q[s, h][None], K, V, vis, scale)
            o[s, h], lse[s, h] = oo[0], ll[0]
    return o, lse


def split_partials(q, k, v, bounds, scale: float):
    """Attention of query rows over each key range [a, b) of ``bounds`` alone.

    q: [R, d]; k, v: [Sk, d]; bounds: list of (a, b).  Each partial is the
    plain definition restricted to its keys: ``(o_s [R,d], lse_s [R])``; an
    empty range gives o_s = 0 and lse_s = -inf.
    """
    out = []
    q, k, v = _as64(q), _as64(k), _as64(v)
    for a, b in bounds:
        vis = np.ones((q.shape[0], b - a), dtype=bool)
        o, l, _ = _attend(q, k[a:b], v[a:b], vis, scale)
        out.append((o, l))
    return out


def merge_partials(partials):
    """Combine per-range results into the result over the union of the ranges.

    This is the online-softmax update of "Hardware Co-Design" applied to whole
    ranges: with M = max_s lse_s and w_s = e^(lse_s - M),
    lse = M + ln sum_s w_s and o = sum_s w_s o_s / sum_s w_s.  Ranges with
    lse_s = -inf carry no weight; if every range is empty, o = 0, lse = -inf.
    """
    os_ = np.stack([_as64(o) for o, _ in partials])       # [n, R, d]
    ls = np.stack([_as64(l) for _, l in partials])        # [n, R]
    M = ls.max(axis=0)
    live = np.isfinite(M)
    M_safe = np.where(live, M, 0.0)
    w = np.exp(ls - M_safe[None])                         # 0 for empty ranges
    W = w.sum(axis=0)
    o = np.zeros(os_.shape[1:])
    lse = np.full(M.shape, -np.inf)
    o[live] = (np.einsum("nr,nrd->rd", w, os_)[live]) / W[live, None]
    lse[live] = M_safe[live] + np.log(W[live])
    return o, lse


def _attend_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, vis: np.ndarray, scale: float):
    """Gradients of one head of standard attention with respect to Q, K, V.

    The pages keep only O and the per-row log-sum-exp for the backward pass
    and recompute the scores and probabilities from Q, K, V ("Fast Inference
    and Training at Scale", section 6.21, Idea 2; "Week 13. GPUs and
    FlashAttention", Step 2).  What is computed is the gradient of the
    definition in ``_attend`` by the chain rule, one step per line:
    O = P V gives dV = P^T dO and dP = dO V^T; the softmax of each row gives
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik); S = scale Q K^T gives
    dQ = scale dS K and dK = scale dS^T Q.  Masked pairs have P = 0, so they
    get no gradient; a row with no visible key has a zero P row.

    Returns (dQ [R,d], dK [Sk,d], dV [Sk,d]).
    """
    _, _, P = _attend(q, k, v, vis, scale)
    dV = P.T @ do
    dP = do @ v.T
    D = (P * dP).sum(axis=1)                   # sum_k P_ik dP_ik per row
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV


def sdpa_backward(q, k, v, do, causal: bool, scale: float):
    """Gradients of ``sum(dO * O)`` for ``O = softmax(scale Q K^T) V``.

    q, do: [B, Hq, Sq, d]; k, v: [B, Hkv, Sk, d].  Returns
    ``(dq [B,Hq,Sq,d], dk [B,Hkv,Sk,d], dv [B,Hkv,Sk,d])`` in fp64.  Under
    grouped-query attention a K/V head is read by several query heads, so its
    gradients are the sums over those heads.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Hkv, Sq, Sk, d = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"do {do.shape} must have the shape of q {q.shape}")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    vis = _visible(np.arange(Sq), Sq, Sk, causal)
    for b in range(B):
        for hq in range(Hq):
            kvh = kv_head_of(hq, Hq, Hkv)
            gq, gk, gv = _attend_grad(q[b, hq], k[b, kvh], v[b, kvh], do[b, hq], vis, scale)
            dq[b, hq] = gq
            dk[b, kvh] += gk
            dv[b, kvh] += gv
    return dq, dk, dv
