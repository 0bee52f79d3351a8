"""Naive, fully materialised fp64 attention and its analytic backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed.  The pages name the operation without writing it out: ARK's
pipeline runs "multi-head SDPA attention" with the causal mask fused into the
SDPA (ARK, pipeline list, "Accelerated forward pass"), cites Vaswani et al.
2017 for it (ARK, references), and Forge hand-writes flash attention forward
and backward following FlashAttention-2 (Forge, "What this is" and
"Acknowledgements").  Flash attention reaches exactly (up to rounding order)
the plain definition below, so the oracle is that definition, one (b, h)
head at a time, with every S x S matrix materialised:

  forward   S = scale * Q K^T ; S_ij = -inf where (i, j) is not allowed
            m_i = max_j S_ij ; E = exp(S - m) ; l_i = sum_j E_ij ; P = E / l
            O = P V ; LSE_i = m_i + ln l_i
  backward  dV = P^T dO ; dP = dO V^T ; Delta_i = sum_j P_ij dP_ij
            dS = P o (dP - Delta) ; dQ = scale * dS K ; dK = scale * dS^T Q

The softmax is the three-pass, underflow-safe form (maximum, shifted
exponential sum, normalise) that ARK's softmax kernel uses (ARK, kernel list
of asm/kern.s); LSE is the max-shifted log-sum-exp ARK uses for its loss.

Readings where the pages are silent (each is listed in the design notes):
  * mask values are -inf, so masked weights are exactly 0;
  * causal means key j <= query i, diagonal included, queries and keys the
    same sequence (no cache offset);
  * packed documents (Cort33x, "Preserving context in the data") attend
    block-diagonally: j <= i and doc(i) == doc(j);
  * LSE uses the natural logarithm;
  * Delta is the row sum of P o dP; for the exact forward this equals
    rowsum(dO o O), which the kernels use (``delta_ref``).

All arrays are float64 in [B, H, S, D] (LSE and Delta [B, H, S]).

Grouped-query attention (Forge, "Architecture": attention with GQA behind an
interface): K and V may have H_kv heads, H_kv dividing H; query head h then
reads K/V head h // (H / H_kv) (consecutive query heads share one K/V head).
The definition is plain attention with each K/V head repeated for its query
heads; dK and dV of a K/V head are the sums of the gradients of its copies.
"""
from __future__ import annotations

import numpy as np

MASK_CAUSAL = 0
MASK_DOC_CAUSAL = 1


def _doc_ids(S, cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != S or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, never decrease and end at S")
    # row s belongs to the last document starting at or before it (an empty
    # document starts where the next one does and owns no row)
    return np.searchsorted(cu, np.arange(S), side="right") - 1


def allowed_mask(S, mask_mode=MASK_CAUSAL, cu_seqlens=None):
    """Boolean [S, S] matrix: entry (i, j) is True when query i may attend key j.

    Causal: j <= i.  Packed documents: j <= i and both in the same document.
    """
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    allowed = j <= i
    if mask_mode == MASK_DOC_CAUSAL:
        if cu_seqlens is None:
            raise ValueError("packed-document mask needs cu_seqlens")
        doc = _doc_ids(S, cu_seqlens)
        allowed = allowed & (doc[:, None] == doc[None, :])
    elif mask_mode != MASK_CAUSAL:
        raise ValueError(f"unknown mask mode {mask_mode}")
    return allowed


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _head_forward(q, k, v, scale, allowed):
    """Forward for one head: q, k, v are [S, D]. Returns (P, O, LSE)."""
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)                       # pass 1: row maximum
    e = np.exp(s - m[:, None])              # pass 2: shifted exponentials ...
    l = e.sum(axis=1)                       #         ... and their sum
    p = e / l[:, None]                      # pass 3: normalise
    o = p @ v
    lse = m + np.log(l)
    return p, o, lse


def _heads(B, H, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return list(heads)


def _group(q, k, v):
    """Query heads per K/V head (1 for plain multi-head attention)."""
    H, H_kv = q.shape[1], k.shape[1]
    if H_kv < 1 or H % H_kv != 0 or v.shape[1] != H_kv:
        raise ValueError("K/V heads must divide the query heads")
    return H // H_kv


def attention_fwd_ref(q, k, v, scale, mask_mode=MASK_CAUSAL, cu_seqlens=None, heads=None):
    """Forward attention.  Returns (O [B,H,S,D], LSE [B,H,S]) in float64.

    ``heads``: optional list of (b, h) to compute; other heads are left NaN.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, S, D = q.shape
    G = _group(q, k, v)
    allowed = allowed_mask(S, mask_mode, cu_seqlens)
    o = np.full((B, H, S, D), np.nan)
    lse = np.full((B, H, S), np.nan)
    for b, h in _heads(B, H, heads):
        _, o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, allowed)
    return o, lse


def attention_bwd_ref(q, k, v, do, scale, mask_mode=MASK_CAUSAL, cu_seqlens=None, heads=None):
    """Forward and analytic backward.  Returns a dict of float64 arrays:
    ``o, lse, dq, dk, dv, delta`` (``delta`` = rowsum(P o dP)).

    ``heads``: optional list of (b, h) to compute; other heads are left NaN
    (plain multi-head attention only: with grouped heads dK and dV need every
    query head of a group).  dk and dv have K's shape.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, S, D = q.shape
    G = _group(q, k, v)
    if G > 1 and heads is not None:
        raise ValueError("head selection needs plain multi-head attention")
    allowed = allowed_mask(S, mask_mode, cu_seqlens)
    out = {name: np.full((B, H, S, D), np.nan) for name in ("o", "dq")}
    for name in ("dk", "dv"):
        out[name] = np.full(k.shape, np.nan) if G == 1 else np.zeros(k.shape)
    out["lse"] = np.full((B, H, S), np.nan)
    out["delta"] = np.full((B, H, S), np.nan)
    for b, h in _heads(B, H, heads):
        qh, kh, vh, doh = q[b, h], k[b, h // G], v[b, h // G], do[b, h]
        p, o, lse = _head_forward(qh, kh, vh, scale, allowed)
        dv = p.T @ doh
        dp = doh @ vh.T
        delta = (p * dp).sum(axis=1)
        ds = p * (dp - delta[:, None])
        out["o"][b, h] = o
        out["lse"][b, h] = lse
        out["dq"][b, h] = scale * (ds @ kh)
        if G == 1:
            out["dv"][b, h] = dv
            out["dk"][b, h] = scale * (ds.T @ qh)
        else:  # this head's share of its K/V head's gradient
            out["dv"][b, h // G] += dv
            out["dk"][b, h // G] += scale * (ds.T @ qh)
        out["delta"][b, h] = delta
    return out


def delta_ref(do, o):
    """Delta_i = sum_d dO_id * O_id (the backward preprocess), float64 [B,H,S]."""
    return np.sum(_as64(do) * _as64(o), axis=-1)


def _row_probs(qh, kh, scale, allowed_row_mask, i):
    s = scale * (kh @ qh[i])
    s = np.where(allowed_row_mask, s, -np.inf)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return e / l, m + np.log(l)


def attention_fwd_rows_ref(q, k, v, scale, b, h, rows, mask_mode=MASK_CAUSAL, cu_seqlens=None):
    """O and LSE of selected query rows of head (b, h), one row at a time.

    Each row needs only its own scores, so this checks any sequence length
    in O(S * D) per row.  Returns (O [len(rows), D], LSE [len(rows)]).
    """
    qh, kh, vh = _as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h])
    S = qh.shape[0]
    doc = _doc_ids(S, cu_seqlens) if mask_mode == MASK_DOC_CAUSAL else None
    o_rows, lse_rows = [], []
    j = np.arange(S)
    for i in rows:
        allowed = j <= i
        if doc is not None:
            allowed = allowed & (doc == doc[i])
        p, lse = _row_probs(qh, kh, scale, allowed, i)
        o_rows.append(p @ vh)
        lse_rows.append(lse)
    return np.array(o_rows), np.array(lse_rows)


def attention_dq_rows_ref(q, k, v, do, scale, b, h, rows, mask_mode=MASK_CAUSAL, cu_seqlens=None):
    """dQ of selected query rows of head (b, h), one row at a time.

    Row i of dQ needs only row i of P and of dP:
      dQ_i = scale * sum_j P_ij (dP_ij - Delta_i) K_j,  dP_ij = dO_i . V_j,
      Delta_i = sum_j P_ij dP_ij.
    Returns [len(rows), D].
    """
    qh, kh, vh, doh = _as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), _as64(do[b, h])
    S = qh.shape[0]
    doc = _doc_ids(S, cu_seqlens) if mask_mode == MASK_DOC_CAUSAL else None
    j = np.arange(S)
    out = []
    for i in rows:
        allowed = j <= i
        if doc is not None:
            allowed = allowed & (doc == doc[i])
        p, _ = _row_probs(qh, kh, scale, allowed, i)
        dp = vh @ doh[i]
        delta = np.sum(p * dp)
        ds = p * (dp - delta)
        out.append(scale * (ds @ kh))
    return np.array(out)


def attention_dkdv_rows_ref(q, k, v, do, scale, b, h, cols, mask_mode=MASK_CAUSAL, cu_seqlens=None):
    """dK and dV of selected key rows of head (b, h).

    Key row j collects from every query i that attends it, so each query's
    softmax statistics (its LSE) and Delta are needed; they are computed row
    by row, then
      dV_j = sum_i P_ij dO_i,  dK_j = scale * sum_i P_ij (dP_ij - Delta_i) Q_i.
    Returns (dK [len(cols), D], dV [len(cols), D]).
    """
    qh, kh, vh, doh = _as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), _as64(do[b, h])
    S = qh.shape[0]
    doc = _doc_ids(S, cu_seqlens) if mask_mode == MASK_DOC_CAUSAL else None
    jj = np.arange(S)
    cols = list(cols)
    dk = np.zeros((len(cols), qh.shape[1]))
    dv = np.zeros((len(cols), qh.shape[1]))
    if not cols:
        return dk, dv
    # Only queries at or after the first requested key, in one of its
    # documents, give these keys a nonzero weight; every other row adds zero.
    rows = np.arange(min(cols), S)
    if doc is not None:
        rows = rows[np.isin(doc[rows], doc[cols])]
    for i in rows:
        allowed = jj <= i
        if doc is not None:
            allowed = allowed & (doc == doc[i])
        p, _ = _row_probs(qh, kh, scale, allowed, i)
        dp = vh @ doh[i]
        delta = np.sum(p * dp)
        for c, j in enumerate(cols):
            if p[j] != 0.0:
                dv[c] += p[j] * doh[i]
                dk[c] += scale * p[j] * (dp[j] - delta) * qh[i]
    return dk, dv


def attention_decode_ref(q, k_cache, v_cache, cache_lens, scale):
    """Decode step with a key/value cache: one new query per (batch entry b, head h)
    attending keys 0 .. cache_lens[b] - 1 of its K/V head (the query is the newest
    token, its own key already in the cache, so causality admits every cached key).

    q: [B, H, D]; k_cache, v_cache: [B, H_kv, S_max, D] (H_kv divides H; query head
    h reads K/V head h // (H / H_kv)); cache_lens: B integers in 1 .. S_max.
    Returns (O [B, H, D], LSE [B, H]) in float64: the plain softmax over the
    cached keys' scaled scores, its weighted sum of values, and its natural-log
    normaliser.
    """
    q, k_cache, v_cache = _as64(q), _as64(k_cache), _as64(v_cache)
    B, H, D = q.shape
    H_kv = k_cache.shape[1]
    if H % H_kv != 0:
        raise ValueError("K/V heads must divide the query heads")
    G = H // H_kv
    o = np.zeros((B, H, D))
    lse = np.zeros((B, H))
    for b in range(B):
        n = int(cache_lens[b])
        if not 1 <= n <= k_cache.shape[2]:
            raise ValueError("cache length out of range")
        for h in range(H):
            kh, vh = k_cache[b, h // G, :n], v_cache[b, h // G, :n]
            s = scale * (kh @ q[b, h])
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o[b, h] = (e / l) @ vh
            lse[b, h] = m + np.log(l)
    return o, lse
