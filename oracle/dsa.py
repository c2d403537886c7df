"""DSA oracle: lightweight indexer, causal top-k selection, sparse attention.

Source: ERNIE 5.5 Flash Base pages -- mirrorspeed page, section "Hybrid sparse
attention, 1/7 full context access" (an indexer scores historical positions
per query; core attention only on the top-k highest-scoring positions);
ai-club.cn page, section on hybrid attention MLA + HCA (256-wide heads in the
full-context layers).

Readings of what the pages leave open:

* Indexer: s(t, u) = sum_h w[t, h] * max(0, <qI[t, h], kI[u]>) over a few
  small dot-product heads, for u <= t (causal); one index key per position
  shared by the index heads; no scale (a positive scale keeps the order).
* Selection: if t + 1 <= k every u <= t is selected.  Otherwise the k
  positions with the largest score, ties broken by the smaller position.  The
  ranking decision is taken in float32 (the kernel's precision): the exact
  float64 score is rounded to float32 and -0 is canonicalised to +0 before
  ranking.  The order inside a row's index list is unspecified; this oracle
  returns it ascending and pads with -1.
* Attention: softmax(scale * <q[t, h], k[u]>) over the selected u, times v[u];
  query head h reads KV head h // (H_q / H_kv) (the DSA workload has one
  shared K/V head, MQA).
"""
from __future__ import annotations

import numpy as np

_U32 = 2.0 ** -24  # unit roundoff of float32


def index_scores_row(qI_t: np.ndarray, kI: np.ndarray, w_t: np.ndarray, t: int) -> np.ndarray:
    """Indexer scores of query t against positions 0..t (float64)."""
    dots = np.asarray(kI[: t + 1], dtype=np.float64) @ np.asarray(qI_t, dtype=np.float64).T  # [t+1, hi]
    return np.maximum(dots, 0.0) @ np.asarray(w_t, dtype=np.float64)


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k best scores (float32 ranking, smaller position wins ties), ascending."""
    n = scores.shape[0]
    if n <= k:
        return np.arange(n)
    s32 = scores.astype(np.float32)
    s32[s32 == 0] = np.float32(0.0)  # -0 -> +0
    order = np.lexsort((np.arange(n), -s32.astype(np.float64)))
    return np.sort(order[:k])


def index_topk(qI, kI, w, k: int, rows=None) -> np.ndarray:
    """idx [B, len(rows), k] int32: selected positions ascending, then -1 padding."""
    B, S = kI.shape[0], kI.shape[1]
    rows = list(range(S)) if rows is None else [int(r) for r in rows]
    out = np.full((B, len(rows), k), -1, dtype=np.int32)
    for b in range(B):
        for ri, t in enumerate(rows):
            sel = topk_row(index_scores_row(qI[b, t], kI[b], w[b, t], t), k)
            out[b, ri, : sel.shape[0]] = sel
    return out


def sparse_attention(q, k, v, idx, scale: float, rows=None):
    """o [B, len(rows), Hq, dv], lse [B, Hq, len(rows)] over the positions listed in idx (-1 skipped).

    Query head h reads KV head h // (Hq / Hkv) (one shared head, MQA, in the
    DSA workload; grouped heads otherwise)."""
    B, S, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv or v.shape[2] != Hkv:
        raise ValueError("query heads must be a multiple of the KV heads")
    group = Hq // Hkv
    dv = v.shape[3]
    rows = list(range(S)) if rows is None else [int(r) for r in rows]
    o = np.zeros((B, len(rows), Hq, dv))
    lse = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for ri, t in enumerate(rows):
            sel = np.asarray(idx[b, ri] if idx.shape[1] == len(rows) else idx[b, t])
            sel = sel[sel >= 0]
            qt = np.asarray(q[b, t], dtype=np.float64)              # [Hq, d]
            for g in range(Hkv):
                hs = slice(g * group, (g + 1) * group)
                keys = np.asarray(k[b, sel, g], dtype=np.float64)
                vals = np.asarray(v[b, sel, g], dtype=np.float64)
                logits = scale * (qt[hs] @ keys.T)                  # [group, n]
                m = logits.max(axis=1, keepdims=True)
                p = np.exp(logits - m)
                den = p.sum(axis=1, keepdims=True)
                o[b, ri, hs] = (p @ vals) / den
                lse[b, hs, ri] = (m + np.log(den))[:, 0]
    return o, lse


def sparse_attention_bwd(q, k, v, idx, scale: float, dout):
    """Gradients of sparse_attention's output (all rows) given dout = dL/do:
    (dq, dk, dv) shaped like q, k, v.  The chain rule through the softmax over
    each query's selected positions (the pages give the forward only): with
    p = softmax(scale q K_sel^T), ds = p (dout V_sel^T - <dout, o>),
    dq = scale ds K_sel, dk_sel += scale ds^T q, dv_sel += p^T dout; a position
    listed by several queries sums their contributions.  Query head h reads KV
    head h // (Hq / Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, _ = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for t in range(S):
            sel = np.asarray(idx[b, t])
            sel = sel[sel >= 0]
            for g in range(Hkv):
                keys = np.asarray(k[b, sel, g], dtype=np.float64)
                vals = np.asarray(v[b, sel, g], dtype=np.float64)
                hs = slice(g * group, (g + 1) * group)
                logits = scale * (q[b, t, hs] @ keys.T)               # [group, n]
                p = np.exp(logits - logits.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                o = p @ vals
                dp = dout[b, t, hs] @ vals.T
                ds = p * (dp - np.sum(dout[b, t, hs] * o, axis=1, keepdims=True))
                dq[b, t, hs] = scale * (ds @ keys)
                np.add.at(dk[b, :, g], sel, scale * (ds.T @ q[b, t, hs]))
                np.add.at(dv[b, :, g], sel, p.T @ dout[b, t, hs])
    return dq, dk, dv


def score_error_bounds(qI_t, kI, w_t, t: int, margin: float = 2.0):
    """Exact scores s, a bound r on |s_fp32 - s| for any float32 evaluation order, and which
    positions are exact zeros in every float32 evaluation (all index-head dots certainly < 0).

    Bound: one float32 dot over d_i terms errs by at most d_i*u*sum|terms|; the
    weighted sum over h_i heads adds (h_i + 1)*u of its magnitude, and the
    float32 rounding of the result one more u.  ``margin`` widens the bound.
    """
    qI_t = np.asarray(qI_t, dtype=np.float64)
    K = np.asarray(kI[: t + 1], dtype=np.float64)
    w_t = np.asarray(w_t, dtype=np.float64)
    hi, di = qI_t.shape
    dots = K @ qI_t.T                                  # [n, hi]
    absdots = np.abs(K) @ np.abs(qI_t).T               # sum_i |qI * kI|
    gamma = margin * (di + hi + 2) * _U32
    s = np.maximum(dots, 0.0) @ w_t
    r = gamma * (absdots @ np.abs(w_t))
    certain_neg = dots < -(margin * di * _U32) * absdots
    zero = certain_neg.all(axis=1)
    return s, r, zero


def tie_free_row(qI_t, kI, w_t, t: int, k: int) -> bool:
    """True when every float32 evaluation of row t's scores yields the same top-k set."""
    if t + 1 <= k:
        return True
    s, r, zero = score_error_bounds(qI_t, kI, w_t, t)
    sel = np.zeros(t + 1, dtype=bool)
    sel[topk_row(s, k)] = True
    a = sel & ~zero
    bn = ~sel & ~zero
    lo_sel = (s - r)[a].min() if a.any() else np.inf
    hi_uns = (s + r)[bn].max() if bn.any() else -np.inf
    if not lo_sel > hi_uns:
        return False
    if (sel & zero).any() and not hi_uns < 0.0:
        return False
    if (~sel & zero).any() and not lo_sel > 0.0:
        return False
    return True


def tie_free_rows(qI, kI, w, k: int, rows=None, batch: int = 0) -> np.ndarray:
    S = kI.shape[1]
    rows = range(S) if rows is None else rows
    return np.array([tie_free_row(qI[batch, t], kI[batch], w[batch, t], int(t), k) for t in rows], dtype=bool)


def valid_topk_row(got, qI_t, kI, w_t, t: int, k: int) -> bool:
    """Whether an index list is a correct top-k of row t for SOME float32 evaluation order.

    The list must hold min(t+1, k) distinct positions <= t (then -1 padding);
    no unselected position may be certainly better than a selected one; exact
    zeros compare by position.
    """
    got = np.asarray(got)
    n_valid = min(t + 1, k)
    if (got[n_valid:] != -1).any():
        return False
    g = got[:n_valid]
    if (g < 0).any() or (g > t).any() or np.unique(g).shape[0] != n_valid:
        return False
    if t + 1 <= k:
        return True
    s, r, zero = score_error_bounds(qI_t, kI, w_t, t)
    sel = np.zeros(t + 1, dtype=bool)
    sel[g] = True
    # non-zero selected vs anything unselected
    lo = np.where(zero, 0.0, s - r)
    hi = np.where(zero, 0.0, s + r)
    if sel.all():
        return True
    worst_sel = lo[sel].min()
    best_uns = hi[~sel].max()
    if worst_sel > best_uns:
        return True
    # pairwise check only where intervals overlap
    sel_idx = np.nonzero(sel)[0]
    uns_idx = np.nonzero(~sel)[0]
    cand_u = uns_idx[hi[uns_idx] >= worst_sel]
    cand_s = sel_idx[lo[sel_idx] <= best_uns]
    for u in cand_u:
        for v_ in cand_s:
            if zero[u] and zero[v_]:
                if u < v_:
                    return False
            elif lo[u] > hi[v_]:
                return False
    return True
