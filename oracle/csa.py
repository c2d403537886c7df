"""CSA oracle: compressed sparse attention -- the history compressed by a
factor of 4, then a top-k selection over the compressed entries.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ERNIE 5.5 Flash Base pages -- mirrorspeed page, section "Hybrid sparse
attention, 1/7 full context access" (the common CSA + HCA design compresses
the history 4x and then selects sparsely; the model puts its budget in MLA
layers instead); besthub page, section "Core Architectural Innovations -- 1.
Hybrid Sparse Attention" (HCA + MLA against CSA + HCA under an equal KV-cache
budget).

Readings of what the pages leave open (the plainest ones that reuse the
compressor and the DSA indexer as defined in ``hca.py`` and ``dsa.py``):

* Compression: the K rows, the V rows and the indexer keys of every ``block``
  (4) consecutive positions become one entry, by the per-head weighted sum of
  ``compress_kv``.
* Visibility: entry j (positions block*j .. block*j + block - 1) belongs to
  the history of position t once its block is complete, i.e.
  block*j + block - 1 <= t, so t sees entries j < (t + 1) // block.
* Indexer and selection: the DSA indexer over the visible entries' compressed
  index keys, s(t, j) = sum_h w[t, h] * max(0, <qI[t, h], kIc[j]>), and the
  DSA ranking (float32 decision, the smaller entry index wins a tie).
* Attention: softmax over the selected entries' compressed keys, times their
  compressed values (query head h reads KV head h // (H_q / H_kv); the
  workload has one shared K/V head as in DSA).  A position with no
  complete block yet (t < block - 1) selects nothing: o = 0, lse = -inf.
"""
from __future__ import annotations

import numpy as np

from .dsa import index_scores_row, topk_row, tie_free_row
from .hca import compress_kv


def visible_entries(t: int, block: int) -> int:
    """Number of compressed entries in the history of position t: (t + 1) // block."""
    return (t + 1) // block


def csa_index_topk(qI, kIc, w, k: int, block: int, rows=None) -> np.ndarray:
    """idx [B, len(rows), k] int32: the selected entries of each query (ascending), then -1.

    qI [B, S, h_i, d_i], w [B, S, h_i] per position; kIc [B, n_entries, d_i] per entry."""
    B, S = qI.shape[0], qI.shape[1]
    rows = list(range(S)) if rows is None else [int(r) for r in rows]
    out = np.full((B, len(rows), k), -1, dtype=np.int32)
    for b in range(B):
        for ri, t in enumerate(rows):
            n = visible_entries(t, block)
            if n == 0:
                continue
            sel = topk_row(index_scores_row(qI[b, t], kIc[b], w[b, t], n - 1), k)
            out[b, ri, : sel.shape[0]] = sel
    return out


def csa_attention(q, kc, vc, idx, scale: float):
    """o [B, S, Hq, dv], lse [B, Hq, S]: attention of each query over the entries listed in its
    row of idx (-1 skipped); a row listing none gives o = 0, lse = -inf.  Query head h reads
    KV head h // (Hq / Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, _ = q.shape
    Hkv = kc.shape[2]
    if Hq % Hkv or vc.shape[2] != Hkv:
        raise ValueError("query heads must be a multiple of the KV heads")
    group = Hq // Hkv
    dv = vc.shape[3]
    o = np.zeros((B, S, Hq, dv))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        for t in range(S):
            sel = np.asarray(idx[b, t])
            sel = sel[sel >= 0]
            if sel.size == 0:
                continue
            for g in range(Hkv):
                hs = slice(g * group, (g + 1) * group)
                keys = np.asarray(kc[b, sel, g], dtype=np.float64)
                vals = np.asarray(vc[b, sel, g], dtype=np.float64)
                logits = scale * (q[b, t, hs] @ keys.T)            # [group, n]
                m = logits.max(axis=1, keepdims=True)
                p = np.exp(logits - m)
                den = p.sum(axis=1, keepdims=True)
                o[b, t, hs] = (p @ vals) / den
                lse[b, hs, t] = (m + np.log(den))[:, 0]
    return o, lse


def csa_forward(q, k, v, qI, kI, w, w_kv, w_i, *, topk: int, block: int, scale: float):
    """The whole CSA step: compress K, V (weights w_kv [1, block]) and the index keys (w_i
    [1, block]) by ``block``, select top-k entries per query, attend.  Returns
    (kc, vc, kIc, idx, o, lse)."""
    kc = compress_kv(np.asarray(k, dtype=np.float64), w_kv, block)
    vc = compress_kv(np.asarray(v, dtype=np.float64), w_kv, block)
    kIc = compress_kv(np.asarray(kI, dtype=np.float64)[:, :, None, :], w_i, block)[:, :, 0, :]
    idx = csa_index_topk(qI, kIc, w, topk, block)
    o, lse = csa_attention(q, kc, vc, idx, scale)
    return kc, vc, kIc, idx, o, lse


def csa_tie_free_row(qI_t, kIc, w_t, t: int, k: int, block: int) -> bool:
    """True when every float32 evaluation of query t's entry scores yields the same top-k set."""
    n = visible_entries(t, block)
    return True if n == 0 else tie_free_row(qI_t, kIc, w_t, n - 1, k)
