"""HCA oracle: block compression and attention over compressed entries plus a raw window.

Source: ERNIE 5.5 Flash Base pages -- mirrorspeed page, section "Hybrid sparse
attention, 1/7 full context access" (128 tokens per cache entry; attention on
the compressed entries plus a recent short uncompressed window); ai-club.cn
page, section on hybrid attention MLA + HCA (dense attention over that
sequence; 512-wide heads).

Readings of what the pages leave open:

* Compressor: cache entry j of head h is the weighted sum over the 128 rows of
  block j with per-head weights w[h, :]; the same form is applied to K and V.
* Window: the W most recent positions up to and including the query
  position t, i.e. [lo(t), t] with lo(t) = max(0, t - W + 1).
* Compressed entries visible to t: the blocks that end before the window
  starts, j < n_c(t) = floor(lo(t) / block), so no block overlaps the window.
  Positions between the last visible block and the window are seen by neither.
* Softmax scale is an input (the configs use 1/sqrt(d)); no positional term.
* GQA/MQA: query head h reads KV head h // (H_q / H_kv).
"""
from __future__ import annotations

import numpy as np


def compress_kv(x: np.ndarray, w: np.ndarray, block: int) -> np.ndarray:
    """Weighted block sum: out[b, j, h, :] = sum_i w[h, i] * x[b, j*block + i, h, :].

    x: [B, S, H, d]; w: [H, block].  A trailing partial block is not compressed.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, S, H, d = x.shape
    n = S // block
    xb = x[:, : n * block].reshape(B, n, block, H, d)
    return np.einsum("bnihd,hi->bnhd", xb, w)


def window_bounds(t: int, window: int, block: int) -> tuple[int, int]:
    """(lo, n_c) for query position t: raw window [lo, t] and compressed entries [0, n_c)."""
    lo = max(0, t - window + 1)
    return lo, lo // block


def visible_positions(t: int, window: int, block: int) -> tuple[list[int], list[int]]:
    """Enumerate what position t sees: compressed block ids and raw positions."""
    lo, n_c = window_bounds(t, window, block)
    return list(range(n_c)), list(range(lo, t + 1))


def attend_row(qv: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of one query over a key set: returns (output row, natural-log LSE)."""
    logits = scale * (keys @ qv)
    m = logits.max()
    p = np.exp(logits - m)
    denom = p.sum()
    return (p @ values) / denom, m + np.log(denom)


def hca_attention(q, k, v, kc, vc, *, window: int, block: int, scale: float,
                  q_pos0: int = 0, kv_pos0: int = 0, rows=None):
    """HCA attention for queries at positions q_pos0 + i.

    q: [B, Sq, Hq, d]; k, v: raw K/V [B, Skv, Hkv, d] covering positions
    kv_pos0 .. kv_pos0 + Skv - 1; kc, vc: compressed entries [B, nb, Hkv, d].
    rows: the query indices i to compute (default all).  Returns (o, lse) with
    o [B, len(rows), Hq, dv] and lse [B, Hq, len(rows)]; lse uses natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    dv = v.shape[3]
    rows = list(range(Sq)) if rows is None else [int(r) for r in rows]
    o = np.zeros((B, len(rows), Hq, dv))
    lse = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for ri, i in enumerate(rows):
            t = q_pos0 + i
            lo, n_c = window_bounds(t, window, block)
            if n_c > kc.shape[1] or lo < kv_pos0 or t >= kv_pos0 + k.shape[1]:
                raise ValueError(f"query position {t} needs keys outside the given cache")
            for h in range(Hq):
                g = h // group
                keys = np.concatenate([np.asarray(kc[b, :n_c, g], dtype=np.float64),
                                       np.asarray(k[b, lo - kv_pos0: t - kv_pos0 + 1, g], dtype=np.float64)])
                vals = np.concatenate([np.asarray(vc[b, :n_c, g], dtype=np.float64),
                                       np.asarray(v[b, lo - kv_pos0: t - kv_pos0 + 1, g], dtype=np.float64)])
                o[b, ri, h], lse[b, h, ri] = attend_row(q[b, i, h], keys, vals, scale)
    return o, lse
