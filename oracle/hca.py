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


# ---------------------------------------------------------------- gradients
#
# The pages describe the forward only; the gradients below are the chain rule
# through the definitions above (softmax attention, weighted block sum).  They
# are pinned against central finite differences of those definitions.

def attend_row_bwd(qv: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float, dout: np.ndarray):
    """Gradients of attend_row's output row, given the gradient dout of that row,
    with respect to the query, every key and every value: (dq, dkeys, dvalues).

    p = softmax(scale * keys q); o = p values.  d/dp_x = <dout, v_x>; through the
    softmax ds_x = p_x (d/dp_x - <dout, o>); then dq = scale sum_x ds_x k_x,
    dk_x = scale ds_x q, dv_x = p_x dout.
    """
    logits = scale * (keys @ qv)
    p = np.exp(logits - logits.max())
    p /= p.sum()
    dp = values @ dout
    ds = p * (dp - dp @ p)
    return scale * (ds @ keys), scale * np.outer(ds, qv), np.outer(p, dout)


def hca_attention_bwd(q, k, v, kc, vc, dout, *, window: int, block: int, scale: float,
                      q_pos0: int = 0, kv_pos0: int = 0):
    """Gradients of hca_attention's output o (all rows) given dout = dL/do.

    Returns (dq, dk, dv, dkc, dvc) shaped like q, k, v, kc, vc: the raw keys and
    values receive the gradient of the window positions that see them, the
    compressed entries that of the queries whose blocks they are.
    """
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dkc = np.zeros(kc.shape)
    dvc = np.zeros(vc.shape)
    for b in range(B):
        for i in range(Sq):
            t = q_pos0 + i
            lo, n_c = window_bounds(t, window, block)
            r0, r1 = lo - kv_pos0, t - kv_pos0 + 1
            for h in range(Hq):
                g = h // group
                keys = np.concatenate([np.asarray(kc[b, :n_c, g], dtype=np.float64),
                                       np.asarray(k[b, r0:r1, g], dtype=np.float64)])
                vals = np.concatenate([np.asarray(vc[b, :n_c, g], dtype=np.float64),
                                       np.asarray(v[b, r0:r1, g], dtype=np.float64)])
                gq, gk, gv = attend_row_bwd(q[b, i, h], keys, vals, scale, dout[b, i, h])
                dq[b, i, h] = gq
                dkc[b, :n_c, g] += gk[:n_c]
                dvc[b, :n_c, g] += gv[:n_c]
                dk[b, r0:r1, g] += gk[n_c:]
                dv[b, r0:r1, g] += gv[n_c:]
    return dq, dk, dv, dkc, dvc


def compress_kv_bwd(x: np.ndarray, w: np.ndarray, dout: np.ndarray, block: int):
    """Gradients of compress_kv given dout = dL/d(out) [B, S // block, H, d]:
    dx[b, j*block + i, h] = w[h, i] dout[b, j, h] (zero past the last whole
    block) and dw[h, i] = sum_{b, j} <dout[b, j, h], x[b, j*block + i, h]>."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, H, d = x.shape
    n = S // block
    dx = np.zeros(x.shape)
    dx[:, : n * block] = np.einsum("hi,bnhd->bnihd", w, dout).reshape(B, n * block, H, d)
    xb = x[:, : n * block].reshape(B, n, block, H, d)
    dw = np.einsum("bnihd,bnhd->hi", xb, dout)
    return dx, dw
