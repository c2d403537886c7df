"""Attention-output epilogue oracle: the low-rank output gate and Virtual Head
Attention (VHA) cross-head mixing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ERNIE 5.5 Flash Base pages -- mirrorspeed page, section "More
structural improvements, data, and infrastructure" (the output gate is
computed from the low-rank query latent the layer already produces, a quarter
of the hidden size, so the gate projection has a quarter of the parameters;
VHA mixes the heads through a lightweight low-rank map with an identity skip
and can be folded into the attention operator); besthub page, section "Core
Architectural Innovations" (low-rank gated attention; VHA, fuseable into
kernels at near-zero overhead).

Readings of what the pages leave open:

* Gate: one gate value per output element, g[b, t, h, e] = sigmoid(<c[b, t, :],
  W_g[h*d_v + e, :]>), from the query latent c [B, S, d_c] (d_c = hidden / 4)
  and a projection W_g [H*d_v, d_c] (the [out, in] layout of a linear layer).
* VHA: z[b, t, h, :] = o[b, t, h, :] + sum_h' (U V)[h, h'] o[b, t, h', :] with
  U [H, r], V [r, H] (rank r); the identity term is the skip.
* Order: the heads are mixed first, then gated: y = g * z, the layer's
  attention output before its output projection.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gate_values(c, w_g, h: int, d_v: int):
    """g [B, S, H, d_v] = sigmoid(c W_g^T) for c [B, S, d_c], W_g [H*d_v, d_c]."""
    c = np.asarray(c, dtype=np.float64)
    w = np.asarray(w_g, dtype=np.float64)
    B, S, _ = c.shape
    return sigmoid(c @ w.T).reshape(B, S, h, d_v)


def vha_mix(o, u, v):
    """z = o + (U V) o across the head axis of o [B, S, H, d]."""
    o = np.asarray(o, dtype=np.float64)
    m = np.asarray(u, dtype=np.float64) @ np.asarray(v, dtype=np.float64)   # [H, H]
    return o + np.einsum("gh,bshd->bsgd", m, o)


def gated_vha_output(o, c, w_g, u, v):
    """y = gate(c) * vha_mix(o): the attention output after both epilogues."""
    H, d_v = o.shape[2], o.shape[3]
    return gate_values(c, w_g, H, d_v) * vha_mix(o, u, v)
