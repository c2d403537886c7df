"""Seeded draws for every workload.

Draw order per workload (all from ``numpy.random.default_rng(seed)``, float32
standard normals, scaled by the config's std in float32, then rounded to
bfloat16 with round-to-nearest-even when the workload is bf16):

* HCA prefill: Q, K, V, then z [h_kv, block]; compressor weights are
  softmax(z) per head, computed in float64 and rounded to float32.  The same
  weights serve K and V.
* HCA decode: q, kc, vc, kw, vw (cache contents are drawn directly).
* DSA: Q, K, V (bf16), then qI, kI, w (float32, never rounded).  A row t of qI
  and w can be redrawn from the sub-stream (seed, b, t, attempt) so that a
  caller can replace rows whose top-k boundary is too close to call.

* CSA: Q, K, V (bf16), then qI, kI, w (float32) as DSA, then z_kv and z_i
  [1, block]; the compressor weights of K/V and of the index keys are
  softmax(z) as for HCA.  Rows of qI and w are redrawn as for DSA.
* Free-standing tensors (gradients flowing into a backward call, inputs of
  other shapes): ``make_normal(shape, seed, std, bf16)``, one generator per
  call.
* Index lists for sparse attention: ``make_index_lists`` draws, per row t, a
  random set of distinct positions <= t (a random permutation's prefix),
  optionally repeats some entries of the row, and pads with -1.

Large arrays are drawn in chunks; a Generator's normal stream does not depend
on how the draw is split, so chunking does not change any value.
"""
from __future__ import annotations

import numpy as np

from .configs import HcaPrefillConfig, HcaDecodeConfig, DsaConfig, CsaConfig

_CHUNK = 1 << 24


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, as_bf16: bool) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if as_bf16 else np.float32)
    s = np.float32(std)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        x = rng.standard_normal(m, dtype=np.float32)
        if s != np.float32(1.0):
            x *= s
        out[i:i + m] = bf16_round_bits(x) if as_bf16 else x
    return out.reshape(shape)


def _softmax_weights(z: np.ndarray) -> np.ndarray:
    z64 = z.astype(np.float64)
    e = np.exp(z64 - z64.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make_prefill(cfg: HcaPrefillConfig) -> dict:
    """Q [B,S,Hq,d], K/V [B,S,Hkv,d] and compressor weights w [Hkv, block].

    bf16 tensors are returned as uint16 bit patterns, f32 tensors as float32.
    """
    rng = np.random.default_rng(cfg.seed)
    bf = cfg.dtype == "bf16"
    q = _normal(rng, (cfg.batch, cfg.seqlen, cfg.h_q, cfg.head_dim), cfg.std, bf)
    k = _normal(rng, (cfg.batch, cfg.seqlen, cfg.h_kv, cfg.head_dim), cfg.std, bf)
    v = _normal(rng, (cfg.batch, cfg.seqlen, cfg.h_kv, cfg.head_dim), cfg.std, bf)
    z = rng.standard_normal((cfg.h_kv, cfg.block), dtype=np.float32)
    return {"cfg": cfg, "q": q, "k": k, "v": v, "w": _softmax_weights(z), "bf16": bf}


def make_decode(cfg: HcaDecodeConfig) -> dict:
    """q [B,1,Hq,d]; compressed cache kc/vc [B,n_blocks,Hkv,d]; raw window kw/vw [B,W,Hkv,d] (bf16 bits)."""
    rng = np.random.default_rng(cfg.seed)
    d = cfg.head_dim
    q = _normal(rng, (cfg.batch, 1, cfg.h_q, d), cfg.std, True)
    kc = _normal(rng, (cfg.batch, cfg.n_blocks, cfg.h_kv, d), cfg.std, True)
    vc = _normal(rng, (cfg.batch, cfg.n_blocks, cfg.h_kv, d), cfg.std, True)
    kw = _normal(rng, (cfg.batch, cfg.window, cfg.h_kv, d), cfg.std, True)
    vw = _normal(rng, (cfg.batch, cfg.window, cfg.h_kv, d), cfg.std, True)
    return {"cfg": cfg, "q": q, "kc": kc, "vc": vc, "kw": kw, "vw": vw}


def make_dsa(cfg: DsaConfig) -> dict:
    """q [B,S,Hq,dqk], k [B,S,1,dqk], v [B,S,1,dv] (bf16 bits); qI [B,S,hi,di], kI [B,S,di], w [B,S,hi] (float32)."""
    rng = np.random.default_rng(cfg.seed)
    B, S = cfg.batch, cfg.seqlen
    q = _normal(rng, (B, S, cfg.h_q, cfg.d_qk), 1.0, True)
    k = _normal(rng, (B, S, 1, cfg.d_qk), 1.0, True)
    v = _normal(rng, (B, S, 1, cfg.d_v), 1.0, True)
    qI = _normal(rng, (B, S, cfg.h_i, cfg.d_i), 1.0, False)
    kI = _normal(rng, (B, S, cfg.d_i), 1.0, False)
    w = _normal(rng, (B, S, cfg.h_i), 1.0, False)
    return {"cfg": cfg, "q": q, "k": k, "v": v, "qI": qI, "kI": kI, "w": w,
            "redraws": np.zeros((B, S), dtype=np.int32)}


def redraw_dsa_rows(inp: dict, rows, attempt: int) -> None:
    """Replace qI[b,t] and w[b,t] for each (b, t) in ``rows`` from sub-stream (seed, b, t, attempt)."""
    cfg: DsaConfig = inp["cfg"]
    for b, t in rows:
        r = np.random.default_rng([cfg.seed, int(b), int(t), int(attempt)])
        inp["qI"][b, t] = r.standard_normal((cfg.h_i, cfg.d_i), dtype=np.float32)
        inp["w"][b, t] = r.standard_normal(cfg.h_i, dtype=np.float32)
        inp["redraws"][b, t] = attempt


def make_normal(shape, seed: int, std: float = 1.0, bf16: bool = False) -> np.ndarray:
    """N(0, std^2) float32 draws of the given shape (bf16 bit patterns when bf16)."""
    return _normal(np.random.default_rng(seed), tuple(shape), std, bf16)


def make_index_lists(batch: int, seqlen: int, topk: int, seed: int, n_valid=None, dup_per_row: int = 0
                     ) -> np.ndarray:
    """int32 [batch, seqlen, topk]: row t lists min(t + 1, n_valid(t), topk) distinct positions in [0, t]
    in random order (n_valid: an int, or None for topk), then, when dup_per_row > 0, that many of its
    entries are overwritten with copies of other entries of the same row (rows with at least two
    entries), and the rest of the row is -1."""
    rng = np.random.default_rng(seed)
    out = np.full((batch, seqlen, topk), -1, dtype=np.int32)
    cap = topk if n_valid is None else min(int(n_valid), topk)
    for b in range(batch):
        for t in range(seqlen):
            n = min(t + 1, cap)
            row = rng.permutation(t + 1)[:n].astype(np.int32)
            if dup_per_row and n >= 2:
                for _ in range(dup_per_row):
                    src, dst = rng.choice(n, 2, replace=False)
                    row[dst] = row[src]
            out[b, t, :n] = row
    return out


def make_index_lists_long(batch: int, seqlen: int, topk: int, seed: int) -> np.ndarray:
    """int32 [batch, seqlen, topk]: row t lists min(t + 1, topk) distinct positions in [0, t] in random
    order, then -1 -- make_index_lists without padding or duplicates, drawing each long row without
    replacement instead of permuting its whole prefix (fast enough for 65536-position sequences)."""
    rng = np.random.default_rng(seed)
    out = np.full((batch, seqlen, topk), -1, dtype=np.int32)
    for b in range(batch):
        for t in range(seqlen):
            if t + 1 <= topk:
                out[b, t, : t + 1] = rng.permutation(t + 1)
            else:
                out[b, t] = rng.choice(t + 1, size=topk, replace=False)
    return out


def make_csa(cfg: CsaConfig) -> dict:
    """make_dsa's tensors for the CSA shapes plus compressor weights w_kv, w_i [1, block] (float32)."""
    rng = np.random.default_rng(cfg.seed)
    B, S = cfg.batch, cfg.seqlen
    q = _normal(rng, (B, S, cfg.h_q, cfg.d_qk), 1.0, True)
    k = _normal(rng, (B, S, 1, cfg.d_qk), 1.0, True)
    v = _normal(rng, (B, S, 1, cfg.d_v), 1.0, True)
    qI = _normal(rng, (B, S, cfg.h_i, cfg.d_i), 1.0, False)
    kI = _normal(rng, (B, S, cfg.d_i), 1.0, False)
    w = _normal(rng, (B, S, cfg.h_i), 1.0, False)
    z_kv = rng.standard_normal((1, cfg.block), dtype=np.float32)
    z_i = rng.standard_normal((1, cfg.block), dtype=np.float32)
    return {"cfg": cfg, "q": q, "k": k, "v": v, "qI": qI, "kI": kI, "w": w,
            "w_kv": _softmax_weights(z_kv), "w_i": _softmax_weights(z_i),
            "redraws": np.zeros((B, S), dtype=np.int32)}
