"""Pins for the HCA oracle: closed forms, special cases that reduce to dense causal
attention (computed by torch), brute force on tiny inputs and a hand-derived golden case."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _dense_causal_torch(q, k, v, scale):
    """Textbook dense causal attention via torch SDPA in float64 (library cross-check)."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    mask = torch.triu(torch.ones(S, S, dtype=torch.bool), 1)
    lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


# ---------------------------------------------------------------- compression

def test_compress_brute_force_loop():
    rng = np.random.default_rng(1)
    B, S, H, d, bs = 2, 13, 3, 4, 4
    x = _rand(rng, B, S, H, d)
    w = _rand(rng, H, bs)
    got = oracle.compress_kv(x, w, bs)
    assert got.shape == (B, S // bs, H, d)
    for b in range(B):
        for j in range(S // bs):
            for h in range(H):
                for c in range(d):
                    acc = 0.0
                    for i in range(bs):
                        acc += w[h, i] * x[b, j * bs + i, h, c]
                    assert abs(got[b, j, h, c] - acc) < 1e-12


def test_compress_one_hot_is_row_copy():
    rng = np.random.default_rng(2)
    x = _rand(rng, 1, 512, 2, 8)
    w = np.zeros((2, 128))
    w[0, 5] = 1.0
    w[1, 127] = 1.0
    got = oracle.compress_kv(x, w, 128)
    np.testing.assert_array_equal(got[0, :, 0], x[0, 5::128, 0])
    np.testing.assert_array_equal(got[0, :, 1], x[0, 127::128, 1])


def test_compress_uniform_is_block_mean_and_cache_is_128x_smaller():
    rng = np.random.default_rng(3)
    x = _rand(rng, 1, 1024, 2, 16)
    w = np.full((2, 128), 1.0 / 128)
    got = oracle.compress_kv(x, w, 128)
    ref = x.reshape(1, 8, 128, 2, 16).mean(axis=2)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)
    # 128 tokens -> one cache entry
    assert got.size * 128 == x.size


def test_compress_is_linear_and_ignores_partial_tail():
    rng = np.random.default_rng(4)
    x, y = _rand(rng, 1, 300, 2, 4), _rand(rng, 1, 300, 2, 4)
    w = _rand(rng, 2, 128)
    a, b = 0.75, -2.5
    np.testing.assert_allclose(oracle.compress_kv(a * x + b * y, w, 128),
                               a * oracle.compress_kv(x, w, 128) + b * oracle.compress_kv(y, w, 128), atol=1e-11)
    x2 = x.copy()
    x2[:, 256:] = 1e6
    np.testing.assert_array_equal(oracle.compress_kv(x2, w, 128), oracle.compress_kv(x, w, 128))


# ---------------------------------------------------------------- visibility

@pytest.mark.parametrize("window,block", [(1, 1), (3, 2), (5, 4), (128, 128), (256, 128), (7, 16)])
def test_visible_sets_by_enumeration(window, block):
    for t in range(0, 700):
        blocks, raw = oracle.visible_positions(t, window, block)
        # raw window: the W most recent positions including t
        assert raw == [p for p in range(t + 1) if t - p < window]
        lo = raw[0]
        # visible blocks: exactly those lying entirely before the window
        assert blocks == [j for j in range(t // block + 1) if (j + 1) * block <= lo]
        # the unseen gap between the last visible block and the window is shorter than a block
        covered_to = len(blocks) * block
        assert 0 <= lo - covered_to < block


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("window", [1, 3, 8])
def test_block_one_is_dense_causal(window):
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, d = 2, 19, 4, 2, 8
    q, k, v = _rand(rng, B, S, Hq, d), _rand(rng, B, S, Hkv, d), _rand(rng, B, S, Hkv, d)
    w = np.ones((Hkv, 1))
    kc, vc = oracle.compress_kv(k, w, 1), oracle.compress_kv(v, w, 1)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=window, block=1, scale=0.3)
    ro, rlse = _dense_causal_torch(q, k, v, 0.3)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, atol=1e-12)


def test_window_covering_sequence_is_dense_causal():
    rng = np.random.default_rng(6)
    B, S, H, d = 1, 40, 3, 16
    q, k, v = _rand(rng, B, S, H, d), _rand(rng, B, S, H, d), _rand(rng, B, S, H, d)
    w = _rand(rng, H, 8)
    kc, vc = oracle.compress_kv(k, w, 8), oracle.compress_kv(v, w, 8)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=S, block=8, scale=0.25)
    ro, rlse = _dense_causal_torch(q, k, v, 0.25)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, atol=1e-12)


def test_equal_keys_give_uniform_weights():
    rng = np.random.default_rng(7)
    B, S, H, d, bs, W = 1, 700, 2, 8, 128, 200
    q = _rand(rng, B, S, H, d)
    kstar = _rand(rng, H, d)
    k = np.broadcast_to(kstar, (B, S, H, d)).copy()
    v = _rand(rng, B, S, H, d)
    w = np.full((H, bs), 1.0 / bs)
    kc, vc = oracle.compress_kv(k, w, bs), oracle.compress_kv(v, w, bs)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=W, block=bs, scale=0.125)
    for t in [0, 1, 127, 199, 200, 327, 328, 455, 456, 699]:
        lo = max(0, t - W + 1)
        n_c = lo // bs
        for h in range(H):
            vis = np.concatenate([vc[0, :n_c, h], v[0, lo:t + 1, h]])
            np.testing.assert_allclose(o[0, t, h], vis.mean(axis=0), atol=1e-12)
            assert abs(lse[0, h, t] - (0.125 * q[0, t, h] @ kstar[h] + math.log(n_c + t + 1 - lo))) < 1e-12


def test_golden_tiny_case():
    g = json.load(open(os.path.join(GOLD, "hca_tiny.json")))
    k = np.array(g["k"]).reshape(1, 5, 1, 1)
    v = np.array(g["v"]).reshape(1, 5, 1, 1)
    q = np.array(g["q"]).reshape(1, 5, 1, 1)
    w = np.array([[0.5, 0.5]])
    kc, vc = oracle.compress_kv(k, w, 2), oracle.compress_kv(v, w, 2)
    np.testing.assert_allclose(kc.ravel(), g["kc"], atol=1e-14)
    np.testing.assert_allclose(vc.ravel(), g["vc"], atol=1e-14)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=2, block=2, scale=1.0)
    np.testing.assert_allclose(o.ravel(), g["o"], rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(lse.ravel(), g["lse"], atol=1e-13)


def test_decode_equals_prefill_row():
    cfg = synth.small_prefill("c1", seqlen=600, h_q=4, h_kv=2, head_dim=16, window=100, block=64)
    inp = synth.make_prefill(cfg)
    q, k, v = (inp[n].astype(np.float64) for n in ("q", "k", "v"))
    kc, vc = oracle.compress_kv(k, inp["w"], 64), oracle.compress_kv(v, inp["w"], 64)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=100, block=64, scale=0.25)
    for t in [0, 99, 163, 164, 599]:
        lo = max(0, t - 99)
        od, lsed = oracle.hca_attention(q[:, t:t + 1], k[:, lo:t + 1], v[:, lo:t + 1], kc, vc,
                                        window=100, block=64, scale=0.25, q_pos0=t, kv_pos0=lo)
        np.testing.assert_allclose(od[:, 0], o[:, t], atol=1e-13)
        np.testing.assert_allclose(lsed[..., 0], lse[..., t], atol=1e-13)


def test_cache_too_short_is_rejected():
    z = np.zeros((1, 300, 1, 2))
    kc = np.zeros((1, 1, 1, 2))
    with pytest.raises(ValueError):
        oracle.hca_attention(z, z, z, kc, kc, window=10, block=128, scale=1.0)
