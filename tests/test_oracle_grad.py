"""Pins of the oracle's gradients: every analytic gradient equals the central
finite difference of the oracle's own forward definition (float64), so a
dropped term, a wrong sign or a transposed operand in the chain rule fails."""
import numpy as np
import pytest

import oracle


def _fd(f, x, eps=1e-6):
    """Central finite differences of the scalar f() with respect to every element of x (in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        x0 = x[i]
        x[i] = x0 + eps
        fp = f()
        x[i] = x0 - eps
        fm = f()
        x[i] = x0
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_attend_row_bwd_matches_finite_differences():
    rng = np.random.default_rng(0)
    qv, keys, vals, dout = rng.standard_normal(4), rng.standard_normal((6, 4)), rng.standard_normal((6, 3)), \
        rng.standard_normal(3)
    loss = lambda: float(dout @ oracle.attend_row(qv, keys, vals, 0.7)[0])
    gq, gk, gv = oracle.attend_row_bwd(qv, keys, vals, 0.7, dout)
    for got, x in ((gq, qv), (gk, keys), (gv, vals)):
        assert np.allclose(got, _fd(loss, x), rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("q_pos0,kv_pos0,Sq,Skv", [(0, 0, 9, 9), (6, 4, 3, 5)])
def test_hca_attention_bwd_matches_finite_differences(q_pos0, kv_pos0, Sq, Skv):
    """Every input of the attention (queries, raw window keys/values, compressed
    entries) at a tiny size with GQA, block 2, window 3, including a chunk whose
    queries and raw keys start mid-sequence."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, d, nb = 2, 4, 2, 3, 4
    q, dout = rng.standard_normal((B, Sq, Hq, d)), rng.standard_normal((B, Sq, Hq, d))
    k, v = rng.standard_normal((B, Skv, Hkv, d)), rng.standard_normal((B, Skv, Hkv, d))
    kc, vc = rng.standard_normal((B, nb, Hkv, d)), rng.standard_normal((B, nb, Hkv, d))
    kw = dict(window=3, block=2, scale=0.8, q_pos0=q_pos0, kv_pos0=kv_pos0)
    loss = lambda: float(np.sum(dout * oracle.hca_attention(q, k, v, kc, vc, **kw)[0]))
    grads = oracle.hca_attention_bwd(q, k, v, kc, vc, dout, **kw)
    for got, x in zip(grads, (q, k, v, kc, vc)):
        assert np.allclose(got, _fd(loss, x), rtol=1e-5, atol=1e-8)


def test_compress_kv_bwd_matches_finite_differences():
    rng = np.random.default_rng(2)
    x, w = rng.standard_normal((2, 7, 2, 3)), rng.standard_normal((2, 3))
    dout = rng.standard_normal((2, 2, 2, 3))        # 7 rows, block 3: two blocks, one trailing row
    loss = lambda: float(np.sum(dout * oracle.compress_kv(x, w, 3)))
    dx, dw = oracle.compress_kv_bwd(x, w, dout, 3)
    assert np.allclose(dx, _fd(loss, x), rtol=1e-6, atol=1e-8)
    assert np.allclose(dw, _fd(loss, w), rtol=1e-6, atol=1e-8)
    assert not dx[:, 6].any()                       # the trailing row feeds no entry


def test_hca_chain_through_compression_matches_finite_differences():
    """The raw keys and values reach the output twice, through the window and
    through the compressed entries built from them: the full gradient is the
    attention gradient of the raw rows plus the compressor's backward of the
    entries' gradient, and the weights' gradient comes from the entries."""
    rng = np.random.default_rng(3)
    B, S, Hq, Hkv, d, blk, W = 1, 10, 2, 1, 3, 2, 3
    q, dout = rng.standard_normal((B, S, Hq, d)), rng.standard_normal((B, S, Hq, d))
    k, v = rng.standard_normal((B, S, Hkv, d)), rng.standard_normal((B, S, Hkv, d))
    wk, wv = rng.standard_normal((Hkv, blk)), rng.standard_normal((Hkv, blk))

    def loss():
        kc, vc = oracle.compress_kv(k, wk, blk), oracle.compress_kv(v, wv, blk)
        return float(np.sum(dout * oracle.hca_attention(q, k, v, kc, vc, window=W, block=blk, scale=0.9)[0]))

    kc, vc = oracle.compress_kv(k, wk, blk), oracle.compress_kv(v, wv, blk)
    dq, dk, dv, dkc, dvc = oracle.hca_attention_bwd(q, k, v, kc, vc, dout, window=W, block=blk, scale=0.9)
    dk2, dwk = oracle.compress_kv_bwd(k, wk, dkc, blk)
    dv2, dwv = oracle.compress_kv_bwd(v, wv, dvc, blk)
    assert np.allclose(dq, _fd(loss, q), rtol=1e-5, atol=1e-8)
    assert np.allclose(dk + dk2, _fd(loss, k), rtol=1e-5, atol=1e-8)
    assert np.allclose(dv + dv2, _fd(loss, v), rtol=1e-5, atol=1e-8)
    assert np.allclose(dwk, _fd(loss, wk), rtol=1e-5, atol=1e-8)
    assert np.allclose(dwv, _fd(loss, wv), rtol=1e-5, atol=1e-8)


def test_sparse_attention_bwd_matches_finite_differences():
    """Selected positions with -1 padding, a position chosen by several queries
    and two KV heads each shared by two query heads."""
    rng = np.random.default_rng(4)
    B, S, Hq, Hkv, d = 1, 5, 4, 2, 3
    q, dout = rng.standard_normal((B, S, Hq, d)), rng.standard_normal((B, S, Hq, d))
    k, v = rng.standard_normal((B, S, Hkv, d)), rng.standard_normal((B, S, Hkv, d))
    idx = np.array([[[0, -1, -1], [1, 0, -1], [2, 0, 1], [3, 1, -1], [4, 0, 2]]], dtype=np.int32)

    def fwd():
        o = np.zeros((B, S, Hq, d))
        for g in range(Hkv):       # the forward oracle reads KV head 0: run it per KV head
            hs = slice(g * 2, g * 2 + 2)
            o[:, :, hs] = oracle.sparse_attention(q[:, :, hs], k[:, :, g:g + 1], v[:, :, g:g + 1], idx, 0.6)[0]
        return o

    loss = lambda: float(np.sum(dout * fwd()))
    dq, dk, dv = oracle.sparse_attention_bwd(q, k, v, idx, 0.6, dout)
    for got, x in ((dq, q), (dk, k), (dv, v)):
        assert np.allclose(got, _fd(loss, x), rtol=1e-5, atol=1e-8)
