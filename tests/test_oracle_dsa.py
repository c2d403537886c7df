"""Pins for the DSA oracle: hand-derived golden values, brute-force scores and sorting,
the k >= context special case against torch dense causal attention, and the tie rules."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_scores_and_selection():
    g = json.load(open(os.path.join(GOLD, "dsa_tiny.json")))
    kI = np.array(g["kI"]).reshape(4, 1)
    qI = np.array([[1.0], [-1.0]])
    w = np.array([1.0, 0.5])
    np.testing.assert_array_equal(oracle.index_scores_row(qI, kI, w, 3), g["scores_t3"])
    for c in g["cases"]:
        sel = oracle.topk_row(oracle.index_scores_row(qI, kI, w, c["t"]), c["k"])
        assert sel.tolist() == c["sel"], c["why"]
    a = g["attention"]
    q = np.ones((1, 1, 1, 1))
    k = np.array(a["k_sel"]).reshape(1, 2, 1, 1)
    v = np.array(a["v_sel"]).reshape(1, 2, 1, 1)
    idx = np.array([[[0, 1, -1]]])
    o, lse = oracle.sparse_attention(q, k, v, idx, 1.0)
    assert abs(o[0, 0, 0, 0] - a["o"]) < 1e-13 and abs(lse[0, 0, 0] - a["lse"]) < 1e-13


def test_scores_brute_force_loops():
    rng = np.random.default_rng(11)
    S, hi, di = 9, 3, 5
    qI, kI, w = rng.standard_normal((S, hi, di)), rng.standard_normal((S, di)), rng.standard_normal((S, hi))
    for t in range(S):
        got = oracle.index_scores_row(qI[t], kI, w[t], t)
        assert got.shape == (t + 1,)
        for u in range(t + 1):
            acc = 0.0
            for h in range(hi):
                dot = 0.0
                for i in range(di):
                    dot += qI[t, h, i] * kI[u, i]
                acc += w[t, h] * (dot if dot > 0 else 0.0)
            assert abs(got[u] - acc) < 1e-12


def test_topk_matches_stable_sort():
    rng = np.random.default_rng(12)
    for n, k in [(50, 7), (200, 64), (33, 33), (10, 40)]:
        s = np.round(rng.standard_normal(n) * 3) / 2   # many exact ties
        s[::5] = 0.0
        s[1::7] = -0.0
        got = oracle.topk_row(s, k)
        keyed = sorted(range(n), key=lambda u: (-float(np.float32(s[u])), u))
        assert got.tolist() == sorted(keyed[:min(k, n)])


def test_equal_index_keys_select_first_positions():
    S, k = 40, 8
    kI = np.ones((1, S, 4))
    qI = np.ones((1, S, 2, 4))
    w = np.ones((1, S, 2))
    idx = oracle.index_topk(qI, kI, w, k)
    for t in range(S):
        n = min(t + 1, k)
        assert idx[0, t, :n].tolist() == list(range(n))
        assert (idx[0, t, n:] == -1).all()


def test_relu_drops_negative_heads():
    kI = np.array([[1.0], [2.0], [-3.0]])
    qI = np.array([[1.0], [-1.0]])
    s = oracle.index_scores_row(qI, kI, np.array([1.0, 1.0]), 2)
    np.testing.assert_array_equal(s, [1.0, 2.0, 3.0])
    s = oracle.index_scores_row(qI, kI, np.array([1.0, -1.0]), 2)
    np.testing.assert_array_equal(s, [1.0, 2.0, -3.0])


def test_k_at_least_context_is_dense_causal_mqa():
    rng = np.random.default_rng(13)
    B, S, Hq, d = 1, 24, 4, 16
    q = rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, 1, d))
    v = rng.standard_normal((B, S, 1, d))
    qI = rng.standard_normal((B, S, 2, 8))
    kI = rng.standard_normal((B, S, 8))
    w = rng.standard_normal((B, S, 2))
    idx = oracle.index_topk(qI, kI, w, S)
    o, lse = oracle.sparse_attention(q, k, v, idx, 0.25)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, Hq, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, Hq, axis=2)).permute(0, 2, 1, 3)
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
    np.testing.assert_allclose(o, ro.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    logits = (qt @ kt.transpose(-1, -2)) * 0.25
    rl = torch.logsumexp(logits.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf), -1)
    np.testing.assert_allclose(lse, rl.numpy(), atol=1e-12)


def test_k_at_least_context_is_dense_causal_gqa():
    """Grouped KV heads (Hq = 6 on Hkv = 3): query head h must read KV head
    h // 2.  With k >= context the selection is every past position, so each
    head's output is torch's causal attention against its own KV head."""
    rng = np.random.default_rng(21)
    B, S, Hq, Hkv, d = 2, 20, 6, 3, 8
    q = rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    idx = np.full((B, S, S + 3), -1, dtype=np.int32)
    for t in range(S):
        idx[:, t, : t + 1] = rng.permutation(t + 1)
    o, lse = oracle.sparse_attention(q, k, v, idx, 0.35)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.35)
    np.testing.assert_allclose(o, ro.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    logits = (qt @ kt.transpose(-1, -2)) * 0.35
    rl = torch.logsumexp(logits.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf), -1)
    np.testing.assert_allclose(lse, rl.numpy(), atol=1e-12)
    # heads of one group share keys: swapping the KV heads changes the outputs of exactly the affected groups
    o2, _ = oracle.sparse_attention(q, k[:, :, [1, 0, 2]], v[:, :, [1, 0, 2]], idx, 0.35)
    assert not np.allclose(o2[:, :, :4], o[:, :, :4])
    np.testing.assert_allclose(o2[:, :, 4:], o[:, :, 4:], atol=0)


def test_sparse_attention_ignores_index_order_and_padding():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 3, 2, 8))
    k = rng.standard_normal((1, 30, 1, 8))
    v = rng.standard_normal((1, 30, 1, 8))
    a = np.array([[[3, 17, 5, -1, -1], [0, 1, 2, 3, 4], [29, -1, 7, -1, 11]]])
    b = np.array([[[5, 3, 17, -1, -1], [4, 3, 2, 1, 0], [-1, 11, -1, 29, 7]]])
    oa, la = oracle.sparse_attention(q, k, v, a, 0.3)
    ob, lb = oracle.sparse_attention(q, k, v, b, 0.3)
    np.testing.assert_allclose(oa, ob, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)


def test_tie_rules():
    # an exact tie at the boundary is not tie-free; a clear gap is
    kI = np.array([[1.0], [2.0], [2.0], [0.5]])
    qI = np.array([[1.0]])
    assert not oracle.tie_free_row(qI, kI, np.array([1.0]), 3, 1)   # 2.0 vs 2.0 at the cut
    assert oracle.tie_free_row(qI, kI, np.array([1.0]), 3, 2)       # the tie lies inside the set
    assert oracle.tie_free_row(qI, kI, np.array([1.0]), 3, 3)
    # exact zeros (all dots certainly negative) are ordered by position
    kI = np.array([[5.0], [-1.0], [-2.0], [-3.0]])
    assert oracle.tie_free_row(qI, kI, np.array([1.0]), 3, 2)
    assert oracle.index_topk(qI[None, None].repeat(4, 1), kI[None], np.ones((1, 4, 1)), 2)[0, 3].tolist() == [0, 1]
    assert oracle.valid_topk_row([0, 1], qI, kI, np.array([1.0]), 3, 2)
    assert not oracle.valid_topk_row([0, 2], qI, kI, np.array([1.0]), 3, 2)
    # an index list that swaps elements inside the error bound is valid; far outside is not
    kI = np.array([[1.0], [1.0 + 1e-9], [3.0], [0.1]])
    assert oracle.valid_topk_row([2, 0], qI, kI, np.array([1.0]), 3, 2)
    assert oracle.valid_topk_row([1, 2], qI, kI, np.array([1.0]), 3, 2)
    assert not oracle.valid_topk_row([2, 3], qI, kI, np.array([1.0]), 3, 2)
    assert not oracle.valid_topk_row([2, 2], qI, kI, np.array([1.0]), 3, 2)
    assert not oracle.valid_topk_row([2, 0, 1], qI, kI, np.array([1.0]), 3, 2)


def test_tie_free_generation_converges_on_synthetic_rows():
    cfg = synth.small_dsa(seqlen=400, topk=64)
    inp = synth.make_dsa(cfg)
    for attempt in range(1, 8):
        bad = np.nonzero(~oracle.tie_free_rows(inp["qI"], inp["kI"], inp["w"], cfg.topk))[0]
        if bad.size == 0:
            break
        synth.redraw_dsa_rows(inp, [(0, t) for t in bad], attempt)
    assert oracle.tie_free_rows(inp["qI"], inp["kI"], inp["w"], cfg.topk).all()
