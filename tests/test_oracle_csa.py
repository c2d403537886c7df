"""Pins of the CSA oracle (history compressed by a block of positions, top-k
over the compressed entries), against definitions it does not share code with:
explicit loops, the DSA special case, and dense attention computed by torch."""
import numpy as np
import pytest
import torch

import oracle


def _inputs(S=40, block=4, hi=4, di=8, seed=0):
    rng = np.random.default_rng(seed)
    qI = rng.standard_normal((1, S, hi, di))
    kIc = rng.standard_normal((1, S // block + 1, di))
    w = rng.standard_normal((1, S, hi))
    return qI, kIc, w


def test_visible_entries_by_enumeration():
    for block in (1, 2, 3, 4, 7):
        for t in range(40):
            complete = [j for j in range(40) if block * j + block - 1 <= t]   # every position of the block <= t
            assert oracle.visible_entries(t, block) == len(complete)


def test_block_one_is_dsa():
    rng = np.random.default_rng(1)
    qI = rng.standard_normal((2, 30, 4, 8))
    kI = rng.standard_normal((2, 30, 8))
    w = rng.standard_normal((2, 30, 4))
    for k in (1, 5, 30):
        np.testing.assert_array_equal(oracle.csa_index_topk(qI, kI, w, k, 1), oracle.index_topk(qI, kI, w, k))


@pytest.mark.parametrize("block,k", [(4, 3), (4, 100), (3, 2), (5, 1)])
def test_selection_against_explicit_loops(block, k):
    qI, kIc, w = _inputs(block=block)
    idx = oracle.csa_index_topk(qI, kIc, w, k, block)
    for t in range(qI.shape[1]):
        n = sum(1 for j in range(kIc.shape[1]) if block * (j + 1) - 1 <= t)
        scores = []
        for j in range(n):
            s = 0.0
            for h in range(qI.shape[2]):
                dot = sum(qI[0, t, h, i] * kIc[0, j, i] for i in range(qI.shape[3]))
                s += w[0, t, h] * max(dot, 0.0)
            scores.append(s)
        # rank: larger float32 score first, smaller entry index on a tie
        order = sorted(range(n), key=lambda j: (-float(np.float32(scores[j])), j))
        want = sorted(order[:k])
        got = idx[0, t]
        assert list(got[: len(want)]) == want
        assert (got[len(want):] == -1).all()


def test_equal_index_keys_select_the_first_entries():
    qI, kIc, w = _inputs(block=4)
    kIc[:] = kIc[0, 0]
    idx = oracle.csa_index_topk(qI, kIc, w, 3, 4)
    for t in range(qI.shape[1]):
        n = min((t + 1) // 4, 3)
        assert list(idx[0, t, :n]) == list(range(n))


def test_k_covering_every_entry_is_dense_block_causal_attention():
    """With k >= the number of entries, CSA is dense attention over the compressed
    rows with a block-causal mask (entry j visible to t iff 4j + 3 <= t)."""
    rng = np.random.default_rng(2)
    S, block, Hq, d = 45, 4, 3, 8
    q = rng.standard_normal((1, S, Hq, d))
    k = rng.standard_normal((1, S, 1, d))
    v = rng.standard_normal((1, S, 1, d))
    qI = rng.standard_normal((1, S, 2, 4))
    kI = rng.standard_normal((1, S, 4))
    w = rng.standard_normal((1, S, 2))
    wk = rng.random((1, block))
    wi = rng.random((1, block))
    kc, vc, kIc, idx, o, lse = oracle.csa_forward(q, k, v, qI, kI, w, wk, wi, topk=64, block=block, scale=0.4)
    n = S // block
    # the compressed rows themselves, by explicit sums
    for j in range(n):
        np.testing.assert_allclose(kc[0, j, 0], sum(wk[0, i] * k[0, block * j + i, 0] for i in range(block)))
    mask = torch.tensor([[block * j + block - 1 <= t for j in range(n)] for t in range(S)])
    rows = [t for t in range(S) if t >= block - 1]
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)[:, rows]                 # [Hq, rows, d]
    kt = torch.from_numpy(kc[0, :, 0])[None].expand(Hq, -1, -1)
    vt = torch.from_numpy(vc[0, :, 0])[None].expand(Hq, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[rows][None], scale=0.4)
    np.testing.assert_allclose(o[0, rows].transpose(1, 0, 2), ref.numpy(), rtol=1e-12, atol=1e-12)
    logits = 0.4 * np.einsum("thd,jd->htj", q[0], kc[0, :, 0])
    logits[:, ~mask.numpy()] = -np.inf
    with np.errstate(divide="ignore"):
        want_lse = np.log(np.exp(logits).sum(axis=2))
    np.testing.assert_allclose(lse[0][:, rows], want_lse[:, rows], rtol=1e-12)
    # positions before the first complete block attend to nothing
    assert (o[0, : block - 1] == 0).all() and np.isneginf(lse[0, :, : block - 1]).all()


def test_csa_attention_grouped_heads_against_torch():
    """Grouped KV heads: query head h attends over KV head h // (Hq / Hkv) of the
    listed entries; with every visible entry listed this is torch's attention
    under the block-causal mask, per KV group."""
    rng = np.random.default_rng(31)
    S, Hq, Hkv, d, block = 22, 4, 2, 8, 4
    n = S // block
    q = rng.standard_normal((1, S, Hq, d))
    kc = rng.standard_normal((1, n, Hkv, d))
    vc = rng.standard_normal((1, n, Hkv, d))
    idx = np.full((1, S, n + 2), -1, dtype=np.int32)
    for t in range(S):
        m = (t + 1) // block
        idx[0, t, :m] = rng.permutation(m)
    o, lse = oracle.csa_attention(q, kc, vc, idx, 0.3)
    mask = torch.tensor([[block * j + block - 1 <= t for j in range(n)] for t in range(S)])
    rows = [t for t in range(S) if t >= block - 1]
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)[:, rows]                  # [Hq, rows, d]
    kt = torch.from_numpy(np.repeat(kc[0], Hq // Hkv, axis=1)).permute(1, 0, 2)  # [Hq, n, d]
    vt = torch.from_numpy(np.repeat(vc[0], Hq // Hkv, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[rows][None], scale=0.3)
    np.testing.assert_allclose(o[0, rows].transpose(1, 0, 2), ref.numpy(), rtol=1e-12, atol=1e-12)
    assert (o[0, : block - 1] == 0).all() and np.isneginf(lse[0, :, : block - 1]).all()


def test_tie_free_rows_reduce_to_dsa_on_the_visible_prefix():
    qI, kIc, w = _inputs(block=4)
    for t in range(qI.shape[1]):
        n = (t + 1) // 4
        want = True if n == 0 else oracle.tie_free_row(qI[0, t], kIc[0], w[0, t], n - 1, 3)
        assert oracle.csa_tie_free_row(qI[0, t], kIc[0], w[0, t], t, 3, 4) == want
