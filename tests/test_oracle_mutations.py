"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each."""
import numpy as np
import pytest

import oracle
import oracle.dsa as odsa
import oracle.hca as ohca
import test_oracle_dsa as tdsa
import test_oracle_hca as thca


def _expect_caught(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail("no pin caught the planted mistake")


def test_window_off_by_one(monkeypatch):
    monkeypatch.setattr(ohca, "window_bounds", lambda t, W, bs: (max(0, t - W), max(0, t - W) // bs))
    _expect_caught([lambda: thca.test_block_one_is_dense_causal(3), thca.test_golden_tiny_case])


def test_blocks_overlapping_window(monkeypatch):
    def wb(t, W, bs):
        lo = max(0, t - W + 1)
        return lo, -(-lo // bs)     # ceil: lets a block overlap the window
    monkeypatch.setattr(ohca, "window_bounds", wb)
    _expect_caught([thca.test_golden_tiny_case, thca.test_equal_keys_give_uniform_weights])


def test_missing_scale(monkeypatch):
    real = ohca.attend_row
    monkeypatch.setattr(ohca, "attend_row", lambda q, k, v, s: real(q, k, v, 1.0))
    _expect_caught([lambda: thca.test_block_one_is_dense_causal(1)])


def test_transposed_compress_weights(monkeypatch):
    def bad(x, w, block):
        x = np.asarray(x, dtype=np.float64)
        B, S, H, d = x.shape
        n = S // block
        return np.einsum("bnihd,hi->bnhd", x[:, : n * block].reshape(B, n, block, H, d), np.asarray(w)[:, ::-1])
    monkeypatch.setattr(oracle, "compress_kv", bad)
    _expect_caught([thca.test_compress_brute_force_loop, thca.test_compress_one_hot_is_row_copy])


def test_relu_dropped(monkeypatch):
    monkeypatch.setattr(odsa, "index_scores_row",
                        lambda qI_t, kI, w_t, t: (np.asarray(kI[: t + 1], float) @ np.asarray(qI_t, float).T) @ np.asarray(w_t, float))
    monkeypatch.setattr(oracle, "index_scores_row", odsa.index_scores_row)
    _expect_caught([tdsa.test_golden_scores_and_selection, tdsa.test_relu_drops_negative_heads])


def test_tie_break_reversed(monkeypatch):
    def bad(scores, k):
        n = scores.shape[0]
        if n <= k:
            return np.arange(n)
        order = np.lexsort((-np.arange(n), -scores.astype(np.float32).astype(np.float64)))
        return np.sort(order[:k])
    monkeypatch.setattr(odsa, "topk_row", bad)
    monkeypatch.setattr(oracle, "topk_row", bad)
    _expect_caught([tdsa.test_golden_scores_and_selection, tdsa.test_topk_matches_stable_sort])


def test_non_causal_indexer(monkeypatch):
    real = odsa.index_scores_row
    monkeypatch.setattr(odsa, "index_scores_row", lambda qI_t, kI, w_t, t: real(qI_t, kI, w_t, min(t + 1, kI.shape[0] - 1)))
    _expect_caught([tdsa.test_k_at_least_context_is_dense_causal_mqa, tdsa.test_equal_index_keys_select_first_positions])


# ---------------------------------------------------------------- gradients

import test_oracle_grad as tgrad  # noqa: E402


def test_softmax_jacobian_missing_mean_term(monkeypatch):
    def bad(qv, keys, values, scale, dout):
        logits = scale * (keys @ qv)
        p = np.exp(logits - logits.max())
        p /= p.sum()
        ds = p * (values @ dout)            # drops the <dout, o> term
        return scale * (ds @ keys), scale * np.outer(ds, qv), np.outer(p, dout)
    monkeypatch.setattr(ohca, "attend_row_bwd", bad)        # used by hca_attention_bwd
    monkeypatch.setattr(oracle, "attend_row_bwd", bad)
    _expect_caught([tgrad.test_attend_row_bwd_matches_finite_differences])
    _expect_caught([lambda: tgrad.test_hca_attention_bwd_matches_finite_differences(0, 0, 9, 9)])


def test_compressed_entries_gradient_dropped_from_raw_keys(monkeypatch):
    real = ohca.compress_kv_bwd
    monkeypatch.setattr(oracle, "compress_kv_bwd", lambda x, w, d, b: (0 * real(x, w, d, b)[0], real(x, w, d, b)[1]))
    _expect_caught([tgrad.test_hca_chain_through_compression_matches_finite_differences])


def test_sparse_bwd_value_gradient_transposed(monkeypatch):
    real = odsa.sparse_attention_bwd

    def bad(q, k, v, idx, scale, dout):
        dq, dk, dv = real(q, k, v, idx, scale, dout)
        return dq, dv, dk                    # key and value gradients swapped
    monkeypatch.setattr(oracle, "sparse_attention_bwd", bad)
    _expect_caught([tgrad.test_sparse_attention_bwd_matches_finite_differences])


# ---------------------------------------------------------------- CSA
import oracle.csa as ocsa  # noqa: E402
import test_oracle_csa as tcsa  # noqa: E402


def test_csa_visibility_counts_the_open_block(monkeypatch):
    monkeypatch.setattr(ocsa, "visible_entries", lambda t, block: (t + block) // block)  # block not yet complete
    _expect_caught([lambda: tcsa.test_selection_against_explicit_loops(4, 3),
                    tcsa.test_k_covering_every_entry_is_dense_block_causal_attention])


def test_csa_visibility_one_block_late(monkeypatch):
    monkeypatch.setattr(ocsa, "visible_entries", lambda t, block: t // block)
    _expect_caught([lambda: tcsa.test_selection_against_explicit_loops(4, 100),
                    tcsa.test_k_covering_every_entry_is_dense_block_causal_attention])


def test_csa_attention_reads_the_wrong_entries(monkeypatch):
    real = ocsa.csa_attention
    # every selected entry replaced by entry 0
    monkeypatch.setattr(ocsa, "csa_attention", lambda q, kc, vc, idx, scale: real(q, kc, vc, np.minimum(idx, 0), scale))
    _expect_caught([tcsa.test_k_covering_every_entry_is_dense_block_causal_attention])


# ---------------------------------------------------------------- epilogues
import oracle.epilogue as oepi  # noqa: E402
import test_oracle_epilogue as tepi  # noqa: E402


def test_vha_mixing_matrix_transposed(monkeypatch):
    def bad(o, u, v):
        m = (np.asarray(u) @ np.asarray(v)).T
        return np.asarray(o) + np.einsum("gh,bshd->bsgd", m, np.asarray(o))
    monkeypatch.setattr(oepi, "vha_mix", bad)
    monkeypatch.setattr(oracle, "vha_mix", bad)
    _expect_caught([tepi.test_vha_against_explicit_loops, tepi.test_vha_special_cases])


def test_gate_applied_before_mixing(monkeypatch):
    def bad(o, c, w_g, u, v):
        return oepi.vha_mix(oepi.gate_values(c, w_g, o.shape[2], o.shape[3]) * o, u, v)
    monkeypatch.setattr(oepi, "gated_vha_output", bad)
    monkeypatch.setattr(oracle, "gated_vha_output", bad)
    _expect_caught([tepi.test_output_is_gate_times_mixed])


def test_gate_tanh_for_sigmoid(monkeypatch):
    monkeypatch.setattr(oepi, "sigmoid", lambda x: np.tanh(np.asarray(x, dtype=np.float64)))
    _expect_caught([tepi.test_gate_closed_forms, tepi.test_gate_against_explicit_loops_and_torch])


def test_sparse_attention_every_head_reads_kv_head_zero(monkeypatch):
    """The MQA shortcut (every query head reading KV head 0) must fail the
    grouped-head pin."""
    real = odsa.sparse_attention

    def bad(q, k, v, idx, scale, rows=None):
        Hq = q.shape[2]
        k0 = np.repeat(np.asarray(k)[:, :, :1], k.shape[2], axis=2)
        v0 = np.repeat(np.asarray(v)[:, :, :1], v.shape[2], axis=2)
        return real(q, k0, v0, idx, scale, rows)
    monkeypatch.setattr(oracle, "sparse_attention", bad)
    _expect_caught([tdsa.test_k_at_least_context_is_dense_causal_gqa])
