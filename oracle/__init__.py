"""Plain float64 CPU oracle for the hybrid sparse attention forward path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package; only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark call it.  It shares no code with the HIP path.

Every function is the plain definition written out in numpy float64, one query
row at a time, following the ERNIE 5.5 Flash Base pages:

* HCA (heavily compressed attention): every 128 tokens of K/V become one cache
  entry; a query attends densely over the compressed entries plus a short
  recent uncompressed window (mirrorspeed page, section "Hybrid sparse
  attention, 1/7 full context access"; ai-club.cn page, section on hybrid
  attention MLA + HCA).
* DSA: a lightweight indexer scores past positions per query and core
  attention runs on the top-k only (same sections; besthub page, section
  "1. Hybrid Sparse Attention").
* CSA: the history compressed 4x, then a top-k selection over the compressed
  entries (mirrorspeed page, same section; besthub page, same section).
* Attention-output epilogues: the output gate from the low-rank query latent
  and Virtual Head Attention's low-rank cross-head mixing (mirrorspeed page,
  section "More structural improvements, data, and infrastructure"; besthub
  page, section "Core Architectural Innovations").

Points the pages leave open are fixed as stated in each module's docstring.
The gradients (``*_bwd``) are the chain rule through these definitions (the
pages describe the forward only), pinned against central finite differences.
Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (closed forms, special cases reducing to dense
causal attention computed by torch, brute-force loops and hand-derived golden
values); none is "parity unpinned".
"""
from .hca import (compress_kv, window_bounds, attend_row, hca_attention, visible_positions,
                  attend_row_bwd, hca_attention_bwd, compress_kv_bwd)
from .dsa import (index_scores_row, topk_row, index_topk, sparse_attention, sparse_attention_bwd,
                  score_error_bounds, tie_free_row, tie_free_rows, valid_topk_row)
from .csa import visible_entries, csa_index_topk, csa_attention, csa_forward, csa_tie_free_row
from .epilogue import sigmoid, gate_values, vha_mix, gated_vha_output

__all__ = [
    "compress_kv", "window_bounds", "attend_row", "hca_attention", "visible_positions",
    "attend_row_bwd", "hca_attention_bwd", "compress_kv_bwd", "sparse_attention_bwd",
    "index_scores_row", "topk_row", "index_topk", "sparse_attention",
    "score_error_bounds", "tie_free_row", "tie_free_rows", "valid_topk_row",
    "visible_entries", "csa_index_topk", "csa_attention", "csa_forward", "csa_tie_free_row",
    "sigmoid", "gate_values", "vha_mix", "gated_vha_output",
]
