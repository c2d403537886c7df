"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This package holds workload shapes and random-number draws only: it draws
normals, rounds them to bfloat16, builds per-head compressor weights as a
softmax of normal draws, and draws random index lists.  It performs none of
the attention, compression, indexing or selection arithmetic of the method
itself, and it imports neither the HIP binding nor the oracle.
"""
from .configs import (HcaPrefillConfig, HcaDecodeConfig, DsaConfig, CsaConfig, CONFIGS, CSA_CONFIGS,
                      small_prefill, small_decode, small_dsa, small_csa)
from .gen import (bf16_round_bits, bf16_bits_to_f32, make_prefill, make_decode,
                  make_dsa, make_csa, redraw_dsa_rows, make_normal, make_index_lists,
                  make_index_lists_long)

__all__ = [
    "HcaPrefillConfig", "HcaDecodeConfig", "DsaConfig", "CsaConfig", "CONFIGS", "CSA_CONFIGS",
    "small_prefill", "small_decode", "small_dsa", "small_csa",
    "bf16_round_bits", "bf16_bits_to_f32", "make_prefill", "make_decode",
    "make_dsa", "make_csa", "redraw_dsa_rows", "make_normal", "make_index_lists", "make_index_lists_long",
]
