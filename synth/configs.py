"""The five workloads of the hybrid-attention forward path, as typed records.

Shapes follow the ERNIE 5.5 Flash Base pages: HCA layers compress every 128
tokens into one cache entry and use 512-wide heads (ai-club.cn page, section on
hybrid attention MLA + HCA); DSA layers use 256-wide heads and a top-k indexer
(same section); inference context reaches 1M tokens (mirrorspeed page,
opening summary).  The remaining sizes (window, batch, head counts, k) are the
stated synthetic choices of this library.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class HcaPrefillConfig:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    seqlen: int
    h_q: int
    h_kv: int
    head_dim: int
    block: int
    window: int
    std: float            # Q/K/V ~ N(0, std^2)
    include_compress: bool
    seed: int = 0

    @property
    def n_blocks(self) -> int:
        return self.seqlen // self.block

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class HcaDecodeConfig:
    name: str
    batch: int
    h_q: int
    h_kv: int
    head_dim: int
    n_blocks: int
    block: int
    window: int
    std: float
    seed: int = 0

    @property
    def kv_pos0(self) -> int:
        # the raw window starts right after the last compressed block
        return self.n_blocks * self.block

    @property
    def q_pos(self) -> int:
        # the query is the newest token of the window
        return self.kv_pos0 + self.window - 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class DsaConfig:
    name: str
    batch: int
    seqlen: int
    h_q: int
    d_qk: int
    d_v: int
    h_i: int
    d_i: int
    topk: int
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


@dataclass(frozen=True)
class CsaConfig:
    """CSA: the DSA shapes with K, V and the index keys compressed per block."""
    name: str
    batch: int
    seqlen: int
    h_q: int
    d_qk: int
    d_v: int
    h_i: int
    d_i: int
    topk: int
    block: int
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def n_entries(self) -> int:
        return self.seqlen // self.block


_S512 = 1.0 / math.sqrt(512.0)

CONFIGS = {
    # fp32 parity case, N(0,1) inputs, seed 0
    "c1": HcaPrefillConfig("c1", "f32", 1, 2048, 2, 2, 128, 128, 128, 1.0, True),
    # bf16 prefill, 256 compressed entries, W=128
    "c2": HcaPrefillConfig("c2", "bf16", 1, 32768, 16, 16, 512, 128, 128, _S512, True),
    # bf16 prefill, 1024 compressed entries, W=256, compression over the full sequence
    "c3": HcaPrefillConfig("c3", "bf16", 1, 131072, 16, 16, 512, 128, 256, _S512, True),
    # bf16 decode: 64 sequences, 8192 compressed entries + 128 raw, 16 heads on one KV head
    "c4": HcaDecodeConfig("c4", 64, 16, 1, 512, 8192, 128, 128, _S512),
    # DSA prefill: 64 query heads on one KV head, d 256, indexer 4 x 64 fp32, k=2048
    "c5": DsaConfig("c5", 1, 65536, 64, 256, 256, 4, 64, 2048),
}

# CSA workload (no config of its own in the headline list): c5's shapes with
# the history compressed by blocks of 4 (16384 entries), top-2048 entries.
CSA_CONFIGS = {
    "csa64k": CsaConfig("csa64k", 1, 65536, 64, 256, 256, 4, 64, 2048, 4),
}


def small_prefill(base: str = "c2", **kw) -> HcaPrefillConfig:
    """A reduced copy of a prefill config (for parity at oracle-friendly sizes)."""
    return replace(CONFIGS[base], name=kw.pop("name", base + "-small"), **kw)


def small_decode(**kw) -> HcaDecodeConfig:
    return replace(CONFIGS["c4"], name=kw.pop("name", "c4-small"), **kw)


def small_dsa(**kw) -> DsaConfig:
    return replace(CONFIGS["c5"], name=kw.pop("name", "c5-small"), **kw)


def small_csa(**kw) -> CsaConfig:
    return replace(CSA_CONFIGS["csa64k"], name=kw.pop("name", "csa-small"), **kw)
