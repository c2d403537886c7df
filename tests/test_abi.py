"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import sparse_attention_hca_amd as hca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hca.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hca.LIB_PATH), reason="libhca.so not built")

S = hca.Strides
Z = S(0, 0, 0)
FAKE = ctypes.c_void_p(1 << 20)   # aligned non-null pointer; never dereferenced on these paths


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:hca|dsa|csa|attn)_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_exports_agree():
    names = _declared()
    assert set(names) == set(hca.EXPORTS)
    lib = hca.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert hca.hca_abi_version() == 1


def _lib():
    return hca.load_library()


def test_append_rejects_bad_arguments():
    lib = _lib()
    ring_k, ring_v = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31)
    kc, vc = ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 33)

    def st(**kw):
        return lib.hca_append_kv(kw.get("dt", 1), kw.get("kn", FAKE), S(0, 512, 512), FAKE, S(0, 512, 512),
                                 kw.get("kr", ring_k), S(0, 512, 512), ring_v, S(0, 512, 512), kw.get("ring", 128),
                                 kw.get("wk", FAKE), FAKE, kc, S(0, 512, 512), vc, S(0, 512, 512),
                                 kw.get("nb", 4), kw.get("t", 127), 1, 1, kw.get("d", 512), kw.get("block", 128),
                                 None)
    assert st(dt=5) == hca.HCA_ERR_INVALID
    assert st(ring=64) == hca.HCA_ERR_INVALID                  # the ring cannot hold a block
    assert "whole block" in hca.hca_last_error()
    assert st(t=5 * 128 - 1) == hca.HCA_ERR_INVALID            # closes block 4, kc holds 4
    assert st(t=-1) == hca.HCA_ERR_INVALID
    assert st(d=96) == hca.HCA_ERR_UNSUPPORTED
    assert st(kn=None) == hca.HCA_ERR_INVALID
    assert st(wk=None) == hca.HCA_ERR_INVALID                  # t = 127 closes block 0
    assert st(kr=ring_v) == hca.HCA_ERR_INVALID                # the two rings alias
    assert "overlap" in hca.hca_last_error()
    assert st(t=1 << 31) == hca.HCA_ERR_UNSUPPORTED


def test_compress_rejects_bad_arguments():
    lib = _lib()
    st = lambda **kw: lib.hca_compress_kv(kw.get("dt", 1), kw.get("k", FAKE), kw.get("sk", S(0, 512, 512)),
                                          kw.get("v", FAKE), S(0, 512, 512), kw.get("wk", FAKE), FAKE,
                                          kw.get("kc", ctypes.c_void_p(1 << 30)), S(0, 512, 512),
                                          ctypes.c_void_p(1 << 31), S(0, 512, 512), 1, kw.get("s", 256), 1,
                                          kw.get("d", 512), kw.get("block", 128), None)
    assert st(dt=7) == hca.HCA_ERR_INVALID
    assert st(k=None) == hca.HCA_ERR_INVALID
    assert st(wk=None) == hca.HCA_ERR_INVALID
    assert st(block=0) == hca.HCA_ERR_INVALID
    assert st(s=-1) == hca.HCA_ERR_INVALID
    assert st(d=96) == hca.HCA_ERR_UNSUPPORTED
    assert st(k=ctypes.c_void_p((1 << 20) + 2)) == hca.HCA_ERR_INVALID          # misaligned
    assert st(sk=S(0, 500, 512)) == hca.HCA_ERR_INVALID                          # stride not 16-byte multiple
    assert st(kc=FAKE) == hca.HCA_ERR_INVALID                                    # output aliases input
    assert "overlap" in hca.hca_last_error()


def _attn(lib, **kw):
    q = kw.get("q", FAKE)
    return lib.hca_attn_fwd(kw.get("dt", 1), q, S(0, 512 * 4, 512), FAKE, S(0, 512 * 4, 512), FAKE,
                            S(0, 512 * 4, 512), kw.get("kc", FAKE), S(0, 512, 512), kw.get("kc", FAKE),
                            S(0, 512, 512), kw.get("o", ctypes.c_void_p(1 << 34)), S(0, 512 * 4, 512),
                            kw.get("lse", None), 1, kw.get("sq", 300), kw.get("qp", 0), kw.get("skv", 300),
                            kw.get("kvp", 0), kw.get("nb", 2), kw.get("hq", 4), kw.get("hkv", 4),
                            kw.get("d", 512), kw.get("block", 128), kw.get("window", 64), kw.get("scale", 0.05),
                            kw.get("ws", None), kw.get("wsb", 0), None)


def test_attn_rejects_bad_arguments():
    lib = _lib()
    assert _attn(lib, hq=6, hkv=4) == hca.HCA_ERR_INVALID
    assert _attn(lib, window=0) == hca.HCA_ERR_INVALID
    assert _attn(lib, block=0) == hca.HCA_ERR_INVALID
    assert _attn(lib, q=None) == hca.HCA_ERR_INVALID
    assert _attn(lib, scale=float("nan")) == hca.HCA_ERR_INVALID
    assert _attn(lib, kvp=5) == hca.HCA_ERR_INVALID           # window of query 0 starts before the raw K/V
    assert _attn(lib, skv=200) == hca.HCA_ERR_INVALID         # raw K/V end before the last query
    assert _attn(lib, o=FAKE) == hca.HCA_ERR_INVALID          # output aliases q
    assert _attn(lib, lse=ctypes.c_void_p((1 << 34) + 2)) == hca.HCA_ERR_INVALID
    assert _attn(lib, dt=0, d=520) == hca.HCA_ERR_UNSUPPORTED
    # decode needs a workspace of the size the query reports
    need = lib.hca_attn_fwd_workspace_size(1, 1, 4, 4, 512, 2, 64)
    assert need > 0
    assert _attn(lib, sq=1, qp=299, kvp=236, skv=64, ws=None, wsb=0) == hca.HCA_ERR_WORKSPACE
    assert _attn(lib, sq=1, qp=299, kvp=236, skv=64, ws=ctypes.c_void_p(1 << 36), wsb=need - 1) == hca.HCA_ERR_WORKSPACE
    assert lib.hca_attn_fwd_workspace_size(1, 5, 4, 4, 512, 2, 64) == 0


def test_attn_needs_enough_compressed_entries():
    lib = _lib()
    # last query t=299, window 64 -> lo = 236 -> n_c = 1; query 0 sees none
    assert _attn(lib, nb=0, kc=None) == hca.HCA_ERR_INVALID
    assert "compressed" in hca.hca_last_error()


def test_dsa_rejects_bad_arguments():
    lib = _lib()
    ws = lib.dsa_index_topk_workspace_size(1, 1000, 64)
    assert ws > 0
    call = lambda **kw: lib.dsa_index_topk(kw.get("q", FAKE), FAKE, FAKE, kw.get("idx", ctypes.c_void_p(1 << 34)),
                                           1, 1000, kw.get("hi", 4), kw.get("di", 64), kw.get("k", 64),
                                           kw.get("ws", ctypes.c_void_p(1 << 36)), kw.get("wsb", ws), None)
    assert call(q=None) == hca.HCA_ERR_INVALID
    assert call(di=65) == hca.HCA_ERR_UNSUPPORTED
    assert call(hi=9) == hca.HCA_ERR_UNSUPPORTED
    assert call(k=0) == hca.HCA_ERR_INVALID
    assert call(wsb=ws - 1) == hca.HCA_ERR_WORKSPACE
    assert call(idx=FAKE) == hca.HCA_ERR_INVALID
    sp = lambda **kw: lib.dsa_sparse_attn_fwd(kw.get("dt", 1), FAKE, S(0, 64 * 256, 256), FAKE, S(0, 256, 256),
                                              FAKE, S(0, 256, 256), kw.get("idx", ctypes.c_void_p(1 << 33)),
                                              ctypes.c_void_p(1 << 34), S(0, 64 * 256, 256), None, 1, 100,
                                              kw.get("hq", 64), 1, kw.get("d", 256), 256, kw.get("k", 16), 0.0625,
                                              None)
    assert sp(idx=None) == hca.HCA_ERR_INVALID
    assert sp(d=128) == hca.HCA_ERR_UNSUPPORTED
    assert sp(hq=32) == hca.HCA_ERR_UNSUPPORTED
    assert sp(dt=0) == hca.HCA_ERR_UNSUPPORTED
    assert sp(k=4097) == hca.HCA_ERR_UNSUPPORTED


def test_dsa_decode_rejects_bad_arguments():
    lib = _lib()
    ws = lib.dsa_index_topk_decode_workspace_size(2, 200000, 2048)
    # one score row per sequence, 4 segments of first-stage winners, the ordered candidates
    assert ws >= 2 * 200064 * 4 + 2 * 4 * 2048 * 4 + 2 * 8192 * 8
    assert lib.dsa_index_topk_decode_workspace_size(2, 5000, 2048) == 2 * 5120 * 4  # one segment: scores only
    call = lambda **kw: lib.dsa_index_topk_decode(kw.get("q", FAKE), FAKE, FAKE,
                                                  kw.get("idx", ctypes.c_void_p(1 << 34)), 2, kw.get("n", 200000),
                                                  kw.get("hi", 4), kw.get("di", 64), kw.get("k", 2048),
                                                  kw.get("ws", ctypes.c_void_p(1 << 36)), kw.get("wsb", ws), None)
    assert call(q=None) == hca.HCA_ERR_INVALID
    assert call(hi=6) == hca.HCA_ERR_UNSUPPORTED
    assert call(di=72) == hca.HCA_ERR_UNSUPPORTED
    assert call(k=4097) == hca.HCA_ERR_UNSUPPORTED
    assert call(n=0) == hca.HCA_ERR_INVALID
    assert call(n=1 << 30) == hca.HCA_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == hca.HCA_ERR_WORKSPACE
    assert call(ws=None) == hca.HCA_ERR_WORKSPACE
    assert call(idx=FAKE) == hca.HCA_ERR_INVALID       # idx aliases the query
    sp = lambda **kw: lib.dsa_sparse_attn_decode(kw.get("dt", 1), FAKE, S(0, 64 * 256, 256), FAKE, S(0, 256, 256),
                                                 FAKE, S(0, 256, 256), kw.get("idx", ctypes.c_void_p(1 << 33)),
                                                 kw.get("o", ctypes.c_void_p(1 << 34)), S(0, 64 * 256, 256), None,
                                                 1, kw.get("n", 100000), 64, 1, kw.get("d", 256), 256,
                                                 kw.get("k", 16), 0.0625, kw.get("ws", None), kw.get("wsb", 0), None)
    assert sp(idx=None) == hca.HCA_ERR_INVALID
    assert sp(n=0) == hca.HCA_ERR_INVALID
    assert sp(d=128) == hca.HCA_ERR_UNSUPPORTED
    assert sp(o=FAKE) == hca.HCA_ERR_INVALID           # o aliases q
    assert sp(o=ctypes.c_void_p((1 << 20) + 4096)) == hca.HCA_ERR_INVALID  # o inside the 100000 key rows
    # the split decode: 1 sequence x 64 heads, top-2048 -> 32 slices of 64 positions
    wsd = lib.dsa_sparse_attn_decode_workspace_size(1, 64, 2048)
    assert wsd == 32 * 64 * 256 * 2 + 64 * 32 * 4
    assert lib.dsa_sparse_attn_decode_workspace_size(16, 64, 2048) == 16 * 16 * 64 * 256 * 2 + 16 * 64 * 16 * 4
    assert lib.dsa_sparse_attn_decode_workspace_size(1, 64, 100) == 0      # slices under 64 positions: no split
    assert lib.dsa_sparse_attn_decode_workspace_size(256, 64, 2048) == 0   # a full chip already
    big = ctypes.c_void_p(1 << 36)
    assert sp(k=2048, ws=big, wsb=wsd - 1) == hca.HCA_ERR_WORKSPACE
    assert sp(k=2048, ws=ctypes.c_void_p((1 << 36) + 8), wsb=wsd) == hca.HCA_ERR_INVALID  # misaligned
    assert sp(k=2048, ws=FAKE, wsb=wsd) == hca.HCA_ERR_INVALID             # workspace overlaps q


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16)
    w = torch.zeros(1, 128)
    with pytest.raises(ValueError):
        hca.hca_compress_kv(x, x, w, w, 128)


def test_hca_bwd_rejects_bad_arguments():
    lib = _lib()
    need = lib.hca_attn_bwd_workspace_size(0, 1, 300, 0, 4, 4, 4, 128, 64, 64)
    assert need >= 300 * 4 * 4
    assert lib.hca_attn_bwd_workspace_size(0, 0, 300, 0, 4, 4, 4, 128, 64, 64) == 0
    # bf16 / head_dim 512: D plus the compressed-entry partials; 32K queries, 256 entries, window 128:
    # entry tiles of 64 start at positions 255, 8447, 16639, 24831 -> 32 + 24 + 16 + 8 chunks of 32 query tiles
    big = lib.hca_attn_bwd_workspace_size(1, 1, 32768, 0, 256, 16, 16, 512, 128, 128)
    assert big == 32768 * 16 * 4 + 2 * 16 * (32 + 24 + 16 + 8) * 64 * 512 * 4
    g = [ctypes.c_void_p((1 << 34) + (i << 28)) for i in range(5)]   # distinct, non-overlapping gradient buffers
    sf = S(0, 128 * 4, 128)

    def call(**kw):
        return lib.hca_attn_bwd(kw.get("dt", 0), kw.get("q", FAKE), sf, FAKE, sf, FAKE, sf, FAKE, S(0, 128, 128),
                                FAKE, S(0, 128, 128), FAKE, sf, kw.get("lse", ctypes.c_void_p(1 << 33)), FAKE, sf,
                                kw.get("dq", g[0]), sf, kw.get("dk", g[1]), sf, g[2], sf, g[3], S(0, 128, 128), g[4],
                                S(0, 128, 128), 1, kw.get("sq", 300), 0, kw.get("skv", 300), kw.get("kvp", 0),
                                kw.get("nb", 4), 4, kw.get("hkv", 4), kw.get("d", 128), 64, kw.get("window", 64),
                                0.1, kw.get("ws", ctypes.c_void_p(1 << 40)), kw.get("wsb", need), None)
    assert call(dt=3) == hca.HCA_ERR_INVALID
    assert call(hkv=3) == hca.HCA_ERR_INVALID
    assert call(window=0) == hca.HCA_ERR_INVALID
    assert call(q=None) == hca.HCA_ERR_INVALID
    assert call(lse=None) == hca.HCA_ERR_INVALID
    assert call(d=516) == hca.HCA_ERR_UNSUPPORTED
    assert call(kvp=10) == hca.HCA_ERR_INVALID              # raw K/V start after query 0's window
    assert call(nb=2) == hca.HCA_ERR_INVALID                # last query (t = 299) needs floor(236 / 64) = 3 entries
    assert "compressed" in hca.hca_last_error()
    assert call(dq=FAKE) == hca.HCA_ERR_INVALID             # gradient aliases an input
    assert "overlap" in hca.hca_last_error()
    assert call(dk=g[0]) == hca.HCA_ERR_INVALID             # two gradients alias
    assert call(wsb=need - 1) == hca.HCA_ERR_WORKSPACE
    assert call(ws=None) == hca.HCA_ERR_WORKSPACE
    assert call(window=20000, sq=20000, skv=20000) == hca.HCA_ERR_UNSUPPORTED   # > 16384 keys per query


def test_compress_bwd_rejects_bad_arguments():
    lib = _lib()
    sf = S(0, 512, 512)

    def call(**kw):
        return lib.hca_compress_kv_bwd(kw.get("dt", 1), kw.get("k", FAKE), S(0, 512, 512), FAKE, S(0, 512, 512),
                                       ctypes.c_void_p(1 << 30), sf, ctypes.c_void_p(1 << 31), sf,
                                       kw.get("wk", FAKE), FAKE, kw.get("dk", ctypes.c_void_p(1 << 34)), sf,
                                       ctypes.c_void_p(1 << 35), sf, kw.get("dwk", ctypes.c_void_p(1 << 36)),
                                       ctypes.c_void_p(1 << 37), 1, 256, 1, kw.get("d", 512), kw.get("block", 128),
                                       None)
    assert call(dt=4) == hca.HCA_ERR_INVALID
    assert call(k=None) == hca.HCA_ERR_INVALID
    assert call(wk=None) == hca.HCA_ERR_INVALID
    assert call(dwk=None) == hca.HCA_ERR_INVALID
    assert call(block=0) == hca.HCA_ERR_INVALID
    assert call(d=510) == hca.HCA_ERR_UNSUPPORTED
    assert call(d=516) == hca.HCA_ERR_UNSUPPORTED
    assert call(dk=ctypes.c_void_p(1 << 35)) == hca.HCA_ERR_INVALID    # dk aliases dv
    assert call(dk=ctypes.c_void_p(1 << 30)) == hca.HCA_ERR_INVALID    # dk aliases dkc


def test_dsa_bwd_rejects_bad_arguments():
    lib = _lib()
    need = lib.dsa_sparse_attn_bwd_workspace_size(0, 1, 100, 8, 2, 64, 64, 16)
    assert need >= 100 * 8 * 4 + 100 * 16 * 4
    # the bf16 / 256-wide path keeps one chunk of position-ordered contribution rows (1 KB per entry here)
    assert lib.dsa_sparse_attn_bwd_workspace_size(1, 1, 300, 64, 1, 256, 256, 16) >= 300 * 16 * 1024
    # two buffer sets (chunks are pipelined), each at most 8 GiB of rows plus its index
    assert lib.dsa_sparse_attn_bwd_workspace_size(1, 1, 1 << 16, 64, 1, 256, 256, 2048) < (18 << 30)
    # one chunk only: one buffer set
    one = lib.dsa_sparse_attn_bwd_workspace_size(1, 1, 300, 64, 1, 256, 256, 16)
    assert one < 2 * 300 * 16 * 1024 + (1 << 20)
    assert lib.dsa_sparse_attn_bwd_workspace_size(7, 1, 100, 8, 2, 64, 64, 16) == 0
    sq = S(0, 8 * 64, 64)
    skv = S(0, 2 * 64, 64)

    def call(**kw):
        return lib.dsa_sparse_attn_bwd(kw.get("dt", 0), FAKE, sq, FAKE, skv, FAKE, skv,
                                       kw.get("idx", ctypes.c_void_p(1 << 33)), FAKE, sq, ctypes.c_void_p(1 << 32),
                                       FAKE, sq, kw.get("dq", ctypes.c_void_p(1 << 34)), sq,
                                       kw.get("dk", ctypes.c_void_p(1 << 35)), skv, ctypes.c_void_p(1 << 36), skv,
                                       1, 100, 8, kw.get("hkv", 2), kw.get("d", 64), 64, kw.get("k", 16), 0.125,
                                       kw.get("ws", ctypes.c_void_p(1 << 40)), kw.get("wsb", need), None)
    assert call(dt=2) == hca.HCA_ERR_INVALID
    assert call(hkv=3) == hca.HCA_ERR_INVALID
    assert call(idx=None) == hca.HCA_ERR_INVALID
    assert call(d=1024) == hca.HCA_ERR_UNSUPPORTED
    assert call(k=4097) == hca.HCA_ERR_UNSUPPORTED
    assert call(dq=FAKE) == hca.HCA_ERR_INVALID
    assert call(dk=ctypes.c_void_p(1 << 34)) == hca.HCA_ERR_INVALID
    assert call(wsb=need - 1) == hca.HCA_ERR_WORKSPACE


def test_attn_compress_bwd_rejects_bad_arguments():
    lib = _lib()
    need = lib.hca_attn_bwd_workspace_size(1, 1, 256, 0, 2, 2, 2, 512, 128, 128)
    sq = S(0, 2 * 512, 512)
    sc = S(0, 2 * 512, 512)
    g = [ctypes.c_void_p((1 << 34) + (i << 28)) for i in range(7)]

    def call(**kw):
        return lib.hca_attn_compress_bwd(1, FAKE, sq, FAKE, sq, FAKE, sq, FAKE, sc, FAKE, sc, FAKE, sq,
                                         ctypes.c_void_p(1 << 33), FAKE, sq, kw.get("wk", FAKE), FAKE, g[0], sq,
                                         g[1], sq, g[2], sq, g[3], sc, g[4], sc, kw.get("dwk", g[5]), g[6], 1,
                                         kw.get("s", 256), kw.get("nb", 2), 2, 2, 512, 128, 128, 0.04,
                                         ctypes.c_void_p(1 << 40), need, None)
    assert call(wk=None) == hca.HCA_ERR_INVALID
    assert call(dwk=None) == hca.HCA_ERR_INVALID
    assert call(nb=3) == hca.HCA_ERR_INVALID          # 3 blocks of 128 > 256 rows
    assert "n_blocks" in hca.hca_last_error()
    assert call(dwk=g[0]) == hca.HCA_ERR_INVALID      # dw_k inside dq
    assert call(s=0) == hca.HCA_ERR_INVALID


def test_csa_rejects_bad_arguments():
    lib = _lib()
    ws = lib.csa_index_topk_workspace_size(1, 4096, 1024, 256)
    assert ws >= 1024 * 4 and lib.csa_index_topk_workspace_size(1, 4096, 0, 256) == 0
    call = lambda **kw: lib.csa_index_topk(kw.get("q", FAKE), ctypes.c_void_p(1 << 33), ctypes.c_void_p(1 << 34),
                                           kw.get("idx", ctypes.c_void_p(1 << 36)), 1, 4096, kw.get("n", 1024),
                                           kw.get("block", 4), kw.get("hi", 4), 64, kw.get("k", 256),
                                           kw.get("ws", ctypes.c_void_p(1 << 40)), kw.get("wsb", ws), None)
    assert call(q=None) == hca.HCA_ERR_INVALID
    assert call(n=1023) == hca.HCA_ERR_INVALID           # position 4095 needs 1024 entries
    assert "entries" in hca.hca_last_error()
    assert call(block=0) == hca.HCA_ERR_INVALID
    assert call(hi=6) == hca.HCA_ERR_UNSUPPORTED
    assert call(k=5000) == hca.HCA_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == hca.HCA_ERR_WORKSPACE
    assert call(idx=FAKE) == hca.HCA_ERR_INVALID         # idx aliases q_idx
    sp = lambda **kw: lib.csa_sparse_attn_fwd(1, FAKE, S(0, 64 * 256, 256), ctypes.c_void_p(1 << 33),
                                              S(0, 256, 256), ctypes.c_void_p(1 << 34), S(0, 256, 256),
                                              kw.get("idx", ctypes.c_void_p(1 << 35)), kw.get("o", ctypes.c_void_p(1 << 36)),
                                              S(0, 64 * 256, 256), None, 1, 4096, kw.get("n", 1024), 64, 1, 256,
                                              256, 64, 0.0625, None)
    assert sp(idx=None) == hca.HCA_ERR_INVALID
    assert sp(n=0) == hca.HCA_ERR_INVALID
    assert sp(o=FAKE) == hca.HCA_ERR_INVALID             # o aliases q


def test_epilogue_rejects_bad_arguments():
    lib = _lib()
    so = S(0, 16 * 512, 512)
    sc = S(0, 2048, 2048)

    def call(**kw):
        return lib.attn_output_epilogue(kw.get("dt", 1), FAKE, so, ctypes.c_void_p(1 << 33), kw.get("sc", sc),
                                        ctypes.c_void_p(1 << 34), ctypes.c_void_p(1 << 35), ctypes.c_void_p(1 << 36),
                                        kw.get("y", ctypes.c_void_p(1 << 37)), so, kw.get("b", 1), 100,
                                        kw.get("h", 16), kw.get("dv", 512), kw.get("dc", 2048), kw.get("r", 4), None)
    assert call(dt=0) == hca.HCA_ERR_UNSUPPORTED
    assert call(h=12) == hca.HCA_ERR_UNSUPPORTED
    assert call(r=17) == hca.HCA_ERR_UNSUPPORTED
    assert call(dc=2000) == hca.HCA_ERR_UNSUPPORTED
    assert call(dv=40) == hca.HCA_ERR_UNSUPPORTED                  # not a multiple of 256 / h = 16
    assert call(h=8, dv=48) == hca.HCA_ERR_UNSUPPORTED             # not a multiple of 256 / h = 32
    assert call(r=0) == hca.HCA_ERR_INVALID
    assert call(y=FAKE) == hca.HCA_ERR_INVALID                     # y aliases o
    assert call(y=ctypes.c_void_p((1 << 37) + 8)) == hca.HCA_ERR_INVALID   # y misaligned


def test_noalloc_rejects_oversized_scratch_before_touching_the_gpu():
    """hca_attn_fwd_noalloc checks its fixed scratch size first: 512 decode
    sequences x 16 heads over 8320 keys need more than 16 MiB of partials."""
    lib = _lib()
    B, Hq, nb, W, d = 512, 16, 8192, 128, 512
    assert lib.hca_attn_fwd_workspace_size(B, 1, Hq, 1, d, nb, W) > hca.HCA_NOALLOC_SCRATCH_BYTES
    st = lib.hca_attn_fwd_noalloc(1, FAKE, S(Hq * d, Hq * d, d), FAKE, S(W * d, d, d), FAKE, S(W * d, d, d),
                                  FAKE, S(nb * d, d, d), FAKE, S(nb * d, d, d), ctypes.c_void_p(1 << 40),
                                  S(Hq * d, Hq * d, d), None, B, 1, 128 * nb + W - 1, W, 128 * nb, nb, Hq, 1, d,
                                  128, W, 0.04, None)
    assert st == hca.HCA_ERR_WORKSPACE
    assert "scratch" in hca.hca_last_error()
