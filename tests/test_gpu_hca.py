"""GPU parity of the HCA path (compression, prefill attention, decode attention)
against the float64 oracle on the same seeded inputs, called through the C-ABI."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BF16_TOL, F32_TOL, LSE_TOL, dev_bf16, dev_f32, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to_dev(inp, name):
    return dev_bf16(inp[name]) if inp["bf16"] else dev_f32(inp[name])


def _run_prefill(cfg, inp, compress_on_gpu=True):
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    torch.cuda.synchronize()
    return kc, vc, o, lse


def _oracle_prefill(cfg, inp, rows=None, heads=None):
    q, k, v = (f64(inp[n], inp["bf16"]) for n in ("q", "k", "v"))
    if heads is not None:
        q, k, v = q[:, :, heads], k[:, :, heads], v[:, :, heads]
        w = inp["w"][heads]
    else:
        w = inp["w"]
    kc, vc = oracle.compress_kv(k, w, cfg.block), oracle.compress_kv(v, w, cfg.block)
    o, lse = oracle.hca_attention(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale, rows=rows)
    return kc, vc, o, lse


# ------------------------------------------------------------------ compression

@pytest.mark.parametrize("dtype,d,block,S", [("bf16", 512, 128, 1000), ("f32", 128, 128, 2048),
                                             ("bf16", 256, 64, 333), ("f32", 64, 7, 100), ("bf16", 512, 1, 40)])
def test_compress_parity(dtype, d, block, S):
    cfg = synth.small_prefill("c2" if dtype == "bf16" else "c1", dtype=dtype, seqlen=S, h_q=3, h_kv=3,
                              head_dim=d, block=block, batch=2)
    _say("compress", cfg)
    inp = synth.make_prefill(cfg)
    k, v = _to_dev(inp, "k"), _to_dev(inp, "v")
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, block)
    torch.cuda.synchronize()
    rk = oracle.compress_kv(f64(inp["k"], inp["bf16"]), inp["w"], block)
    rv = oracle.compress_kv(f64(inp["v"], inp["bf16"]), inp["w"], block)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert kc.shape == rk.shape
    assert rel_err(host(kc), rk) < tol and rel_err(host(vc), rv) < tol


@pytest.mark.parametrize("dtype,H,d,block,S,B", [("bf16", 4, 512, 128, 1000, 2), ("bf16", 16, 512, 66, 500, 1),
                                                  ("f32", 8, 256, 128, 700, 1), ("f32", 4, 512, 64, 300, 1)])
def test_compress_all_heads_per_workgroup_parity(dtype, H, d, block, S, B):
    """Shapes whose heads fill whole waves (h * d / 16-byte pieces a multiple
    of 256) take the kernel with one workgroup per block covering every head;
    block 66 leaves a tail of rows after the 4-row batches."""
    cfg = synth.small_prefill("c2" if dtype == "bf16" else "c1", dtype=dtype, seqlen=S, h_q=H, h_kv=H,
                              head_dim=d, block=block, batch=B)
    _say("compress rows", cfg)
    inp = synth.make_prefill(cfg)
    k, v = _to_dev(inp, "k"), _to_dev(inp, "v")
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, block)
    torch.cuda.synchronize()
    rk = oracle.compress_kv(f64(inp["k"], inp["bf16"]), inp["w"], block)
    rv = oracle.compress_kv(f64(inp["v"], inp["bf16"]), inp["w"], block)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert kc.shape == rk.shape
    assert rel_err(host(kc), rk) < tol and rel_err(host(vc), rv) < tol


def test_compress_all_heads_one_hot_is_bit_exact_with_strided_heads():
    H = 4
    cfg = synth.small_prefill("c2", seqlen=384, h_q=H, h_kv=H)
    inp = synth.make_prefill(cfg)
    big = torch.zeros(1, 384, 2 * H + 1, 512, dtype=torch.bfloat16, device="cuda:0")
    big[:, :, 1:2 * H + 1:2] = dev_bf16(inp["k"])
    k = big[:, :, 1:2 * H + 1:2]                        # head stride 2 * 512
    w = torch.zeros(H, 128, device="cuda:0")
    for h in range(H):
        w[h, 31 * h + 5] = 1.0
    kc, vc = hca.hca_compress_kv(k, k, w, w, 128)
    torch.cuda.synchronize()
    kd = dev_bf16(inp["k"])
    ref = torch.stack([kd[0, 31 * h + 5::128, h] for h in range(H)], dim=1)[None]
    assert torch.equal(kc, ref) and torch.equal(vc, ref)


def test_compress_one_hot_is_bit_exact_and_strided_views_work():
    cfg = synth.small_prefill("c2", seqlen=640, h_q=2, h_kv=2)
    inp = synth.make_prefill(cfg)
    big = torch.zeros(1, 640, 5, 512, dtype=torch.bfloat16, device="cuda:0")
    big[:, :, 1:3] = dev_bf16(inp["k"])
    k = big[:, :, 1:3]                                  # non-contiguous head stride
    w = torch.zeros(2, 128, device="cuda:0")
    w[0, 17] = 1.0
    w[1, 127] = 1.0
    kc, vc = hca.hca_compress_kv(k, k, w, w, 128)
    torch.cuda.synchronize()
    ref = torch.stack([dev_bf16(inp["k"])[0, 17::128, 0], dev_bf16(inp["k"])[0, 127::128, 1]], dim=1)[None]
    assert torch.equal(kc, ref) and torch.equal(vc, ref)


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    # name, dtype, S, H, Hkv, d, block, W
    ("c1-full", "f32", 2048, 2, 2, 128, 128, 128),
    ("bf16-ragged", "bf16", 1000, 2, 2, 512, 128, 128),
    ("bf16-w200-b64", "bf16", 777, 2, 2, 512, 64, 200),
    ("bf16-gqa", "bf16", 600, 4, 2, 512, 128, 256),
    ("bf16-window-covers", "bf16", 300, 2, 2, 512, 128, 400),
    ("bf16-window1", "bf16", 400, 1, 1, 512, 32, 1),
    ("bf16-block1", "bf16", 150, 1, 1, 512, 1, 5),
    ("bf16-tiny", "bf16", 2, 1, 1, 512, 128, 128),
    ("f32-d64", "f32", 500, 2, 1, 64, 16, 40),
    # the fp32 MFMA kernel: ragged query tiles, grouped heads, degenerate windows
    ("f32-gqa-ragged", "f32", 333, 3, 1, 64, 8, 50),
    ("f32-window1", "f32", 130, 1, 1, 64, 4, 1),
    ("f32-block1", "f32", 97, 2, 2, 128, 1, 3),
    ("f32-window-covers", "f32", 70, 2, 2, 128, 128, 100),
    ("f32-tiny", "f32", 3, 1, 1, 128, 128, 128),
    # the bf16 MFMA kernel for narrower heads (64, 128, 256)
    ("bf16-d128-gqa", "bf16", 700, 4, 2, 128, 64, 100),
    ("bf16-d256", "bf16", 500, 2, 2, 256, 128, 128),
    ("bf16-d64-ragged", "bf16", 333, 3, 1, 64, 8, 50),
    ("bf16-d128-window1", "bf16", 130, 1, 1, 128, 4, 1),
    ("bf16-d256-block1", "bf16", 97, 2, 2, 256, 1, 3),
    ("bf16-d64-window-covers", "bf16", 70, 2, 2, 64, 128, 100),
    ("bf16-d128-tiny", "bf16", 3, 1, 1, 128, 128, 128),
]


@pytest.mark.parametrize("name,dtype,S,H,Hkv,d,block,W", PREFILL_CASES)
def test_prefill_parity(name, dtype, S, H, Hkv, d, block, W):
    base = "c1" if dtype == "f32" else "c2"
    cfg = synth.small_prefill(base, name=name, dtype=dtype, seqlen=S, h_q=H, h_kv=Hkv, head_dim=d, block=block,
                              window=W, std=1.0 if dtype == "f32" else 1.0 / math.sqrt(d))
    _say("prefill", cfg)
    inp = synth.make_prefill(cfg)
    kc, vc, o, lse = _run_prefill(cfg, inp)
    _, _, ro, rlse = _oracle_prefill(cfg, inp)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    err = rel_err(host(o), ro)
    _say(f"  rel err {err:.3e}")
    assert err < tol
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_prefill_bf16_narrow_heads_beyond_generic_key_limit():
    """bf16, head_dim 128, block 1: late queries see ~17000 keys, more than the
    one-query-per-workgroup kernel takes; the MFMA kernel has no key limit.
    Sampled rows (including both sides of 16384 visible keys) against the oracle."""
    cfg = synth.small_prefill("c2", name="long-d128", seqlen=17000, h_q=2, h_kv=1, head_dim=128, block=1,
                              window=4, std=1.0 / math.sqrt(128))
    _say("prefill", cfg)
    inp = synth.make_prefill(cfg)
    kc, vc, o, lse = _run_prefill(cfg, inp)
    rows = [0, 1, 3, 4, 5, 127, 128, 4095, 8191, 16386, 16387, 16388, 16999]
    _, _, ro, rlse = _oracle_prefill(cfg, inp, rows=rows)
    err = rel_err(host(o[:, rows]), ro)
    _say(f"  rel err {err:.3e} on {len(rows)} rows")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse[:, :, rows]) - rlse)) < LSE_TOL


def test_prefill_bf16_narrow_heads_strided_views_batch2():
    """bf16 head_dim 128, two sequences, grouped heads (8 on 2), with q, k, v
    and o as non-contiguous views (padded head and position strides): the
    kernel follows the strides the call passes."""
    cfg = synth.small_prefill("c2", name="strided-d128", seqlen=300, h_q=8, h_kv=2, head_dim=128, block=32,
                              window=50, batch=2, std=1.0 / math.sqrt(128))
    inp = synth.make_prefill(cfg)

    def padded(x):
        B, S, H, d = x.shape
        big = torch.full((B, S + 3, H + 1, d + 64), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        big[:, :S, :H, :d] = x
        return big[:, :S, :H, :d]

    q, k, v = (padded(_to_dev(inp, n)) for n in ("q", "k", "v"))
    assert not q.is_contiguous()
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o = padded(torch.zeros_like(_to_dev(inp, "q")))
    _, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale, o=o)
    torch.cuda.synchronize()
    _, _, ro, rlse = _oracle_prefill(cfg, inp)
    err = rel_err(host(o), ro)
    _say(f"  rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_prefill_bf16_narrow_heads_decode_row():
    """bf16 head_dim 256 decode (one query) runs the same MFMA kernel; it agrees
    with the prefill row of the same position."""
    cfg = synth.small_prefill("c2", name="dec-d256", seqlen=700, h_q=4, h_kv=2, head_dim=256, block=64,
                              window=100, std=1.0 / math.sqrt(256))
    inp = synth.make_prefill(cfg)
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    t = 650
    lo = t - cfg.window + 1
    od, lsed = hca.hca_attn_fwd(q[:, t:t + 1], k[:, lo:t + 1], v[:, lo:t + 1], kc, vc, window=cfg.window,
                                block=cfg.block, scale=cfg.scale, q_pos0=t, kv_pos0=lo)
    torch.cuda.synchronize()
    # same keys, different tile grouping of the online softmax: equal up to rounding
    assert rel_err(host(od[:, 0]), host(o[:, t])) < 1e-2
    assert np.max(np.abs(host(lsed[:, :, 0]) - host(lse[:, :, t]))) < 1e-4


def test_prefill_unit_variance_logits():
    """N(0,1) inputs at d=512 give logits of std ~1, a real softmax test."""
    cfg = synth.small_prefill("c2", name="n01", seqlen=900, h_q=2, h_kv=2, std=1.0, window=128)
    _say("prefill", cfg)
    inp = synth.make_prefill(cfg)
    # feed the oracle the GPU's bf16 cache so only the attention kernel is compared
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    torch.cuda.synchronize()
    ro, rlse = oracle.hca_attention(f64(inp["q"], True), f64(inp["k"], True), f64(inp["v"], True), host(kc),
                                    host(vc), window=cfg.window, block=cfg.block, scale=cfg.scale)
    assert rel_err(host(o), ro) < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_prefill_extreme_logits():
    """Logits with a spread of hundreds: later tiles exceed the first tile's
    maximum by far more than fp32 exp range allows for a fixed reference, so
    the kernel must fall back to its exact-maximum pass.  The oracle is plain
    max-subtracted softmax."""
    cfg = synth.small_prefill("c2", name="extreme", seqlen=640, h_q=2, h_kv=2, std=1.0, window=128)
    _say("prefill", cfg)
    inp = synth.make_prefill(cfg)
    # scale q by 64 (exact in bf16): logit std about 64
    q64 = synth.bf16_round_bits(synth.bf16_bits_to_f32(inp["q"]) * np.float32(64.0))
    q = dev_bf16(q64)
    k, v = dev_bf16(inp["k"]), dev_bf16(inp["v"])
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    torch.cuda.synchronize()
    ro, rlse = oracle.hca_attention(f64(q64, True), f64(inp["k"], True), f64(inp["v"], True), host(kc), host(vc),
                                    window=cfg.window, block=cfg.block, scale=cfg.scale)
    assert np.all(np.isfinite(host(o))) and np.all(np.isfinite(host(lse)))
    err = rel_err(host(o), ro)
    _say(f"  rel err {err:.3e}, lse range {rlse.min():.1f} .. {rlse.max():.1f}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_prefill_deterministic_and_writes_every_output():
    cfg = synth.small_prefill("c2", name="det", seqlen=700, h_q=2, h_kv=2, window=128)
    inp = synth.make_prefill(cfg)
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((1, 2, 700), float("nan"), device="cuda:0")
    hca.hca_attn_fwd(q, k, v, kc, vc, window=128, block=128, o=o1, lse=l1)
    o2, l2 = hca.hca_attn_fwd(q, k, v, kc, vc, window=128, block=128)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_chunked_prefill_matches_full_prefill():
    """Queries [400, 700) with raw K/V starting at the first needed window position."""
    cfg = synth.small_prefill("c2", name="chunk", seqlen=700, h_q=2, h_kv=2, window=128)
    inp = synth.make_prefill(cfg)
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o_full, l_full = hca.hca_attn_fwd(q, k, v, kc, vc, window=128, block=128)
    lo = 400 - 127
    o_part, l_part = hca.hca_attn_fwd(q[:, 400:], k[:, lo:], v[:, lo:], kc, vc, window=128, block=128,
                                      q_pos0=400, kv_pos0=lo)
    torch.cuda.synchronize()
    assert rel_err(host(o_part), host(o_full[:, 400:])) < 1e-2
    assert float((l_part - l_full[:, :, 400:]).abs().max()) < 1e-3


# ------------------------------------------------------------------ decode

DECODE_CASES = [
    # B, Hq, Hkv, n_blocks, W, q_pos (None -> newest token of the window after n_blocks blocks)
    (4, 16, 1, 300, 128, None),
    (3, 8, 1, 50, 128, None),          # fewer than 16 heads per KV head
    (2, 32, 2, 77, 64, None),          # two KV heads
    (2, 16, 1, 0, 100, 37),            # early token: no compressed entry yet
    (2, 16, 1, 5, 128, 700),           # window not aligned to a block end
]


@pytest.mark.parametrize("B,Hq,Hkv,nb,W,qpos", DECODE_CASES)
def test_decode_parity(B, Hq, Hkv, nb, W, qpos):
    cfg = synth.small_decode(batch=B, h_q=Hq, h_kv=Hkv, n_blocks=nb, window=W)
    _say("decode", cfg, qpos)
    inp = synth.make_decode(cfg)
    t = cfg.q_pos if qpos is None else qpos
    lo = max(0, t - W + 1)
    n_c = lo // cfg.block
    kw_len = t - lo + 1
    q = dev_bf16(inp["q"])
    kw, vw = dev_bf16(inp["kw"][:, :kw_len]), dev_bf16(inp["vw"][:, :kw_len])
    kc = dev_bf16(inp["kc"]) if nb else None
    vc = dev_bf16(inp["vc"]) if nb else None
    assert n_c <= nb
    o, lse = hca.hca_attn_fwd(q, kw, vw, kc, vc, window=W, block=cfg.block, scale=cfg.scale, q_pos0=t, kv_pos0=lo)
    torch.cuda.synchronize()
    z = np.zeros((B, 1, Hkv, 512))
    ro, rlse = oracle.hca_attention(f64(inp["q"], True), f64(inp["kw"][:, :kw_len], True),
                                    f64(inp["vw"][:, :kw_len], True),
                                    f64(inp["kc"], True) if nb else z, f64(inp["vc"], True) if nb else z,
                                    window=W, block=cfg.block, scale=cfg.scale, q_pos0=t, kv_pos0=lo)
    err = rel_err(host(o), ro)
    _say(f"  rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_decode_workspace_reuse_across_calls_and_shapes():
    """One workspace serves consecutive decode calls of different shapes
    (different chunk counts), each call fully overwriting what it uses."""
    shapes = [(4, 16, 1, 300, 128), (2, 32, 2, 77, 64), (3, 16, 1, 20, 128), (4, 16, 1, 300, 128)]
    cfgs = [synth.small_decode(batch=B, h_q=Hq, h_kv=Hkv, n_blocks=nb, window=W, seed=10 + i)
            for i, (B, Hq, Hkv, nb, W) in enumerate(shapes)]
    wsz = max(hca.hca_attn_fwd_workspace_size(c.batch, 1, c.h_q, c.h_kv, 512, c.n_blocks, c.window) for c in cfgs)
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda:0")
    for cfg in cfgs:
        _say("decode reuse", cfg)
        inp = synth.make_decode(cfg)
        q, kw, vw, kc, vc = (dev_bf16(inp[n]) for n in ("q", "kw", "vw", "kc", "vc"))
        o, lse = hca.hca_attn_fwd(q, kw, vw, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale,
                                  q_pos0=cfg.q_pos, kv_pos0=cfg.kv_pos0, workspace=ws)
        torch.cuda.synchronize()
        ro, rlse = oracle.hca_attention(*(f64(inp[n], True) for n in ("q", "kw", "vw", "kc", "vc")),
                                        window=cfg.window, block=cfg.block, scale=cfg.scale, q_pos0=cfg.q_pos,
                                        kv_pos0=cfg.kv_pos0)
        assert rel_err(host(o), ro) < BF16_TOL
        assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_decode_equals_prefill_row():
    cfg = synth.small_prefill("c2", name="dec-vs-pre", seqlen=1100, h_q=4, h_kv=1, window=128, std=1.0)
    inp = synth.make_prefill(cfg)
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=128, block=128)
    for t in (0, 127, 128, 700, 1099):
        lo = max(0, t - 127)
        od, ld = hca.hca_attn_fwd(q[:, t:t + 1], k[:, lo:t + 1], v[:, lo:t + 1], kc, vc, window=128, block=128,
                                  q_pos0=t, kv_pos0=lo)
        torch.cuda.synchronize()
        assert rel_err(host(od[:, 0]), host(o[:, t])) < 1e-2
        assert float((ld[..., 0] - lse[..., t]).abs().max()) < 1e-3


# ------------------------------------------------------------------ decode-time cache upkeep

APPEND_CASES = [
    # dtype, d, Hq, Hkv, window, ring
    ("bf16", 512, 16, 1, 128, 128),    # the decode configuration's shape, ring = window = block
    ("bf16", 512, 4, 2, 64, 160),      # ring larger than the block, window not a multiple of it
    ("f32", 128, 2, 2, 100, 128),      # fp32 caches (compressor and generic attention)
]


@pytest.mark.parametrize("dtype,d,Hq,Hkv,W,R", APPEND_CASES)
def test_append_streams_history(dtype, d, Hq, Hkv, W, R):
    """Positions 0..T-1 appended one at a time: the ring window equals the
    last rows exactly, every closed block equals hca_compress_kv over the whole
    history bit for bit (same kernel, same block) and the oracle within the
    compression tolerance, and decode attention read from the ring matches
    the oracle at several positions."""
    T = 3 * 128 + 45
    cfg = synth.small_prefill("c2" if dtype == "bf16" else "c1", name="append", dtype=dtype, seqlen=T, h_q=Hq,
                              h_kv=Hkv, head_dim=d, window=W, block=128, batch=2)
    _say("append", cfg, R)
    inp = synth.make_prefill(cfg)
    q, k, v = (_to_dev(inp, n) for n in ("q", "k", "v"))
    w = dev_f32(inp["w"])
    B, nb = cfg.batch, T // 128
    k_ring = torch.zeros((B, 2 * R, Hkv, d), dtype=k.dtype, device=k.device)
    v_ring = torch.zeros_like(k_ring)
    kc = torch.zeros((B, nb, Hkv, d), dtype=k.dtype, device=k.device)
    vc = torch.zeros_like(kc)
    rk = oracle.compress_kv(f64(inp["k"], inp["bf16"]), inp["w"], 128)
    rv = oracle.compress_kv(f64(inp["v"], inp["bf16"]), inp["w"], 128)
    checks = {0, 1, 63, 100, 127, 128, 129, 255, 256, 300, T - 1}
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for t in range(T):
        hca.hca_append_kv(k[:, t:t + 1], v[:, t:t + 1], k_ring, v_ring, t, 128, w, w, kc, vc)
        if t not in checks:
            continue
        torch.cuda.synchronize()
        lo = max(0, t - W + 1)
        s0, n = lo % R, t - lo + 1
        assert torch.equal(k_ring[:, s0:s0 + n], k[:, lo:t + 1]) and torch.equal(v_ring[:, s0:s0 + n], v[:, lo:t + 1])
        o, lse = hca.hca_attn_fwd(q[:, t:t + 1], k_ring[:, s0:s0 + n], v_ring[:, s0:s0 + n], kc, vc, window=W,
                                  block=128, scale=cfg.scale, q_pos0=t, kv_pos0=lo)
        torch.cuda.synchronize()
        ro, rlse = oracle.hca_attention(f64(inp["q"][:, t:t + 1], inp["bf16"]), f64(inp["k"][:, :t + 1], inp["bf16"]),
                                        f64(inp["v"][:, :t + 1], inp["bf16"]), rk, rv, window=W, block=128,
                                        scale=cfg.scale, q_pos0=t, kv_pos0=0)
        err = rel_err(host(o), ro)
        _say(f"  t={t} decode rel err {err:.3e}")
        assert err < tol
        assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL
    kc_full, vc_full = hca.hca_compress_kv(k, v, w, w, 128)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc_full) and torch.equal(vc, vc_full)
    assert rel_err(host(kc), rk) < tol and rel_err(host(vc), rv) < tol


# ------------------------------------------------------------------ full-size configurations, sampled

def _sample_rows(S, W, n=24, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, W - 1, W, W + 127, W + 128, S // 2, S - 129, S - 128, S - 1]
    return sorted(set(fixed) | set(rng.integers(0, S, n).tolist()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c2", "c3"])
def test_full_size_prefill_sampled(name):
    cfg = synth.CONFIGS[name]
    _say("full-size", cfg)
    inp = synth.make_prefill(cfg)
    kc, vc, o, lse = _run_prefill(cfg, inp)
    heads = [0, cfg.h_q // 2, cfg.h_q - 1]
    rows = _sample_rows(cfg.seqlen, cfg.window)
    # compression on the sampled heads, every block (convert only those heads)
    q, k, v = (f64(inp[n][:, :, heads], True) for n in ("q", "k", "v"))
    kch = oracle.compress_kv(k, inp["w"][heads], cfg.block)
    vch = oracle.compress_kv(v, inp["w"][heads], cfg.block)
    assert rel_err(host(kc[:, :, heads]), kch) < BF16_TOL
    assert rel_err(host(vc[:, :, heads]), vch) < BF16_TOL
    ro, rlse = oracle.hca_attention(q, k, v, kch, vch, window=cfg.window,
                                    block=cfg.block, scale=cfg.scale, rows=rows)
    got = host(o[:, rows][:, :, heads])
    err = rel_err(got, ro)
    _say(f"  rel err {err:.3e} on {len(rows)} rows x {len(heads)} heads")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse[:, heads][:, :, rows]) - rlse)) < LSE_TOL
    assert not torch.isnan(o).any()


@pytest.mark.timeout(600)
def test_full_size_decode_every_sequence():
    """c4 at full size: every one of the 64 sequences (16 heads each) against the oracle."""
    cfg = synth.CONFIGS["c4"]
    _say("full-size", cfg)
    inp = synth.make_decode(cfg)
    q, kc, vc, kw, vw = (dev_bf16(inp[n]) for n in ("q", "kc", "vc", "kw", "vw"))
    o, lse = hca.hca_attn_fwd(q, kw, vw, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale,
                              q_pos0=cfg.q_pos, kv_pos0=cfg.kv_pos0)
    torch.cuda.synchronize()
    _say(f"  checking all {cfg.batch} sequences")
    for b in range(cfg.batch):
        ro, rlse = oracle.hca_attention(f64(inp["q"][b:b + 1], True), f64(inp["kw"][b:b + 1], True),
                                        f64(inp["vw"][b:b + 1], True), f64(inp["kc"][b:b + 1], True),
                                        f64(inp["vc"][b:b + 1], True), window=cfg.window, block=cfg.block,
                                        scale=cfg.scale, q_pos0=cfg.q_pos, kv_pos0=cfg.kv_pos0)
        assert rel_err(host(o[b:b + 1]), ro) < BF16_TOL
        assert np.max(np.abs(host(lse[b:b + 1]) - rlse)) < LSE_TOL
