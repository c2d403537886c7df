"""hca_attn_fwd_noalloc (the entry point for callers that cannot allocate)
against hca_attn_fwd with a caller workspace, through the C-ABI: two calls in
a row on the library's fixed scratch array, the second smaller, each equal to
the workspace path and within the bf16 tolerance of the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BF16_TOL, LSE_TOL, dev_bf16, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _decode_case(B, Hq, Hkv, nb, W, seed):
    d, block = 512, 128
    std = float(1.0 / np.sqrt(d))
    q = synth.make_normal((B, 1, Hq, d), seed, std, bf16=True)
    kc = synth.make_normal((B, nb, Hkv, d), seed + 1, std, bf16=True)
    vc = synth.make_normal((B, nb, Hkv, d), seed + 2, std, bf16=True)
    kw = synth.make_normal((B, W, Hkv, d), seed + 3, std, bf16=True)
    vw = synth.make_normal((B, W, Hkv, d), seed + 4, std, bf16=True)
    kv_pos0 = block * nb
    return dict(q=q, kc=kc, vc=vc, kw=kw, vw=vw, kv_pos0=kv_pos0, q_pos=kv_pos0 + W - 1, W=W, block=block,
                scale=float(1.0 / np.sqrt(d)))


def _run_both(c):
    q, kc, vc, kw, vw = (dev_bf16(c[n]) for n in ("q", "kc", "vc", "kw", "vw"))
    kw_args = dict(window=c["W"], block=c["block"], scale=c["scale"], q_pos0=c["q_pos"], kv_pos0=c["kv_pos0"])
    o_ref, lse_ref = hca.hca_attn_fwd(q, kw, vw, kc, vc, **kw_args)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], 1), float("nan"), dtype=torch.float32, device=q.device)
    hca.hca_attn_fwd_noalloc(q, kw, vw, kc, vc, o, lse, **kw_args)
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref


def test_noalloc_decode_two_calls_second_smaller():
    cases = [("first", _decode_case(16, 16, 1, 2000, 128, 301)),     # 2128 keys, 16 heads on one KV head
             ("second, smaller", _decode_case(3, 8, 2, 300, 64, 311))]  # 364 keys, GQA 8 on 2
    for name, c in cases:
        B, _, Hq, _ = c["q"].shape
        Hkv, nb = c["kc"].shape[2], c["kc"].shape[1]
        need = hca.hca_attn_fwd_workspace_size(B, 1, Hq, Hkv, 512, nb, c["W"])
        _say(f"noalloc decode {name}: B={B} Hq={Hq} Hkv={Hkv} keys={nb + c['W']} scratch={need}")
        assert 0 < need <= hca.HCA_NOALLOC_SCRATCH_BYTES
        o, lse, o_ref, lse_ref = _run_both(c)
        # the same kernels on the same inputs: identical bits
        assert torch.equal(o, o_ref)
        assert torch.equal(lse, lse_ref)
        ro, rlse = oracle.hca_attention(f64(c["q"], True), f64(c["kw"], True), f64(c["vw"], True),
                                        f64(c["kc"], True), f64(c["vc"], True), window=c["W"], block=c["block"],
                                        scale=c["scale"], q_pos0=c["q_pos"], kv_pos0=c["kv_pos0"])
        err = rel_err(host(o), ro)
        _say(f"  rel err vs oracle {err:.2e}")
        assert err < BF16_TOL
        assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_noalloc_prefill_needs_no_scratch():
    """seqlen_q > 1 runs the prefill kernel, which uses no scratch."""
    cfg = synth.small_prefill(seqlen=600, h_q=2, h_kv=2, window=128)
    inp = synth.make_prefill(cfg)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    w = torch.from_numpy(inp["w"]).to("cuda:0")
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o_ref, lse_ref = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    hca.hca_attn_fwd_noalloc(q, k, v, kc, vc, o, lse, window=cfg.window, block=cfg.block, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """512 sequences x 16 heads over 8320 keys need 16.8 MB of partials: a clear
    HCA_ERR_WORKSPACE, nothing launched, o untouched."""
    B, Hq, nb, W, d = 512, 16, 8192, 128, 512
    assert hca.hca_attn_fwd_workspace_size(B, 1, Hq, 1, d, nb, W) > hca.HCA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda:0")
    kw = torch.zeros((B, W, 1, d), dtype=torch.bfloat16, device="cuda:0")
    kc = torch.zeros((B, nb, 1, d), dtype=torch.bfloat16, device="cuda:0")
    o = torch.full_like(q, 7.0)
    with pytest.raises(hca.HcaError) as e:
        hca.hca_attn_fwd_noalloc(q, kw, kw, kc, kc, o, None, window=W, block=128, q_pos0=128 * nb + W - 1,
                                 kv_pos0=128 * nb)
    assert e.value.status == hca.HCA_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (o == 7.0).all()
