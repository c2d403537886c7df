"""GPU parity of the attention-output epilogue (low-rank output gate + VHA
cross-head mixing) against the float64 oracle on the same seeded bf16 inputs,
through the C-ABI."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BF16_TOL, dev_bf16, dev_f32, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(B, S, H, dv, dc, r, seed):
    o = synth.make_normal((B, S, H, dv), seed, bf16=True)
    c = synth.make_normal((B, S, dc), seed + 1, bf16=True)
    # projection scaled so the gate pre-activations are O(1)
    w = synth.make_normal((H * dv, dc), seed + 2, std=1.0 / np.sqrt(dc), bf16=True)
    u = synth.make_normal((H, r), seed + 3, std=0.5)
    v = synth.make_normal((r, H), seed + 4, std=0.5)
    return o, c, w, u, v


@pytest.mark.parametrize("B,S,H,dv,dc,r", [(1, 300, 16, 512, 2048, 4), (2, 130, 8, 64, 256, 3),
                                           (1, 77, 64, 256, 512, 16), (1, 64, 32, 128, 64, 8)])
def test_epilogue_parity(B, S, H, dv, dc, r):
    _say("epilogue", B, S, H, dv, dc, r)
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 101)
    y = hca.attn_output_epilogue(dev_bf16(o), dev_bf16(c), dev_bf16(w), dev_f32(u), dev_f32(v))
    torch.cuda.synchronize()
    ref = oracle.gated_vha_output(f64(o, True), f64(c, True), f64(w, True), u, v)
    err = rel_err(host(y), ref)
    _say(f"  rel err {err:.2e}")
    assert err < BF16_TOL


def test_epilogue_special_cases():
    """A zero projection gates everything by 1/2; zero U leaves only the skip."""
    B, S, H, dv, dc, r = 1, 150, 16, 64, 128, 4
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 202)
    od, cd = dev_bf16(o), dev_bf16(c)
    y0 = hca.attn_output_epilogue(od, cd, torch.zeros(H * dv, dc, dtype=torch.bfloat16, device="cuda:0"),
                                  dev_f32(u), dev_f32(v))
    y1 = hca.attn_output_epilogue(od, cd, dev_bf16(w), torch.zeros(H, r, device="cuda:0"), dev_f32(v))
    torch.cuda.synchronize()
    ref0 = 0.5 * oracle.vha_mix(f64(o, True), u, v)
    assert rel_err(host(y0), ref0) < BF16_TOL
    ref1 = oracle.gate_values(f64(c, True), f64(w, True), H, dv) * f64(o, True)
    assert rel_err(host(y1), ref1) < BF16_TOL


def test_epilogue_strided_output_of_attention():
    """o may be a head-strided view (e.g. one half of a fused tensor)."""
    B, S, H, dv, dc, r = 1, 140, 16, 128, 256, 4
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 303)
    big = torch.zeros(B, S, 2 * H, dv, dtype=torch.bfloat16, device="cuda:0")
    big[:, :, H:] = dev_bf16(o)
    y = hca.attn_output_epilogue(big[:, :, H:], dev_bf16(c), dev_bf16(w), dev_f32(u), dev_f32(v))
    torch.cuda.synchronize()
    ref = oracle.gated_vha_output(f64(o, True), f64(c, True), f64(w, True), u, v)
    assert rel_err(host(y), ref) < BF16_TOL


def test_epilogue_head_strided_output():
    """y whose heads are not contiguous within a token (head stride 2 d_v):
    only the addressed half is written."""
    B, S, H, dv, dc, r = 1, 300, 16, 256, 512, 4
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 505)
    big = torch.zeros(B, S, H, 2 * dv, dtype=torch.bfloat16, device="cuda:0")
    y = hca.attn_output_epilogue(dev_bf16(o), dev_bf16(c), dev_bf16(w), dev_f32(u), dev_f32(v), y=big[..., :dv])
    torch.cuda.synchronize()
    ref = oracle.gated_vha_output(f64(o, True), f64(c, True), f64(w, True), u, v)
    assert rel_err(host(y), ref) < BF16_TOL
    assert (host(big[..., dv:]) == 0).all()


def test_epilogue_batch_strided_latent_and_output():
    """Several sequences whose latent and output rows are not token-contiguous
    across the batch (each sequence padded to a longer buffer), with a token
    count that is not a multiple of the 256-token tile."""
    B, S, H, dv, dc, r = 3, 200, 16, 128, 256, 4
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 606)
    cbig = torch.zeros(B, S + 37, dc, dtype=torch.bfloat16, device="cuda:0")
    cbig[:, :S] = dev_bf16(c)
    ybig = torch.zeros(B, S + 11, H, dv, dtype=torch.bfloat16, device="cuda:0")
    y = hca.attn_output_epilogue(dev_bf16(o), cbig[:, :S], dev_bf16(w), dev_f32(u), dev_f32(v), y=ybig[:, :S])
    torch.cuda.synchronize()
    ref = oracle.gated_vha_output(f64(o, True), f64(c, True), f64(w, True), u, v)
    assert rel_err(host(y), ref) < BF16_TOL
    assert (host(ybig[:, S:]) == 0).all()


@pytest.mark.timeout(600)
def test_full_size_epilogue_sampled():
    """The epilogue at the 32768-token HCA shape (16 heads x 512, latent 2048,
    rank 4): sampled tokens against the oracle."""
    B, S, H, dv, dc, r = 1, 32768, 16, 512, 2048, 4
    o, c, w, u, v = _inputs(B, S, H, dv, dc, r, 404)
    y = hca.attn_output_epilogue(dev_bf16(o), dev_bf16(c), dev_bf16(w), dev_f32(u), dev_f32(v))
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 127, 128, 4095, 16384, S - 1]) | set(np.random.default_rng(6).integers(0, S, 9).tolist()))
    sel = torch.tensor(rows, device=y.device)
    got = host(y.index_select(1, sel))
    ref = oracle.gated_vha_output(f64(o[:, rows], True), f64(c[:, rows], True), f64(w, True), u, v)
    assert rel_err(got, ref) < BF16_TOL
