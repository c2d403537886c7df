"""GPU parity of the backward path -- HCA attention, the block compressor and
DSA sparse attention -- against the float64 oracle gradients on the same seeded
inputs, called through the C-ABI.

fp32 cases feed the kernels the oracle's own forward (o, lse rounded to fp32),
so they test the backward arithmetic alone at the fp32 tolerance.  bf16 cases
chain the library's forward and backward and compare with the oracle's
gradients of the exact (fp64) forward at the bf16 tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BF16_TOL, F32_TOL, dev_bf16, dev_f32, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x, bf16):
    return dev_bf16(x) if bf16 else dev_f32(x)


def _softmax_w(h, block, seed):
    z = synth.make_normal((h, block), seed).astype(np.float64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _check(name, got, ref, tol):
    err = rel_err(host(got), ref)
    _say(f"  {name}: rel err {err:.2e} (tol {tol:.0e})")
    assert err < tol, name


# ------------------------------------------------------------------ HCA attention

@pytest.mark.parametrize("B,Sq,Skv,q_pos0,kv_pos0,Hq,Hkv,d,block,window,nb", [
    (2, 300, 300, 0, 0, 4, 2, 64, 64, 48, 4),         # prefill, GQA, ragged tail, block > window
    (1, 130, 190, 400, 340, 2, 1, 128, 32, 61, 15),   # a chunk mid-sequence, raw K/V starting before it
    (1, 1, 40, 999, 960, 8, 8, 256, 128, 40, 7),      # one decode query
    (1, 70, 70, 0, 0, 2, 2, 512, 16, 200, 0),         # window covers everything: no compressed entry
])
def test_hca_attn_bwd_f32(B, Sq, Skv, q_pos0, kv_pos0, Hq, Hkv, d, block, window, nb):
    _say("hca bwd f32", B, Sq, Skv, q_pos0, kv_pos0, Hq, Hkv, d, block, window, nb)
    q = synth.make_normal((B, Sq, Hq, d), 11)
    k = synth.make_normal((B, Skv, Hkv, d), 12)
    v = synth.make_normal((B, Skv, Hkv, d), 13)
    kc = synth.make_normal((B, nb, Hkv, d), 14)
    vc = synth.make_normal((B, nb, Hkv, d), 15)
    dout = synth.make_normal((B, Sq, Hq, d), 16)
    scale = float(1.0 / np.sqrt(d))
    kw = dict(window=window, block=block, scale=scale, q_pos0=q_pos0, kv_pos0=kv_pos0)
    args64 = [x.astype(np.float64) for x in (q, k, v, kc, vc)]
    o, lse = oracle.hca_attention(*args64, **kw)
    ref = oracle.hca_attention_bwd(*args64, dout.astype(np.float64), **kw)
    dkc_dev = dev_f32(kc) if nb else None
    dvc_dev = dev_f32(vc) if nb else None
    got = hca.hca_attn_bwd(dev_f32(q), dev_f32(k), dev_f32(v), dkc_dev, dvc_dev, dev_f32(o), dev_f32(lse),
                           dev_f32(dout), **kw)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv", "dkc", "dvc"), got, ref):
        if r.size == 0:
            assert g is None
            continue
        _check(name, g, r, F32_TOL)


def test_hca_attn_bwd_unseen_rows_are_zero_and_strided_views_work():
    """Raw rows past the last query and compressed entries no query reaches
    get zero gradients; inputs and gradients may be head-strided views."""
    B, S, H, d, block, window, nb = 1, 200, 2, 64, 32, 40, 8
    q = synth.make_normal((B, S, H, d), 21)
    kv = synth.make_normal((B, S + 30, 2 * H, d), 22)       # K and V interleaved per head, 30 extra rows
    kc = synth.make_normal((B, nb, H, d), 23)
    dout = synth.make_normal((B, S, H, d), 24)
    k, v = kv[:, :, :H], kv[:, :, H:]
    kw = dict(window=window, block=block, scale=0.125)
    o, lse = oracle.hca_attention(q, k, v, kc, kc, **kw)
    ref = oracle.hca_attention_bwd(q, k, v, kc, kc, dout, **kw)
    kv_dev = dev_f32(kv)
    got = hca.hca_attn_bwd(dev_f32(q), kv_dev[:, :, :H], kv_dev[:, :, H:], dev_f32(kc), dev_f32(kc), dev_f32(o),
                           dev_f32(lse), dev_f32(dout), **kw)
    torch.cuda.synchronize()
    dq, dk, dv, dkc, dvc = (host(x) for x in got)
    assert (dk[:, S:] == 0).all() and (dv[:, S:] == 0).all()
    # last query t = 199: lo = 160 -> entries 0..4 seen; 5..7 never
    assert (dkc[:, 5:] == 0).all() and (dvc[:, 5:] == 0).all()
    for name, g, r in zip(("dq", "dk", "dv", "dkc", "dvc"), (dq, dk, dv, dkc, dvc), ref):
        err = rel_err(g, r)
        _say(f"  {name}: {err:.2e}")
        assert err < F32_TOL, name


@pytest.mark.parametrize("S,H,d,block,window", [(600, 2, 512, 128, 128), (333, 3, 256, 64, 100)])
def test_hca_training_step_bf16_chain(S, H, d, block, window):
    """bf16 forward (compression + attention) then backward (attention, then the
    compressor into the raw K/V gradients and the weights) against the oracle's
    gradients of the whole chain."""
    _say("hca chain bf16", S, H, d, block, window)
    B = 1
    q = synth.make_normal((B, S, H, d), 31, bf16=True)
    k = synth.make_normal((B, S, H, d), 32, bf16=True)
    v = synth.make_normal((B, S, H, d), 33, bf16=True)
    dout = synth.make_normal((B, S, H, d), 34, bf16=True)
    wk, wv = _softmax_w(H, block, 35), _softmax_w(H, block, 36)
    scale = float(1.0 / np.sqrt(d))
    kw = dict(window=window, block=block, scale=scale)
    # library: forward then backward
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, dout))
    wkd, wvd = dev_f32(wk), dev_f32(wv)
    kcd, vcd = hca.hca_compress_kv(kd, vd, wkd, wvd, block)
    o, lse = hca.hca_attn_fwd(qd, kd, vd, kcd, vcd, **kw)
    dq, dk, dv, dkc, dvc = hca.hca_attn_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, **kw)
    dk, dv, dwk, dwv = hca.hca_compress_kv_bwd(kd, vd, dkc, dvc, wkd, wvd, block, dk=dk, dv=dv)
    torch.cuda.synchronize()
    # oracle
    q64, k64, v64, g64 = (f64(x, True) for x in (q, k, v, dout))
    kc64, vc64 = oracle.compress_kv(k64, wk, block), oracle.compress_kv(v64, wv, block)
    rq, rk, rv, rkc, rvc = oracle.hca_attention_bwd(q64, k64, v64, kc64, vc64, g64, **kw)
    ck, rwk = oracle.compress_kv_bwd(k64, wk, rkc, block)
    cv, rwv = oracle.compress_kv_bwd(v64, wv, rvc, block)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk + ck), ("dv", dv, rv + cv), ("dkc", dkc, rkc),
                       ("dvc", dvc, rvc), ("dw_k", dwk, rwk), ("dw_v", dwv, rwv)):
        _check(name, g, r, BF16_TOL)


@pytest.mark.parametrize("B,Sq,Skv,q_pos0,kv_pos0,Hq,Hkv,block,window,nb", [
    (1, 3000, 3000, 0, 0, 2, 1, 16, 40, 187),    # GQA; compressed tiles cut into several chunks of queries
    (2, 1200, 1200, 0, 0, 2, 2, 32, 64, 36),     # two sequences: batch strides, per-sequence item ranges
    (1, 1100, 1100, 0, 0, 1, 1, 128, 128, 7),    # the c2 block / window at a small length, ragged tiles
    (1, 130, 190, 400, 340, 2, 2, 32, 61, 15),   # a chunk mid-sequence, raw K/V starting before it
    (2, 1, 40, 999, 960, 4, 1, 128, 40, 7),      # one decode query per sequence
    (1, 70, 70, 0, 0, 2, 2, 16, 200, 0),         # window covers everything: no compressed entry
])
def test_hca_attn_bwd_bf16_512(B, Sq, Skv, q_pos0, kv_pos0, Hq, Hkv, block, window, nb):
    """The MFMA path (bf16, head_dim 512): the library's forward, then its
    backward, against the oracle's gradients on the same bf16 inputs."""
    _say("hca bwd bf16 d512", B, Sq, Skv, q_pos0, kv_pos0, Hq, Hkv, block, window, nb)
    d = 512
    q = synth.make_normal((B, Sq, Hq, d), 81, bf16=True)
    k = synth.make_normal((B, Skv, Hkv, d), 82, bf16=True)
    v = synth.make_normal((B, Skv, Hkv, d), 83, bf16=True)
    kc = synth.make_normal((B, nb, Hkv, d), 84, bf16=True)
    vc = synth.make_normal((B, nb, Hkv, d), 85, bf16=True)
    dout = synth.make_normal((B, Sq, Hq, d), 86, bf16=True)
    scale = float(1.0 / np.sqrt(d))
    kw = dict(window=window, block=block, scale=scale, q_pos0=q_pos0, kv_pos0=kv_pos0)
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, dout))
    kcd = dev_bf16(kc) if nb else None
    vcd = dev_bf16(vc) if nb else None
    o, lse = hca.hca_attn_fwd(qd, kd, vd, kcd, vcd, **kw)
    got = hca.hca_attn_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, **kw)
    torch.cuda.synchronize()
    ref = oracle.hca_attention_bwd(*(f64(x, True) for x in (q, k, v, kc, vc, dout)), **kw)
    for name, g, r in zip(("dq", "dk", "dv", "dkc", "dvc"), got, ref):
        if r.size == 0:
            assert g is None
            continue
        _check(name, g, r, BF16_TOL)


@pytest.mark.parametrize("dtype,B,S,H,d,block,window", [("bf16", 1, 1100, 2, 512, 128, 128),
                                                        ("bf16", 2, 700, 1, 512, 64, 100),
                                                        ("f32", 2, 300, 2, 64, 32, 40)])
def test_hca_attn_compress_bwd(dtype, B, S, H, d, block, window):
    """The fused layer backward (compressor share added inside the key-tile
    kernel on the MFMA path) against the oracle's chain, and against the
    two-call path (hca_attn_bwd then hca_compress_kv_bwd).  S is not a whole
    number of blocks, so the rows past the last block take the window part
    only."""
    _say("attn+compress bwd", dtype, B, S, H, d, block, window)
    bf = dtype == "bf16"
    q = synth.make_normal((B, S, H, d), 91, bf16=bf)
    k = synth.make_normal((B, S, H, d), 92, bf16=bf)
    v = synth.make_normal((B, S, H, d), 93, bf16=bf)
    dout = synth.make_normal((B, S, H, d), 94, bf16=bf)
    wk, wv = _softmax_w(H, block, 95), _softmax_w(H, block, 96)
    scale = float(1.0 / np.sqrt(d))
    kw = dict(window=window, block=block, scale=scale)
    qd, kd, vd, gd = (_dev(x, bf) for x in (q, k, v, dout))
    wkd, wvd = dev_f32(wk), dev_f32(wv)
    kcd, vcd = hca.hca_compress_kv(kd, vd, wkd, wvd, block)
    o, lse = hca.hca_attn_fwd(qd, kd, vd, kcd, vcd, **kw)
    fused = hca.hca_attn_compress_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, wkd, wvd, **kw)
    two = list(hca.hca_attn_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, **kw))
    dk2, dv2, dwk2, dwv2 = hca.hca_compress_kv_bwd(kd, vd, two[3], two[4], wkd, wvd, block, dk=two[1], dv=two[2])
    torch.cuda.synchronize()
    q64, k64, v64, g64 = (f64(x, bf) for x in (q, k, v, dout))
    kc64, vc64 = oracle.compress_kv(k64, wk, block), oracle.compress_kv(v64, wv, block)
    rq, rk, rv, rkc, rvc = oracle.hca_attention_bwd(q64, k64, v64, kc64, vc64, g64, **kw)
    ck, rwk = oracle.compress_kv_bwd(k64, wk, rkc, block)
    cv, rwv = oracle.compress_kv_bwd(v64, wv, rvc, block)
    tol = BF16_TOL if bf else F32_TOL
    ref = (rq, rk + ck, rv + cv, rkc, rvc, rwk, rwv)
    for name, g, r in zip(("dq", "dk", "dv", "dkc", "dvc", "dw_k", "dw_v"), fused, ref):
        _check(name, g, r, tol)
    # same arithmetic as the two-call path up to fp32 rounding of the final add
    for name, a_, b_ in (("dq", fused[0], two[0]), ("dk", fused[1], dk2), ("dv", fused[2], dv2),
                         ("dw_k", fused[5], dwk2), ("dw_v", fused[6], dwv2)):
        err = rel_err(host(a_), host(b_))
        _say(f"  fused vs two-call {name}: {err:.2e}")
        assert err < 1e-5, name


# ------------------------------------------------------------------ compressor

@pytest.mark.parametrize("dtype,S,H,d,block", [("f32", 100, 2, 64, 7), ("bf16", 1000, 3, 512, 128),
                                               ("f32", 256, 1, 128, 1), ("bf16", 50, 2, 256, 64)])
def test_compress_kv_bwd(dtype, S, H, d, block):
    """dk/dv accumulate onto what they held; rows past the last whole block keep it."""
    _say("compress bwd", dtype, S, H, d, block)
    bf = dtype == "bf16"
    B, nb = 2, S // block
    k = synth.make_normal((B, S, H, d), 41, bf16=bf)
    v = synth.make_normal((B, S, H, d), 42, bf16=bf)
    dkc = synth.make_normal((B, nb, H, d), 43)
    dvc = synth.make_normal((B, nb, H, d), 44)
    base_k = synth.make_normal((B, S, H, d), 45)
    base_v = synth.make_normal((B, S, H, d), 46)
    wk, wv = _softmax_w(H, block, 47), _softmax_w(H, block, 48)
    dk, dv, dwk, dwv = hca.hca_compress_kv_bwd(_dev(k, bf), _dev(v, bf), dev_f32(dkc), dev_f32(dvc), dev_f32(wk),
                                               dev_f32(wv), block, dk=dev_f32(base_k), dv=dev_f32(base_v))
    torch.cuda.synchronize()
    rk, rwk = oracle.compress_kv_bwd(f64(k, bf), wk, dkc, block)
    rv, rwv = oracle.compress_kv_bwd(f64(v, bf), wv, dvc, block)
    hk, hv = host(dk), host(dv)
    assert (hk[:, nb * block:] == base_k[:, nb * block:]).all()
    for name, g, r in (("dk", hk, rk + base_k), ("dv", hv, rv + base_v), ("dw_k", host(dwk), rwk),
                       ("dw_v", host(dwv), rwv)):
        err = rel_err(g, r)
        _say(f"  {name}: {err:.2e}")
        assert err < F32_TOL, name      # fp32 arithmetic on exact (bf16-representable) inputs


# ------------------------------------------------------------------ DSA sparse attention

def _oracle_dsa_fwd(q, k, v, idx, scale):
    """Oracle forward per KV head (the oracle's sparse_attention reads one KV head)."""
    B, S, Hq, _ = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    o = np.zeros((B, S, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, S))
    for g in range(Hkv):
        hs = slice(g * group, (g + 1) * group)
        og, lg = oracle.sparse_attention(q[:, :, hs], k[:, :, g:g + 1], v[:, :, g:g + 1], idx, scale)
        o[:, :, hs], lse[:, hs] = og, lg
    return o, lse


@pytest.mark.parametrize("B,S,Hq,Hkv,dqk,dv,topk,n_valid,dup", [
    (2, 200, 4, 2, 64, 32, 24, 20, 0),       # GQA, -1 padding after 20 entries, d_v != d_qk
    (1, 150, 6, 1, 256, 256, 40, None, 3),   # duplicates in every row with >= 2 entries
    (1, 97, 2, 2, 128, 64, 128, None, 0),    # topk > S: every row lists its whole causal prefix
])
def test_dsa_sparse_attn_bwd_f32(B, S, Hq, Hkv, dqk, dv, topk, n_valid, dup):
    _say("dsa bwd f32", B, S, Hq, Hkv, dqk, dv, topk, n_valid, dup)
    q = synth.make_normal((B, S, Hq, dqk), 51).astype(np.float64)
    k = synth.make_normal((B, S, Hkv, dqk), 52).astype(np.float64)
    v = synth.make_normal((B, S, Hkv, dv), 53).astype(np.float64)
    dout = synth.make_normal((B, S, Hq, dv), 54).astype(np.float64)
    idx = synth.make_index_lists(B, S, topk, seed=55, n_valid=n_valid, dup_per_row=dup)
    scale = float(1.0 / np.sqrt(dqk))
    o, lse = _oracle_dsa_fwd(q, k, v, idx, scale)
    rq, rk, rv = oracle.sparse_attention_bwd(q, k, v, idx, scale, dout)
    got = hca.dsa_sparse_attn_bwd(dev_f32(q), dev_f32(k), dev_f32(v), torch.from_numpy(idx).cuda(), dev_f32(o),
                                  dev_f32(lse), dev_f32(dout), scale=scale)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        _check(name, g, r, F32_TOL)


def test_dsa_bwd_skips_empty_and_out_of_range_entries():
    """A row whose list holds no valid entry (forward: o = 0, lse = -inf) gets
    dq = 0 and adds nothing to dk/dv, whatever its dout; entries at or past
    seqlen are skipped.  The expected values are the oracle's with that row's
    dout set to zero (every gradient is linear in dout)."""
    B, S, Hq, d, topk = 1, 80, 4, 64, 16
    q = synth.make_normal((B, S, Hq, d), 61).astype(np.float64)
    k = synth.make_normal((B, S, 1, d), 62).astype(np.float64)
    v = synth.make_normal((B, S, 1, d), 63).astype(np.float64)
    dout = synth.make_normal((B, S, Hq, d), 64).astype(np.float64)
    idx = synth.make_index_lists(B, S, topk, seed=65)
    scale = 0.125
    o, lse = _oracle_dsa_fwd(q, k, v, idx, scale)
    dz = dout.copy()
    dz[0, 30] = 0.0
    rq, rk, rv = oracle.sparse_attention_bwd(q, k, v, idx, scale, dz)
    bad = idx.copy()
    bad[0, 30] = -1                      # empty row
    o[0, 30], lse[0, :, 30] = 0.0, -np.inf
    bad[0, 5, 10] = S + 7                # row 5 lists 6 valid entries then -1s: one padding slot out of range
    got = hca.dsa_sparse_attn_bwd(dev_f32(q), dev_f32(k), dev_f32(v), torch.from_numpy(bad).cuda(), dev_f32(o),
                                  dev_f32(lse), dev_f32(dout), scale=scale)
    torch.cuda.synchronize()
    dq, dk, dv = (host(x) for x in got)
    assert (dq[0, 30] == 0).all()
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = rel_err(g, r)
        _say(f"  {name}: {err:.2e}")
        assert err < F32_TOL, name


@pytest.mark.parametrize("S,topk", [(256, 64), (300, 256)])
def test_dsa_training_step_bf16_chain(S, topk):
    """bf16 DSA forward (64 query heads on one KV head, d 256) then backward,
    against the oracle's gradients."""
    _say("dsa chain bf16", S, topk)
    B, Hq, d = 1, 64, 256
    q = synth.make_normal((B, S, Hq, d), 71, bf16=True)
    k = synth.make_normal((B, S, 1, d), 72, bf16=True)
    v = synth.make_normal((B, S, 1, d), 73, bf16=True)
    dout = synth.make_normal((B, S, Hq, d), 74, bf16=True)
    idx = synth.make_index_lists(B, S, topk, seed=75)
    scale = float(1.0 / np.sqrt(d))
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, dout))
    idd = torch.from_numpy(idx).cuda()
    o, lse = hca.dsa_sparse_attn_fwd(qd, kd, vd, idd, scale=scale)
    dq, dk, dv = hca.dsa_sparse_attn_bwd(qd, kd, vd, idd, o, lse, gd, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.sparse_attention_bwd(f64(q, True), f64(k, True), f64(v, True), idx, scale, f64(dout, True))
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check(name, g, r, BF16_TOL)


def _dsa_bwd_bf16_case(B, S, Hq, Hkv, idx, seed, empty_rows=()):
    """bf16 inputs, the oracle's forward (o rounded to bf16, lse fp32) as the
    forward outputs, the library's backward against the oracle's gradients.
    Entries at or past S are skipped (the oracle sees -1 there).  Rows in
    empty_rows reach the library as all -1 with the empty row's forward
    (o = 0, lse = -inf); the oracle keeps their lists but gets zero dout for
    them, which gives the same gradients (every gradient is linear in dout)."""
    d = 256
    q = synth.make_normal((B, S, Hq, d), seed, bf16=True)
    k = synth.make_normal((B, S, Hkv, d), seed + 1, bf16=True)
    v = synth.make_normal((B, S, Hkv, d), seed + 2, bf16=True)
    dout = synth.make_normal((B, S, Hq, d), seed + 3, bf16=True)
    scale = float(1.0 / np.sqrt(d))
    q64, k64, v64, g64 = (f64(x, True) for x in (q, k, v, dout))
    idx_o = np.where(idx < S, idx, -1)
    o, lse = _oracle_dsa_fwd(q64, k64, v64, idx_o, scale)
    idx_k = idx.copy()
    for b, t in empty_rows:
        g64[b, t] = 0.0
        idx_k[b, t] = -1
        o[b, t], lse[b, :, t] = 0.0, -np.inf
    got = hca.dsa_sparse_attn_bwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(idx_k).cuda(),
                                  torch.from_numpy(o).to(torch.bfloat16).cuda(), dev_f32(lse), dev_bf16(dout),
                                  scale=scale)
    torch.cuda.synchronize()
    ref = oracle.sparse_attention_bwd(q64, k64, v64, idx_o, scale, g64)
    return got, ref


@pytest.mark.parametrize("B,S,Hq,Hkv,topk,n_valid,dup", [
    (2, 200, 64, 1, 40, 35, 2),      # topk not a multiple of 32, -1 padding, duplicates, two sequences
    (1, 150, 128, 2, 64, None, 0),   # two KV heads of 64 query heads each
    (1, 130, 128, 1, 100, None, 0),  # two 64-head groups on one KV head (their contributions add)
])
def test_dsa_bwd_mfma_path(B, S, Hq, Hkv, topk, n_valid, dup):
    """The bf16 / 256-wide kernels (64 heads per workgroup, position-ordered
    contribution rows) on ragged, padded and grouped shapes."""
    _say("dsa bwd mfma", B, S, Hq, Hkv, topk, n_valid, dup)
    idx = synth.make_index_lists(B, S, topk, seed=95, n_valid=n_valid, dup_per_row=dup)
    got, ref = _dsa_bwd_bf16_case(B, S, Hq, Hkv, idx, 90)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, g, r, BF16_TOL)


def test_dsa_bwd_mfma_empty_and_out_of_range_rows():
    """An all -1 row adds nothing and gets dq = 0; an entry past the sequence is skipped."""
    B, S, Hq, Hkv, topk = 1, 96, 64, 1, 48
    idx = synth.make_index_lists(B, S, topk, seed=96)
    idx[0, 70, 3] = S + 5
    got, ref = _dsa_bwd_bf16_case(B, S, Hq, Hkv, idx, 97, empty_rows=[(0, 40)])
    assert (host(got[0])[0, 40] == 0).all()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, g, r, BF16_TOL)


@pytest.mark.timeout(900)
def test_full_size_dsa_backward_sampled():
    """The DSA backward at the 65536-token workload (64 heads x 256 on one KV
    head, top-2048; the contribution rows go through 16 chunks of 4096
    queries): dq on sampled rows, dk and dv on sampled positions, against the
    oracle's gradients of the same selections."""
    cfg = synth.CONFIGS["c5"]
    _say("full-size dsa backward", cfg)
    inp = synth.make_dsa(cfg)
    S, Hq, d = cfg.seqlen, cfg.h_q, cfg.d_qk
    idx = synth.make_index_lists_long(1, S, cfg.topk, seed=98)
    dout = synth.make_normal((1, S, Hq, d), 99, bf16=True)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    idd = torch.from_numpy(idx).cuda()
    o, lse = hca.dsa_sparse_attn_fwd(q, k, v, idd, scale=cfg.scale)
    dq, dk, dv = hca.dsa_sparse_attn_bwd(q, k, v, idd, o, lse, dev_bf16(dout), scale=cfg.scale)
    torch.cuda.synchronize()
    _say("  backward done")
    k64, v64 = f64(inp["k"], True), f64(inp["v"], True)
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 2047, 2048, 4095, 4096, 40000, S - 1]) | set(rng.integers(0, S, 6).tolist()))
    rq, _, _ = oracle.sparse_attention_bwd(f64(inp["q"][:, rows], True), k64, v64, idx[:, rows], cfg.scale,
                                           f64(dout[:, rows], True))
    err = rel_err(host(dq[:, rows]), rq)
    _say(f"  dq on {len(rows)} rows: {err:.3e}")
    assert err < BF16_TOL
    for u in (S - 1, S - 2, S - 37, S - 700, S - 3000):
        sel = np.nonzero((idx[0] == u).any(axis=1))[0]
        _, rk, rv = oracle.sparse_attention_bwd(f64(inp["q"][:, sel], True), k64, v64, idx[:, sel], cfg.scale,
                                                f64(dout[:, sel], True))
        ek = rel_err(host(dk[:, u]), rk[:, u])
        ev = rel_err(host(dv[:, u]), rv[:, u])
        _say(f"  position {u}: {len(sel)} selecting queries, dk {ek:.2e}, dv {ev:.2e}")
        assert ek < BF16_TOL and ev < BF16_TOL
    # a position no query selects gets zeros (every position of a full row is selected by some later
    # query with overwhelming probability, so check the structure instead: dk, dv finite everywhere)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


@pytest.mark.timeout(900)
def test_full_size_backward_c2_shape():
    """The backward calls the benchmark times, at their shape (32768 tokens, 16
    heads x 512, block 128, window 128; the c2 inputs plus a seeded dO): one
    head's gradients checked in full against the oracle (every dq row, every raw
    K/V row, every compressed entry, the compressor weights), and dq of sampled
    rows on two more heads.  With MHA, head h only meets KV head h, so the
    one-head oracle is exact for that head."""
    cfg = synth.CONFIGS["c2"]
    _say("full-size backward", cfg)
    inp = synth.make_prefill(cfg)
    dout = synth.make_normal((cfg.batch, cfg.seqlen, cfg.h_q, cfg.head_dim), cfg.seed + 1, cfg.std, bf16=True)
    kw = dict(window=cfg.window, block=cfg.block, scale=cfg.scale)
    qd, kd, vd, gd = (dev_bf16(x) for x in (inp["q"], inp["k"], inp["v"], dout))
    wd = dev_f32(inp["w"])
    kcd, vcd = hca.hca_compress_kv(kd, vd, wd, wd, cfg.block)
    o, lse = hca.hca_attn_fwd(qd, kd, vd, kcd, vcd, **kw)
    attn = hca.hca_attn_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, **kw)
    layer = hca.hca_attn_compress_bwd(qd, kd, vd, kcd, vcd, o, lse, gd, wd, wd, **kw)
    torch.cuda.synchronize()
    del qd, kd, vd, gd, kcd, vcd, o, lse
    h = 5
    q, k, v, g = (f64(x[:, :, [h]], True) for x in (inp["q"], inp["k"], inp["v"], dout))
    wh = inp["w"][[h]]
    kc, vc = oracle.compress_kv(k, wh, cfg.block), oracle.compress_kv(v, wh, cfg.block)
    rq, rk, rv, rkc, rvc = oracle.hca_attention_bwd(q, k, v, kc, vc, g, **kw)
    ck, rwk = oracle.compress_kv_bwd(k, wh, rkc, cfg.block)
    cv, rwv = oracle.compress_kv_bwd(v, wh, rvc, cfg.block)
    sl = lambda t: t[:, :, h:h + 1]
    for name, got, ref in (("dq", sl(attn[0]), rq), ("dk", sl(attn[1]), rk), ("dv", sl(attn[2]), rv),
                           ("dkc", sl(attn[3]), rkc), ("dvc", sl(attn[4]), rvc)):
        _check("attn " + name, got, ref, BF16_TOL)
    dq, dk, dv, dkc, dvc, dwk, dwv = layer
    for name, got, ref in (("dq", sl(dq), rq), ("dk", sl(dk), rk + ck), ("dv", sl(dv), rv + cv),
                           ("dkc", sl(dkc), rkc), ("dvc", sl(dvc), rvc),
                           ("dw_k", dwk[h:h + 1], rwk), ("dw_v", dwv[h:h + 1], rwv)):
        _check("layer " + name, got, ref, BF16_TOL)
    # dq of sampled rows on two more heads
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 127, 128, 255, 256, 16383, cfg.seqlen - 1]) | set(rng.integers(0, cfg.seqlen, 8).tolist()))
    for h2 in (0, cfg.h_q - 1):
        q2, k2, v2, g2 = (f64(x[:, :, h2], True)[0] for x in (inp["q"], inp["k"], inp["v"], dout))
        kc2 = oracle.compress_kv(k2[None, :, None], inp["w"][[h2]], cfg.block)[0, :, 0]
        vc2 = oracle.compress_kv(v2[None, :, None], inp["w"][[h2]], cfg.block)[0, :, 0]
        ref = np.zeros((len(rows), cfg.head_dim))
        for i, t in enumerate(rows):
            lo, n_c = oracle.window_bounds(t, cfg.window, cfg.block)
            keys = np.concatenate([kc2[:n_c], k2[lo:t + 1]])
            vals = np.concatenate([vc2[:n_c], v2[lo:t + 1]])
            ref[i] = oracle.attend_row_bwd(q2[t], keys, vals, cfg.scale, g2[t])[0]
        _check(f"dq head {h2} sampled rows", attn[0][0, rows, h2], ref, BF16_TOL)
        _check(f"layer dq head {h2} sampled rows", dq[0, rows, h2], ref, BF16_TOL)
