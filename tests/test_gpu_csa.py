"""GPU parity of the CSA path -- K, V and the index keys compressed per block,
indexer + top-k over the compressed entries, sparse attention over them --
against the float64 oracle on the same seeded inputs, through the C-ABI.

The compressed index keys come from the library's compressor (fp32); the
oracle ranks those same fp32 values, so index sets are compared exactly on
rows whose top-k boundary is clear of the fp32 error bound (other rows are
redrawn)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BF16_TOL, LSE_TOL, dev_bf16, dev_f32, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sorted_rows(idx):
    out = np.full_like(idx, -1)
    for b in range(idx.shape[0]):
        for t in range(idx.shape[1]):
            v = np.sort(idx[b, t][idx[b, t] >= 0])
            out[b, t, : v.shape[0]] = v
    return out


def _compress_index_keys(kI, w_i, block):
    """Compressed index keys [B, n, d_i] from the library's compressor (one fp32 head)."""
    kd = dev_f32(kI)[:, :, None, :]
    wd = dev_f32(w_i)
    kc, _ = hca.hca_compress_kv(kd, kd, wd, wd, block)
    kc = kc[:, :, 0].contiguous()
    torch.cuda.synchronize()
    return kc


def _make_tie_free(inp, kIc_host, cfg, rows=None):
    S = cfg.seqlen
    rows = range(S) if rows is None else rows
    for attempt in range(1, 13):
        bad = [(b, t) for b in range(cfg.batch) for t in rows
               if not oracle.csa_tie_free_row(inp["qI"][b, t], kIc_host[b], inp["w"][b, t], t, cfg.topk, cfg.block)]
        if not bad:
            return
        synth.redraw_dsa_rows(inp, bad, attempt)
    raise RuntimeError("could not make the CSA rows tie-free")


@pytest.mark.parametrize("S,topk,block,B", [(300, 16, 4, 1), (1000, 64, 4, 2), (2500, 100, 4, 1), (777, 32, 2, 1),
                                            (900, 8, 8, 1), (203, 512, 4, 1)])
def test_csa_index_topk_exact_sets(S, topk, block, B):
    cfg = synth.small_csa(seqlen=S, topk=topk, block=block, batch=B)
    _say("csa index_topk", cfg)
    inp = synth.make_csa(cfg)
    kIc = _compress_index_keys(inp["kI"], inp["w_i"], block)
    kIc_h = kIc.cpu().numpy()
    _make_tie_free(inp, kIc_h, cfg)
    idx = hca.csa_index_topk(dev_f32(inp["qI"]), kIc, dev_f32(inp["w"]), topk, block)
    torch.cuda.synchronize()
    got = _sorted_rows(idx.cpu().numpy())
    ref = oracle.csa_index_topk(inp["qI"], kIc_h, inp["w"], topk, block)
    assert np.array_equal(got, ref)


def test_csa_index_topk_long_rows_exact():
    """Rows of more than 4096 entries take the sampling selection path."""
    S, k, block = 20000, 512, 4
    cfg = synth.small_csa(seqlen=S, topk=k, block=block)
    _say("csa index_topk long rows", cfg)
    inp = synth.make_csa(cfg)
    kIc = _compress_index_keys(inp["kI"], inp["w_i"], block)
    kIc_h = kIc.cpu().numpy()
    rows = list(range(4 * 4096, S, 13)) + [S - 1]
    _make_tie_free(inp, kIc_h, cfg, rows)
    idx = hca.csa_index_topk(dev_f32(inp["qI"]), kIc, dev_f32(inp["w"]), k, block)
    got = _sorted_rows(idx.cpu().numpy())
    ref = oracle.csa_index_topk(inp["qI"], kIc_h, inp["w"], k, block, rows=rows)
    assert np.array_equal(got[:, rows], ref)


def test_csa_block_one_is_dsa():
    """block 1 with one key per position is exactly the DSA selection."""
    cfg = synth.small_dsa(seqlen=1200, topk=64)
    inp = synth.make_dsa(cfg)
    qI, kI, w = dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"])
    a = hca.csa_index_topk(qI, kI, w, 64, 1)
    b = hca.dsa_index_topk(qI, kI, w, 64)
    torch.cuda.synchronize()
    assert np.array_equal(_sorted_rows(a.cpu().numpy()), _sorted_rows(b.cpu().numpy()))


def _run_chain(cfg, inp):
    """The CSA step on the GPU: compress K, V (bf16) and the index keys, select, attend."""
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wkv = dev_f32(inp["w_kv"])
    kc, vc = hca.hca_compress_kv(k, v, wkv, wkv, cfg.block)
    kIc = _compress_index_keys(inp["kI"], inp["w_i"], cfg.block)
    idx = hca.csa_index_topk(dev_f32(inp["qI"]), kIc, dev_f32(inp["w"]), cfg.topk, cfg.block)
    o, lse = hca.csa_sparse_attn_fwd(q, kc, vc, idx, scale=cfg.scale)
    torch.cuda.synchronize()
    return kc, vc, kIc, idx, o, lse


@pytest.mark.parametrize("S,topk", [(500, 32), (1300, 256)])
def test_csa_chain_parity(S, topk):
    cfg = synth.small_csa(seqlen=S, topk=topk)
    _say("csa chain", cfg)
    inp = synth.make_csa(cfg)
    kc, vc, kIc, idx, o, lse = _run_chain(cfg, inp)
    kIc_h = kIc.cpu().numpy()
    idx_h = idx.cpu().numpy()
    # every row is a valid top-k of its visible entries for some fp32 evaluation order
    for t in range(S):
        n = oracle.visible_entries(t, cfg.block)
        row = idx_h[0, t]
        if n == 0:
            assert (row == -1).all()
        else:
            assert oracle.valid_topk_row(row, inp["qI"][0, t], kIc_h[0], inp["w"][0, t], n - 1, topk)
    # the compressed rows against the oracle's compressor
    rk = oracle.compress_kv(f64(inp["k"], True), inp["w_kv"], cfg.block)
    assert rel_err(host(kc), rk) < BF16_TOL
    # attention over the GPU's compressed rows and selection
    ro, rlse = oracle.csa_attention(f64(inp["q"], True), host(kc), host(vc), idx_h, cfg.scale)
    on, ln = host(o), host(lse)
    assert rel_err(on, ro) < BF16_TOL
    first = cfg.block - 1
    assert np.max(np.abs(ln[:, :, first:] - rlse[:, :, first:])) < LSE_TOL
    assert (on[0, :first] == 0).all() and np.isneginf(ln[0, :, :first]).all()


@pytest.mark.timeout(900)
def test_full_size_csa_sampled():
    """The CSA workload at full size (65536 positions, 16384 entries, top-2048,
    64 heads x 256): sampled rows' index sets exactly, attention rows against
    the oracle."""
    cfg = synth.CSA_CONFIGS["csa64k"]
    _say("full-size", cfg)
    inp = synth.make_csa(cfg)
    kIc = _compress_index_keys(inp["kI"], inp["w_i"], cfg.block)
    kIc_h = kIc.cpu().numpy()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 3, 4, 8190, 8191, 8192, 8195, 20000, cfg.seqlen - 1]) |
                  set(rng.integers(0, cfg.seqlen, 12).tolist()))
    _make_tie_free(inp, kIc_h, cfg, rows)
    kc, vc, _, idx, o, lse = _run_chain(cfg, inp)
    idx_h = idx.cpu().numpy()
    got = _sorted_rows(idx_h[:, rows])
    ref = oracle.csa_index_topk(inp["qI"], kIc_h, inp["w"], cfg.topk, cfg.block, rows=rows)
    assert np.array_equal(got, ref)
    q64 = f64(inp["q"][:, rows], True)
    ro, rlse = oracle.csa_attention(q64, host(kc), host(vc), idx_h[:, rows], cfg.scale)
    sel = torch.tensor(rows, device=o.device)
    o_rows, lse_rows = host(o.index_select(1, sel)), host(lse.index_select(2, sel))
    assert rel_err(o_rows, ro) < BF16_TOL
    ok = [i for i, t in enumerate(rows) if t >= cfg.block - 1]
    assert np.max(np.abs(lse_rows[:, :, ok] - rlse[:, :, ok])) < LSE_TOL
    first = [i for i, t in enumerate(rows) if t < cfg.block - 1]
    assert (o_rows[:, first] == 0).all() and np.isneginf(lse_rows[:, :, first]).all()
