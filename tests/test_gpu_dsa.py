"""GPU parity of the DSA path (indexer + causal top-k, sparse attention) against
the float64 oracle on the same seeded inputs, called through the C-ABI."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from dsa_inputs import make_tie_free
from helpers import BF16_TOL, LSE_TOL, dev_bf16, dev_f32, f64, host, rel_err

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("sparse_attention_hca_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sorted_rows(idx):
    """Per row: the valid entries sorted ascending, then the -1 padding."""
    out = np.full_like(idx, -1)
    for b in range(idx.shape[0]):
        for t in range(idx.shape[1]):
            v = np.sort(idx[b, t][idx[b, t] >= 0])
            out[b, t, : v.shape[0]] = v
    return out


@pytest.mark.parametrize("S,topk,B", [(1500, 256, 1), (700, 64, 2), (300, 512, 1), (1000, 100, 1), (500, 48, 5)])
def test_index_topk_exact_sets(S, topk, B):
    """Exact sets on tie-free rows; more than one chunk (here one per sequence)
    runs each chunk's selection on the side stream beside the next chunk's
    scores, with the two score buffers reused in turn (B = 5)."""
    cfg = synth.small_dsa(seqlen=S, topk=topk, batch=B)
    _say("index_topk", cfg)
    inp = make_tie_free(cfg)
    idx = hca.dsa_index_topk(dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"]), topk)
    torch.cuda.synchronize()
    got = _sorted_rows(idx.cpu().numpy())
    ref = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], topk)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("h_i,d_i", [(4, 16), (4, 32), (4, 48), (8, 16), (8, 32), (4, 80), (8, 128)])
def test_index_topk_indexer_shapes(h_i, d_i):
    """The other indexer shapes the library takes (h_i 4 or 8, d_i a multiple of
    16 up to 128): the query-stationary score kernels of the small shapes and the
    per-tile kernel of the rest, over several key blocks, give the oracle's sets."""
    S, topk = 1800, 128
    cfg = synth.small_dsa(seqlen=S, topk=topk, h_i=h_i, d_i=d_i)
    _say("index_topk shape", cfg)
    inp = make_tie_free(cfg)
    idx = hca.dsa_index_topk(dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"]), topk)
    torch.cuda.synchronize()
    got = _sorted_rows(idx.cpu().numpy())
    ref = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], topk)
    assert np.array_equal(got, ref)


def test_index_topk_on_other_streams_and_back_to_back():
    """The chunk pipeline orders its side stream against whatever stream the
    caller runs on: a call on a second torch stream, and two calls queued back
    to back on it (the second rewrites the same workspace and output while the
    first's selections may still run), give the default stream's sets."""
    cfg = synth.small_dsa(seqlen=500, topk=48, batch=5)
    _say("index_topk streams", cfg)
    inp = make_tie_free(cfg)
    qI, kI, w = dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"])
    ref = hca.dsa_index_topk(qI, kI, w, cfg.topk)
    torch.cuda.synchronize()
    ref = _sorted_rows(ref.cpu().numpy())
    s = torch.cuda.Stream()
    ws = torch.empty(hca.dsa_index_topk_workspace_size(cfg.batch, cfg.seqlen, cfg.topk), dtype=torch.uint8,
                     device="cuda:0")
    out = torch.full((cfg.batch, cfg.seqlen, cfg.topk), -7, dtype=torch.int32, device="cuda:0")
    with torch.cuda.stream(s):
        hca.dsa_index_topk(qI, kI, w, cfg.topk, idx=out, workspace=ws)
        first = out.clone()
        hca.dsa_index_topk(qI, kI, w, cfg.topk, idx=out, workspace=ws)
        second = out.clone()
    s.synchronize()
    assert np.array_equal(_sorted_rows(first.cpu().numpy()), ref)
    assert np.array_equal(_sorted_rows(second.cpu().numpy()), ref)


def test_index_topk_long_rows_exact():
    """Rows of 4096+ positions take the sampling selection path; tie-free rows
    must give exactly the oracle's sets."""
    S, k = 6000, 512
    cfg = synth.small_dsa(seqlen=S, topk=k)
    _say("index_topk long rows", cfg)
    inp = synth.make_dsa(cfg)
    rows = list(range(4096, S, 7)) + [S - 1]
    for attempt in range(1, 13):
        bad = [(0, t) for t in rows if not oracle.tie_free_row(inp["qI"][0, t], inp["kI"][0], inp["w"][0, t], t, k)]
        if not bad:
            break
        synth.redraw_dsa_rows(inp, bad, attempt)
    assert not bad
    idx = hca.dsa_index_topk(dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"]), k)
    got = _sorted_rows(idx.cpu().numpy())
    ref = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], k, rows=rows)
    assert np.array_equal(got[:, rows], ref)


def test_index_topk_long_rows_heavy_ties():
    """Integer-valued scores with thousands of ties per value on long rows: the
    tie-break by position must be exact on every selection path."""
    S, k = 6000, 512
    rng = np.random.default_rng(11)
    kI = np.zeros((1, S, 64), dtype=np.float32)
    kI[0, np.arange(S), np.arange(S) % 8] = 1.0
    qI = rng.integers(0, 2, (1, S, 4, 64)).astype(np.float32)
    w = rng.integers(1, 3, (1, S, 4)).astype(np.float32)
    idx = hca.dsa_index_topk(dev_f32(qI), dev_f32(kI), dev_f32(w), k)
    got = _sorted_rows(idx.cpu().numpy())
    rows = list(range(4090, S, 13)) + [S - 1]
    ref = oracle.index_topk(qI, kI, w, k, rows=rows)
    assert np.array_equal(got[:, rows], ref)


def test_index_topk_long_rows_zero_mass_at_the_boundary():
    """Most index keys are zero, so most scores are exactly 0, and the weights
    are negative, so every other score is below 0: on rows past ~4800
    positions the zeros outnumber the candidate buffer and the k-th key is a
    tie among thousands of zeros (the lowest positions win)."""
    S, k = 6000, 512
    rng = np.random.default_rng(21)
    kI = rng.standard_normal((1, S, 64)).astype(np.float32)
    kI[0, rng.random(S) < 0.8] = 0.0
    qI = rng.standard_normal((1, S, 4, 64)).astype(np.float32)
    w = -np.abs(rng.standard_normal((1, S, 4))).astype(np.float32) - 0.1
    idx = hca.dsa_index_topk(dev_f32(qI), dev_f32(kI), dev_f32(w), k)
    got = _sorted_rows(idx.cpu().numpy())
    rows = list(range(4095, S, 37)) + [S - 1]
    ref = oracle.index_topk(qI, kI, w, k, rows=rows)
    assert np.array_equal(got[:, rows], ref)


def test_index_topk_ties_break_by_position():
    """Equal index keys make every score equal: the first k positions win."""
    S, k = 600, 64
    qI = np.ones((1, S, 4, 64), dtype=np.float32)
    kI = np.full((1, S, 64), 0.5, dtype=np.float32)
    w = np.ones((1, S, 4), dtype=np.float32)
    idx = hca.dsa_index_topk(dev_f32(qI), dev_f32(kI), dev_f32(w), k)
    got = _sorted_rows(idx.cpu().numpy())
    for t in range(S):
        n = min(t + 1, k)
        assert got[0, t, :n].tolist() == list(range(n))
        assert (got[0, t, n:] == -1).all()


def test_index_topk_all_zero_scores_and_negative_weights():
    """ReLU zeros everywhere (qI = -kI direction) plus negative weights: exact zeros order by position."""
    rng = np.random.default_rng(5)
    S, k = 500, 32
    kI = np.abs(rng.standard_normal((1, S, 64))).astype(np.float32)
    qI = -np.abs(rng.standard_normal((1, S, 4, 64))).astype(np.float32)
    w = -np.abs(rng.standard_normal((1, S, 4))).astype(np.float32)
    idx = hca.dsa_index_topk(dev_f32(qI), dev_f32(kI), dev_f32(w), k)
    got = _sorted_rows(idx.cpu().numpy())
    assert np.array_equal(got, oracle.index_topk(qI, kI, w, k))


def _sparse_case(cfg, inp, idx_np):
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).to("cuda:0")
    o, lse = hca.dsa_sparse_attn_fwd(q, k, v, idx, scale=cfg.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("S,topk", [(400, 128), (256, 300)])
def test_sparse_attention_parity(S, topk):
    cfg = synth.small_dsa(seqlen=S, topk=topk)
    _say("sparse", cfg)
    inp = make_tie_free(cfg)
    idx = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], topk)
    # scramble the order inside each row: any order is accepted
    rng = np.random.default_rng(1)
    idx = np.stack([np.stack([rng.permutation(r) for r in idx[b]]) for b in range(idx.shape[0])])
    o, lse = _sparse_case(cfg, inp, idx)
    ro, rlse = oracle.sparse_attention(f64(inp["q"], True), f64(inp["k"], True), f64(inp["v"], True), idx, cfg.scale)
    err = rel_err(host(o), ro)
    _say(f"  rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_sparse_attention_k_covers_context_is_dense():
    cfg = synth.small_dsa(seqlen=200, topk=256)
    inp = synth.make_dsa(cfg)
    idx = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], 256)
    o, lse = _sparse_case(cfg, inp, idx)
    q, k, v = (torch.from_numpy(f64(inp[n], True)) for n in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), k.expand(-1, -1, 64, -1).permute(0, 2, 1, 3),
        v.expand(-1, -1, 64, -1).permute(0, 2, 1, 3), is_causal=True, scale=cfg.scale).permute(0, 2, 1, 3)
    assert rel_err(host(o), ref.numpy()) < BF16_TOL


def test_sparse_attention_bad_index_poisons_row():
    cfg = synth.small_dsa(seqlen=64, topk=16)
    inp = synth.make_dsa(cfg)
    idx = np.tile(np.arange(16, dtype=np.int32), (1, 64, 1))
    idx[0, 5, 3] = 64          # out of range
    idx[0, 9, :] = -1          # empty row
    o, lse = _sparse_case(cfg, inp, idx)
    on = host(o)
    assert np.isnan(on[0, 5]).all()
    assert (on[0, 9] == 0).all() and np.isneginf(host(lse)[0, :, 9]).all()
    others = [t for t in range(64) if t not in (5, 9)]
    assert not np.isnan(on[0, others]).any()


def _oracle_rows(inp, idx, scale, rows):
    return oracle.sparse_attention(f64(inp["q"][:, rows], True), f64(inp["k"], True), f64(inp["v"], True),
                                   idx[:, rows], scale, rows=list(range(len(rows))))


def test_sparse_attention_holes_and_empty_tiles():
    """-1 entries anywhere in a row: a hole in every row, whole 32-entry tiles of
    -1 between valid ones, rows whose valid entries stop early, and a row with
    none (o = 0, lse = -inf)."""
    S, topk = 300, 200
    cfg = synth.small_dsa(seqlen=S, topk=topk)
    _say("holes", cfg)
    inp = synth.make_dsa(cfg)
    rng = np.random.default_rng(11)
    idx = np.full((1, S, topk), -1, dtype=np.int32)
    for t in range(S):
        n = min(S, topk)
        idx[0, t, :n] = rng.permutation(S)[:n]
    idx[0, :, 37] = -1
    idx[0, 250:, 64:128] = -1
    idx[0, 200:220, 40:] = -1
    idx[0, 123] = -1
    o, lse = _sparse_case(cfg, inp, idx)
    on, ln = host(o), host(lse)
    assert (on[0, 123] == 0).all() and np.isneginf(ln[0, :, 123]).all()
    keep = [t for t in range(S) if t != 123]
    ro, rlse = _oracle_rows(inp, idx, cfg.scale, keep)
    err = rel_err(on[:, keep], ro)
    _say(f"  rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(ln[:, :, keep] - rlse)) < LSE_TOL


def test_sparse_attention_late_dominant_keys():
    """Two keys met in the second tile (of four) score about 2^135 above every
    logit of the first tile, so the softmax reference of those rows is replaced
    (the row runs again; without it the probabilities would overflow fp32); the
    two differ slightly, so the output mixes their values."""
    S, topk = 160, 128
    cfg = synth.small_dsa(seqlen=S, topk=topk)
    inp = synth.make_dsa(cfg)
    q = synth.bf16_bits_to_f32(inp["q"]).copy()
    k = synth.bf16_bits_to_f32(inp["k"]).copy()
    rows = [3, 77, 140]
    q[0, rows] = 1.0
    k[0, 150] = 6.0
    k[0, 151] = 6.0
    k[0, 151, 0, :8] = 5.875
    inp = dict(inp, q=synth.bf16_round_bits(q), k=synth.bf16_round_bits(k))
    rng = np.random.default_rng(12)
    idx = np.stack([rng.permutation(150)[:topk] for _ in range(S)])[None].astype(np.int32)
    idx[0, rows, 40] = 150
    idx[0, rows, 60] = 151
    o, lse = _sparse_case(cfg, inp, idx)
    ro, rlse = _oracle_rows(inp, idx, cfg.scale, list(range(S)))
    on = host(o)
    assert not np.isnan(on).any()
    err = rel_err(on, ro)
    _say(f"  rel err {err:.3e}")
    assert err < BF16_TOL
    assert rel_err(on[:, rows], ro[:, rows]) < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_sparse_attention_negative_scale():
    cfg = synth.small_dsa(seqlen=200, topk=96)
    inp = synth.make_dsa(cfg)
    idx = synth.make_index_lists(1, 200, 96, seed=13)
    o, lse = hca.dsa_sparse_attn_fwd(dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]),
                                     torch.from_numpy(idx).to("cuda:0"), scale=-cfg.scale)
    torch.cuda.synchronize()
    valid = [t for t in range(200) if (idx[0, t] >= 0).any()]
    ro, rlse = _oracle_rows(inp, idx, -cfg.scale, valid)
    assert rel_err(host(o)[:, valid], ro) < BF16_TOL
    assert np.max(np.abs(host(lse)[:, :, valid] - rlse)) < LSE_TOL


def test_sparse_attention_wide_position_stride():
    """K and V rows 16 MiB apart (position stride 2^23 elements): the gather
    takes 64-bit addresses."""
    S, topk = 24, 40
    cfg = synth.small_dsa(seqlen=S, topk=topk)
    inp = synth.make_dsa(cfg)
    st = 1 << 23
    views = []
    for name in ("k", "v"):
        buf = torch.zeros(S * st, dtype=torch.bfloat16, device="cuda:0")
        t = buf.as_strided((1, S, 1, 256), (S * st, st, 256, 1))
        t.copy_(dev_bf16(inp[name]))
        views.append(t)
    rng = np.random.default_rng(14)
    idx = np.full((1, S, topk), -1, dtype=np.int32)
    for t in range(S):
        idx[0, t, :S] = rng.permutation(S)
    o, lse = hca.dsa_sparse_attn_fwd(dev_bf16(inp["q"]), views[0], views[1], torch.from_numpy(idx).to("cuda:0"),
                                     scale=cfg.scale)
    torch.cuda.synchronize()
    ro, rlse = _oracle_rows(inp, idx, cfg.scale, list(range(S)))
    assert rel_err(host(o), ro) < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse)) < LSE_TOL


def test_sparse_attention_rows_longer_than_2048():
    """topk in (2048, 4096] runs the one-workgroup-per-CU configuration (a
    4-stage ring and 4096-entry rows); rows shorter than topk end in -1."""
    S, topk = 3300, 3000
    cfg = synth.small_dsa(seqlen=S, topk=topk)
    _say("long rows", cfg)
    inp = synth.make_dsa(cfg)
    idx = synth.make_index_lists(1, S, topk, seed=15)
    o, lse = _sparse_case(cfg, inp, idx)
    rows = sorted(set([0, 1, 31, 32, 2047, 2999, 3000, S - 1]) | set(np.random.default_rng(16).integers(0, S, 8).tolist()))
    ro, rlse = _oracle_rows(inp, idx, cfg.scale, rows)
    assert rel_err(host(o)[:, rows], ro) < BF16_TOL
    assert np.max(np.abs(host(lse)[:, :, rows] - rlse)) < LSE_TOL


@pytest.mark.timeout(900)
def test_full_size_dsa_sampled():
    """c5 at full size (65536 positions, top-2048, 64 heads x 256) in the launch
    configuration the benchmark times.  The sampled rows are made tie-free
    first (their qI and w redrawn from their own sub-streams, which touches no
    other row), so every sampled index set must equal the oracle's exactly."""
    cfg = synth.CONFIGS["c5"]
    _say("full-size", cfg)
    inp = synth.make_dsa(cfg)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, 2046, 2047, 2048, 2049, 5000, 40000, cfg.seqlen - 1]) |
                  set(rng.integers(0, cfg.seqlen, 12).tolist()))
    for attempt in range(1, 13):
        bad = [(0, t) for t in rows
               if not oracle.tie_free_row(inp["qI"][0, t], inp["kI"][0], inp["w"][0, t], t, cfg.topk)]
        if not bad:
            break
        synth.redraw_dsa_rows(inp, bad, attempt)
    assert not bad, "could not make the sampled rows tie-free"
    _say(f"  sampled rows redrawn: {int((inp['redraws'][0, rows] > 0).sum())} of {len(rows)}")
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    qI, kI, w = dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"])
    idx = hca.dsa_index_topk(qI, kI, w, cfg.topk)
    o, lse = hca.dsa_sparse_attn_fwd(q, k, v, idx, scale=cfg.scale)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    got = _sorted_rows(idx_np[:, rows])
    ref = oracle.index_topk(inp["qI"], inp["kI"], inp["w"], cfg.topk, rows=rows)
    for i, t in enumerate(rows):
        assert np.array_equal(got[0, i], ref[0, i]), t
    _say(f"  {len(rows)}/{len(rows)} sampled rows exact")
    ro, rlse = oracle.sparse_attention(f64(inp["q"][:, rows], True)[:, :, :, :], f64(inp["k"], True),
                                       f64(inp["v"], True), idx_np[:, rows], cfg.scale,
                                       rows=list(range(len(rows))))
    err = rel_err(host(o[:, rows]), ro)
    _say(f"  sparse attention rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse[:, :, rows]) - rlse)) < LSE_TOL


# ------------------------------------------------------------------ decode: one query per sequence

def _decode_indexer_inputs(B, n, k, seed, di=64, hi=4, max_attempts=20):
    """Keys ~ N(0,1); each sequence's query and weights are redrawn until its
    row is tie-free (the same top-k set for every fp32 evaluation order)."""
    rng = np.random.default_rng(seed)
    kI = rng.standard_normal((B, n, di)).astype(np.float32)
    qI = np.zeros((B, 1, hi, di), dtype=np.float32)
    w = np.zeros((B, 1, hi), dtype=np.float32)
    for b in range(B):
        for _ in range(max_attempts):
            qI[b, 0] = rng.standard_normal((hi, di)).astype(np.float32)
            w[b, 0] = rng.standard_normal(hi).astype(np.float32)
            if oracle.tie_free_row(qI[b, 0], kI[b], w[b, 0], n - 1, k):
                break
        else:
            raise AssertionError("no tie-free draw")
    return qI, kI, w


@pytest.mark.parametrize("B,n,topk", [(2, 1000, 2048), (2, 5000, 512), (3, 70000, 2048), (2, 150001, 2048),
                                      (1, 131072, 4096), (4, 262144, 2048)])
def test_index_topk_decode_exact_sets(B, n, topk):
    """One query per sequence over n keys, through one segment (n <= 65536) or
    the two-stage selection (several segments, the last one ragged).  The
    sixteen full segments of the last case include one whose sampled bracket
    admits ~4300 candidates (more than the prefill selection's LDS holds)."""
    _say("index_topk_decode", B, n, topk)
    qI, kI, w = _decode_indexer_inputs(B, n, topk, seed=n + topk)
    idx = hca.dsa_index_topk_decode(dev_f32(qI), dev_f32(kI), dev_f32(w), topk)
    got = _sorted_rows(idx.cpu().numpy())
    for b in range(B):
        ref = oracle.topk_row(oracle.index_scores_row(qI[b, 0], kI[b], w[b, 0], n - 1), topk)
        m = min(n, topk)
        assert got[b, 0, :m].tolist() == np.sort(ref).tolist()
        assert (got[b, 0, m:] == -1).all()


def test_index_topk_decode_heavy_ties_across_segments():
    """Integer scores with tens of thousands of ties per value over three
    segments: the winners of every segment and of the merge break ties by
    position exactly."""
    n, k = 150001, 2048
    rng = np.random.default_rng(12)
    kI = np.zeros((2, n, 64), dtype=np.float32)
    kI[:, np.arange(n), np.arange(n) % 8] = 1.0
    qI = rng.integers(0, 2, (2, 1, 4, 64)).astype(np.float32)
    w = rng.integers(1, 3, (2, 1, 4)).astype(np.float32)
    idx = hca.dsa_index_topk_decode(dev_f32(qI), dev_f32(kI), dev_f32(w), k)
    got = _sorted_rows(idx.cpu().numpy())
    for b in range(2):
        ref = oracle.topk_row(oracle.index_scores_row(qI[b, 0], kI[b], w[b, 0], n - 1), k)
        assert got[b, 0].tolist() == np.sort(ref).tolist()


def test_index_topk_decode_equals_prefill_last_row():
    """The decode selection of a query equals the prefill selection of the
    same query's row (same keys)."""
    cfg = synth.small_dsa(seqlen=3000, topk=256, batch=2)
    inp = make_tie_free(cfg)
    S, k = cfg.seqlen, cfg.topk
    full = _sorted_rows(hca.dsa_index_topk(dev_f32(inp["qI"]), dev_f32(inp["kI"]), dev_f32(inp["w"]), k).cpu().numpy())
    for t in (S - 1, 1700):
        qI = np.ascontiguousarray(inp["qI"][:, t:t + 1])
        w = np.ascontiguousarray(inp["w"][:, t:t + 1])
        kI = np.ascontiguousarray(inp["kI"][:, :t + 1])
        dec = _sorted_rows(hca.dsa_index_topk_decode(dev_f32(qI), dev_f32(kI), dev_f32(w), k).cpu().numpy())
        assert np.array_equal(dec[:, 0], full[:, t])


@pytest.mark.parametrize("n,topk", [(5000, 2048), (70000, 512)])
def test_sparse_attention_decode_parity(n, topk):
    """One query per sequence, 64 heads on one KV head, over positions chosen
    from a history longer than the query sequence (-1 padding included)."""
    B, Hq, d = 2, 64, 256
    rng = np.random.default_rng(n)
    q = synth.bf16_round_bits(rng.standard_normal((B, 1, Hq, d)))
    k = synth.bf16_round_bits(rng.standard_normal((B, n, 1, d)))
    v = synth.bf16_round_bits(rng.standard_normal((B, n, 1, d)))
    idx = np.full((B, 1, topk), -1, dtype=np.int32)
    for b in range(B):
        m = topk - 37 * b
        idx[b, 0, :m] = rng.choice(n, m, replace=False)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o, lse = hca.dsa_sparse_attn_decode(qd, kd, vd, torch.from_numpy(idx).cuda(), scale=1.0 / 16)
    torch.cuda.synchronize()
    ro, rlse = oracle.sparse_attention(f64(q, True), f64(k, True), f64(v, True), idx, 1.0 / 16, rows=[0])
    err = rel_err(host(o), ro)
    _say(f"sparse decode n={n} rel err {err:.3e}")
    assert err < BF16_TOL
    assert np.max(np.abs(host(lse) - rlse[:, :, 0])) < LSE_TOL


def test_sparse_attention_decode_rejects_out_of_range_positions():
    """A position >= n_keys poisons its row with NaN instead of reading past the keys."""
    B, Hq, d, n, topk = 2, 64, 256, 300, 64
    q = torch.randn(B, 1, Hq, d, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, n, 1, d, device="cuda").to(torch.bfloat16)
    v = torch.randn_like(k)
    idx = torch.arange(topk, dtype=torch.int32, device="cuda").repeat(B, 1, 1).contiguous()
    idx[1, 0, 5] = n
    o, lse = hca.dsa_sparse_attn_decode(q, k, v, idx)
    torch.cuda.synchronize()
    assert torch.isfinite(o[0].float()).all() and torch.isnan(o[1].float()).all()


@pytest.mark.gpu
def test_sparse_attention_decode_split_matches_oracle_and_single_pass():
    """The split decode (index row in slices, merged by log-sum-exp) against
    the oracle and the single-pass kernel: full rows, a row padded with -1
    so that most slices are empty, and a row with no position at all."""
    B, Hq, d, n, topk = 4, 64, 256, 70000, 2048
    rng = np.random.default_rng(91)
    q = synth.bf16_round_bits(rng.standard_normal((B, 1, Hq, d)))
    k = synth.bf16_round_bits(rng.standard_normal((B, n, 1, d)))
    v = synth.bf16_round_bits(rng.standard_normal((B, n, 1, d)))
    idx = np.full((B, 1, topk), -1, dtype=np.int32)
    for b, m in enumerate((topk, topk - 37, 100, 0)):
        idx[b, 0, :m] = rng.choice(n, m, replace=False)
    assert hca.dsa_sparse_attn_decode_workspace_size(B, Hq, topk) > 0
    _say("sparse decode split", B, n, topk)
    qd, kd, vd, ix = dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(idx).cuda()
    o, lse = hca.dsa_sparse_attn_decode(qd, kd, vd, ix, scale=1.0 / 16)
    o1, lse1 = hca.dsa_sparse_attn_decode(qd, kd, vd, ix, scale=1.0 / 16, split=False)
    torch.cuda.synchronize()
    ro, rlse = oracle.sparse_attention(f64(q[:3], True), f64(k[:3], True), f64(v[:3], True), idx[:3], 1.0 / 16,
                                       rows=[0])
    assert rel_err(host(o)[:3], ro) < BF16_TOL
    assert np.max(np.abs(host(lse)[:3] - rlse[:, :, 0])) < LSE_TOL
    assert rel_err(host(o)[:3], host(o1)[:3]) < BF16_TOL
    # no position: zero output, lse -inf, as the single-pass kernel writes it
    assert (host(o)[3] == 0).all() and np.isneginf(host(lse)[3]).all()
    assert (host(o1)[3] == 0).all() and np.isneginf(host(lse1)[3]).all()


@pytest.mark.gpu
def test_sparse_attention_decode_split_poisons_row():
    """An out-of-range position in one slice poisons the whole merged row."""
    B, Hq, d, n, topk = 2, 64, 256, 3000, 2048
    assert hca.dsa_sparse_attn_decode_workspace_size(B, Hq, topk) > 0
    q = torch.randn(B, 1, Hq, d, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, n, 1, d, device="cuda").to(torch.bfloat16)
    v = torch.randn_like(k)
    idx = torch.arange(topk, dtype=torch.int32, device="cuda").repeat(B, 1, 1).contiguous()
    idx[1, 0, 1500] = n
    o, lse = hca.dsa_sparse_attn_decode(q, k, v, idx)
    torch.cuda.synchronize()
    assert torch.isfinite(o[0].float()).all() and torch.isfinite(lse[0]).all()
    assert torch.isnan(o[1].float()).all() and torch.isnan(lse[1]).all()
