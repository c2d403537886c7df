"""The seeded input generators: determinism, rounding against torch, shapes."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, -1e-38, 3.3895314e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_round_bits(x), ref)
    back = synth.bf16_bits_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_prefill_draws_are_deterministic_and_shaped():
    cfg = synth.small_prefill("c2", seqlen=300, h_q=2, h_kv=2)
    a, b = synth.make_prefill(cfg), synth.make_prefill(cfg)
    for n in ("q", "k", "v", "w"):
        np.testing.assert_array_equal(a[n], b[n])
    assert a["q"].shape == (1, 300, 2, 512) and a["q"].dtype == np.uint16
    np.testing.assert_allclose(a["w"].sum(axis=1), 1.0, rtol=1e-6)
    vals = synth.bf16_bits_to_f32(a["k"])
    assert abs(vals.std() * np.sqrt(512) - 1.0) < 0.02


def test_dsa_row_redraw_is_local():
    cfg = synth.small_dsa(seqlen=64, h_q=2, topk=8)
    a = synth.make_dsa(cfg)
    b = synth.make_dsa(cfg)
    synth.redraw_dsa_rows(b, [(0, 10), (0, 33)], attempt=1)
    changed = np.nonzero((a["qI"] != b["qI"]).any(axis=(2, 3))[0])[0].tolist()
    assert changed == [10, 33]
    np.testing.assert_array_equal(a["kI"], b["kI"])
    c = synth.make_dsa(cfg)
    synth.redraw_dsa_rows(c, [(0, 10), (0, 33)], attempt=1)
    np.testing.assert_array_equal(b["qI"], c["qI"])


def test_index_lists_are_causal_distinct_and_padded():
    idx = synth.make_index_lists(2, 50, 8, seed=4, n_valid=6)
    assert idx.shape == (2, 50, 8) and idx.dtype == np.int32
    for b in range(2):
        for t in range(50):
            row = idx[b, t]
            n = min(t + 1, 6)
            assert (row[n:] == -1).all()
            assert len(set(row[:n].tolist())) == n and row[:n].min() >= 0 and row[:n].max() <= t
    dup = synth.make_index_lists(1, 40, 8, seed=4, dup_per_row=2)
    assert any(len(set(dup[0, t][dup[0, t] >= 0].tolist())) < min(t + 1, 8) for t in range(40))
    assert (dup[dup >= 0] <= np.arange(40)[None, :, None].repeat(8, 2)[dup >= 0]).all()
    np.testing.assert_array_equal(synth.make_index_lists(2, 50, 8, seed=4, n_valid=6), idx)


def test_long_index_lists_are_distinct_causal_prefix_samples():
    x = synth.make_index_lists_long(2, 300, 64, seed=9)
    assert x.shape == (2, 300, 64) and x.dtype == np.int32
    for b in range(2):
        for t in (0, 5, 63, 64, 65, 299):
            n = min(t + 1, 64)
            row = x[b, t]
            assert (row[n:] == -1).all()
            assert len(np.unique(row[:n])) == n and row[:n].min() >= 0 and row[:n].max() <= t
    assert np.array_equal(x, synth.make_index_lists_long(2, 300, 64, seed=9))
