"""Pins of the attention-output epilogue oracle (low-rank output gate, VHA
cross-head mixing) against explicit loops, closed forms and special cases."""
import math

import numpy as np
import torch

import oracle


def _draw(B=2, S=5, H=4, d=3, dc=6, r=2, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, H, d)), rng.standard_normal((B, S, dc)),
            rng.standard_normal((H * d, dc)), rng.standard_normal((H, r)), rng.standard_normal((r, H)))


def test_gate_against_explicit_loops_and_torch():
    o, c, w, u, v = _draw()
    g = oracle.gate_values(c, w, 4, 3)
    for b in range(2):
        for t in range(5):
            for h in range(4):
                for e in range(3):
                    x = sum(c[b, t, k] * w[h * 3 + e, k] for k in range(6))
                    assert abs(g[b, t, h, e] - 1.0 / (1.0 + math.exp(-x))) < 1e-14
    ref = torch.sigmoid(torch.nn.functional.linear(torch.from_numpy(c), torch.from_numpy(w))).numpy()
    np.testing.assert_allclose(g.reshape(2, 5, 12), ref, rtol=1e-13)


def test_gate_closed_forms():
    o, c, w, u, v = _draw()
    assert (oracle.gate_values(c, 0 * w, 4, 3) == 0.5).all()              # zero projection: gate 1/2
    g, gn = oracle.gate_values(c, w, 4, 3), oracle.gate_values(c, -w, 4, 3)
    np.testing.assert_allclose(g + gn, 1.0, rtol=1e-14)                      # sigmoid(x) + sigmoid(-x) = 1


def test_vha_against_explicit_loops():
    o, c, w, u, v = _draw()
    z = oracle.vha_mix(o, u, v)
    for b in range(2):
        for t in range(5):
            for h in range(4):
                for e in range(3):
                    s = o[b, t, h, e]
                    for h2 in range(4):
                        s += sum(u[h, j] * v[j, h2] for j in range(2)) * o[b, t, h2, e]
                    assert abs(z[b, t, h, e] - s) < 1e-12


def test_vha_special_cases():
    o, c, w, u, v = _draw(r=4)
    np.testing.assert_array_equal(oracle.vha_mix(o, 0 * u, v), o)          # no mixing: the identity skip alone
    np.testing.assert_allclose(oracle.vha_mix(o, -np.eye(4), np.eye(4)), 0.0, atol=1e-15)   # U V = -I cancels it
    # a rank-1 map that copies head 0 into head 2
    u1, v1 = np.zeros((4, 1)), np.zeros((1, 4))
    u1[2, 0], v1[0, 0] = 1.0, 1.0
    z = oracle.vha_mix(o, u1, v1)
    np.testing.assert_allclose(z[:, :, 2], o[:, :, 2] + o[:, :, 0])
    np.testing.assert_array_equal(z[:, :, [0, 1, 3]], o[:, :, [0, 1, 3]])


def test_output_is_gate_times_mixed():
    o, c, w, u, v = _draw()
    y = oracle.gated_vha_output(o, c, w, u, v)
    np.testing.assert_allclose(y, oracle.gate_values(c, w, 4, 3) * oracle.vha_mix(o, u, v))
    # with a zero projection and no mixing the output is o / 2
    np.testing.assert_allclose(oracle.gated_vha_output(o, c, 0 * w, 0 * u, v), o / 2)
