"""Pins for the oracle's attention forward (the forward whose logits give the
per-head S_max).  Each check comes from the definition of softmax attention,
not from the oracle's own code path:
  * brute force: scalar Python loops over (b, h, i, j) with math.exp;
  * identical keys give uniform weights, so causal row i is the mean of
    v_0 .. v_i;
  * all-ones values give all-ones outputs (each weight row sums to one);
  * the first causal query sees only itself: o_0 = v_0 exactly;
  * a dominant logit selects its value row;
  * exp(lse_i) equals the sum of exp(s_ij) over the allowed keys.
"""
import math

import numpy as np
import pytest

from oracle import muon_oracle as O


def brute(Q, K, V, scale, causal):
    B, T, H, d = Q.shape
    out = np.zeros(Q.shape[:3] + (V.shape[3],))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            for i in range(T):
                js = range(i + 1) if causal else range(T)
                s = [scale * sum(Q[b, i, h, t] * K[b, j, h, t] for t in range(d)) for j in js]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for c in range(V.shape[3]):
                    out[b, i, h, c] = sum(wj * V[b, j, h, c] for wj, j in zip(w, js)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force(causal):
    g = np.random.default_rng(3)
    Q, K, V = (g.standard_normal((2, 5, 2, 4)) for _ in range(3))
    o, lse, smax = O.attention_forward(Q, K, V, 0.5, causal)
    ob, lb = brute(Q, K, V, 0.5, causal)
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-12)


def test_identical_keys_average_values():
    g = np.random.default_rng(4)
    Q = g.standard_normal((1, 6, 1, 8))
    K = np.tile(g.standard_normal((1, 1, 1, 8)), (1, 6, 1, 1))
    V = g.standard_normal((1, 6, 1, 3))
    o, _, _ = O.attention_forward(Q, K, V, 1.0, True)
    for i in range(6):
        assert np.allclose(o[0, i, 0], V[0, :i + 1, 0].mean(axis=0), atol=1e-12)


def test_ones_values_and_first_query():
    g = np.random.default_rng(5)
    Q, K = g.standard_normal((2, 2, 7, 3, 16))
    o, _, _ = O.attention_forward(Q, K, np.ones((2, 7, 3, 5)), 0.25, True)
    assert np.allclose(o, 1.0, atol=1e-12)
    V = g.standard_normal((2, 7, 3, 5))
    o, _, _ = O.attention_forward(Q, K, V, 0.25, True)
    assert np.array_equal(o[:, 0], V[:, 0])


def test_dominant_logit_selects_value():
    T, d = 5, 4
    Q = np.zeros((1, T, 1, d)); Q[0, :, 0, 0] = 1.0
    K = np.zeros((1, T, 1, d)); K[0, 2, 0, 0] = 80.0
    V = np.arange(T * 2, dtype=float).reshape(1, T, 1, 2)
    o, _, smax = O.attention_forward(Q, K, V, 1.0, False)
    assert np.allclose(o[0, :, 0], V[0, 2, 0], atol=1e-30)
    assert smax[0] == 80.0


def test_lse_closed_form():
    g = np.random.default_rng(6)
    Q, K, V = (g.standard_normal((1, 4, 2, 3)) for _ in range(3))
    _, lse, _ = O.attention_forward(Q, K, V, 0.7, True)
    for h in range(2):
        for i in range(4):
            s = [0.7 * float(Q[0, i, h] @ K[0, j, h]) for j in range(i + 1)]
            assert math.isclose(math.exp(lse[0, h, i]), sum(math.exp(x) for x in s), rel_tol=1e-12)
