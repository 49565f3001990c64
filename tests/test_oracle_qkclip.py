"""Pins for the oracle's QK-Clip (CPU).

  * S_max by brute force: plain Python loops over batch, heads and token
    pairs on tiny inputs ("Muon and MuonClip", "The exploding-logit problem":
    S_max^h = (1/sqrt(d)) max over samples, i, j of q_i . k_j), causal and not.
  * worked examples from the pages (tests/golden/qkclip_examples.json):
    400 -> gamma 0.25 -> each side x0.5 (MLA: rotary query x0.25, shared
    rotary key untouched); 80 -> untouched.
  * invariant: the logit scales by exactly gamma, so re-measuring on the
    rescaled weights gives min(S_max, tau) ("Muon and MuonClip", MuonClip
    section; "About Muon: Muon At Scale", "When Softmax Collapses").
  * general alpha: the q side gets gamma^alpha, the k side gamma^(1-alpha).
  * tie and non-finite readings: S_max == tau untouched, NaN/Inf flagged -1.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import muon_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute_smax(Q, K, scale, causal):
    B, T, H, d = Q.shape
    out = []
    for h in range(H):
        best = -math.inf
        for b in range(B):
            for i in range(T):
                for j in range(T):
                    if causal and j > i:
                        continue
                    s = 0.0
                    for t in range(d):
                        s += float(Q[b, i, h, t]) * float(K[b, j, h, t])
                    best = max(best, s * scale)
        out.append(best)
    return np.array(out)


@pytest.mark.parametrize("causal", [True, False])
def test_smax_brute_force(causal):
    rng = np.random.default_rng(1)
    B, T, H, d = 2, 6, 3, 4
    Q = rng.standard_normal((B, T, H, d))
    K = rng.standard_normal((B, T, H, d))
    # make the unmasked upper triangle hold the largest logit so that a
    # missing causal mask would change the answer
    K[:, -1] *= 10.0
    got = O.smax_per_head(Q, K, 1 / math.sqrt(d), causal)
    exp = brute_smax(Q, K, 1 / math.sqrt(d), causal)
    assert np.allclose(got, exp, rtol=1e-14, atol=1e-14)


def test_worked_examples():
    gold = json.load(open(os.path.join(GOLD, "qkclip_examples.json")))
    tau, alpha = gold["tau"], gold["alpha"]
    d_head, d_model = 3, 5
    rng = np.random.default_rng(2)
    for case in gold["cases"]:
        Wq = rng.standard_normal((2 * d_head, d_model))
        Wk = rng.standard_normal((2 * d_head, d_model))
        s_max = np.array([case["s_max"], 10.0])
        q2, k2, gamma, flag = O.qkclip_rescale(Wq, Wk, s_max, tau, alpha, d_head)
        assert gamma[0] == pytest.approx(case["gamma"], abs=0)
        assert flag[0] == case["clipped"] and flag[1] == 0
        assert np.allclose(q2[:d_head], Wq[:d_head] * case["q_scale"], rtol=1e-15)
        assert np.allclose(k2[:d_head], Wk[:d_head] * case["k_scale"], rtol=1e-15)
        assert np.array_equal(q2[d_head:], Wq[d_head:])
        assert np.array_equal(k2[d_head:], Wk[d_head:])
        # MLA
        d_c, d_r = 4, 2
        Wqc = rng.standard_normal((2 * d_c, d_model))
        Wkc = rng.standard_normal((2 * d_c, d_model))
        Wqr = rng.standard_normal((2 * d_r, d_model))
        Wkr = rng.standard_normal((d_r, d_model))
        a, b, c, dd, g2, f2 = O.qkclip_rescale_mla(Wqc, Wkc, Wqr, Wkr, s_max, tau, d_c, d_r)
        m = case["mla"]
        assert np.allclose(a[:d_c], Wqc[:d_c] * m["q_content"], rtol=1e-15)
        assert np.allclose(b[:d_c], Wkc[:d_c] * m["k_content"], rtol=1e-15)
        assert np.allclose(c[:d_r], Wqr[:d_r] * m["q_rotary"], rtol=1e-15)
        assert np.array_equal(dd, Wkr * m["k_rotary_shared"])
        assert np.array_equal(a[d_c:], Wqc[d_c:]) and np.array_equal(c[d_r:], Wqr[d_r:])


@pytest.mark.parametrize("alpha", [0.5, 0.3, 1.0])
def test_remeasure_invariant(alpha):
    rng = np.random.default_rng(3)
    B, T, H, d, dm = 2, 16, 4, 8, 24
    X = rng.standard_normal((B * T, dm))
    Wq = rng.standard_normal((H * d, dm)) / math.sqrt(dm)
    Wk = rng.standard_normal((H * d, dm)) / math.sqrt(dm)
    Wq[:d] *= 12.0
    Wk[:d] *= 12.0           # head 0 far above tau
    Wq[2 * d:3 * d] *= 5.0   # head 2 moderately above
    Wk[2 * d:3 * d] *= 5.0
    scale = 1 / math.sqrt(d)

    def measure(wq, wk):
        Q = (X @ wq.T).reshape(B, T, H, d)
        K = (X @ wk.T).reshape(B, T, H, d)
        return O.smax_per_head(Q, K, scale, True)

    tau = 30.0
    s0 = measure(Wq, Wk)
    assert s0[0] > tau and s0[2] > tau
    q2, k2, gamma, flag = O.qkclip_rescale(Wq, Wk, s0, tau, alpha, d)
    s1 = measure(q2, k2)
    assert np.allclose(s1, np.minimum(s0, tau), rtol=1e-12)
    assert np.all(s1 <= tau * (1 + 1e-6))
    # the product of the two factors is exactly gamma
    hq = np.linalg.norm(q2[:d]) / np.linalg.norm(Wq[:d])
    hk = np.linalg.norm(k2[:d]) / np.linalg.norm(Wk[:d])
    assert hq == pytest.approx(gamma[0] ** alpha, rel=1e-12)
    assert hk == pytest.approx(gamma[0] ** (1 - alpha), rel=1e-12)


def test_tie_and_nonfinite():
    gamma, flag = O.qkclip_factors(np.array([100.0, np.nan, np.inf, -np.inf, 100.0001, 99.0]), 100.0)
    assert list(flag) == [0, -1, -1, -1, 1, 0]
    assert gamma[0] == 1.0 and gamma[1] == 1.0 and gamma[2] == 1.0
    assert gamma[4] == pytest.approx(100.0 / 100.0001)
