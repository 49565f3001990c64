"""Pins for the oracle's momentum, scale, update and number formats (CPU).

  * momentum: after t steps the recurrence equals the unrolled sum
    sum_k mu^(t-k) G_k ("MuonClip", section 02 momentum equation).
  * Nesterov lookahead: with a constant gradient both the momentum and the
    lookahead converge to G / (1 - mu); with mu = 0 the lookahead is G.
  * pure weight decay: G = 0 gives W_t = (1 - lr wd)^t W_0 exactly
    ("MuonClip", section 03 decoupled decay).
  * descent: with wd = 0 the step decreases <G, W> (the update opposes G).
  * RMS identity: RMS(scale * O) = 0.2 sqrt(mean sigma_i(O)^2) for the
    Moonlight scale, and it sits near 0.2 for a full-rank input ("About
    Muon: Muon At Scale", Moonlight bullet; "MuonClip", section 03).
  * spectral scale: sqrt(rows / cols) (Bernstein bullet, same page).
  * bf16 rounding: brute force against exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon_oracle as O


def test_momentum_unrolled_sum():
    rng = np.random.default_rng(1)
    mu = 0.95
    Gs = [rng.standard_normal((4, 3)) for _ in range(7)]
    M = np.zeros((4, 3))
    for G in Gs:
        M = O.momentum_update(M, G, mu)
    t = len(Gs)
    expect = sum(mu ** (t - 1 - k) * Gs[k] for k in range(t))
    assert np.allclose(M, expect, atol=1e-13)


def test_nesterov_steady_state_and_mu_zero():
    mu = 0.9
    G = np.array([[1.0, -2.0], [0.5, 3.0]])
    M = np.zeros_like(G)
    for _ in range(400):
        M = O.momentum_update(M, G, mu)
    U = O.nesterov_lookahead(M, G, mu, True)
    assert np.allclose(M, G / (1 - mu), rtol=1e-12)
    assert np.allclose(U, G / (1 - mu), rtol=1e-12)
    M0 = O.momentum_update(np.ones_like(G), G, 0.0)
    assert np.array_equal(O.nesterov_lookahead(M0, G, 0.0, True), G)
    assert np.array_equal(O.nesterov_lookahead(M0, G, 0.0, False), G)


def test_pure_weight_decay():
    rng = np.random.default_rng(2)
    W0 = rng.standard_normal((6, 9)) * 0.02
    W = W0.copy()
    M = np.zeros_like(W)
    for _ in range(10):
        W, M, _ = O.muon_step(W, M, np.zeros_like(W), lr=0.02, momentum=0.95,
                              weight_decay=0.1)
    assert np.allclose(W, (1 - 0.02 * 0.1) ** 10 * W0, rtol=1e-14, atol=0)


@pytest.mark.parametrize("shape", [(8, 5), (5, 8), (16, 16)])
def test_update_is_a_descent_direction(shape):
    rng = np.random.default_rng(3)
    G = rng.standard_normal(shape)
    W = rng.standard_normal(shape)
    W1, _, _ = O.muon_step(W, np.zeros(shape), G, lr=0.01, momentum=0.95,
                           weight_decay=0.0, nesterov=False)
    assert np.sum(G * (W1 - W)) < 0


@pytest.mark.parametrize("shape", [(256, 128), (64, 200), (96, 96)])
def test_rms_identity_and_level(shape):
    rng = np.random.default_rng(4)
    G = rng.standard_normal(shape)
    W = np.zeros(shape)
    lr = 0.5
    W1, _, O_ = O.muon_step(W, np.zeros(shape), G, lr=lr, momentum=0.95, weight_decay=0.0)
    upd = -(W1 - W) / lr
    rms = np.sqrt(np.mean(upd ** 2))
    sv = np.linalg.svd(O_, compute_uv=False)
    assert abs(rms - 0.2 * np.sqrt(np.mean(sv ** 2))) < 1e-12
    # 0.2 x the tuned iteration's output band of about 0.68 to 1.2 ("Muon and
    # MuonClip: orthogonalised updates for LLM training", "Newton-Schulz: an
    # odd polynomial on singular values"), widened slightly: a full-rank
    # Gaussian input puts only most of its normalised singular values above
    # the 0.0015 floor that band assumes
    assert 0.13 <= rms <= 0.25


def test_spectral_scale():
    assert O.update_scale(512, 128, "spectral") == pytest.approx(2.0)
    assert O.update_scale(256, 128, "moonlight") == pytest.approx(0.2 * 16.0)
    assert O.update_scale(128, 256, "moonlight") == pytest.approx(0.2 * 16.0)
    assert O.update_scale(3, 4, "none") == 1.0


def _nearest_bf16_exact(x: float) -> int:
    """Brute force: scan the bf16 neighbours of x and pick the nearest, ties to
    the even bit pattern."""
    f = Fraction(x)
    b0 = int(np.float32(x).view(np.uint32) >> 16)
    best = None
    for b in range(max(0, (b0 & 0x7FFF) - 2), min(0x7F80, (b0 & 0x7FFF) + 3)):
        v = Fraction(float(O.bf16_bits_to_f64(np.array([b], dtype=np.uint16))[0]))
        d = abs(v - abs(f))
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1] | (0x8000 if x < 0 else 0)


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(300) * np.exp(rng.uniform(-60, 60, 300)))
    # exact ties: halfway between two bf16 values, both parities
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7), 1.5 + 2.0 ** -8]
    xs += [1e-40, -3e-39, 2.0 ** -133, 1.7e38]
    got = O.f64_to_bf16_bits(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _nearest_bf16_exact(float(x)), x


def test_bf16_specials():
    b = O.f64_to_bf16_bits(np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 3.5e38]))
    assert list(b[[0, 1, 3, 4, 5]]) == [0x7F80, 0xFF80, 0x0000, 0x8000, 0x7F80]
    assert (b[2] & 0x7F80) == 0x7F80 and (b[2] & 0x7F) != 0
    w = O.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001], dtype=np.uint16))
    assert list(w) == [1.0, -2.0, 2.0 ** -133]


def _closed_form_ns(U, steps=5, abc=(3.4445, -4.7750, 2.0315), eps=1e-7):
    """Newton-Schulz of U in closed form from NumPy's SVD: the iteration maps
    each normalised singular value s to the composed odd polynomial p^steps(s)
    and keeps the singular vectors ("Muon and MuonClip: orthogonalised
    updates for LLM training", "Newton-Schulz: an odd polynomial on singular
    values")."""
    a, b, c = abc
    Uu, S, Vt = np.linalg.svd(U, full_matrices=False)
    s = S / (np.linalg.norm(U) + eps)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (Uu * s) @ Vt


@pytest.mark.parametrize("shape", [(12, 7), (7, 12), (9, 9)])
def test_lookahead_uses_the_new_momentum(shape):
    """A warm momentum buffer that is not parallel to the gradient.  "MuonClip",
    section 02 writes the momentum M_t = mu M_{t-1} + G_t; the lookahead adds
    mu M_t to the gradient, so Newton-Schulz acts on
        U = G_t + mu (mu M_{t-1} + G_t) = (1 + mu) G_t + mu^2 M_{t-1}.
    The oracle's O must equal the SVD closed form of that matrix, and the
    stored momentum must be mu M_{t-1} + G_t.  Building U from M_{t-1} instead
    (U = G_t + mu M_{t-1}) moves O far outside the closed form's rounding,
    which the last assertion checks, so this pin catches that mistake.  A
    second step repeats the check with the first step's momentum as M_{t-1}."""
    rng = np.random.default_rng(11)
    mu = 0.9
    W = rng.standard_normal(shape) * 0.02
    M0 = rng.standard_normal(shape) * 3.0
    G1 = rng.standard_normal(shape)
    W1, M1, O1 = O.muon_step(W, M0, G1, lr=0.02, momentum=mu, weight_decay=0.1, nesterov=True)
    assert np.allclose(M1, mu * M0 + G1, rtol=0, atol=1e-14)
    expect = _closed_form_ns((1 + mu) * G1 + mu * mu * M0)
    assert np.linalg.norm(O1 - expect) <= 1e-11 * np.linalg.norm(expect)
    wrong = _closed_form_ns(G1 + mu * M0)
    assert np.linalg.norm(O1 - wrong) >= 1e-2 * np.linalg.norm(expect)
    # second step, fresh gradient, warm M1
    G2 = rng.standard_normal(shape)
    _, M2, O2 = O.muon_step(W1, M1, G2, lr=0.02, momentum=mu, weight_decay=0.1, nesterov=True)
    assert np.allclose(M2, mu * M1 + G2, rtol=0, atol=1e-13)
    expect2 = _closed_form_ns((1 + mu) * G2 + mu * mu * M1)
    assert np.linalg.norm(O2 - expect2) <= 1e-11 * np.linalg.norm(expect2)
    # without the lookahead Newton-Schulz acts on the momentum itself
    _, _, O3 = O.muon_step(W, M0, G1, lr=0.02, momentum=mu, weight_decay=0.1, nesterov=False)
    expect3 = _closed_form_ns(mu * M0 + G1)
    assert np.linalg.norm(O3 - expect3) <= 1e-11 * np.linalg.norm(expect3)
