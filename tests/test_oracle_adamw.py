"""Pins for the oracle's AdamW companion step (CPU).

  * first step: whatever beta1 and beta2, the bias-corrected moments are g and
    g^2, so the step is lr * g / (|g| + eps): elementwise sign descent
    ("Muon and MuonClip", "Adam, seen as steepest descent": with the moving
    averages switched off Adam's update is g/|g|).
  * entry RMS of that step is lr for |g| >> eps ("About Muon: Muon At
    Scale", Moonlight bullet: AdamW's step has entry RMS about eta).
  * constant gradient: the moments stay at g and g^2 after bias correction,
    so every step is the same sign step (a closed form over t steps).
  * decoupled decay: g = 0 shrinks p by exactly (1 - lr wd) per step.
"""
import numpy as np
import pytest

from oracle import muon_oracle as O

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)


@pytest.mark.parametrize("b1,b2", [(0.9, 0.999), (0.5, 0.5), (0.0, 0.0)])
def test_first_step_is_sign_descent(b1, b2):
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000) * np.exp(rng.uniform(-5, 5, 1000))
    p0 = rng.standard_normal(1000)
    hp = dict(HP, beta1=b1, beta2=b2, eps=0.0)
    p1, m, v = O.adamw_step(p0, g, np.zeros(1000), np.zeros(1000), step=1, **hp)
    assert np.allclose(p1, p0 - hp["lr"] * np.sign(g), rtol=0, atol=1e-15)
    rms = np.sqrt(np.mean((p1 - p0) ** 2))
    assert rms == pytest.approx(hp["lr"], rel=1e-12)


def test_constant_gradient_closed_form():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(50)
    p = rng.standard_normal(50)
    p0 = p.copy()
    m = np.zeros(50)
    v = np.zeros(50)
    T = 25
    for t in range(1, T + 1):
        p, m, v = O.adamw_step(p, g, m, v, step=t, **dict(HP, eps=0.0))
    assert np.allclose(p, p0 - T * HP["lr"] * np.sign(g), rtol=0, atol=1e-12)


def test_decoupled_decay():
    p0 = np.linspace(-1, 1, 11)
    p, m, v = O.adamw_step(p0, np.zeros(11), np.zeros(11), np.zeros(11), step=1,
                           **dict(HP, weight_decay=0.1))
    assert np.allclose(p, p0 * (1 - 1e-3 * 0.1), rtol=1e-15, atol=0)


def test_moment_recurrences():
    rng = np.random.default_rng(3)
    gs = [rng.standard_normal(7) for _ in range(6)]
    m = np.zeros(7)
    v = np.zeros(7)
    p = np.zeros(7)
    for t, g in enumerate(gs, start=1):
        p, m, v = O.adamw_step(p, g, m, v, step=t, **HP)
    b1, b2 = HP["beta1"], HP["beta2"]
    n = len(gs)
    assert np.allclose(m, sum((1 - b1) * b1 ** (n - 1 - k) * gs[k] for k in range(n)), atol=1e-15)
    assert np.allclose(v, sum((1 - b2) * b2 ** (n - 1 - k) * gs[k] ** 2 for k in range(n)), atol=1e-15)
