"""Pins for the oracle's Newton-Schulz (CPU only).

What each test pins, and against what:
  * closed form: the matrix iteration equals U p^N(S / (||G||_F + eps)) V^T,
    with p the scalar odd polynomial composed N times, computed from NumPy's
    SVD ("Muon and MuonClip", section 2, "Newton-Schulz: an odd polynomial on
    singular values").  Catches a dropped term, a wrong sign, X^T X in place
    of X X^T, a misplaced coefficient.
  * singular vectors kept: U^T O V is diagonal (same subsection; "MuonClip"
    section 02, ideal polar factor).
  * textbook special case: the classic cubic and the simple quintic, iterated
    to convergence, give the polar factor U V^T of numpy.linalg.svd.
  * the page's demo numbers (tests/golden/ns_demo.json) and the Polar
    Express aside (tests/golden/polar_express_aside.json).
  * band: outputs stay in [0.68, 1.2025] for inputs >= 0.0015 (demo text).
  * orientation: the transposed input gives the transposed output.
  * decoupling: on a scaled partial permutation (coordinate singular vectors)
    the full iteration equals the per-element scalar map and keeps every
    other element zero, which the full-size GPU checks at the element limit
    rely on.
"""
import json
import os

import numpy as np
import pytest

from oracle import muon_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TUNED = (3.4445, -4.7750, 2.0315)


def scalar_composed(s, n, abc):
    a, b, c = abc
    s = np.array(s, dtype=np.float64)
    for _ in range(n):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def with_spectrum(rng, rows, cols, sigma):
    k = min(rows, cols)
    U, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    return (U * np.asarray(sigma)) @ V.T


@pytest.mark.parametrize("shape", [(6, 4), (4, 6), (5, 5), (24, 10), (10, 24), (1, 7), (7, 1)])
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_closed_form_matches_svd(shape, steps):
    rng = np.random.default_rng(hash(shape) % 1000 + steps)
    G = rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, shape))
    eps = 1e-7
    out = O.newton_schulz(G, steps, *TUNED, eps=eps)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    expect = (U * scalar_composed(S / (np.linalg.norm(G) + eps), steps, TUNED)) @ Vt
    assert np.linalg.norm(out - expect) <= 1e-12 * max(1.0, np.linalg.norm(expect))


def test_singular_vectors_preserved():
    rng = np.random.default_rng(3)
    G = with_spectrum(rng, 20, 12, np.geomspace(1, 1e-2, 12))
    out = O.newton_schulz(G)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    D = U.T @ out @ Vt.T
    off = D - np.diag(np.diag(D))
    assert np.abs(off).max() < 1e-12
    assert np.all(np.diag(D) > 0)


@pytest.mark.parametrize("abc,steps", [((1.5, -0.5, 0.0), 80), ((2.0, -1.5, 0.5), 40)])
def test_textbook_coefficients_converge_to_polar_factor(abc, steps):
    rng = np.random.default_rng(7)
    G = with_spectrum(rng, 9, 14, np.geomspace(1.0, 0.05, 9))
    out = O.newton_schulz(G, steps, *abc)
    U, _, Vt = np.linalg.svd(G, full_matrices=False)
    assert np.linalg.norm(out - U @ Vt) < 1e-10


def demo_spectrum(gold):
    n, cond = gold["n_values"], gold["condition_number"]
    return np.geomspace(1.0, 1.0 / cond, n)


def test_demo_numbers():
    gold = json.load(open(os.path.join(GOLD, "ns_demo.json")))
    pr, tol = gold["printed"], gold["tolerance"]
    rng = np.random.default_rng(11)
    sig = demo_spectrum(gold)
    G = with_spectrum(rng, 16, 24, sig)

    def sv(abc, steps):
        return np.linalg.svd(O.newton_schulz(G, steps, *abc, eps=0.0), compute_uv=False)

    # smallest input after normalisation is about 0.001, as the page says
    assert abs(sig.min() / np.linalg.norm(sig) - pr["tuned_5_smallest_before"]) < 5e-4
    t5 = sv(gold["coefficients"]["tuned"], 5)
    assert abs(t5.min() - pr["tuned_5_smallest_after"]) <= tol["tuned_5_smallest_after"]
    assert abs(t5.max() - pr["tuned_5_largest_after"]) <= tol["tuned_5_largest_after"]
    s5 = sv(gold["coefficients"]["simple_quintic"], 5)
    assert abs(s5.min() - pr["simple_5_smallest_after"]) <= tol["simple_5_smallest_after"]
    s10 = sv(gold["coefficients"]["simple_quintic"], 10)
    assert abs(s10.min() - pr["simple_10_smallest_after"]) <= tol["simple_10_smallest_after"]
    # the classic cubic is slower still
    c5 = sv(gold["coefficients"]["classic_cubic"], 5)
    assert c5.min() < s5.min()


def test_polar_express_aside():
    gold = json.load(open(os.path.join(GOLD, "polar_express_aside.json")))
    s_in = gold["sigma_in"]
    sig = np.array([np.sqrt(1.0 - s_in ** 2), s_in])   # Frobenius norm exactly 1
    rng = np.random.default_rng(5)
    G = with_spectrum(rng, 2, 5, sig)
    out = np.linalg.svd(O.newton_schulz(G, gold["steps"], *gold["coefficients"], eps=0.0),
                        compute_uv=False)
    assert abs(out.min() - gold["printed_out"]) <= gold["tolerance"]


def test_output_band():
    gold = json.load(open(os.path.join(GOLD, "ns_demo.json")))
    lo, hi = gold["printed"]["tuned_band_low"], gold["printed"]["tuned_band_high"]
    rng = np.random.default_rng(13)
    sig = np.concatenate([np.geomspace(0.0015, 1.0, 60), rng.uniform(0.0015, 1.0, 40)])
    # scale so the normalised spectrum is exactly sig / ||sig||, then check the
    # outputs for the normalised values that are >= 0.0015
    G = with_spectrum(rng, 100, 130, sig)
    S_in = np.linalg.svd(G, compute_uv=False) / np.linalg.norm(G)
    out = np.sort(np.linalg.svd(O.newton_schulz(G, eps=0.0), compute_uv=False))
    keep = np.sort(S_in) >= 0.0015
    assert out[keep].min() >= lo - 1e-3 and out.max() <= hi + 3e-3


def test_orientation_transpose_consistency():
    rng = np.random.default_rng(17)
    G = rng.standard_normal((30, 11))
    a = O.newton_schulz(G)
    b = O.newton_schulz(G.T)
    assert np.allclose(a, b.T, rtol=0, atol=1e-13)


def test_zero_input_gives_zero():
    out = O.newton_schulz(np.zeros((5, 8)))
    assert np.all(out == 0.0)


def test_scale_invariance():
    rng = np.random.default_rng(19)
    G = rng.standard_normal((12, 20))
    a = O.newton_schulz(G, eps=0.0)
    b = O.newton_schulz(G * 1234.5, eps=0.0)
    assert np.allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("shape", [(24, 60), (60, 24), (16, 16)])
def test_partial_permutation_decouples(shape):
    """One nonzero per row of the wide view, at distinct columns: the matrix
    is U diag(s) V^T with coordinate vectors U, V, so the iteration keeps the
    pattern and maps each nonzero through the scalar polynomial alone.  The
    full-size GPU checks rest on this: the oracle's iteration on the 1 x 1
    matrix [[x / ||G||_F]] must equal the oracle's full-matrix result at that
    element, and every other element must stay exactly zero."""
    from synthetic import generators as gen
    rows, cols = shape
    g = gen.rng(rows * 1000 + cols)
    ri, ci, v = gen.partial_permutation(g, rows, cols, gen.log_spaced_levels(min(rows, cols), 4))
    G = np.zeros(shape)
    G[ri, ci] = v
    assert np.count_nonzero(G) == min(rows, cols)
    assert np.linalg.matrix_rank(G) == min(rows, cols)
    full = O.newton_schulz(G)
    x = O.frobenius_normalize(v[None, :], 1e-7)[0]
    per = np.array([O.newton_schulz_iterate(np.array([[t]]), 5, *TUNED)[0, 0] for t in x])
    assert np.array_equal(full != 0, G != 0)
    assert np.allclose(full[ri, ci], per, rtol=1e-13, atol=0)
    assert np.allclose(per, scalar_composed(x, 5, TUNED), rtol=1e-13, atol=0)
