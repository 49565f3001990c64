"""GPU parity of the rank-r Dion step ("About Muon: Muon At Scale", "What
Breaks at Scale", "The Matrix Does Not Fit") through the C ABI, against the
fp64 oracle on identical seeded inputs.

Tolerances, from the arithmetic (fp32 products, Gram matrices and Cholesky
factors in fp64, Cholesky-QR applied twice):
  * M' = B - (1 - mu) P R^T: relative Frobenius error <= 1e-5 (the fp32 bar;
    the rank-r term enters scaled by 1 - mu).
  * Q' = ColNorm(R) and the update Delta W = -lr P Q'^T: relative Frobenius
    error <= 1e-5, the fp32 bar (fp32 sums over up to 1000 terms, the
    orthogonalisation about cond(B Q) x 1e-7 before its second pass; measured
    2e-7 to 2e-6, the low-rank-plus-noise case included).
  * bf16 parameters: each element within half a bf16 step of the exact
    update, plus 1e-5 of the update's RMS (the product's error scale), plus
    the fp32 rounding of the element.
Every case prints its name first.
"""
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from synthetic import generators as gen
from tests.gpu_util import rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_orthogonalizing_optimizer_muon_amd as m
    m.load_library()
    return m


def widen(a, dtype):
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def make_inputs(seed, batch, rows, cols, rank, dtype, grad="normal"):
    g = gen.rng(seed)
    W = gen._cast(gen.gaussian(g, (batch, rows, cols), 0.02), dtype)
    if grad == "normal":
        G = gen._cast(gen.gaussian(g, (batch, rows, cols), 1.0), dtype)
    else:
        G = gen._cast(np.stack([gen.low_rank_plus_noise(g, rows, cols, rank=8) for _ in range(batch)]), dtype)
    M = gen.gaussian(g, (batch, rows, cols), 0.5 if grad == "normal" else 0.0).astype(np.float32)
    Q = gen.gaussian(g, (batch, cols, rank), 1.0).astype(np.float32)
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    return W, G, M, Q


def check(W0, G, M0, Q0, Wg, Mg, Qg, dtype, mu, lr, tol):
    for b in range(W0.shape[0]):
        Xr, Mr, Qr, _, _ = O.dion_step(widen(W0[b], dtype), widen(G[b], dtype), M0[b].astype(np.float64),
                                       Q0[b].astype(np.float64), mu=mu, lr=lr)
        em = rel_fro(Mg[b], Mr)
        eq = rel_fro(Qg[b], Qr)
        dref = Xr - widen(W0[b], dtype)
        if dtype == "f32":
            ew = rel_fro(Wg[b].astype(np.float64) - widen(W0[b], dtype), dref)
            wok = ew <= tol
        else:
            x = O.bf16_bits_to_f64(Wg[b])
            _, e = np.frexp(np.abs(Xr))
            # the update term's error is relative to the update's scale, not
            # to each element of it: tol x its RMS
            rms = np.sqrt(np.mean(dref * dref))
            bound = np.ldexp(1.0, e - 9) + tol * rms + 2.0 ** -22 * np.abs(Xr) + 1e-12
            ew = int(np.count_nonzero(np.abs(x - Xr) > bound))
            wok = ew == 0
        say(f"   matrix {b}: M {em:.2e}  Q {eq:.2e}  W {ew}")
        assert em <= 1e-5 and eq <= tol and wok


CASES = [(2, 64, 96, 16, "f32"), (1, 200, 136, 32, "bf16"), (3, 96, 64, 8, "bf16"), (1, 256, 512, 128, "f32"),
         (2, 512, 256, 40, "bf16"), (1, 1000, 600, 128, "bf16"),
         # padded rank 96 (does not divide the 256 threads of the norm pass)
         (2, 96, 200, 72, "f32"),
         # 8 rows, 4096 columns: the column-norm partials outgrow the Gram partials
         (1, 8, 4096, 8, "bf16")]


@pytest.mark.parametrize("batch,rows,cols,rank,dtype", CASES)
def test_dion_step_matches_oracle(mm, batch, rows, cols, rank, dtype):
    import torch
    say(f"[dion] batch={batch} {rows}x{cols} rank={rank} {dtype}")
    dev = torch.device("cuda:0")
    W, G, M, Q = make_inputs(rows * 7 + cols + rank, batch, rows, cols, rank, dtype)
    Wd, Gd, Md, Qd = (to_dev(x, dev) for x in (W, G, M, Q))
    mm.dion_step(Wd, Gd, Md, Qd, lr=0.02, mu=0.95)
    torch.cuda.synchronize()
    check(W, G, M, Q, to_host(Wd), to_host(Md), to_host(Qd), dtype, 0.95, 0.02, 1e-5)


def test_dion_low_rank_gradient(mm):
    """Low-rank-plus-noise gradient (rank 8, singular values i^-1.5, noise
    0.01) with rank 32: B Q is ill-conditioned (8 strong directions, 24 at
    noise level), the case a single Cholesky-QR pass in fp32 would lose."""
    import torch
    say("[dion] low-rank-plus-noise gradient, rank 32")
    dev = torch.device("cuda:0")
    W, G, M, Q = make_inputs(5, 2, 384, 512, 32, "f32", grad="lowrank")
    Wd, Gd, Md, Qd = (to_dev(x, dev) for x in (W, G, M, Q))
    mm.dion_step(Wd, Gd, Md, Qd, lr=0.02, mu=0.95)
    torch.cuda.synchronize()
    check(W, G, M, Q, to_host(Wd), to_host(Md), to_host(Qd), "f32", 0.95, 0.02, 1e-5)


def test_dion_exact_rank_r_closed_form(mm):
    """B of exact rank r with Q its right singular vectors: P = U, so
    M' = mu B, Q' = V and W' = W - lr U V^T, independent of the oracle."""
    import torch
    say("[dion] exact rank-r closed form")
    dev = torch.device("cuda:0")
    g = np.random.default_rng(11)
    m, n, r = 256, 192, 16
    U = np.linalg.qr(g.standard_normal((m, r)))[0]
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    s = np.linspace(4.0, 1.0, r)
    B = (U * s) @ V.T
    G = (0.4 * B).astype(np.float32)
    M = (B - G.astype(np.float64)).astype(np.float32)
    Bx = M.astype(np.float64) + G.astype(np.float64)
    W = np.zeros((m, n), dtype=np.float32)     # W' is then the update itself, with no fp32 rounding of W
    Wd, Gd, Md, Qd = (to_dev(x, dev) for x in (W, G, M, V.astype(np.float32)))
    mm.dion_step(Wd, Gd, Md, Qd, lr=0.05, mu=0.9)
    torch.cuda.synchronize()
    assert rel_fro(to_host(Md), 0.9 * Bx) <= 1e-5
    assert rel_fro(to_host(Qd), V) <= 1e-5
    assert rel_fro(to_host(Wd).astype(np.float64), -0.05 * U @ V.T) <= 1e-5


def test_dion_zero_input_and_nan(mm):
    """B = 0: every pivot is dropped, so Q' = 0, M' = 0 and W is untouched
    (the oracle's QR picks arbitrary directions there, all with R = 0).  A NaN
    in G propagates into M, Q and W."""
    import torch
    say("[dion] zero input; NaN propagation")
    dev = torch.device("cuda:0")
    W, G, M, Q = make_inputs(9, 1, 64, 64, 16, "f32")
    Wd = to_dev(W, dev)
    Gd = torch.zeros_like(Wd)
    Md = torch.zeros_like(Wd)
    Qd = to_dev(Q, dev)
    mm.dion_step(Wd, Gd, Md, Qd, lr=0.02, mu=0.95)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(Wd), W)
    assert not to_host(Md).any() and not to_host(Qd).any()
    G2 = G.copy()
    G2[0, 3, 5] = np.nan
    Wd, Gd, Md, Qd = (to_dev(x, dev) for x in (W, G2, M, Q))
    mm.dion_step(Wd, Gd, Md, Qd, lr=0.02, mu=0.95)
    torch.cuda.synchronize()
    assert np.isnan(to_host(Md)[0, 3, 5]) and np.isnan(to_host(Qd)).any() and np.isnan(to_host(Wd)).any()


def test_dion_three_warm_started_steps(mm):
    """Three consecutive steps with fresh gradients, Q and M carried on the
    GPU; each step is checked against the oracle from the GPU's own state."""
    import torch
    say("[dion] three warm-started steps")
    dev = torch.device("cuda:0")
    W, G, M, Q = make_inputs(13, 2, 256, 320, 32, "bf16")
    Wd, Md, Qd = to_dev(W, dev), to_dev(M, dev), to_dev(Q, dev)
    g = gen.rng(14)
    for step in range(3):
        Gs = gen._cast(gen.gaussian(g, W.shape, 1.0), "bf16")
        W0, M0, Q0 = to_host(Wd), to_host(Md), to_host(Qd)
        mm.dion_step(Wd, to_dev(Gs, dev), Md, Qd, lr=0.02, mu=0.95)
        torch.cuda.synchronize()
        say(f"   step {step}")
        check(W0, Gs, M0, Q0, to_host(Wd), to_host(Md), to_host(Qd), "bf16", 0.95, 0.02, 1e-5)
