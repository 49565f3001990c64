"""GPU parity for the rows beyond the core step: MLA QK-Clip (separate and
fused projection layouts), the companion AdamW group, and the other
Newton-Schulz coefficient sets, each through the C ABI against the fp64
oracle on identical seeded inputs.

Tolerances:
  * rescaled weights: bf16 within 1 bf16 step of the oracle's rounding of the
    exact product (the factors 1/2 and 1/4 of the worked example are exact,
    so that head is bit-exact); fp32 relative Frobenius error <= 1e-6.
    Untouched rows are bit-identical.
  * AdamW moments (fp32): relative Frobenius error <= 1e-6.  Parameters: the
    change p_new - p is within 1e-5 relative Frobenius error of the oracle's
    change (fp32 params); bf16 params are a faithful bf16 rounding of the
    exact result (at most 1 bf16 step from the oracle's rounding).
  * Newton-Schulz with the cubic and the simple quintic: the same 2e-2
    relative Frobenius bound as the tuned quintic.
"""
import json
import math
import os
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from synthetic import generators as gen
from tests.gpu_util import bf16_ulp_diff, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


@pytest.fixture(scope="module")
def dev(mm):
    import torch
    return torch.device("cuda:0")


def widen(a, dtype):
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def assert_close_weights(got, ref, orig, dtype, untouched_rows):
    if dtype == "bf16":
        d = bf16_ulp_diff(got, O.f64_to_bf16_bits(ref))
        assert d.max() <= 1, f"max bf16 step difference {d.max()}"
    else:
        assert rel_fro(got, ref) <= 1e-6
    for rows in untouched_rows:
        assert np.array_equal(got[rows], orig[rows])


# ---------------------------------------------------------------------------
# MLA QK-Clip
# ---------------------------------------------------------------------------

MLA_SMAX = np.array([400.0, 80.0, 100.0, np.nan, 1.0e4, 133.0], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("q_in,kv_in", [(96, 40), (1536, 512), (70, 37)])
def test_qk_rescale_mla_matches_oracle(mm, dev, dtype, q_in, kv_in):
    import torch
    H, d_c, d_r = len(MLA_SMAX), 128, 64
    say(f"[mla] dtype={dtype} q_in={q_in} kv_in={kv_in} H={H} d_c={d_c} d_r={d_r}")
    g = gen.rng(31 + q_in + kv_in)
    Wqc = gen._cast(gen.gaussian(g, (H * d_c, q_in), 0.05), dtype)
    Wkc = gen._cast(gen.gaussian(g, (H * d_c, kv_in), 0.05), dtype)
    Wqr = gen._cast(gen.gaussian(g, (H * d_r, q_in), 0.05), dtype)
    Wkr = gen._cast(gen.gaussian(g, (d_r, kv_in), 0.05), dtype)
    dq, dk, dr = to_dev(Wqc, dev), to_dev(Wkc, dev), to_dev(Wqr, dev)
    flags = mm.qkclip_rescale_mla(dq, dk, dr, to_dev(MLA_SMAX, dev), d_c=d_c, d_r=d_r, tau=100.0)
    torch.cuda.synchronize()
    rq, rk, rr, rkr, gamma, fl = O.qkclip_rescale_mla(widen(Wqc, dtype), widen(Wkc, dtype), widen(Wqr, dtype),
                                                      widen(Wkr, dtype), MLA_SMAX.astype(np.float64), 100.0,
                                                      d_c, d_r)
    assert list(to_host(flags)) == list(fl) == [1, 0, 0, -1, 1, 1]
    assert np.array_equal(rkr, widen(Wkr, dtype))          # the shared rotary key never moves
    untouched = [h for h in range(H) if fl[h] != 1]
    c_rows = [slice(h * d_c, (h + 1) * d_c) for h in untouched]
    r_rows = [slice(h * d_r, (h + 1) * d_r) for h in untouched]
    assert_close_weights(to_host(dq), rq, Wqc, dtype, c_rows)
    assert_close_weights(to_host(dk), rk, Wkc, dtype, c_rows)
    assert_close_weights(to_host(dr), rr, Wqr, dtype, r_rows)


def test_qk_rescale_mla_worked_example_is_exact(mm, dev):
    """400 against tau 100: gamma 1/4, content rows x 1/2, rotary query rows
    x 1/4 (powers of two, so every bf16 product is exact)."""
    import torch
    gold = json.load(open(os.path.join(GOLDEN, "qkclip_examples.json")))
    case = gold["cases"][0]
    H, d_c, d_r, q_in, kv_in = 2, 128, 64, 64, 32
    say("[mla] worked example")
    g = gen.rng(77)
    Wqc = gen.f32_to_bf16_bits(gen.gaussian(g, (H * d_c, q_in), 0.05))
    Wkc = gen.f32_to_bf16_bits(gen.gaussian(g, (H * d_c, kv_in), 0.05))
    Wqr = gen.f32_to_bf16_bits(gen.gaussian(g, (H * d_r, q_in), 0.05))
    s = np.array([case["s_max"], gold["cases"][1]["s_max"]], dtype=np.float32)
    dq, dk, dr = to_dev(Wqc, dev), to_dev(Wkc, dev), to_dev(Wqr, dev)
    mm.qkclip_rescale_mla(dq, dk, dr, to_dev(s, dev), d_c=d_c, d_r=d_r, tau=gold["tau"])
    torch.cuda.synchronize()
    f = O.bf16_bits_to_f64
    m = case["mla"]
    assert np.array_equal(f(to_host(dq))[:d_c], f(Wqc)[:d_c] * m["q_content"])
    assert np.array_equal(f(to_host(dk))[:d_c], f(Wkc)[:d_c] * m["k_content"])
    assert np.array_equal(f(to_host(dr))[:d_r], f(Wqr)[:d_r] * m["q_rotary"])
    assert np.array_equal(to_host(dq)[d_c:], Wqc[d_c:])
    assert np.array_equal(to_host(dr)[d_r:], Wqr[d_r:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qk_rescale_slices_fused_projection_layout(mm, dev, dtype):
    """Fused projections whose per-head blocks interleave parts: the query
    up-projection holds [content d_c | rotary d_r] per head, the key/value
    up-projection [content key d_c | value d_v] per head.  Three slices give
    the MLA rule; value rows must stay bit-identical."""
    import torch
    H, d_c, d_r, d_v, q_in, kv_in = 5, 128, 64, 128, 192, 136
    say(f"[slices] fused MLA layout dtype={dtype}")
    s = MLA_SMAX[:H].copy()
    g = gen.rng(55)
    Wq = gen._cast(gen.gaussian(g, (H * (d_c + d_r), q_in), 0.05), dtype)
    Wkv = gen._cast(gen.gaussian(g, (H * (d_c + d_v), kv_in), 0.05), dtype)
    dq, dkv = to_dev(Wq, dev), to_dev(Wkv, dev)
    flags = mm.qkclip_rescale_slices([(dq, 0, d_c + d_r, d_c, 0.5), (dq, d_c, d_c + d_r, d_r, 1.0),
                                      (dkv, 0, d_c + d_v, d_c, 0.5)], to_dev(s, dev), tau=100.0)
    torch.cuda.synchronize()
    # de-interleave on the host, apply the oracle, re-interleave
    wq, wkv = widen(Wq, dtype), widen(Wkv, dtype)
    q3 = wq.reshape(H, d_c + d_r, q_in)
    kv3 = wkv.reshape(H, d_c + d_v, kv_in)
    rq, rk, rr, _, _, fl = O.qkclip_rescale_mla(q3[:, :d_c].reshape(H * d_c, q_in),
                                                kv3[:, :d_c].reshape(H * d_c, kv_in),
                                                q3[:, d_c:].reshape(H * d_r, q_in),
                                                np.zeros((d_r, kv_in)), s.astype(np.float64), 100.0, d_c, d_r)
    ref_q = np.concatenate([rq.reshape(H, d_c, q_in), rr.reshape(H, d_r, q_in)], axis=1).reshape(wq.shape)
    ref_kv = np.concatenate([rk.reshape(H, d_c, kv_in), kv3[:, d_c:]], axis=1).reshape(wkv.shape)
    assert list(to_host(flags)) == list(fl)
    value_rows = [slice(h * (d_c + d_v) + d_c, (h + 1) * (d_c + d_v)) for h in range(H)]
    assert_close_weights(to_host(dq), ref_q, Wq, dtype, [])
    assert_close_weights(to_host(dkv), ref_kv, Wkv, dtype, value_rows)


def test_qk_rescale_slices_matches_mha_entry(mm, dev):
    """The MHA entry point is the two-slice case with exponents alpha, 1 - alpha."""
    import torch
    H, d, dm = 4, 64, 72
    say("[slices] MHA equivalence")
    g = gen.rng(8)
    Wq = gen.f32_to_bf16_bits(gen.gaussian(g, (H * d, dm), 0.05))
    Wk = gen.f32_to_bf16_bits(gen.gaussian(g, (H * d, dm), 0.05))
    s = to_dev(np.array([250.0, 50.0, 1000.0, 101.0], dtype=np.float32), dev)
    a1, b1, a2, b2 = (to_dev(x, dev) for x in (Wq, Wk, Wq, Wk))
    mm.qkclip_rescale(a1, b1, s, d_head=d, tau=100.0, alpha=0.3)
    mm.qkclip_rescale_slices([(a2, 0, d, d, 0.3), (b2, 0, d, d, 0.7)], s, tau=100.0)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(a1), to_host(a2)) and np.array_equal(to_host(b1), to_host(b2))


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

ADAMW_SIZES = [1, 7, 8, 2048, 2049, 100003, 300 * 257, 4096 * 64]


def adamw_inputs(g, sizes, dtype, warm):
    ps, gs, ms, vs = [], [], [], []
    for n in sizes:
        ps.append(gen._cast(gen.gaussian(g, (n,), 0.02), dtype))
        gs.append(gen._cast(gen.gaussian(g, (n,), 1e-3), dtype))
        if warm:
            ms.append(gen.gaussian(g, (n,), 1e-3))
            vs.append((gen.gaussian(g, (n,), 1e-3) ** 2).astype(np.float32))
        else:
            ms.append(np.zeros(n, np.float32))
            vs.append(np.zeros(n, np.float32))
    return ps, gs, ms, vs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("step,warm", [(1, False), (7, True)])
def test_adamw_matches_oracle(mm, dev, dtype, step, warm):
    import torch
    say(f"[adamw] dtype={dtype} step={step} sizes={ADAMW_SIZES}")
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    g = gen.rng(100 + step)
    ps, gs, ms, vs = adamw_inputs(g, ADAMW_SIZES, dtype, warm)
    P = [to_dev(x, dev) for x in ps]
    G = [to_dev(x, dev) for x in gs]
    M = [to_dev(x, dev) for x in ms]
    V = [to_dev(x, dev) for x in vs]
    mm.adamw_step(P, G, M, V, step=step, **hp)
    torch.cuda.synchronize()
    for i, n in enumerate(ADAMW_SIZES):
        p0 = widen(ps[i], dtype)
        rp, rm, rv = O.adamw_step(p0, widen(gs[i], dtype), ms[i], vs[i], step=step, **hp)
        assert rel_fro(to_host(M[i]), rm) <= 1e-6, f"exp_avg of tensor {i}"
        assert rel_fro(to_host(V[i]), rv) <= 1e-6, f"exp_avg_sq of tensor {i}"
        got = to_host(P[i])
        if dtype == "f32":
            assert rel_fro(got.astype(np.float64) - p0, rp - p0) <= 1e-5, f"param of tensor {i}"
        else:
            d = bf16_ulp_diff(got, O.f64_to_bf16_bits(rp))
            assert d.max() <= 1, f"param of tensor {i}: {d.max()} bf16 steps"


def test_adamw_many_tensors_and_empty(mm, dev):
    """More tensors than one launch's argument block holds, with empty ones
    mixed in: every tensor is updated exactly once."""
    import torch
    sizes = [0 if i % 17 == 5 else (i * 37) % 3001 for i in range(130)]
    say(f"[adamw] {len(sizes)} tensors")
    hp = dict(lr=1e-3, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.0)
    g = gen.rng(5)
    ps, gs, ms, vs = adamw_inputs(g, sizes, "f32", True)
    P = [to_dev(x, dev) for x in ps]
    G = [to_dev(x, dev) for x in gs]
    M = [to_dev(x, dev) for x in ms]
    V = [to_dev(x, dev) for x in vs]
    mm.adamw_step(P, G, M, V, step=3, **hp)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        rp, rm, rv = O.adamw_step(ps[i], gs[i], ms[i], vs[i], step=3, **hp)
        if sizes[i] == 0:
            continue
        assert rel_fro(to_host(M[i]), rm) <= 1e-6 and rel_fro(to_host(V[i]), rv) <= 1e-6
        assert rel_fro(to_host(P[i]).astype(np.float64) - ps[i], rp - ps[i]) <= 1e-5


def test_adamw_unaligned_views(mm, dev):
    """Views that start one element into their storage take the unvectorised path."""
    import torch
    n = 5000
    say("[adamw] unaligned views")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    g = gen.rng(6)
    ps, gs, ms, vs = adamw_inputs(g, [n + 1], "bf16", True)
    P, G, M, V = (to_dev(x, dev)[1:] for x in (ps[0], gs[0], ms[0], vs[0]))
    mm.adamw_step([P], [G], [M], [V], step=2, **hp)
    torch.cuda.synchronize()
    rp, rm, rv = O.adamw_step(widen(ps[0][1:], "bf16"), widen(gs[0][1:], "bf16"), ms[0][1:], vs[0][1:],
                              step=2, **hp)
    assert rel_fro(to_host(M), rm) <= 1e-6 and rel_fro(to_host(V), rv) <= 1e-6
    assert bf16_ulp_diff(to_host(P), O.f64_to_bf16_bits(rp)).max() <= 1


# ---------------------------------------------------------------------------
# other Newton-Schulz coefficient sets
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["classic_cubic", "simple_quintic"])
@pytest.mark.parametrize("shape", [(96, 160), (300, 600), (520, 260)])
def test_ns_coefficient_variants(mm, dev, name, shape):
    import torch
    coeffs = tuple(json.load(open(os.path.join(GOLDEN, "ns_demo.json")))["coefficients"][name])
    r, c = shape
    say(f"[ns] {name} {coeffs} shape={shape}")
    g = gen.rng(r * 7 + c)
    X = gen.f32_to_bf16_bits(gen.gaussian(g, (2, r, c), 1.0))
    out = mm.ns_orthogonalize(to_dev(X, dev), coeffs=coeffs)
    torch.cuda.synchronize()
    got = O.bf16_bits_to_f64(to_host(out))
    for b in range(2):
        ref = O.newton_schulz(O.bf16_bits_to_f64(X[b]), a=coeffs[0], b=coeffs[1], c=coeffs[2])
        err = rel_fro(got[b], ref)
        say(f"   matrix {b}: rel err {err:.3e}")
        assert err <= 2e-2


def test_muon_step_with_cubic_matches_ns_entry(mm, dev):
    """The full step with the cubic routes through the same two-product
    iteration as ns_orthogonalize: the O it leaves in the workspace equals
    ns_orthogonalize of the same normalised input bit for bit."""
    import torch
    r, c = 200, 330
    say("[step] cubic coefficients")
    g = gen.rng(12)
    W = gen.f32_to_bf16_bits(gen.gaussian(g, (r, c), 0.02))
    G = gen.f32_to_bf16_bits(gen.gaussian(g, (r, c), 1.0))
    Wd, Gd = to_dev(W, dev), to_dev(G, dev)
    Md = torch.zeros((r, c), dtype=torch.float32, device=dev)
    cubic = (1.5, -0.5, 0.0)
    hp = mm.HParams(ns_steps=5, ns_coeffs=cubic, nesterov=False, momentum=0.0)
    groups = [(Wd, Gd, Md)]
    ws = mm.muon_step(groups, hp)
    torch.cuda.synchronize()
    o, _, _ = mm.workspace_views(groups, 0, ws, ns_steps=5)
    O_step = to_host(o)[0]
    O_ns = to_host(mm.ns_orthogonalize(Gd, coeffs=cubic))
    torch.cuda.synchronize()
    assert np.array_equal(O_step, O_ns.reshape(O_step.shape))
    ref = O.newton_schulz(O.bf16_bits_to_f64(G), a=1.5, b=-0.5, c=0.0)
    assert rel_fro(O.bf16_bits_to_f64(O_step), ref) <= 2e-2
