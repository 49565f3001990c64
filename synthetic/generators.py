"""Seeded synthetic inputs for the Muon step and QK-Clip workloads.

This module serves both sides of every parity check (the HIP path and the
fp64 oracle) and therefore holds none of the method's arithmetic: no
momentum, normalisation, Newton-Schulz, scaling, logit maximum or clip
factor.  It only draws seeded random numbers, shapes them into the
workloads' matrices and casts them to the storage formats the workloads name.

Randomness: NumPy PCG64, seed = 1000 * workload + stream, unless a test asks
for another seed.  Bulk fills of the large workloads may instead use torch's
seeded generator on the GPU (`bulk_normal_torch`); those bytes are then
copied to the host whenever the oracle needs them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (input cast)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# matrix recipes
# ----------------------------------------------------------------------------

def gaussian(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def low_rank_plus_noise(g: np.random.Generator, rows: int, cols: int,
                        rank: int = 32, decay: float = 1.5,
                        noise_std: float = 0.01,
                        magnitude: float = 1.0) -> np.ndarray:
    """G = magnitude * (U_r diag(i^-decay) V_r^T + N(0, noise_std^2)),
    U_r, V_r orthonormal (QR of seeded Gaussians), i = 1..rank."""
    r = min(rank, rows, cols)
    Ur, _ = np.linalg.qr(g.standard_normal((rows, r)))
    Vr, _ = np.linalg.qr(g.standard_normal((cols, r)))
    s = np.arange(1, r + 1, dtype=np.float64) ** (-decay)
    G = (Ur * s) @ Vr.T
    G = G.astype(np.float32)
    G += gaussian(g, (rows, cols), noise_std)
    if magnitude != 1.0:
        G *= np.float32(magnitude)
    return G


def with_spectrum(g: np.random.Generator, rows: int, cols: int, sigma) -> np.ndarray:
    """A rows x cols matrix whose singular values are exactly `sigma` (length
    min(rows, cols)) up to float64 rounding: diag(sigma) between two fast
    orthogonal transforms (the orthonormal DCT-II along each side) with
    seeded random sign flips of the rows and columns.  O(rows cols log) work,
    so full-size spectra stay cheap to draw."""
    from scipy.fft import dct
    k = min(rows, cols)
    sigma = np.asarray(sigma, dtype=np.float64)
    assert sigma.shape == (k,)
    Z = np.zeros((rows, cols))
    Z[np.arange(k), np.arange(k)] = sigma
    Z = dct(Z, type=2, norm="ortho", axis=0)
    Z = dct(Z, type=2, norm="ortho", axis=1)
    sr = np.where(g.random(rows) < 0.5, -1.0, 1.0)
    sc = np.where(g.random(cols) < 0.5, -1.0, 1.0)
    return np.ascontiguousarray((Z * sr[:, None]) * sc[None, :])


def log_spaced_levels(k: int, levels: int = 16, cond: float = 1000.0) -> np.ndarray:
    """k singular values on `levels` log-spaced levels from 1 down to 1/cond
    (the interactive Newton-Schulz demo's spread), each level repeated
    k / levels times (the remainder on the top levels)."""
    lv = np.logspace(0.0, -np.log10(cond), levels)
    reps = np.full(levels, k // levels)
    reps[: k % levels] += 1
    return np.repeat(lv, reps)


def partial_permutation(g: np.random.Generator, rows: int, cols: int, sigma):
    """A rows x cols matrix with one nonzero per row of its wide view
    (min(rows, cols) nonzeros, no two in one row or column): the nonzero of
    wide-view row i sits at a seeded distinct position along the long side,
    which always includes the last one, and holds sigma[i] with a seeded sign.
    Returned as (row index, column index, value) arrays in the matrix's own
    layout, so that a full-size matrix never has to exist on the host.  Its
    singular values are |sigma| and its singular vectors coordinate vectors."""
    k, n = min(rows, cols), max(rows, cols)
    sigma = np.asarray(sigma, dtype=np.float64)
    assert sigma.shape == (k,)
    long_idx = g.choice(n, size=k, replace=False)
    if not np.any(long_idx == n - 1):
        long_idx[g.integers(k)] = n - 1
    vals = sigma[g.permutation(k)] * np.where(g.random(k) < 0.5, -1.0, 1.0)
    short_idx = np.arange(k)
    if rows <= cols:
        return short_idx, long_idx.astype(np.int64), vals
    return long_idx.astype(np.int64), short_idx, vals


def zipf_magnitudes(g: np.random.Generator, n: int, s: float = 1.1) -> np.ndarray:
    """Per-expert magnitude rank^-s over a seeded permutation of ranks 1..n
    (the largest is 1)."""
    ranks = g.permutation(n) + 1
    return ranks.astype(np.float64) ** (-s)


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------

@dataclass
class Group:
    """`batch` same-shape matrices [rows, cols] (a PyTorch Linear weight
    layout: rows = fan-out)."""
    name: str
    batch: int
    rows: int
    cols: int


@dataclass
class Workload:
    name: str
    groups: list
    dtype: str                  # parameter and gradient storage: "f32" | "bf16"
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    nesterov: bool = True
    ns_steps: int = 5
    ns_coeffs: tuple = (3.4445, -4.7750, 2.0315)
    ns_eps: float = 1e-7
    rms_target: float = 0.2
    grad_kind: str = "normal"   # "normal" | "lowrank" | "lowrank_zipf"
    weight_std: float = 0.02
    steps: int = 1
    extra: dict = field(default_factory=dict)


def workload(idx: int) -> Workload:
    """The five workloads, 1-based as they are listed."""
    if idx == 1:
        return Workload("single 256x128 fp32 matrix, 10 steps",
                        [Group("W", 1, 256, 128)], "f32", steps=10)
    if idx == 2:
        h = 2048
        return Workload("one transformer layer, hidden 2048",
                        [Group("attn_qkvo", 4, h, h), Group("mlp_up_gate", 2, 4 * h, h),
                         Group("mlp_down", 1, h, 4 * h)], "bf16", grad_kind="lowrank")
    if idx == 3:
        L, h, kv, f = 24, 4096, 1024, 14336
        return Workload("24-layer dense decoder Muon group, hidden 4096",
                        [Group("attn_qo", 2 * L, h, h), Group("attn_kv", 2 * L, kv, h),
                         Group("mlp_up_gate", 2 * L, f, h), Group("mlp_down", L, h, f)],
                        "bf16", grad_kind="normal")
    if idx == 4:
        E = 64
        return Workload("64-expert MoE stack",
                        [Group("expert_up_gate", 2 * E, 2048, 7168),
                         Group("expert_down", E, 7168, 2048)], "bf16",
                        grad_kind="lowrank_zipf")
    if idx == 5:
        d_model, H, dh = 7168, 64, 128
        return Workload("MuonClip attention layer, hidden 7168, 64 heads x 128",
                        [Group("attn_qkv", 3, H * dh, d_model), Group("attn_o", 1, d_model, H * dh)],
                        "bf16", grad_kind="normal",
                        extra=dict(d_model=d_model, heads=H, d_head=dh, batch=4, seq=4096,
                                   tau=100.0, alpha=0.5, n_designated=8,
                                   targets=(120.0, 150.0, 200.0, 300.0, 400.0, 600.0, 1000.0, 2000.0)))
    raise ValueError(idx)


def small_workload(rows_cols=((96, 160), (200, 72), (128, 128)), batch=2, dtype="bf16",
                   seed_name="small") -> Workload:
    """A few-tile workload with ragged shapes for CPU-sized parity checks."""
    gs = [Group(f"g{i}", batch, r, c) for i, (r, c) in enumerate(rows_cols)]
    return Workload(seed_name, gs, dtype)


# ----------------------------------------------------------------------------
# materialisation on the host
# ----------------------------------------------------------------------------

def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def group_params(wl: Workload, gi: int, seed: int) -> np.ndarray:
    grp = wl.groups[gi]
    g = rng(seed * 100 + gi)
    return _cast(gaussian(g, (grp.batch, grp.rows, grp.cols), wl.weight_std), wl.dtype)


def group_momentum(wl: Workload, gi: int, seed: int, warm: bool = True) -> np.ndarray:
    """Initial fp32 momentum: a warm buffer (seeded like a gradient, scale 0.5)
    so the first step exercises mu * M; zeros when warm=False."""
    grp = wl.groups[gi]
    if not warm:
        return np.zeros((grp.batch, grp.rows, grp.cols), dtype=np.float32)
    g = rng(seed * 100 + 50 + gi)
    return gaussian(g, (grp.batch, grp.rows, grp.cols), 0.5)


def group_grads(wl: Workload, gi: int, seed: int, step: int = 0) -> np.ndarray:
    """Gradients in the storage dtype.  'normal': N(0,1); 'lowrank': rank-32
    with singular values i^-1.5 plus N(0, 0.01^2); 'lowrank_zipf': the same
    per expert times a Zipf(1.1) magnitude."""
    grp = wl.groups[gi]
    g = rng(seed * 100000 + step * 100 + 10 + gi)
    shape = (grp.batch, grp.rows, grp.cols)
    if wl.grad_kind == "normal":
        G = gaussian(g, shape, 1.0)
    elif wl.grad_kind in ("lowrank", "lowrank_zipf"):
        mags = zipf_magnitudes(rng(seed * 7 + 3), grp.batch) if wl.grad_kind == "lowrank_zipf" \
            else np.ones(grp.batch)
        G = np.empty(shape, dtype=np.float32)
        for e in range(grp.batch):
            G[e] = low_rank_plus_noise(g, grp.rows, grp.cols, magnitude=float(mags[e]))
    else:
        raise ValueError(wl.grad_kind)
    return _cast(G, wl.dtype)


# ----------------------------------------------------------------------------
# QK-Clip inputs: activations, projections, designated heads
# ----------------------------------------------------------------------------

def expected_gaussian_max(n_pairs: float) -> float:
    """Rough size of the largest of n standard-normal logits, sqrt(2 ln n);
    used only to pick weight scales that put designated heads far above and
    the others far below the threshold."""
    return math.sqrt(2.0 * math.log(n_pairs))


def qk_inputs(seed: int, batch: int, seq: int, heads: int, d_head: int, d_model: int,
              designated: int, targets, causal: bool = True):
    """X_act ~ N(0,1) [batch*seq, d_model]; W_q, W_k ~ N(0, 1/d_model)
    [heads*d_head, d_model]; `designated` seeded heads get their W_q and W_k
    rows multiplied by sqrt(target / m0), with m0 the rough Gaussian maximum,
    so their logit maximum lands near `target`.  All bf16 bit patterns.
    Returns dict(X, Wq, Wk, designated_heads, head_scale)."""
    g = rng(seed)
    X = f32_to_bf16_bits(gaussian(g, (batch * seq, d_model), 1.0))
    std = 1.0 / math.sqrt(d_model)
    Wq = gaussian(g, (heads * d_head, d_model), std)
    Wk = gaussian(g, (heads * d_head, d_model), std)
    heads_sel = np.sort(g.choice(heads, size=designated, replace=False))
    pairs = batch * (seq * (seq + 1) / 2 if causal else seq * seq)
    m0 = expected_gaussian_max(pairs)
    scales = np.ones(heads)
    for h, t in zip(heads_sel, list(targets)[:designated]):
        s = math.sqrt(float(t) / m0)
        scales[h] = s
        Wq[h * d_head:(h + 1) * d_head] *= np.float32(s)
        Wk[h * d_head:(h + 1) * d_head] *= np.float32(s)
    return dict(X=X, Wq=f32_to_bf16_bits(Wq), Wk=f32_to_bf16_bits(Wk),
                designated_heads=heads_sel, head_scale=scales)


def project_host(X_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """The forward's projection Q = X W^T (float32 matmul of the bf16 values,
    result held as bf16), on the host.  Model forward, not the optimizer."""
    return f32_to_bf16_bits(bf16_bits_to_f32(X_bits) @ bf16_bits_to_f32(W_bits).T)


def random_qk(seed: int, batch: int, seq: int, heads: int, d_head: int, std: float = 1.0):
    """Plain Gaussian Q, K [batch, seq, heads, d_head] as bf16 bit patterns."""
    g = rng(seed)
    Q = f32_to_bf16_bits(gaussian(g, (batch, seq, heads, d_head), std))
    K = f32_to_bf16_bits(gaussian(g, (batch, seq, heads, d_head), std))
    return Q, K


# ----------------------------------------------------------------------------
# bulk fills on the GPU (large workloads); torch's seeded generator
# ----------------------------------------------------------------------------

def bulk_normal_torch(shape, std, seed, device, dtype):
    """N(0, std^2) of `shape` drawn on `device` from a torch generator seeded
    with `seed`, cast (nearest-even) to `dtype`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def qk_inputs_torch(seed, batch, seq, heads, d_head, d_model, designated, targets, device,
                    causal=True):
    """The same recipe as qk_inputs, drawn on the GPU: X_act, W_q, W_k (bf16)
    with `designated` seeded heads scaled towards `targets`.  Returns
    dict(X, Wq, Wk, designated_heads)."""
    import torch
    X = bulk_normal_torch((batch * seq, d_model), 1.0, seed, device, torch.bfloat16)
    std = 1.0 / math.sqrt(d_model)
    Wq = bulk_normal_torch((heads * d_head, d_model), std, seed + 1, device, torch.float32)
    Wk = bulk_normal_torch((heads * d_head, d_model), std, seed + 2, device, torch.float32)
    heads_sel = np.sort(rng(seed).choice(heads, size=designated, replace=False))
    pairs = batch * (seq * (seq + 1) / 2 if causal else seq * seq)
    m0 = expected_gaussian_max(pairs)
    for h, t in zip(heads_sel, list(targets)[:designated]):
        s = math.sqrt(float(t) / m0)
        Wq[h * d_head:(h + 1) * d_head] *= s
        Wk[h * d_head:(h + 1) * d_head] *= s
    return dict(X=X, Wq=Wq.to(torch.bfloat16), Wk=Wk.to(torch.bfloat16), designated_heads=heads_sel)


def lowrank_torch(rows, cols, seed, device, rank=32, decay=1.5, noise_std=0.01, magnitude=1.0):
    """low_rank_plus_noise drawn for the GPU: orthonormal factors from NumPy QR
    of seeded Gaussians (host), the rank-r product and the N(0, noise_std^2)
    noise on the device, times `magnitude`, cast to bf16."""
    import torch
    g = rng(seed)
    r = min(rank, rows, cols)
    Ur, _ = np.linalg.qr(g.standard_normal((rows, r)))
    Vr, _ = np.linalg.qr(g.standard_normal((cols, r)))
    s = np.arange(1, r + 1, dtype=np.float64) ** (-decay)
    U = torch.from_numpy((Ur * s).astype(np.float32)).to(device)
    V = torch.from_numpy(Vr.astype(np.float32)).to(device)
    G = U @ V.t()
    G += bulk_normal_torch((rows, cols), noise_std, seed + 1, device, torch.float32)
    if magnitude != 1.0:
        G *= magnitude
    return G.to(torch.bfloat16)
