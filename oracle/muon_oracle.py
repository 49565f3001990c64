"""fp64 CPU oracle for the Muon optimizer step and MuonClip's QK-Clip.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
constant table or helper with that path.

Everything here is plain NumPy in float64: one matrix at a time, library
matmuls as the only primitive, no blocking, fusion or reordering beyond the
definitions on the pages.  Inputs are widened exactly from the bytes the GPU
receives (bf16 bit patterns or float32 values).

Sources (web pages, cited by title and section):
  [MC]  "MuonClip" (manishklach.github.io), sections "02 / Muon from first
        principles", "03 / Making Muon scale", "05 / QK-Clip",
        "06 / Multi-head latent attention changes the surgery",
        "07 / One complete training step".
  [MM]  "Muon and MuonClip: orthogonalised updates for LLM training"
        (fernfant.github.io), section 2, subsections "Newton-Schulz: an odd
        polynomial on singular values", "The Muon optimizer",
        "The exploding-logit problem", "MuonClip: QK-clip, per head, adapted
        to MLA".
  [MS]  "About Muon: Muon At Scale" (kiungsong.github.io), sections
        "Why Not Bernstein's Multiplier?", "When Softmax Collapses",
        "What Breaks at Scale" (subsection "The Matrix Does Not Fit": Dion).

Readings taken where the pages are silent:
  * Nesterov lookahead: U = G + mu * M_new (sum-form momentum, [MC] 02 says a
    lookahead "may be applied" without giving its form).
  * Normalisation epsilon: X0 = X / (||X||_F + eps), eps = 1e-7 ([MM] writes
    X0 = G / ||G||_F; eps only guards a zero gradient).
  * Orientation: the iteration runs on the transpose when rows > cols, so the
    Gram matrix X X^T is the smaller side ([MC] 02 "cheaper orientation",
    [MM] cost paragraph with m <= n).
  * Update: W <- (1 - lr*wd) * W - lr * scale * O with the pre-update W in
    the decay term, one rounding to the parameter dtype at the end.
  * S_max: signed maximum of q_i . k_j * logit_scale over the batch and the
    causal pairs j <= i (diagonal included), per head.
  * Clip tie/non-finite: a head is clipped iff S_max > tau; a NaN/Inf S_max
    leaves the weights untouched and is flagged -1.
  * Dion: "orthogonalize P" is the Q factor of the thin QR with a positive
    diagonal; ColNorm leaves a zero column zero; the update X - lr P Q'^T has
    no scale factor or weight decay (the pages write none); Q is state the
    caller keeps between steps (the warm start).

Pins: every function here is checked in tests/test_oracle_*.py against
closed forms, printed worked examples, textbook special cases and brute force
(see the header of each test file).  None is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats.  bf16 is the top half of an IEEE binary32; widening is
# exact, narrowing rounds to nearest, ties to even.
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even), returned as bit patterns.

    Rounds once, directly from float64: the magnitude is scaled by a power of
    two onto bf16's integer significand grid (8 significant bits for normals,
    quantum 2^-133 for subnormals), rounded with np.rint (ties to even), and
    scaled back.  All scalings are exact.  Overflow gives +-inf, NaN a quiet
    NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(invalid="ignore", over="ignore"):
        v = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    v = np.where(np.isfinite(a), v, a)
    v = np.where(v >= 2.0 ** 128, np.inf, v)
    with np.errstate(over="ignore"):
        bits = (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits | (np.signbit(x).astype(np.uint16) << np.uint16(15))


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to binary32 (round to nearest even, NumPy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# Muon: momentum, Newton-Schulz, scale, decoupled weight decay.
# ---------------------------------------------------------------------------


def momentum_update(M: np.ndarray, G: np.ndarray, mu: float) -> np.ndarray:
    """M_t = mu * M_{t-1} + G_t  ([MC] 02, momentum equation; [MM] "The Muon
    optimizer", SGD momentum line).  Sum form, no dampening."""
    return mu * M + G


def nesterov_lookahead(M_new: np.ndarray, G: np.ndarray, mu: float,
                       nesterov: bool) -> np.ndarray:
    """The matrix handed to Newton-Schulz.  With the lookahead ([MC] 02: "a
    Nesterov-style lookahead may be applied") it is G + mu * M_t; without it,
    the momentum itself."""
    return G + mu * M_new if nesterov else M_new


def to_wide(U: np.ndarray) -> tuple[np.ndarray, bool]:
    """Orientation: iterate on the side whose Gram matrix is smaller.  Returns
    (X, transposed) with X of shape m x n, m <= n ([MC] 02 quintic step note
    "after choosing the cheaper orientation"; [MM] cost for n x m, m <= n)."""
    if U.shape[0] > U.shape[1]:
        return U.T, True
    return U, False


def frobenius_normalize(X: np.ndarray, eps: float) -> np.ndarray:
    """X_0 = X / (||X||_F + eps): every singular value lands in (0, 1]
    ([MM] Newton-Schulz pseudocode, first line; self-check on dividing by the
    Frobenius norm)."""
    return X / (np.linalg.norm(X, "fro") + eps)


def newton_schulz_iterate(X: np.ndarray, steps: int, a: float, b: float,
                          c: float) -> np.ndarray:
    """Odd-polynomial Newton-Schulz iteration on an m x n matrix (m <= n):
        A = X X^T ;  B = b A + c A A ;  X <- a X + B X
    repeated `steps` times ([MM] "Newton-Schulz: an odd polynomial on singular
    values"; [MC] 02 "quintic NS step").  Each step maps every singular value
    s to a s + b s^3 + c s^5 and keeps the singular vectors."""
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def newton_schulz(U: np.ndarray, steps: int = 5, a: float = 3.4445,
                  b: float = -4.7750, c: float = 2.0315,
                  eps: float = 1e-7) -> np.ndarray:
    """Approximate orthogonalisation of one matrix, in its own layout:
    orient wide, Frobenius-normalise, iterate, orient back."""
    X, transposed = to_wide(np.asarray(U, dtype=np.float64))
    X = frobenius_normalize(X, eps)
    X = newton_schulz_iterate(X, steps, a, b, c)
    return X.T if transposed else X


def update_scale(rows: int, cols: int, mode: str = "moonlight",
                 rms_target: float = 0.2) -> float:
    """Multiplier on the orthogonalised update.
    moonlight: rms_target * sqrt(max(rows, cols))  ([MC] 03 "orthogonalized
               direction"; [MM] scaling-up paragraph; [MS] "Why Not
               Bernstein's Multiplier?").
    spectral:  sqrt(fan_out / fan_in) = sqrt(rows / cols)  ([MS], Bernstein
               bullet; rows = fan-out of a Linear weight).
    none:      1."""
    if mode == "moonlight":
        return rms_target * math.sqrt(max(rows, cols))
    if mode == "spectral":
        return math.sqrt(rows / cols)
    if mode == "none":
        return 1.0
    raise ValueError(mode)


def param_update(W: np.ndarray, O: np.ndarray, lr: float, wd: float,
                 scale: float) -> np.ndarray:
    """Decoupled weight decay plus the scaled direction:
        W_t = W_{t-1} - lr * (scale * O_t + wd * W_{t-1})
    ([MC] 03 "decoupled decay" equation with O_t = NS(M_t) * scale; [MC] 07
    pseudocode; [MS] update fragment: multiply by 1 - lr*wd, add -lr*scale*O).
    """
    return (1.0 - lr * wd) * W - lr * scale * O


def muon_step(W: np.ndarray, M: np.ndarray, G: np.ndarray, *, lr: float,
              momentum: float, weight_decay: float, nesterov: bool = True,
              ns_steps: int = 5, ns_coeffs=(3.4445, -4.7750, 2.0315),
              ns_eps: float = 1e-7, scale_mode: str = "moonlight",
              rms_target: float = 0.2):
    """One Muon step on one matrix in float64 ([MC] 07 pseudocode order:
    momentum -> Newton-Schulz -> scale + decay).  Returns (W_new, M_new, O)
    with O the orthogonalised direction before scaling, in W's layout."""
    W = np.asarray(W, dtype=np.float64)
    M_new = momentum_update(np.asarray(M, dtype=np.float64),
                            np.asarray(G, dtype=np.float64), momentum)
    U = nesterov_lookahead(M_new, np.asarray(G, dtype=np.float64), momentum,
                           nesterov)
    a, b, c = ns_coeffs
    O = newton_schulz(U, ns_steps, a, b, c, ns_eps)
    s = update_scale(W.shape[0], W.shape[1], scale_mode, rms_target)
    W_new = param_update(W, O, lr, weight_decay, s)
    return W_new, M_new, O


# ---------------------------------------------------------------------------
# QK-Clip.
# ---------------------------------------------------------------------------


def smax_per_head(Q: np.ndarray, K: np.ndarray, logit_scale: float,
                  causal: bool = True) -> np.ndarray:
    """S_max^h = logit_scale * max over batch rows b and token pairs (i, j)
    of q_{b,i}^h . k_{b,j}^h, with j <= i when causal ([MM] "The exploding-
    logit problem", S_max definition with 1/sqrt(d); [MC] 05 per-head signal).

    Q, K: [B, T, H, d] (any real dtype; widened to float64).  Returns [H]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, T, H, _ = Q.shape
    out = np.full(H, -np.inf)
    mask = np.tril(np.ones((T, K.shape[1]), dtype=bool)) if causal else None
    for h in range(H):
        best = -np.inf
        for b in range(B):
            S = (Q[b, :, h, :] @ K[b, :, h, :].T) * logit_scale
            if causal:
                S = np.where(mask, S, -np.inf)
            m = S.max()
            if np.isnan(S).any():
                m = np.nan
            best = np.nan if (np.isnan(best) or np.isnan(m)) else max(best, m)
        out[h] = best
    return out


def qkclip_factors(s_max: np.ndarray, tau: float):
    """gamma_h = min(1, tau / S_max^h) ([MC] 05 adaptive factor; [MM]
    MuonClip section; [MS] "When Softmax Collapses").  Returns (gamma, flag)
    with flag 1 = clipped (S_max > tau), 0 = untouched, -1 = non-finite S_max
    (untouched)."""
    s_max = np.asarray(s_max, dtype=np.float64)
    gamma = np.ones_like(s_max)
    flag = np.zeros(s_max.shape, dtype=np.int32)
    finite = np.isfinite(s_max)
    clip = finite & (s_max > tau)
    gamma[clip] = tau / s_max[clip]
    flag[clip] = 1
    flag[~finite] = -1
    return gamma, flag


def qkclip_rescale(Wq: np.ndarray, Wk: np.ndarray, s_max: np.ndarray,
                   tau: float, alpha: float, d_head: int):
    """Balanced MHA rescale: rows of head h in W_q times gamma^alpha, in W_k
    times gamma^(1 - alpha) ([MC] 05 balanced rescale; [MM] MuonClip MHA
    line; [MS] "When Softmax Collapses").  Head h owns rows
    [h*d_head, (h+1)*d_head) of W_q and W_k ([H*d_head, d_model], the rows
    that produce q^h and k^h).  Momentum is not touched ([MC] 07).
    Returns (Wq_new, Wk_new, gamma, flag), float64."""
    Wq = np.array(Wq, dtype=np.float64)
    Wk = np.array(Wk, dtype=np.float64)
    gamma, flag = qkclip_factors(s_max, tau)
    for h in range(len(gamma)):
        if flag[h] != 1:
            continue
        rows = slice(h * d_head, (h + 1) * d_head)
        Wq[rows] *= gamma[h] ** alpha
        Wk[rows] *= gamma[h] ** (1.0 - alpha)
    return Wq, Wk, gamma, flag


def qkclip_rescale_mla(Wqc: np.ndarray, Wkc: np.ndarray, Wqr: np.ndarray,
                       Wkr: np.ndarray, s_max: np.ndarray, tau: float,
                       d_c: int, d_r: int):
    """MLA variant ([MC] 06; [MM] MuonClip MLA lines): per head, the content
    query and content key rows scale by sqrt(gamma), the rotary query rows by
    gamma, and the shared rotary key is left as is.  Head h owns rows
    [h*d_c, (h+1)*d_c) of Wqc and Wkc and rows [h*d_r, (h+1)*d_r) of Wqr.
    Returns (Wqc, Wkc, Wqr, Wkr, gamma, flag), float64."""
    Wqc = np.array(Wqc, dtype=np.float64)
    Wkc = np.array(Wkc, dtype=np.float64)
    Wqr = np.array(Wqr, dtype=np.float64)
    Wkr = np.array(Wkr, dtype=np.float64)
    gamma, flag = qkclip_factors(s_max, tau)
    for h in range(len(gamma)):
        if flag[h] != 1:
            continue
        g = gamma[h]
        Wqc[h * d_c:(h + 1) * d_c] *= math.sqrt(g)
        Wkc[h * d_c:(h + 1) * d_c] *= math.sqrt(g)
        Wqr[h * d_r:(h + 1) * d_r] *= g
    return Wqc, Wkc, Wqr, Wkr, gamma, flag


# ---------------------------------------------------------------------------
# The attention forward that the per-head statistic comes from.
# ---------------------------------------------------------------------------


def attention_forward(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                      logit_scale: float, causal: bool = True):
    """Softmax attention per batch row b and head h, float64: logits
    s_ij = logit_scale * q_i . k_j (j <= i when causal), output
    o_i = sum_j softmax_j(s_ij) v_j, log-sum-exp lse_i = log sum_j exp(s_ij),
    and the per-head maximum logit of smax_per_head.  The pages take S_max
    from this forward ([MC] 05: the per-head signal is read off the forward's
    logits; [MM] "The exploding-logit problem": the logits that feed the
    softmax), so it is the same maximum.

    Q, K, V: [B, T, H, d].  Returns (O [B, T, H, d], lse [B, H, T], s_max [H])."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, T, H, d = Q.shape
    O = np.zeros((B, T, H, V.shape[3]))
    lse = np.zeros((B, H, T))
    mask = np.tril(np.ones((T, T), dtype=bool)) if causal else np.ones((T, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            S = (Q[b, :, h, :] @ K[b, :, h, :].T) * logit_scale
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            O[b, :, h, :] = (P @ V[b, :, h, :]) / l
            lse[b, h, :] = (m + np.log(l))[:, 0]
    return O, lse, smax_per_head(Q, K, logit_scale, causal)


# ---------------------------------------------------------------------------
# AdamW, the companion optimizer for the parameters Muon does not take.
# ---------------------------------------------------------------------------


def adamw_step(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, *,
               lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int):
    """One decoupled AdamW step, float64 ("MuonClip" section 03 and section 07
    pseudocode route embeddings, the head and 1-D parameters to AdamW; the
    pages name it without writing it out, so this is the standard decoupled
    form): p <- p (1 - lr wd); m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
    p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
    `step` is t >= 1 (the step being taken).  Returns (p, m, v)."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    p = p * (1.0 - lr * weight_decay) - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


# ---------------------------------------------------------------------------
# Dion: the rank-r orthonormalised update ([MS] "What Breaks at Scale",
# subsection "The Matrix Does Not Fit").
# ---------------------------------------------------------------------------


def orthonormal_basis(P0: np.ndarray) -> np.ndarray:
    """The Q factor of the thin QR of P0 with a non-negative diagonal of R:
    the Gram-Schmidt basis of P0's columns in order.  [MS] says "orthogonalize
    P" without naming the method; this is the plainest reading and the basis
    every QR or Cholesky-QR variant converges to.  Library QR as the step."""
    Qf, Rf = np.linalg.qr(np.asarray(P0, dtype=np.float64), mode="reduced")
    sgn = np.sign(np.diag(Rf))
    sgn[sgn == 0] = 1.0
    return Qf * sgn[None, :]


def column_normalize(R: np.ndarray) -> np.ndarray:
    """ColNorm: every column divided by its l2 norm; a zero column stays zero
    (the pages give no epsilon)."""
    R = np.asarray(R, dtype=np.float64)
    nrm = np.linalg.norm(R, axis=0)
    safe = np.where(nrm > 0.0, nrm, 1.0)
    return np.where(nrm[None, :] > 0.0, R / safe[None, :], 0.0)


def dion_step(X: np.ndarray, G: np.ndarray, M: np.ndarray, Q: np.ndarray, *,
              mu: float, lr: float):
    """One Dion step on an m x n matrix with rank-r state Q (n x r), float64:
        B = M + G
        P = orth(B Q)                 (one warm-started power step ...
        R = B^T P                      ... PowerIter_1(B; Q))
        M' = B - (1 - mu) P R^T       (error feedback: the rank-r piece leaves M)
        Q' = ColNorm(R)
        X' = X - lr P Q'^T
    in the pages' order and notation.  No scale factor or weight decay: the
    pages' update has neither.  Returns (X', M', Q', P, R)."""
    X = np.asarray(X, dtype=np.float64)
    B = np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    P = orthonormal_basis(B @ np.asarray(Q, dtype=np.float64))
    R = B.T @ P
    M_new = B - (1.0 - mu) * (P @ R.T)
    Q_new = column_normalize(R)
    X_new = X - lr * (P @ Q_new.T)
    return X_new, M_new, Q_new, P, R
