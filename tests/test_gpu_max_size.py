"""GPU parity at the largest matrices the boundary accepts.

A matrix may hold up to about 2^31 elements: every side at most 2^20 and the
padded wide view (max(rows, cols) + 256) x (min(rows, cols) + 256) at most
2^31 elements.  Element indices then come close to 2^31 and byte offsets pass
it (2^32 for the fp32 momentum), so 32-bit index arithmetic anywhere on the
path would misplace, drop or fault on elements.

At that size the oracle cannot run Newton-Schulz on the whole matrix.  The
inputs are therefore scaled partial permutations: one nonzero per row of the
wide view, at distinct columns (including the last), with magnitudes on the
16 log-spaced levels of the Newton-Schulz demo (condition number 1000) and
random signs.  Such a matrix is U diag(s) V^T with coordinate vectors U and V,
so X X^T and A A are diagonal, every other element stays exactly zero, and
each nonzero x follows the scalar map of the iteration; the oracle's iteration
on the 1 x 1 matrix [[x / ||G||_F]] is the exact expected value of that
element (tests/test_oracle_ns.py pins this against the oracle's full-matrix
iteration on small matrices).  The GPU output must hold exactly
min(rows, cols) nonzeros, at the input's positions, their values within the
stated 2e-2 relative Frobenius error.  The Muon step also checks the momentum
(every element), 1 / ||U||_F and the parameter update at the nonzeros and at
a seeded sample of other positions, where the update is the pure decay.
"""
import math
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from synthetic import generators as gen
from tests.gpu_util import rel_fro, to_host
from tests.test_gpu_parity import w_excess

pytestmark = pytest.mark.gpu

TUNED = (3.4445, -4.7750, 2.0315)
NEED_BYTES = 60 << 30   # inputs, outputs and workspace of the largest case, with margin


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info(0)
    if free < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES >> 30} GiB of free device memory")
    import matrix_orthogonalizing_optimizer_muon_amd as m
    m.load_library()
    return m


def structured(rows, cols, seed):
    """Seeded partial permutation: (row idx, col idx, bf16-rounded values)."""
    g = gen.rng(seed)
    ri, ci, v = gen.partial_permutation(g, rows, cols, gen.log_spaced_levels(min(rows, cols)))
    vb = O.bf16_bits_to_f64(O.f64_to_bf16_bits(v))
    return ri, ci, vb


def place(shape, ri, ci, vals, dtype, dev):
    """A dense device tensor of `shape`, zero except vals at (ri, ci)."""
    import torch
    t = torch.zeros(shape, dtype=dtype, device=dev)
    t[torch.from_numpy(ri).to(dev), torch.from_numpy(ci).to(dev)] = torch.from_numpy(vals).to(dev, dtype)
    return t


def expected_ns(vals, eps=1e-7, steps=5):
    """The oracle's iteration on each normalised nonzero alone."""
    x = O.frobenius_normalize(np.asarray(vals, dtype=np.float64)[None, :], eps)[0]
    return np.array([O.newton_schulz_iterate(np.array([[t]]), steps, *TUNED)[0, 0] for t in x])


def check_pattern(out, ri, ci, k):
    """Exactly k nonzeros, all at (ri, ci); returns the values there."""
    import torch
    idx_r = torch.from_numpy(ri).to(out.device)
    idx_c = torch.from_numpy(ci).to(out.device)
    got = out[idx_r, idx_c].float()
    nnz = int(torch.count_nonzero(out).item())
    at = int(torch.count_nonzero(got).item())
    say(f"   nonzeros {nnz} (expected {k}), of which at the input's positions {at}")
    assert nnz == k and at == k
    return got.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("rows,cols", [(8192, 253944), (253944, 8192), (46084, 46084)])
def test_ns_at_the_element_limit(mm, rows, cols):
    import torch
    dev = torch.device("cuda:0")
    say(f"[ns max size] {rows}x{cols} bf16, partial permutation")
    ri, ci, v = structured(rows, cols, rows + 3 * cols)
    X = place((rows, cols), ri, ci, v, torch.bfloat16, dev)
    out = mm.ns_orthogonalize(X)
    torch.cuda.synchronize()
    del X
    got = check_pattern(out, ri, ci, min(rows, cols))
    del out
    err = rel_fro(got, expected_ns(v))
    say(f"   rel err vs oracle {err:.3e}")
    assert err <= 2e-2


def test_muon_step_at_the_element_limit(mm):
    import torch
    dev = torch.device("cuda:0")
    rows, cols = 8192, 253944
    hp = mm.HParams()
    say(f"[muon_step max size] {rows}x{cols} bf16 params, partial-permutation grad and momentum")
    ri, ci, gv = structured(rows, cols, 71)
    mv = gen.rng(72).standard_normal(len(gv)).astype(np.float32).astype(np.float64)
    W = gen.bulk_normal_torch((rows, cols), 0.02, 73, dev, torch.bfloat16)
    G = place((rows, cols), ri, ci, gv, torch.bfloat16, dev)
    M = place((rows, cols), ri, ci, mv, torch.float32, dev)
    # a seeded sample of the dense update, plus the structure's positions and
    # the matrix's last element
    g = gen.rng(74)
    sr = np.concatenate([g.integers(0, rows, 1 << 20), ri, [rows - 1]])
    sc = np.concatenate([g.integers(0, cols, 1 << 20), ci, [cols - 1]])
    tr, tc = torch.from_numpy(sr).to(dev), torch.from_numpy(sc).to(dev)
    W0 = O.bf16_bits_to_f64(to_host(W[tr, tc]))
    ws = mm.muon_step([(W, G, M)], hp)
    o, inv, _ = mm.workspace_views([(W, G, M)], 0, ws, hp.ns_steps)
    torch.cuda.synchronize()
    del G

    # momentum: exactly the structure, holding the fp32 result of mu M + G
    Mr = O.momentum_update(mv, gv, hp.momentum)
    em = rel_fro(check_pattern(M, ri, ci, rows), Mr)
    del M
    U = O.nesterov_lookahead(Mr, gv, hp.momentum, hp.nesterov)
    inv_ref = 1.0 / (np.linalg.norm(U) + hp.ns_eps)
    einv = abs(float(to_host(inv)[0]) - inv_ref) / inv_ref
    # Newton-Schulz output: exactly the structure, each value the scalar map
    og = check_pattern(o[0], ri, ci, rows)
    eo = rel_fro(og, expected_ns(U, hp.ns_eps, hp.ns_steps))
    # update given the GPU's own O: pure decay away from the structure
    Os = O.bf16_bits_to_f64(to_host(o[0][tr, tc]))
    s = O.update_scale(rows, cols, hp.scale_mode, hp.rms_target)
    Wr = O.param_update(W0, Os, hp.lr, hp.weight_decay, s)
    ew = w_excess(to_host(W[tr, tc]), Wr, W0, Os, hp, s)
    say(f"   momentum {em:.2e}  1/|U| {einv:.2e}  O {eo:.3e}  W outside bound {ew} of {len(sr)}")
    assert em <= 1e-5
    assert einv <= 1e-5
    assert eo <= 2e-2
    assert ew == 0


# ---------------------------------------------------------------------------
# S_max past 2^31 elements of Q and K
# ---------------------------------------------------------------------------

def plant(Q, K, h, i, j, vq, vk):
    import torch
    Q[0, i, h] = torch.from_numpy(vq).to(Q.device, Q.dtype)
    K[0, j, h] = torch.from_numpy(vk).to(K.device, K.dtype)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_qk_rowmax_long_context(mm, d):
    """One batch row of 131072 tokens and 16384 / d heads: Q and K hold 2^31
    elements each, so byte offsets reach 2^32.  Q and K are N(0, 1/256) apart
    from two planted pairs per head: an allowed pair (j <= i) whose logit is
    d, and a masked pair (j > i) whose logit is 2.25 d.  Cauchy-Schwarz on the
    measured row norms bounds every other logit below d, so the causal
    statistic is exactly d * logit_scale and the unmasked one 2.25 d *
    logit_scale (integer sums of products of +-1 and +-1.5, exact in fp32).
    Head 0 places its allowed pair at the farthest distance (i = T - 1,
    j = 0) and head 1 on the last diagonal element.  At d = 128 the
    attention forward's S_max export is held to the same value."""
    import torch
    dev = torch.device("cuda:0")
    B, T, H = 1, 131072, 16384 // d
    say(f"[qk long context] B={B} T={T} H={H} d={d}")
    Q = gen.bulk_normal_torch((B, T, H, d), 1.0 / 16, 81 + d, dev, torch.bfloat16)
    K = gen.bulk_normal_torch((B, T, H, d), 1.0 / 16, 82 + d, dev, torch.bfloat16)
    g = gen.rng(83 + d)
    planted = []
    for h in range(H):
        if h == 0:
            i, j = T - 1, 0
        elif h == 1:
            i, j = T - 1, T - 1
        else:
            i = int(g.integers(0, T))
            j = int(g.integers(0, i + 1))
        # the masked pair takes other rows of Q and K than the allowed one
        i2, j2 = i, j
        while i2 == i or j2 == j:
            i2 = int(g.integers(0, T - 1))
            j2 = int(g.integers(i2 + 1, T))
        v = np.where(g.random(d) < 0.5, -1.0, 1.0)
        w = 1.5 * np.where(g.random(d) < 0.5, -1.0, 1.0)
        plant(Q, K, h, i, j, v, v)
        plant(Q, K, h, i2, j2, w, w)
        planted.append((i, j, i2, j2, v, w))
    # Cauchy-Schwarz bound on every pair other than the two planted ones
    qn = Q.float().norm(dim=3)   # [B, T, H]
    kn = K.float().norm(dim=3)
    for h, (i, j, i2, j2, v, w) in enumerate(planted):
        qn[0, i, h] = 0.0
        qn[0, i2, h] = 0.0
        kn[0, j, h] = 0.0
        kn[0, j2, h] = 0.0
    bq, bk = float(qn.max()), float(kn.max())
    del qn, kn
    big = 1.5 * math.sqrt(d)
    for i, j, i2, j2, v, w in planted:
        cross = [abs(float(v @ w))] * 2     # q_i . k_j2 and q_i2 . k_j
        bound = max(bq * bk, big * bq, big * bk, *cross)
        assert bound < 0.9 * d, (bound, d)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    want_c = np.float32(np.float32(scale) * np.float32(d))
    want_n = np.float32(np.float32(scale) * np.float32(2.25 * d))
    got_c = to_host(mm.qkclip_rowmax(Q, K, scale, True))
    got_n = to_host(mm.qkclip_rowmax(Q, K, scale, False))
    torch.cuda.synchronize()
    say(f"   causal {got_c.min():.6g}..{got_c.max():.6g} (want {want_c:.6g}); "
        f"unmasked {got_n.min():.6g}..{got_n.max():.6g} (want {want_n:.6g})")
    assert np.all(got_c == want_c)
    assert np.all(got_n == want_n)
    if d == 128:
        # the attention forward's S_max export reads the same logits (K as V)
        _, sm, _ = mm.attn_fwd(Q, K, K, scale, True)
        got_a = to_host(sm)
        torch.cuda.synchronize()
        say(f"   attention causal {got_a.min():.6g}..{got_a.max():.6g}")
        assert np.all(got_a == want_c)
