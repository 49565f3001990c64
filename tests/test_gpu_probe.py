"""The measurement probes (not part of the optimizer).  The matrix-core probe
(muon_mfma_probe): both operand kinds run and leave finite, reproducible
per-block sums; an unknown operand kind is refused before any launch.  The
HBM stream probe (muon_hbm_probe): every written chunk is the XOR of its
unit's loads with the chunk index in the first word, for every supported
mix and both launch shapes, with the unit count taken from the smaller
stream and ragged tails (3000 units is not a multiple of 1024)."""
import sys

import numpy as np
import pytest

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


@pytest.mark.parametrize("kind", ["random", "smooth"])
def test_probe_runs_and_is_reproducible(mm, kind):
    import torch
    dev = torch.device("cuda:0")
    operands = mm.PROBE_RANDOM if kind == "random" else mm.PROBE_SMOOTH
    blocks, iters = 64, 4
    say(f"[probe] {kind} operands, {blocks} blocks x {iters} iterations")
    runs = []
    for _ in range(2):
        sink = torch.full((blocks,), float("nan"), dtype=torch.float32, device=dev)
        flop = mm.mfma_probe(blocks, iters, sink, operands)
        torch.cuda.synchronize()
        runs.append(sink.cpu().numpy())
    assert flop == blocks * 4 * 32 * iters * 32768
    assert np.all(np.isfinite(runs[0]))
    assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))
    if kind == "smooth":
        # every operand is positive, so every accumulated product is too
        assert np.all(runs[0] > 0)


def test_probe_refuses_unknown_operand_kind(mm):
    import torch
    sink = torch.zeros(4, dtype=torch.float32, device=torch.device("cuda:0"))
    with pytest.raises(Exception):
        mm.mfma_probe(4, 1, sink, 7)


@pytest.mark.parametrize("unroll", [1, 4])
@pytest.mark.parametrize("reads,writes,units,spare_src,spare_dst", [(3, 4, 1000, 40, 0), (2, 1, 777, 0, 48),
                                                                   (1, 1, 256, 16, 8), (1, 1, 3000, 0, 0)])
def test_hbm_probe_writes_the_xor_of_its_loads(mm, reads, writes, units, spare_src, spare_dst, unroll):
    import torch
    dev = torch.device("cuda:0")
    say(f"[hbm probe] reads={reads} writes={writes} units={units} unroll={unroll}")
    g = np.random.default_rng(units)
    src_h = g.integers(0, 2 ** 32, size=(reads * units * 16 + spare_src) // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).to(dev)
    dst = torch.zeros((writes * units * 16 + spare_dst) // 4, dtype=torch.int32, device=dev)
    moved = mm.hbm_probe(src, dst, reads, writes, unroll)
    torch.cuda.synchronize()
    assert moved == units * 16 * (reads + writes)
    chunks = src_h[: reads * units * 4].reshape(reads, units, 4)
    x = np.bitwise_xor.reduce(chunks, axis=0)
    got = dst.cpu().numpy().view(np.uint32)
    for k in range(writes):
        want = x.copy()
        want[:, 0] ^= np.uint32(k)
        assert np.array_equal(got[k * units * 4:(k + 1) * units * 4].reshape(units, 4), want), k
    assert np.all(got[writes * units * 4:] == 0)   # nothing past the last unit


def test_hbm_probe_refuses_other_mixes(mm):
    import torch
    dev = torch.device("cuda:0")
    a = torch.zeros(1024, dtype=torch.int32, device=dev)
    b = torch.zeros(1024, dtype=torch.int32, device=dev)
    with pytest.raises(Exception):
        mm.hbm_probe(a, b, 2, 2)
    with pytest.raises(Exception):
        mm.hbm_probe(a, b, 1, 1, 2)
