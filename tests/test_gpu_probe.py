"""The matrix-core probe (muon_mfma_probe, not part of the optimizer): both
operand kinds run and leave finite, reproducible per-block sums; an unknown
operand kind is refused before any launch."""
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
