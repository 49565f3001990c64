"""qkclip_rowmax_noalloc, the entry point for callers that cannot allocate:
called through the C ABI, it must give the same per-head maxima as
qkclip_rowmax (same kernels, so bit for bit) on two calls in a row, the
second smaller than the first (the scratch keeps the first call's partials),
and refuse a size beyond its scratch before launching anything."""
import ctypes
import math
import sys

import numpy as np
import pytest

from synthetic import generators as gen
from tests.gpu_util import to_dev, to_host

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


def rowmax_abi(mm, lib, Q, K, d, causal, noalloc):
    """One call through the C ABI; returns the fp32 [H] result on the host."""
    import torch
    B, T, H, _ = Q.shape
    out = torch.full((H,), -7.0, dtype=torch.float32, device=Q.device)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.qkclip_rowmax_noalloc(Q.data_ptr(), K.data_ptr(), B, T, H, d, 1.0 / math.sqrt(d), int(causal),
                                       out.data_ptr(), stream)
    else:
        need = lib.qkclip_rowmax_workspace_size(B, T, H)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
        st = lib.qkclip_rowmax(Q.data_ptr(), K.data_ptr(), B, T, H, d, 1.0 / math.sqrt(d), int(causal),
                               out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, mm.load_library().muon_status_string(st)
    torch.cuda.synchronize()
    return to_host(out)


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_rowmax_matches_workspace_entry(mm, causal):
    import torch
    lib = mm.load_library()
    dev = torch.device("cuda:0")
    cases = [(2, 1000, 12, 128, 3), (1, 300, 5, 64, 4)]   # the second call is smaller
    for B, T, H, d, seed in cases:
        say(f"[no-alloc rowmax] B={B} T={T} H={H} d={d} causal={causal}")
        Qb, Kb = gen.random_qk(seed, B, T, H, d)
        Q, K = to_dev(Qb, dev), to_dev(Kb, dev)
        ref = rowmax_abi(mm, lib, Q, K, d, causal, noalloc=False)
        got = rowmax_abi(mm, lib, Q, K, d, causal, noalloc=True)
        say(f"   differing heads: {int(np.count_nonzero(got != ref))} of {H}")
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_noalloc_rowmax_refuses_beyond_its_scratch(mm):
    """B * H * ceil(T / 256) one past the scratch (head dim 64 runs 256-query
    blocks): MUON_ERR_WORKSPACE, decided
    on the host before any launch (the tensors are never read)."""
    import torch
    lib = mm.load_library()
    cap = lib.qkclip_rowmax_noalloc_max_partials()
    assert cap == 1 << 18
    dev = torch.device("cuda:0")
    Q = torch.zeros((1, 16, 64, 64), dtype=torch.bfloat16, device=dev)
    out = torch.zeros(64, dtype=torch.float32, device=dev)
    T = 256 * (cap // 64 + 1)
    st = lib.qkclip_rowmax_noalloc(Q.data_ptr(), Q.data_ptr(), 1, T, 64, 64, 0.125, 1, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mm.MUON_ERR_WORKSPACE
    assert float(out.abs().max()) == 0.0
