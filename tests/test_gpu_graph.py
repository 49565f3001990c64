"""HIP graph capture of the path: the library launches only kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a whole
MuonClip step, and the companion entry points (the allocation-free S_max
pass, the attention forward, AdamW, Dion), can be captured once and
replayed.  Each replay is checked bit for bit against the same number of
eager calls on identical inputs, with eager work and synchronisations
between the replays."""
import math
import sys

import numpy as np
import pytest

from synthetic import generators as gen
from tests.gpu_util import to_dev

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


def make_state(dev):
    import torch
    g = gen.rng(21)
    W1 = to_dev(gen.gaussian(g, (256, 128), 0.02), dev)
    G1 = to_dev(gen.gaussian(g, (256, 128), 1.0), dev)
    M1 = torch.zeros((256, 128), dtype=torch.float32, device=dev)
    W2 = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 300, 520), 0.02)), dev)
    G2 = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 300, 520), 1.0)), dev)
    M2 = to_dev(gen.gaussian(g, (2, 300, 520), 0.5), dev)
    H, d, dm = 4, 128, 256
    Wq = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (H * d, dm), 0.05)), dev)
    Wk = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (H * d, dm), 0.05)), dev)
    Q = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 192, H, d), 1.0)), dev)
    K = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 192, H, d), 1.0)), dev)
    Q[:, :, 1] *= 40.0      # head 1 exceeds tau
    return [W1, G1, M1, W2, G2, M2, Wq, Wk, Q, K]


def test_captured_step_replays_match_eager(mm):
    import torch
    dev = torch.device("cuda:0")
    say("[graph] capture one MuonClip step (S_max, two Muon groups, rescale), replay 3 times")
    eager = make_state(dev)
    static = [t.clone() for t in eager]
    hp = mm.HParams(lr=0.02, momentum=0.95, weight_decay=0.1)

    def buffers(st):
        W1, G1, M1, W2, G2, M2, Wq, Wk, Q, K = st
        return [(W1, G1, M1)], [(W2, G2, M2)], Wq, Wk, Q, K

    def make_step(st):
        g1, g2, Wq, Wk, Q, K = buffers(st)
        ws1 = torch.empty(mm.workspace_size(g1), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(mm.workspace_size(g2), dtype=torch.uint8, device=dev)
        rws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
        s_max = torch.empty(4, dtype=torch.float32, device=dev)
        flags = torch.empty(4, dtype=torch.int32, device=dev)

        def step():
            mm.qkclip_rowmax(Q, K, 1.0 / math.sqrt(128), True, out=s_max, workspace=rws)
            mm.muon_step(g1, hp, workspace=ws1)
            mm.muon_step(g2, hp, workspace=ws2)
            mm.qkclip_rescale(Wq, Wk, s_max, 128, 100.0, 0.5, clipped=flags)
        return step, flags

    eager_step, eager_flags = make_step(eager)
    graph_step, graph_flags = make_step(static)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        graph_step()
    torch.cuda.synchronize()
    # capture records without running: the static state is still the initial one
    for t_e, t_s in zip(eager, static):
        assert torch.equal(t_e, t_s)
    x = torch.randn(512, 512, device=dev)
    for rep in range(3):
        eager_step()
        _ = x @ x                      # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t_e, t_s) in enumerate(zip(eager, static)):
            assert torch.equal(t_e, t_s), f"replay {rep}: buffer {i} differs"
        assert torch.equal(eager_flags, graph_flags)
        say(f"   replay {rep}: identical; flags {graph_flags.tolist()}")
    assert graph_flags.tolist()[1] == 1


def test_captured_companions_replay_match_eager(mm):
    """The other entry points under capture: the allocation-free S_max pass
    (its partials in the library's own scratch), the attention forward with
    its S_max export, a multi-tensor AdamW step and a Dion step, captured once
    and replayed 3 times, each replay bit-identical to the same eager calls,
    with eager work and synchronisations between the replays."""
    import torch
    dev = torch.device("cuda:0")
    say("[graph] capture S_max (no-alloc), attention, AdamW and Dion, replay 3 times")
    g = gen.rng(31)

    def state():
        Q = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 300, 3, 128), 1.0)), dev)
        K = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 300, 3, 128), 1.0)), dev)
        V = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 300, 3, 128), 1.0)), dev)
        ps = [to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (n,), 0.02)), dev) for n in (1000, 4097, 64)]
        gs = [to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (p.numel(),), 1.0)), dev) for p in ps]
        ms = [torch.zeros(p.numel(), dtype=torch.float32, device=dev) for p in ps]
        vs = [torch.zeros(p.numel(), dtype=torch.float32, device=dev) for p in ps]
        W = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 256, 192), 0.02)), dev)
        G = to_dev(gen.f32_to_bf16_bits(gen.gaussian(g, (2, 256, 192), 1.0)), dev)
        M = torch.zeros((2, 256, 192), dtype=torch.float32, device=dev)
        R = gen.gaussian(g, (2, 192, 16), 1.0)
        R /= np.linalg.norm(R, axis=1, keepdims=True)
        Qd = to_dev(R.astype(np.float32), dev)
        return [Q, K, V, ps, gs, ms, vs, W, G, M, Qd]

    first = state()
    eager = [t.clone() if not isinstance(t, list) else [x.clone() for x in t] for t in first]
    static = first

    def make(st):
        Q, K, V, ps, gs, ms, vs, W, G, M, Qd = st
        s_a = torch.empty(3, dtype=torch.float32, device=dev)
        s_b = torch.empty(3, dtype=torch.float32, device=dev)
        out = torch.empty_like(Q)
        aws = torch.empty(max(mm.load_library().attn_fwd_workspace_size(2, 300, 3), 256), dtype=torch.uint8,
                          device=dev)
        dws = torch.empty(max(mm.load_library().dion_workspace_size(2, 256, 192, 16), 256), dtype=torch.uint8,
                          device=dev)

        def step():
            mm.qkclip_rowmax_noalloc(Q, K, 1.0 / math.sqrt(128), True, out=s_a)
            mm.attn_fwd(Q, K, V, 1.0 / math.sqrt(128), True, out=out, s_max=s_b, workspace=aws)
            mm.adamw_step(ps, gs, ms, vs, lr=1e-3, step=1)
            mm.dion_step(W, G, M, Qd, lr=0.01, workspace=dws)
        return step, [s_a, s_b, out]

    eager_step, eager_out = make(eager)
    graph_step, graph_out = make(static)
    # one eager call of every entry point on a third state first, so that
    # nothing is done for the first time inside the capture
    make(state())[0]()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        graph_step()
    torch.cuda.synchronize()

    def flat(st):
        return [x for t in st for x in (t if isinstance(t, list) else [t])]

    x = torch.randn(512, 512, device=dev)
    for rep in range(3):
        eager_step()
        _ = x @ x                      # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t_e, t_s) in enumerate(zip(flat(eager) + eager_out, flat(static) + graph_out)):
            assert torch.equal(t_e, t_s), f"replay {rep}: buffer {i} differs"
        say(f"   replay {rep}: identical; s_max {graph_out[0].tolist()}")
    # the two statistics agree
    assert torch.allclose(graph_out[0], graph_out[1], rtol=1e-6, atol=0)
