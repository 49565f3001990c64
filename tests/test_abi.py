"""CPU checks of the boundary: the C-ABI library loads and exports every
function include/muon.h declares; host-side argument validation returns its
documented status codes without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    if not os.path.exists(mm.library_path()):
        pytest.skip("libmuon.so not built")
    return mm.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["muon_step", "ns_orthogonalize", "qkclip_rowmax", "qkclip_rescale",
              "qkclip_rescale_slices", "qkclip_rescale_mla", "adamw_step", "attn_fwd", "dion_step"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.muon_status_string(s)


def test_host_validation_without_gpu(lib):
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    # null groups
    assert lib.muon_step(None, 1, 0, None, None, 0, None) == mm.MUON_ERR_INVALID_ARG
    g = (mm._Group * 1)()
    g[0] = mm._Group(8, 8, 8, 1, 4, 4, 0, 16)
    hp = mm.HParams().to_c()
    # workspace missing
    assert lib.muon_step(g, 1, mm.DTYPE_F32, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_WORKSPACE
    assert lib.muon_step_workspace_size(g, 1) > 0
    # bad batch stride
    g[0] = mm._Group(8, 8, 8, 1, 4, 4, 0, 15)
    assert lib.muon_step(g, 1, mm.DTYPE_F32, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.muon_step_workspace_size(g, 1) == 0
    # zero rows, bad dtype, bad steps
    g[0] = mm._Group(8, 8, 8, 1, 0, 4, 0, 16)
    assert lib.muon_step(g, 1, mm.DTYPE_F32, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG
    g[0] = mm._Group(8, 8, 8, 1, 4, 4, 0, 16)
    assert lib.muon_step(g, 1, 7, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG
    hp.ns_steps = 0
    assert lib.muon_step(g, 1, mm.DTYPE_F32, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG
    # QK-Clip argument checks
    assert lib.qkclip_rowmax(16, 16, 1, 8, 2, 96, 0.1, 1, 16, 16, 1 << 20, None) == mm.MUON_ERR_UNSUPPORTED
    assert lib.qkclip_rowmax(16, 16, 1, 8, 2, 64, 0.0, 1, 16, 16, 1 << 20, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.qkclip_rowmax(16, 16, 1, 8, 2, 64, 0.1, 1, 16, None, 0, None) == mm.MUON_ERR_WORKSPACE
    assert lib.qkclip_rescale(None, 16, 1, 2, 64, 8, 16, 100.0, 0.5, None, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.qkclip_rescale(16, 16, 1, 2, 64, 8, 16, -1.0, 0.5, None, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.qkclip_rescale(16, 16, 1, 2, 64, 8, 16, 100.0, 1.5, None, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.ns_orthogonalize(16, 0, 16, 1, 4, 4, 16, 5, 3.4, -4.7, 2.0, 1e-7, None, 0, None) == mm.MUON_ERR_WORKSPACE
    # MLA: zero rotary width, bad dtype
    assert lib.qkclip_rescale_mla(16, 16, 16, 1, 2, 64, 0, 8, 8, 16, 100.0, None, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.qkclip_rescale_mla(16, 16, 16, 5, 2, 64, 32, 8, 8, 16, 100.0, None, None) == mm.MUON_ERR_INVALID_ARG
    # slices: too many, pitch below rows, exponent outside [0, 1]
    sl = (mm._Slice * 5)()
    for i in range(5):
        sl[i] = mm._Slice(16, 64, 64, 8, 0.5)
    assert lib.qkclip_rescale_slices(sl, 5, 1, 2, 16, 100.0, None, None) == mm.MUON_ERR_INVALID_ARG
    sl[0] = mm._Slice(16, 32, 64, 8, 0.5)
    assert lib.qkclip_rescale_slices(sl, 1, 1, 2, 16, 100.0, None, None) == mm.MUON_ERR_INVALID_ARG
    sl[0] = mm._Slice(16, 64, 64, 8, 1.5)
    assert lib.qkclip_rescale_slices(sl, 1, 1, 2, 16, 100.0, None, None) == mm.MUON_ERR_INVALID_ARG
    # AdamW: step 0, beta1 = 1, missing moment buffer, misaligned bf16 param
    t = (mm._AdamWTensor * 1)()
    t[0] = mm._AdamWTensor(16, 16, 16, 16, 10)
    hp = mm._AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 0)
    assert lib.adamw_step(t, 1, 1, ctypes.byref(hp), None) == mm.MUON_ERR_INVALID_ARG
    hp = mm._AdamWHParams(1e-3, 1.0, 0.95, 1e-8, 0.1, 1)
    assert lib.adamw_step(t, 1, 1, ctypes.byref(hp), None) == mm.MUON_ERR_INVALID_ARG
    hp = mm._AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    t[0] = mm._AdamWTensor(16, 16, None, 16, 10)
    assert lib.adamw_step(t, 1, 1, ctypes.byref(hp), None) == mm.MUON_ERR_INVALID_ARG
    t[0] = mm._AdamWTensor(17, 16, 16, 16, 10)
    assert lib.adamw_step(t, 1, 1, ctypes.byref(hp), None) == mm.MUON_ERR_INVALID_ARG
    # attention forward: head dim other than 128, missing output, no workspace
    assert lib.attn_fwd(16, 16, 16, 1, 8, 2, 64, 0.1, 1, 16, None, 16, 16, 1 << 20, None) == mm.MUON_ERR_UNSUPPORTED
    assert lib.attn_fwd(16, 16, 16, 1, 8, 2, 128, 0.1, 1, None, None, 16, 16, 1 << 20, None) == mm.MUON_ERR_INVALID_ARG
    assert lib.attn_fwd(16, 16, 16, 1, 8, 2, 128, 0.1, 1, 16, None, 16, None, 0, None) == mm.MUON_ERR_WORKSPACE
    assert lib.attn_fwd_workspace_size(2, 300, 3) >= 2 * 3 * 3 * 4 * 4   # [B][H][query blocks][4 waves] fp32
    # nothing to do is not an error and launches nothing
    assert lib.adamw_step(t, 0, 1, ctypes.byref(hp), None) == mm.MUON_OK
    assert lib.ns_workspace_size(1, 0, 4) == 0


def test_size_limits_without_gpu(lib):
    """The largest matrices accepted: every side <= 2^20 and the padded wide
    view (max + 256) x (min + 256) <= 2^31 elements; one more row or column
    is refused before any launch."""
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    accepted = [(8192, 253944), (253944, 8192), (46084, 46084), (1 << 20, 1), (1, 1 << 20)]
    refused = [(8192, 253945), (253945, 8192), (46085, 46085), ((1 << 20) + 1, 1), (1, (1 << 20) + 1)]
    for r, c in accepted:
        assert lib.ns_workspace_size(1, r, c) > 0, (r, c)
    for r, c in refused:
        assert lib.ns_workspace_size(1, r, c) == 0, (r, c)
        assert lib.ns_orthogonalize(16, mm.DTYPE_BF16, 16, 1, r, c, r * c, 5, 3.4445, -4.775, 2.0315,
                                    1e-7, 256, 1 << 40, None) == mm.MUON_ERR_INVALID_ARG
        g = (mm._Group * 1)()
        g[0] = mm._Group(16, 16, 16, 1, r, c, 0, r * c)
        assert lib.muon_step_workspace_size(g, 1) == 0
        hp = mm.HParams().to_c()
        assert lib.muon_step(g, 1, mm.DTYPE_BF16, ctypes.byref(hp), 256, 1 << 40, None) == mm.MUON_ERR_INVALID_ARG
    # the workspace of the largest square case: four padded copies of X and
    # two of A (46336 x 46336 bf16 each) plus the norm partials
    assert lib.ns_workspace_size(1, 46084, 46084) >= 6 * 46336 * 46336 * 2


def test_workspace_layout_query(lib):
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    g = (mm._Group * 2)()
    g[0] = mm._Group(8, 8, 8, 3, 300, 100, 0, 30000)   # tall
    g[1] = mm._Group(8, 8, 8, 2, 100, 700, 0, 70000)   # wide, tile 128
    lay = mm._WsLayout()
    assert lib.muon_step_workspace_layout(g, 2, 0, 5, ctypes.byref(lay)) == 0
    # tall: O is the transposed buffer, leading dimension = padded cols (128)
    assert lay.o_ld == 128 and lay.x0_ld == 384
    assert lay.o_offset % 256 == 0 and lay.inv_norm_offset % 256 == 0
    assert lib.muon_step_workspace_layout(g, 2, 1, 4, ctypes.byref(lay)) == 0
    assert lay.o_ld == 768 and lay.x0_ld == 768
    assert lib.muon_step_workspace_layout(g, 2, 2, 5, ctypes.byref(lay)) == mm.MUON_ERR_INVALID_ARG
    total = lib.muon_step_workspace_size(g, 2)
    assert lay.o_offset < total


def test_dion_host_validation_without_gpu(lib):
    """dion_step's argument checks run on the host: invalid arguments,
    unsupported shapes and a missing workspace are reported before any launch
    (the fake device pointers are never dereferenced)."""
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    P = 1 << 12           # 16-byte aligned fake pointer, never touched
    ok = dict(dtype=mm.DTYPE_BF16, batch=2, rows=64, cols=96, rank=16, stride=64 * 96, lr=0.01, mu=0.95)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.dion_step(a.get("p", P), a["dtype"], a.get("g", P), a.get("m", P), a.get("q", P), a["batch"],
                             a["rows"], a["cols"], a["rank"], a["stride"], a["lr"], a["mu"], a.get("ws", None),
                             a.get("wsz", 0), None)
    assert lib.dion_workspace_size(2, 64, 96, 16) > 0
    assert lib.dion_workspace_size(0, 64, 96, 16) == 0
    assert call(p=None) == mm.MUON_ERR_INVALID_ARG
    assert call(dtype=7) == mm.MUON_ERR_INVALID_ARG
    assert call(stride=64 * 96 - 8) == mm.MUON_ERR_INVALID_ARG
    assert call(lr=float("nan")) == mm.MUON_ERR_INVALID_ARG
    assert call(rank=12) == mm.MUON_ERR_UNSUPPORTED          # not a multiple of 8
    assert call(rank=136, rows=256, cols=256, stride=65536) == mm.MUON_ERR_UNSUPPORTED   # above 128
    assert call(rank=72) == mm.MUON_ERR_UNSUPPORTED          # above min(rows, cols)
    assert call(cols=100, stride=6400) == mm.MUON_ERR_UNSUPPORTED
    assert call(q=P + 4) == mm.MUON_ERR_UNSUPPORTED          # misaligned
    assert call() == mm.MUON_ERR_WORKSPACE
    assert call(ws=P, wsz=lib.dion_workspace_size(2, 64, 96, 16) - 1) == mm.MUON_ERR_WORKSPACE


def test_workspace_layout_properties(lib):
    """For random group sets (every path: single-workgroup, thin, tiled; wide,
    tall and square; any batch), the regions the layout query names lie inside
    the workspace, are 256-byte aligned, hold every matrix of their group, and
    the O regions of different groups do not overlap (host logic only)."""
    import random
    import matrix_orthogonalizing_optimizer_muon_amd as mm
    rng = random.Random(1234)
    sides = [1, 7, 33, 96, 97, 128, 200, 256, 300, 512, 777, 1024, 2100]
    for _ in range(300):
        n = rng.randint(1, mm.MAX_GROUPS)
        g = (mm._Group * n)()
        shapes = []
        for k in range(n):
            r, c, b = rng.choice(sides), rng.choice(sides), rng.randint(1, 5)
            g[k] = mm._Group(16, 16, 16, b, r, c, 0, r * c + rng.choice([0, 8]))
            shapes.append((b, r, c))
        total = lib.muon_step_workspace_size(g, n)
        assert total > 0
        steps = rng.choice([1, 5])
        o_regions = []
        for k, (b, r, c) in enumerate(shapes):
            lay = mm._WsLayout()
            assert lib.muon_step_workspace_layout(g, n, k, steps, ctypes.byref(lay)) == mm.MUON_OK
            assert lay.o_offset % 256 == 0 and lay.inv_norm_offset % 256 == 0 and lay.x0_offset % 256 == 0
            o_end = lay.o_offset + 2 * ((b - 1) * lay.o_batch_stride + (r - 1) * lay.o_ld + c)
            assert lay.o_ld >= c and lay.o_batch_stride >= r * lay.o_ld and o_end <= total
            assert lay.inv_norm_offset + 4 * b <= total
            m, w = min(r, c), max(r, c)
            assert lay.x0_ld >= w and lay.x0_offset + 2 * ((b - 1) * lay.x0_batch_stride + (m - 1) * lay.x0_ld + w) <= total
            o_regions.append((lay.o_offset, o_end))
        o_regions.sort()
        for (a0, a1), (b0, b1) in zip(o_regions, o_regions[1:]):
            assert a1 <= b0, (a0, a1, b0, b1)
