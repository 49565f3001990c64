"""Muon optimizer step and MuonClip QK-Clip on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libmuon.so (C ABI in include/muon.h).  Every step of
the computation runs in the library's HIP kernels; this module only checks
tensor arguments, passes raw device pointers and torch's current HIP stream,
and allocates workspaces with torch.  There is no fallback: if the library is
missing or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

MUON_OK, MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_ERR_HIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1
SCALE_MODES = {"moonlight": 0, "spectral": 1, "none": 2}
MAX_GROUPS = 16
_MAX_KINDS = 64   # upper bound on the library's kernel kinds (it reports the real count)

# ---------------------------------------------------------------------------
# C structs
# ---------------------------------------------------------------------------


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("ns_steps", ctypes.c_int32), ("ns_a", ctypes.c_float),
                ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("scale_mode", ctypes.c_int32),
                ("rms_target", ctypes.c_float)]


class _Group(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("batch_stride", ctypes.c_int64)]


class _WsLayout(ctypes.Structure):
    _fields_ = [("o_offset", ctypes.c_size_t), ("o_batch_stride", ctypes.c_int64),
                ("o_ld", ctypes.c_int64), ("inv_norm_offset", ctypes.c_size_t),
                ("x0_offset", ctypes.c_size_t), ("x0_batch_stride", ctypes.c_int64),
                ("x0_ld", ctypes.c_int64)]


class _Slice(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("head_pitch", ctypes.c_int64),
                ("rows_per_head", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("exponent", ctypes.c_float)]


class _AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32)]


class _AdamWTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("numel", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libmuon.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    G = ctypes.POINTER(_Group)
    lib.muon_step_workspace_size.argtypes = [G, i32]
    lib.muon_step_workspace_size.restype = sz
    lib.muon_step.argtypes = [G, i32, i32, ctypes.POINTER(_HParams), vp, sz, vp]
    lib.muon_step.restype = i32
    lib.muon_step_workspace_layout.argtypes = [G, i32, i32, i32, ctypes.POINTER(_WsLayout)]
    lib.muon_step_workspace_layout.restype = i32
    lib.ns_workspace_size.argtypes = [i32, i32, i32]
    lib.ns_workspace_size.restype = sz
    lib.ns_orthogonalize.argtypes = [vp, i32, vp, i32, i32, i32, i64, i32, f32, f32, f32, f32, vp, sz, vp]
    lib.ns_orthogonalize.restype = i32
    lib.qkclip_rowmax_workspace_size.argtypes = [i32, i32, i32]
    lib.qkclip_rowmax_workspace_size.restype = sz
    lib.qkclip_rowmax.argtypes = [vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, sz, vp]
    lib.qkclip_rowmax.restype = i32
    lib.qkclip_rowmax_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.qkclip_rowmax_noalloc.restype = i32
    lib.qkclip_rowmax_noalloc_max_partials.argtypes = []
    lib.qkclip_rowmax_noalloc_max_partials.restype = sz
    lib.qkclip_rescale.argtypes = [vp, vp, i32, i32, i32, i32, vp, f32, f32, vp, vp]
    lib.qkclip_rescale.restype = i32
    lib.qkclip_rescale_slices.argtypes = [ctypes.POINTER(_Slice), i32, i32, i32, vp, f32, vp, vp]
    lib.qkclip_rescale_slices.restype = i32
    lib.qkclip_rescale_mla.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, f32, vp, vp]
    lib.qkclip_rescale_mla.restype = i32
    lib.attn_fwd_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_fwd_workspace_size.restype = sz
    lib.attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp]
    lib.attn_fwd.restype = i32
    lib.adamw_step.argtypes = [ctypes.POINTER(_AdamWTensor), i32, i32, ctypes.POINTER(_AdamWHParams), vp]
    lib.dion_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dion_workspace_size.restype = sz
    lib.dion_step.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i64, f32, f32, vp, sz, vp]
    lib.dion_step.restype = i32
    lib.adamw_step.restype = i32
    lib.muon_mfma_probe.argtypes = [i32, i32, i32, vp, vp]
    lib.muon_mfma_probe.restype = i32
    lib.muon_hbm_probe.argtypes = [vp, sz, vp, sz, i32, i32, i32, vp]
    lib.muon_hbm_probe.restype = i64
    lib.muon_status_string.argtypes = [i32]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_profile_enable.argtypes = [i32]
    lib.muon_profile_enable.restype = i32
    lib.muon_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32]
    lib.muon_profile_collect.restype = i32
    lib.muon_kernel_kind_name.argtypes = [i32]
    lib.muon_kernel_kind_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load_library()
        super().__init__(f"{where}: {lib.muon_status_string(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status != MUON_OK:
        raise MuonError(status, where)


# ---------------------------------------------------------------------------
# helpers (torch is used for device memory and the stream handle only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _as3d(t):
    """View a [rows, cols] or [batch, rows, cols] tensor as (batch, rows, cols,
    batch_stride); rows must be contiguous."""
    if t.dim() == 2:
        if not t.is_contiguous():
            raise ValueError("matrices must be row-major contiguous")
        return 1, t.shape[0], t.shape[1], t.shape[0] * t.shape[1]
    if t.dim() == 3:
        b, r, c = t.shape
        # a stride along a dimension of extent 1 is never used (NumPy gives
        # inserted axes stride 0)
        row_ok = (t.stride(2) == 1 or c == 1) and (t.stride(1) == c or r == 1)
        if not row_ok or (b > 1 and t.stride(0) < r * c):
            raise ValueError("each matrix must be row-major contiguous")
        return b, r, c, (t.stride(0) if b > 1 else r * c)
    raise ValueError("expected a 2-D or 3-D tensor")


def _workspace(nbytes: int, device):
    torch = _torch()
    # 256-byte alignment: torch's caching allocator returns >= 512-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


@dataclass
class HParams:
    """Muon hyper-parameters (defaults: the pages' common settings)."""
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    nesterov: bool = True
    ns_steps: int = 5
    ns_coeffs: tuple = (3.4445, -4.7750, 2.0315)
    ns_eps: float = 1e-7
    scale_mode: str = "moonlight"
    rms_target: float = 0.2

    def to_c(self) -> _HParams:
        a, b, c = self.ns_coeffs
        return _HParams(self.lr, self.momentum, self.weight_decay, int(bool(self.nesterov)),
                        int(self.ns_steps), a, b, c, self.ns_eps, SCALE_MODES[self.scale_mode],
                        self.rms_target)


def _groups_c(groups):
    if not 1 <= len(groups) <= MAX_GROUPS:
        raise ValueError(f"1..{MAX_GROUPS} groups per call")
    arr = (_Group * len(groups))()
    dtype = None
    for k, (p, g, m) in enumerate(groups):
        _need_cuda(p, g, m)
        torch = _torch()
        if p.shape != g.shape or p.shape != m.shape:
            raise ValueError("param, grad and momentum must share a shape")
        if p.dtype != g.dtype:
            raise TypeError("grad must have the param dtype")
        if m.dtype != torch.float32:
            raise TypeError("momentum must be float32")
        dc = _dtype_code(p)
        if dtype is None:
            dtype = dc
        elif dc != dtype:
            raise TypeError("all groups of one call share a param dtype")
        b, r, c, st = _as3d(p)
        if _as3d(g)[3] != st or _as3d(m)[3] != st:
            raise ValueError("param, grad and momentum must share the batch stride")
        arr[k] = _Group(p.data_ptr(), g.data_ptr(), m.data_ptr(), b, r, c, 0, st)
    return arr, dtype


def workspace_size(groups) -> int:
    lib = load_library()
    arr, _ = _groups_c(groups)
    return int(lib.muon_step_workspace_size(arr, len(groups)))


def muon_step(groups, hp: HParams | None = None, workspace=None):
    """One Muon step, in place, over a list of (param, grad, momentum) groups
    ([batch, rows, cols] or [rows, cols] tensors).  Returns the workspace
    tensor (reusable for the next call with the same groups)."""
    lib = load_library()
    hp = hp or HParams()
    arr, dtype = _groups_c(groups)
    need = int(lib.muon_step_workspace_size(arr, len(groups)))
    if workspace is None:
        workspace = _workspace(need, groups[0][0].device)
    h = hp.to_c()
    _check(lib.muon_step(arr, len(groups), dtype, ctypes.byref(h), workspace.data_ptr(),
                         workspace.numel(), _stream()), "muon_step")
    return workspace


def workspace_views(groups, g: int, workspace, ns_steps: int = 5):
    """(O, inv_norm, X0) tensors viewing the workspace after muon_step:
    O [batch, rows, cols] bf16 (group layout), inv_norm [batch] fp32 and
    X0 [batch, m, n] bf16 (wide orientation, unnormalised)."""
    torch = _torch()
    lib = load_library()
    arr, _ = _groups_c(groups)
    lay = _WsLayout()
    _check(lib.muon_step_workspace_layout(arr, len(groups), g, ns_steps, ctypes.byref(lay)),
           "muon_step_workspace_layout")
    b, r, c, _ = _as3d(groups[g][0])
    m, n = min(r, c), max(r, c)
    bf = workspace.view(torch.bfloat16) if workspace.numel() % 2 == 0 else None
    o = torch.as_strided(bf, (b, r, c), (lay.o_batch_stride, lay.o_ld, 1), lay.o_offset // 2)
    inv = torch.as_strided(workspace.view(torch.float32), (b,), (1,), lay.inv_norm_offset // 4)
    x0 = torch.as_strided(bf, (b, m, n), (lay.x0_batch_stride, lay.x0_ld, 1), lay.x0_offset // 2)
    return o, inv, x0


def ns_orthogonalize(x, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
                     out=None, workspace=None):
    """Newton-Schulz on each matrix of x ([rows, cols] or [batch, rows, cols],
    float32 or bfloat16); returns bf16 of the same shape."""
    torch = _torch()
    lib = load_library()
    _need_cuda(x)
    b, r, c, st = _as3d(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of x's shape")
    need = int(lib.ns_workspace_size(b, r, c))
    if workspace is None:
        workspace = _workspace(need, x.device)
    a_, b_, c_ = coeffs
    _check(lib.ns_orthogonalize(x.data_ptr(), _dtype_code(x), out.data_ptr(), b, r, c, st, steps,
                                a_, b_, c_, eps, workspace.data_ptr(), workspace.numel(), _stream()),
           "ns_orthogonalize")
    return out


def qkclip_rowmax(Q, K, logit_scale: float | None = None, causal: bool = True, out=None,
                  workspace=None):
    """Per-head maximum logit of bf16 Q, K [B, T, H, d_head]; returns fp32 [H]."""
    torch = _torch()
    lib = load_library()
    _need_cuda(Q, K)
    if Q.dtype != torch.bfloat16 or K.dtype != torch.bfloat16:
        raise TypeError("Q and K must be bfloat16")
    if Q.dim() != 4 or Q.shape != K.shape or not Q.is_contiguous() or not K.is_contiguous():
        raise ValueError("Q and K must be contiguous [B, T, H, d_head] tensors of one shape")
    B, T, H, D = Q.shape
    if logit_scale is None:
        logit_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=Q.device)
    need = int(lib.qkclip_rowmax_workspace_size(B, T, H))
    if workspace is None:
        workspace = _workspace(need, Q.device)
    _check(lib.qkclip_rowmax(Q.data_ptr(), K.data_ptr(), B, T, H, D, logit_scale, int(bool(causal)),
                             out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()),
           "qkclip_rowmax")
    return out


def qkclip_rowmax_noalloc(Q, K, logit_scale: float | None = None, causal: bool = True, out=None):
    """qkclip_rowmax without a workspace: the library's own per-GPU scratch
    holds the partial maxima (B * H * ceil(T / q) of them, q = 512 queries
    per block for d_head 128 and 256 otherwise, at most
    qkclip_rowmax_noalloc_max_partials()).  Calls that overlap on one GPU
    race.  Returns fp32 [H]."""
    torch = _torch()
    lib = load_library()
    _need_cuda(Q, K)
    if Q.dtype != torch.bfloat16 or K.dtype != torch.bfloat16:
        raise TypeError("Q and K must be bfloat16")
    if Q.dim() != 4 or Q.shape != K.shape or not Q.is_contiguous() or not K.is_contiguous():
        raise ValueError("Q and K must be contiguous [B, T, H, d_head] tensors of one shape")
    B, T, H, D = Q.shape
    if logit_scale is None:
        logit_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=Q.device)
    _check(lib.qkclip_rowmax_noalloc(Q.data_ptr(), K.data_ptr(), B, T, H, D, logit_scale, int(bool(causal)),
                                     out.data_ptr(), _stream()), "qkclip_rowmax_noalloc")
    return out


def qkclip_rescale(Wq, Wk, s_max, d_head: int, tau: float = 100.0, alpha: float = 0.5,
                   clipped=None):
    """In-place per-head rescale of Wq, Wk [H*d_head, d_model]; returns the
    int32 [H] flags (1 clipped, 0 untouched, -1 non-finite S_max)."""
    torch = _torch()
    lib = load_library()
    _need_cuda(Wq, Wk, s_max)
    if Wq.shape != Wk.shape or Wq.dim() != 2 or not Wq.is_contiguous() or not Wk.is_contiguous():
        raise ValueError("Wq and Wk must be contiguous 2-D tensors of one shape")
    if Wq.dtype != Wk.dtype:
        raise TypeError("Wq and Wk must share a dtype")
    rows, d_model = Wq.shape
    if rows % d_head:
        raise ValueError("rows of Wq must be a multiple of d_head")
    H = rows // d_head
    if s_max.dtype != torch.float32 or s_max.numel() != H:
        raise ValueError("s_max must be float32 [H]")
    if clipped is None:
        clipped = torch.empty(H, dtype=torch.int32, device=Wq.device)
    _check(lib.qkclip_rescale(Wq.data_ptr(), Wk.data_ptr(), _dtype_code(Wq), H, d_head, d_model,
                              s_max.data_ptr(), tau, alpha, clipped.data_ptr(), _stream()),
           "qkclip_rescale")
    return clipped


def attn_fwd(Q, K, V, logit_scale: float | None = None, causal: bool = True, out=None,
             s_max=None, with_lse: bool = False, workspace=None):
    """Softmax attention forward over bf16 [B, T, H, 128] tensors.  Returns
    (O bf16 [B, T, H, 128], s_max fp32 [H], lse fp32 [B, H, T] or None);
    s_max is the per-head maximum logit that QK-Clip takes."""
    torch = _torch()
    lib = load_library()
    _need_cuda(Q, K, V)
    if Q.dim() != 4 or Q.shape != K.shape or Q.shape != V.shape:
        raise ValueError("Q, K and V must share a [B, T, H, d] shape")
    for t in (Q, K, V):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("Q, K and V must be contiguous bfloat16")
    B, T, H, D = Q.shape
    if logit_scale is None:
        logit_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(Q)
    if out.shape != Q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of Q's shape")
    if s_max is None:
        s_max = torch.empty(H, dtype=torch.float32, device=Q.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=Q.device) if with_lse else None
    need = int(lib.attn_fwd_workspace_size(B, T, H))
    if workspace is None:
        workspace = _workspace(need, Q.device)
    _check(lib.attn_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), B, T, H, D, logit_scale, int(bool(causal)),
                        out.data_ptr(), lse.data_ptr() if lse is not None else None, s_max.data_ptr(),
                        workspace.data_ptr(), workspace.numel(), _stream()), "attn_fwd")
    return out, s_max, lse


def _flags(H, device, clipped):
    torch = _torch()
    if clipped is None:
        clipped = torch.empty(H, dtype=torch.int32, device=device)
    elif clipped.dtype != torch.int32 or clipped.numel() != H:
        raise ValueError("clipped must be int32 [H]")
    return clipped


def qkclip_rescale_slices(slices, s_max, tau: float = 100.0, clipped=None):
    """Per-head rescale over row slices.  Each slice is a tuple
    (W, row_offset, head_pitch, rows_per_head, exponent) with W a contiguous
    2-D tensor; head h owns rows row_offset + h*head_pitch + [0, rows_per_head)
    of W, multiplied by gamma^exponent when the head is clipped.  Returns the
    int32 [H] flags."""
    torch = _torch()
    lib = load_library()
    H = s_max.numel()
    if s_max.dtype != torch.float32 or H < 1:
        raise ValueError("s_max must be float32 [H]")
    _need_cuda(s_max)
    arr = (_Slice * max(len(slices), 1))()
    dtype = None
    for i, (W, off, pitch, rows, expo) in enumerate(slices):
        _need_cuda(W)
        if W.dim() != 2 or not W.is_contiguous():
            raise ValueError("slice matrices must be contiguous 2-D tensors")
        code = _dtype_code(W)
        if dtype is not None and code != dtype:
            raise TypeError("all slices must share a dtype")
        dtype = code
        if off < 0 or rows < 1 or pitch < rows or off + (H - 1) * pitch + rows > W.shape[0]:
            raise ValueError(f"slice {i}: rows of head {H - 1} fall outside the matrix")
        arr[i] = _Slice(W.data_ptr() + off * W.shape[1] * W.element_size(), pitch, rows, W.shape[1],
                        float(expo))
    clipped = _flags(H, s_max.device, clipped)
    _check(lib.qkclip_rescale_slices(arr, len(slices), dtype if dtype is not None else DTYPE_BF16, H,
                                     s_max.data_ptr(), tau, clipped.data_ptr(), _stream()),
           "qkclip_rescale_slices")
    return clipped


def qkclip_rescale_mla(Wqc, Wkc, Wqr, s_max, d_c: int, d_r: int, tau: float = 100.0, clipped=None):
    """MLA QK-Clip in place: content query/key rows of a clipped head scale by
    sqrt(gamma), its rotary query rows by gamma; the shared rotary key is not
    an argument because it never changes.  Wqc [H*d_c, q_in], Wkc
    [H*d_c, kv_in], Wqr [H*d_r, q_in].  Returns the int32 [H] flags."""
    torch = _torch()
    lib = load_library()
    _need_cuda(Wqc, Wkc, Wqr, s_max)
    for W in (Wqc, Wkc, Wqr):
        if W.dim() != 2 or not W.is_contiguous():
            raise ValueError("MLA matrices must be contiguous 2-D tensors")
    if not (Wqc.dtype == Wkc.dtype == Wqr.dtype):
        raise TypeError("MLA matrices must share a dtype")
    H = s_max.numel()
    if s_max.dtype != torch.float32:
        raise ValueError("s_max must be float32 [H]")
    if Wqc.shape[0] != H * d_c or Wkc.shape[0] != H * d_c or Wqr.shape[0] != H * d_r:
        raise ValueError("row counts must be H*d_c (content) and H*d_r (rotary query)")
    if Wqr.shape[1] != Wqc.shape[1]:
        raise ValueError("content and rotary query projections must share their input width")
    clipped = _flags(H, s_max.device, clipped)
    _check(lib.qkclip_rescale_mla(Wqc.data_ptr(), Wkc.data_ptr(), Wqr.data_ptr(), _dtype_code(Wqc), H, d_c, d_r,
                                  Wqc.shape[1], Wkc.shape[1], s_max.data_ptr(), tau, clipped.data_ptr(),
                                  _stream()),
           "qkclip_rescale_mla")
    return clipped


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr: float, beta1: float = 0.9,
               beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.1, step: int = 1):
    """One AdamW step in place over lists of tensors (params and grads of one
    dtype, fp32 or bf16; moments fp32; every tensor contiguous)."""
    torch = _torch()
    lib = load_library()
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have one entry per tensor")
    arr = (_AdamWTensor * max(n, 1))()
    dtype = None
    for i, (p, g, m, v) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
        _need_cuda(p, g, m, v)
        code = _dtype_code(p)
        if dtype is not None and code != dtype:
            raise TypeError("all params must share a dtype")
        dtype = code
        if g.dtype != p.dtype or m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError("grad must match the param dtype; moments must be float32")
        if not (p.numel() == g.numel() == m.numel() == v.numel()):
            raise ValueError(f"tensor {i}: sizes differ")
        for t in (p, g, m, v):
            if not t.is_contiguous():
                raise ValueError("AdamW tensors must be contiguous")
        arr[i] = _AdamWTensor(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), p.numel())
    hp = _AdamWHParams(lr, beta1, beta2, eps, weight_decay, step)
    _check(lib.adamw_step(arr, n, dtype if dtype is not None else DTYPE_F32, ctypes.byref(hp), _stream()),
           "adamw_step")


def dion_step(param, grad, momentum, q, *, lr: float, mu: float = 0.95, workspace=None):
    """One rank-r Dion step in place: param and grad ([rows, cols] or
    [batch, rows, cols], fp32 or bf16, same dtype), momentum fp32 of the same
    shape, q fp32 [cols, rank] or [batch, cols, rank] (the warm-start state,
    replaced by ColNorm(R)).  rank = q.shape[-1]."""
    torch = _torch()
    lib = load_library()
    _need_cuda(param, grad, momentum, q)
    b, r, c, st = _as3d(param)
    if grad.dtype != param.dtype or momentum.dtype != torch.float32 or q.dtype != torch.float32:
        raise TypeError("grad must match the param dtype; momentum and q must be float32")
    if _as3d(grad) != (b, r, c, st) or _as3d(momentum) != (b, r, c, st):
        raise ValueError("param, grad and momentum must share shape and strides")
    rank = q.shape[-1]
    if not q.is_contiguous() or q.numel() != b * c * rank or q.shape[-2] != c:
        raise ValueError("q must be a contiguous [batch, cols, rank] float32 tensor")
    need = int(lib.dion_workspace_size(b, r, c, rank))
    if workspace is None:
        workspace = _workspace(need, param.device)
    _check(lib.dion_step(param.data_ptr(), _dtype_code(param), grad.data_ptr(), momentum.data_ptr(),
                         q.data_ptr(), b, r, c, rank, st, lr, mu, workspace.data_ptr(), workspace.numel(),
                         _stream()), "dion_step")
    return workspace


PROBE_RANDOM = 0
PROBE_SMOOTH = 1


def mfma_probe(blocks: int, iters: int, sink, operands: int = PROBE_RANDOM):
    """Launch the register-only bf16 MFMA loop on the current stream (see
    muon_mfma_probe); sink: a float32 device tensor of >= blocks elements;
    operands: PROBE_RANDOM or PROBE_SMOOTH.  Returns the launch's flop count."""
    _need_cuda(sink)
    if sink.dtype != _torch().float32 or sink.numel() < blocks:
        raise ValueError("sink must be a float32 tensor of at least `blocks` elements")
    _check(load_library().muon_mfma_probe(blocks, iters, int(operands), sink.data_ptr(), _stream()),
           "muon_mfma_probe")
    return blocks * 4 * 32 * iters * 32768


def hbm_probe(src, dst, reads: int, writes: int, unroll: int = 1):
    """Launch the HBM stream probe on the current stream (see muon_hbm_probe):
    src and dst are device tensors (their bytes are the streams), (reads,
    writes) one of (1, 1), (3, 4), (2, 1), unroll 1 or 4 units per thread.
    Returns the bytes the launch moves."""
    _need_cuda(src, dst)
    moved = load_library().muon_hbm_probe(src.data_ptr(), src.numel() * src.element_size(), dst.data_ptr(),
                                          dst.numel() * dst.element_size(), int(reads), int(writes), int(unroll),
                                          _stream())
    if moved < 0:
        _check(int(-moved), "muon_hbm_probe")
    return int(moved)


def profile_enable(on: bool = True):
    load_library().muon_profile_enable(int(bool(on)))


def profile_collect() -> dict:
    """{kernel kind name: (total_ms, launches)} for launches since profile_enable."""
    lib = load_library()
    ms = (ctypes.c_double * _MAX_KINDS)()
    cnt = (ctypes.c_int64 * _MAX_KINDS)()
    n = lib.muon_profile_collect(ms, cnt, _MAX_KINDS)
    if n < 0:
        raise MuonError(-n, "muon_profile_collect")
    n = min(n, _MAX_KINDS)
    return {lib.muon_kernel_kind_name(k).decode(): (ms[k], int(cnt[k])) for k in range(n)}
