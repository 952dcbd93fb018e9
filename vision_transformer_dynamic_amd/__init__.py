"""Bi-Level Routing Attention (BRA) forward for MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libbra.so`` (declared in
``include/bra.h``). This module only marshals arguments: every step of the
computation runs in the library's HIP kernels. PyTorch supplies device memory
and the current stream. If the library has not been built, every call raises
``RuntimeError``; there is no fallback.

    pool(q, k, S)                                      -> (q_r, k_r) region means [B, S*S, C] float32
    route_pooled(q_r, k_r, S, topk)                    -> idx from given region means
    attend_kernel(B, H, W, C, heads, S, topk, dtype)   -> name of the attention kernel launched
    route(q, k, S, topk)                               -> idx [B, S*S, topk] int32
    route_ws(q, k, S, topk, workspace)                 -> the same, in a caller workspace
    attend(q, k, v, idx, heads, S)                     -> o   [B, H, W, C]
    forward(q, k, v, heads, S, topk)                   -> o   [B, H, W, C]
    forward_ws(q, k, v, heads, S, topk, workspace)     -> the same, in a caller workspace
    forward_static(q, k, v, heads, S, topk)            -> the same, in the library's static scratch
    attend_lce(q, k, v, idx, weight, bias, heads, S)   -> o + 5x5 depthwise conv of v
    forward_lce(q, k, v, weight, bias, heads, S, topk) -> o + 5x5 depthwise conv of v
    attend_backward(q, k, v, o, do, idx, heads, S)     -> (dq, dk, dv), routing held fixed
    qkv_pool(x, w_qkv, b_qkv, S)                       -> (q, k, v, q_r, k_r) region means of q, k
    forward_qkv(x, w_qkv, b_qkv, heads, S, topk)       -> (o, q, k, v) from the block input

q, k, v: contiguous [B, H, W, C] tensors on one GPU, float32 or bfloat16;
weight [C, 5, 5] and bias [C] (or None) of the local-context filter in the
same dtype.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BraError",
    "library_path",
    "load_library",
    "workspace_bytes",
    "attend_kernel",
    "pool",
    "route_pooled",
    "route",
    "route_ws",
    "attend",
    "forward",
    "forward_ws",
    "forward_static",
    "attend_lce",
    "forward_lce",
    "attend_backward",
    "qkv_pool",
    "forward_qkv",
    "EXPORTS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_ENV = "BRA_LIBRARY"

BRA_F32 = 0
BRA_BF16 = 1
BRA_OK, BRA_EINVAL, BRA_EUNSUPPORTED, BRA_EHIP, BRA_ENOMEM, BRA_ESCRATCH = range(6)
STATIC_SCRATCH_BYTES = 16 << 20  # BRA_STATIC_SCRATCH_BYTES

# Every symbol include/bra.h declares.
EXPORTS = ("bra_status_string", "bra_attend_kernel", "bra_workspace_bytes", "bra_pool", "bra_route_pooled",
           "bra_route", "bra_route_ws", "bra_attend", "bra_forward", "bra_forward_ws", "bra_forward_static", "bra_attend_lce", "bra_forward_lce", "bra_backward_workspace_bytes", "bra_attend_backward",
           "bra_qkv_pool", "bra_forward_qkv")

_lib = None


class BraError(RuntimeError):
    """A non-success status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"BRA status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.environ.get(_LIB_ENV, os.path.join(_PKG, "libbra.so"))


def load_library():
    """Load libbra.so once; raise RuntimeError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not built: {path} is missing "
            "(run `python -m vision_transformer_dynamic_amd.build`)"
        )
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.bra_status_string.restype = ctypes.c_char_p
    lib.bra_status_string.argtypes = [i32]
    lib.bra_workspace_bytes.restype = sz
    lib.bra_workspace_bytes.argtypes = [i32] * 6
    lib.bra_attend_kernel.restype = ctypes.c_char_p
    lib.bra_attend_kernel.argtypes = [i32] * 7 + [i32, i32]
    lib.bra_pool.restype = i32
    lib.bra_pool.argtypes = [vp] * 4 + [i32] * 5 + [i32, vp]
    lib.bra_route_pooled.restype = i32
    lib.bra_route_pooled.argtypes = [vp] * 3 + [i32] * 4 + [vp]
    lib.bra_route.restype = i32
    lib.bra_route.argtypes = [vp, vp, vp] + [i32] * 6 + [i32, vp]
    lib.bra_route_ws.restype = i32
    lib.bra_route_ws.argtypes = [vp, vp, vp] + [i32] * 6 + [i32, vp, sz, vp]
    lib.bra_attend.restype = i32
    lib.bra_attend.argtypes = [vp, vp, vp, vp, vp] + [i32] * 7 + [i32, vp]
    lib.bra_forward.restype = i32
    lib.bra_forward.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [i32, vp]
    lib.bra_forward_ws.restype = i32
    lib.bra_forward_ws.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [i32, vp, sz, vp]
    lib.bra_forward_static.restype = i32
    lib.bra_forward_static.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [i32, vp]
    lib.bra_attend_lce.restype = i32
    lib.bra_attend_lce.argtypes = [vp, vp, vp, vp, vp, vp, vp] + [i32] * 7 + [i32, vp]
    lib.bra_forward_lce.restype = i32
    lib.bra_forward_lce.argtypes = [vp, vp, vp, vp, vp, vp] + [i32] * 7 + [i32, vp, sz, vp]
    lib.bra_backward_workspace_bytes.restype = sz
    lib.bra_backward_workspace_bytes.argtypes = [i32] * 7
    lib.bra_attend_backward.restype = i32
    lib.bra_attend_backward.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp, sz, vp]
    lib.bra_qkv_pool.restype = i32
    lib.bra_qkv_pool.argtypes = [vp] * 8 + [i32] * 5 + [i32, vp]
    lib.bra_forward_qkv.restype = i32
    lib.bra_forward_qkv.argtypes = [vp] * 7 + [i32] * 7 + [i32, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status == BRA_OK:
        return
    msg = load_library().bra_status_string(status).decode()
    if status == BRA_EINVAL:
        raise ValueError(f"BRA status {status}: {msg}")
    if status == BRA_EUNSUPPORTED:
        raise NotImplementedError(f"BRA status {status}: {msg}")
    raise BraError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return BRA_F32
    if t.dtype == torch.bfloat16:
        return BRA_BF16
    raise NotImplementedError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_maps(*ts: torch.Tensor):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, W, C]")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and out) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, W, C]")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(B: int, H: int, W: int, C: int, S: int, topk: int) -> int:
    n = load_library().bra_workspace_bytes(B, H, W, C, S, topk)
    if n == 0:
        raise ValueError("invalid sizes for BRA")
    return int(n)


def _workspace(q: torch.Tensor, S: int, topk: int, workspace):
    B, H, W, C = q.shape
    need = workspace_bytes(B, H, W, C, S, topk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if (workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous()
            or workspace.device != q.device):
        raise ValueError(f"workspace must be a contiguous buffer of at least {need} bytes on q's device")
    return workspace, need


def attend_kernel(B: int, H: int, W: int, C: int, heads: int, S: int, topk: int, dtype: torch.dtype,
                  with_lce: bool = False) -> str:
    """Name of the attention kernel bra_attend (or bra_attend_lce) launches
    for these sizes, as a profiler lists it."""
    code = BRA_F32 if dtype == torch.float32 else BRA_BF16 if dtype == torch.bfloat16 else -1
    name = load_library().bra_attend_kernel(B, H, W, C, heads, S, topk, code, int(bool(with_lce)))
    if name is None:
        raise ValueError("invalid or unsupported sizes for BRA")
    return name.decode()


def _means_check(t: torch.Tensor, B: int, R: int, C: int, dev):
    if t.dtype != torch.float32 or t.shape != (B, R, C) or not t.is_contiguous() or t.device != dev:
        raise ValueError("region means must be contiguous float32 [B, S*S, C] tensors on the maps' device")


def pool(q: torch.Tensor, k: torch.Tensor, S: int, out=None):
    """Region means (q_r, k_r), float32 [B, S*S, C] (bra_pool)."""
    lib = load_library()
    _check_maps(q, k)
    B, H, W, C = q.shape
    if out is None:
        out = tuple(torch.empty((B, S * S, C), dtype=torch.float32, device=q.device) for _ in range(2))
    qr, kr = out
    for t in (qr, kr):
        _means_check(t, B, S * S, C, q.device)
    _check(lib.bra_pool(q.data_ptr(), k.data_ptr(), qr.data_ptr(), kr.data_ptr(), B, H, W, C, S,
                        _dtype_code(q), _stream(q.device)))
    return qr, kr


def route_pooled(qr: torch.Tensor, kr: torch.Tensor, S: int, topk: int, out=None) -> torch.Tensor:
    """Routing table from given region means (bra_route_pooled)."""
    lib = load_library()
    if qr.dim() != 3:
        raise ValueError("region means must be [B, S*S, C]")
    B, R, C = qr.shape
    for t in (qr, kr):
        _means_check(t, B, S * S, C, qr.device)
    out = _route_out(qr, S, topk, out)
    _check(lib.bra_route_pooled(qr.data_ptr(), kr.data_ptr(), out.data_ptr(), B, S, C, topk, _stream(qr.device)))
    return out


def _route_out(q, S, topk, out):
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, S * S, topk), dtype=torch.int32, device=q.device)
    if out.dtype != torch.int32 or not out.is_contiguous() or out.shape != (B, S * S, topk) or out.device != q.device:
        raise ValueError("out must be a contiguous int32 [B, S*S, topk] tensor on q's device")
    return out


def route(q: torch.Tensor, k: torch.Tensor, S: int, topk: int, out=None, workspace=None) -> torch.Tensor:
    """Routing table [B, S*S, topk] int32 (descending affinity, lower index on
    ties). With a workspace this is bra_route_ws; without, bra_route, which
    allocates its scratch stream-ordered."""
    if workspace is not None:
        return route_ws(q, k, S, topk, workspace, out=out)
    lib = load_library()
    _check_maps(q, k)
    B, H, W, C = q.shape
    out = _route_out(q, S, topk, out)
    _check(lib.bra_route(q.data_ptr(), k.data_ptr(), out.data_ptr(), B, H, W, C, S, topk,
                         _dtype_code(q), _stream(q.device)))
    return out


def route_ws(q: torch.Tensor, k: torch.Tensor, S: int, topk: int, workspace: torch.Tensor, out=None) -> torch.Tensor:
    """route() in a caller workspace of workspace_bytes(...) bytes (bra_route_ws)."""
    lib = load_library()
    _check_maps(q, k)
    B, H, W, C = q.shape
    out = _route_out(q, S, topk, out)
    ws, nbytes = _workspace(q, S, topk, workspace)
    _check(lib.bra_route_ws(q.data_ptr(), k.data_ptr(), out.data_ptr(), B, H, W, C, S, topk,
                            _dtype_code(q), ws.data_ptr(), nbytes, _stream(q.device)))
    return out


def attend(q, k, v, idx: torch.Tensor, heads: int, S: int, out=None) -> torch.Tensor:
    """Attention of every region's queries over the tokens of its routed regions."""
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.dim() != 3 or idx.device != q.device:
        raise ValueError("idx must be a contiguous int32 [B, S*S, topk] tensor on q's device")
    if tuple(idx.shape[:2]) != (B, S * S):
        raise ValueError("idx must be [B, S*S, topk]")
    topk = idx.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    _check(lib.bra_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), out.data_ptr(),
                          B, H, W, C, heads, S, topk, _dtype_code(q), _stream(q.device)))
    return out


def forward(q, k, v, heads: int, S: int, topk: int, out=None, workspace=None) -> torch.Tensor:
    """Full BRA forward (without the local-context dwconv term). With a
    workspace this is bra_forward_ws; without, bra_forward, which allocates
    its scratch stream-ordered."""
    if workspace is not None:
        return forward_ws(q, k, v, heads, S, topk, workspace, out=out)
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    _check(lib.bra_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           B, H, W, C, heads, S, topk, _dtype_code(q), _stream(q.device)))
    return out


def forward_ws(q, k, v, heads: int, S: int, topk: int, workspace: torch.Tensor, out=None) -> torch.Tensor:
    """forward() in a caller workspace of workspace_bytes(...) bytes
    (bra_forward_ws); the routing table is left in it."""
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    ws, nbytes = _workspace(q, S, topk, workspace)
    _check(lib.bra_forward_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              B, H, W, C, heads, S, topk, _dtype_code(q),
                              ws.data_ptr(), nbytes, _stream(q.device)))
    return out


def forward_static(q, k, v, heads: int, S: int, topk: int, out=None) -> torch.Tensor:
    """forward() with the library's static device scratch (bra_forward_static):
    no allocation in the call; calls on one GPU must be ordered."""
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    _check(lib.bra_forward_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  B, H, W, C, heads, S, topk, _dtype_code(q), _stream(q.device)))
    return out


def _lce_args(q: torch.Tensor, weight: torch.Tensor, bias):
    C = q.shape[-1]
    if weight.shape != (C, 5, 5) or weight.dtype != q.dtype or weight.device != q.device or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [C, 5, 5] tensor of q's dtype on q's device")
    if bias is None:
        return weight.data_ptr(), None
    if bias.shape != (C,) or bias.dtype != q.dtype or bias.device != q.device or not bias.is_contiguous():
        raise ValueError("bias must be a contiguous [C] tensor of q's dtype on q's device, or None")
    return weight.data_ptr(), bias.data_ptr()


def attend_lce(q, k, v, idx: torch.Tensor, weight: torch.Tensor, bias, heads: int, S: int, out=None) -> torch.Tensor:
    """attend() plus the local context term: a 5x5 depthwise convolution of v
    (zero padding, optional per-channel bias) over the whole map."""
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.dim() != 3 or idx.device != q.device:
        raise ValueError("idx must be a contiguous int32 [B, S*S, topk] tensor on q's device")
    if tuple(idx.shape[:2]) != (B, S * S):
        raise ValueError("idx must be [B, S*S, topk]")
    topk = idx.shape[2]
    wp, bp = _lce_args(q, weight, bias)
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    _check(lib.bra_attend_lce(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), wp, bp, out.data_ptr(),
                              B, H, W, C, heads, S, topk, _dtype_code(q), _stream(q.device)))
    return out


def forward_lce(q, k, v, weight: torch.Tensor, bias, heads: int, S: int, topk: int, out=None,
                workspace=None) -> torch.Tensor:
    """forward() plus the local context term (the module output of the
    pages' pseudocode, after the projections)."""
    lib = load_library()
    _check_maps(q, k, v)
    B, H, W, C = q.shape
    wp, bp = _lce_args(q, weight, bias)
    if out is None:
        out = torch.empty_like(q)
    _check_maps(q, out)
    ws, nbytes = _workspace(q, S, topk, workspace)
    _check(lib.bra_forward_lce(q.data_ptr(), k.data_ptr(), v.data_ptr(), wp, bp, out.data_ptr(),
                               B, H, W, C, heads, S, topk, _dtype_code(q),
                               ws.data_ptr(), nbytes, _stream(q.device)))
    return out


def backward_workspace_bytes(B: int, H: int, W: int, C: int, heads: int, S: int, topk: int) -> int:
    n = load_library().bra_backward_workspace_bytes(B, H, W, C, heads, S, topk)
    if n == 0:
        raise ValueError("invalid sizes for the BRA backward")
    return int(n)


def attend_backward(q, k, v, o, do, idx: torch.Tensor, heads: int, S: int, out=None, workspace=None):
    """Gradients (dq, dk, dv) of the token attention given dL/dO = do, the
    routing table idx held fixed; o is the forward output for the same idx."""
    lib = load_library()
    _check_maps(q, k, v, o, do)
    B, H, W, C = q.shape
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.dim() != 3 or idx.device != q.device:
        raise ValueError("idx must be a contiguous int32 [B, S*S, topk] tensor on q's device")
    if tuple(idx.shape[:2]) != (B, S * S):
        raise ValueError("idx must be [B, S*S, topk]")
    topk = idx.shape[2]
    if out is None:
        out = tuple(torch.empty_like(q) for _ in range(3))
    dq, dk, dv = out
    _check_maps(q, dq, dk, dv)
    need = backward_workspace_bytes(B, H, W, C, heads, S, topk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer of at least {need} bytes")
    _check(lib.bra_attend_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                   idx.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   B, H, W, C, heads, S, topk, _dtype_code(q),
                                   workspace.data_ptr(), need, _stream(q.device)))
    return dq, dk, dv


def _proj_args(x: torch.Tensor, w_qkv: torch.Tensor, b_qkv):
    C = x.shape[-1]
    if w_qkv.shape != (3 * C, C) or w_qkv.dtype != x.dtype or w_qkv.device != x.device or not w_qkv.is_contiguous():
        raise ValueError("w_qkv must be a contiguous [3C, C] tensor of x's dtype on x's device")
    if b_qkv is None:
        return w_qkv.data_ptr(), None
    if b_qkv.shape != (3 * C,) or b_qkv.dtype != x.dtype or b_qkv.device != x.device or not b_qkv.is_contiguous():
        raise ValueError("b_qkv must be a contiguous [3C] tensor of x's dtype on x's device, or None")
    return w_qkv.data_ptr(), b_qkv.data_ptr()


def qkv_pool(x: torch.Tensor, w_qkv: torch.Tensor, b_qkv, S: int, out=None):
    """Q, K, V = x w_qkv^T + b_qkv (chunked q, k, v) and the region means
    q_r, k_r [B, S*S, C] float32 of the rounded Q and K."""
    lib = load_library()
    _check_maps(x)
    B, H, W, C = x.shape
    wp, bp = _proj_args(x, w_qkv, b_qkv)
    if out is None:
        out = tuple(torch.empty_like(x) for _ in range(3)) + tuple(
            torch.empty((B, S * S, C), dtype=torch.float32, device=x.device) for _ in range(2))
    q, k, v, qr, kr = out
    _check_maps(x, q, k, v)
    for t in (qr, kr):
        if t.dtype != torch.float32 or t.shape != (B, S * S, C) or not t.is_contiguous() or t.device != x.device:
            raise ValueError("q_r, k_r must be contiguous float32 [B, S*S, C] tensors on x's device")
    _check(lib.bra_qkv_pool(x.data_ptr(), wp, bp, q.data_ptr(), k.data_ptr(), v.data_ptr(), qr.data_ptr(),
                            kr.data_ptr(), B, H, W, C, S, _dtype_code(x), _stream(x.device)))
    return q, k, v, qr, kr


def forward_qkv(x: torch.Tensor, w_qkv: torch.Tensor, b_qkv, heads: int, S: int, topk: int, out=None,
                workspace=None):
    """The module from its input x: projection (with the pooling fused),
    routing and attention. Returns (o, q, k, v)."""
    lib = load_library()
    _check_maps(x)
    B, H, W, C = x.shape
    wp, bp = _proj_args(x, w_qkv, b_qkv)
    if out is None:
        out = tuple(torch.empty_like(x) for _ in range(4))
    o, q, k, v = out
    _check_maps(x, o, q, k, v)
    ws, nbytes = _workspace(x, S, topk, workspace)
    _check(lib.bra_forward_qkv(x.data_ptr(), wp, bp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               B, H, W, C, heads, S, topk, _dtype_code(x), ws.data_ptr(), nbytes,
                               _stream(x.device)))
    return o, q, k, v
