"""MI355X (gfx950) attention forward: a thin ctypes binding over ``libfa.so``.

Every entry point of ``include/fa.h`` has a Python function of the same name that
only marshals arguments (torch tensors to device pointers and sizes) and turns
status codes into exceptions. All computation happens in the HIP kernels of the
library; torch supplies device memory and the current stream. There is no CPU
fallback: if the library is missing and cannot be built, importing the binding
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from . import build as _build

__all__ = [
    "FaError", "lib", "fa_fwd", "fa_unfused_fwd", "fa_unfused_workspace_bytes", "fa_select_blocks",
    "fa_check_args", "fa_status_string", "fa_version", "forward", "unfused_forward",
    "fa_decode_fwd", "fa_decode_plan", "fa_decode_check_args", "decode_forward", "DECODE_MAX_NQ",
    "fa_decode_fwd_noalloc", "DECODE_SCRATCH_BYTES",
    "fa_fwd_tile_order", "TILE_ORDERS", "fa_fwd_blocks", "fa_bwd", "fa_bwd_workspace_bytes", "backward",
    "STATUS",
]

DECODE_MAX_NQ = 16  # FA_DECODE_MAX_NQ
DECODE_SCRATCH_BYTES = 32 << 20  # FA_DECODE_SCRATCH_BYTES
TILE_ORDERS = {"xcd": 0, "dispatch": 1, "qtile_major": 2}  # orders of fa_fwd_tile_order

STATUS = {
    "FA_OK": 0, "FA_ERR_NULL": -1, "FA_ERR_SHAPE": -2, "FA_ERR_HEADDIM": -3, "FA_ERR_ALIGN": -4,
    "FA_ERR_SCALE": -5, "FA_ERR_ALIAS": -6, "FA_ERR_OVERFLOW": -7, "FA_ERR_WORKSPACE": -8,
    "FA_ERR_HIP": -9, "FA_ERR_DEVICE": -10, "FA_ERR_SCRATCH": -11,
}
_ARG_ERRORS = {-1, -2, -3, -4, -5, -6, -7, -8, -11}


class FaError(RuntimeError):
    """A non-zero status from libfa. ``code`` is the fa_status value."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_status_string(code)} (status {code})")


class FaArgumentError(FaError, ValueError):
    """An argument error (detected before any HIP call)."""


def _load() -> ctypes.CDLL:
    if not os.path.exists(_build.LIB_PATH):
        _build.build_library()
    _build.check_built()  # a library left from older sources is never loaded
    dll = ctypes.CDLL(_build.LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    dll.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
    dll.fa_fwd.restype = i
    dll.fa_unfused_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    dll.fa_unfused_fwd.restype = i
    dll.fa_unfused_workspace_bytes.argtypes = [i, i, i]
    dll.fa_unfused_workspace_bytes.restype = sz
    dll.fa_select_blocks.argtypes = [i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)]
    dll.fa_select_blocks.restype = i
    dll.fa_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz]
    dll.fa_check_args.restype = i
    dll.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    dll.fa_bwd.restype = i
    dll.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    dll.fa_bwd_workspace_bytes.restype = sz
    dll.fa_fwd_tile_order.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    dll.fa_fwd_tile_order.restype = i
    dll.fa_fwd_blocks.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    dll.fa_fwd_blocks.restype = i
    dll.fa_decode_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz, vp]
    dll.fa_decode_fwd.restype = i
    dll.fa_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    dll.fa_decode_fwd_noalloc.restype = i
    dll.fa_decode_plan.argtypes = [i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(sz)]
    dll.fa_decode_plan.restype = i
    dll.fa_decode_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz]
    dll.fa_decode_check_args.restype = i
    dll.fa_status_string.argtypes = [i]
    dll.fa_status_string.restype = ctypes.c_char_p
    dll.fa_version.argtypes = []
    dll.fa_version.restype = i
    return dll


lib = _load()


def _raise(code: int, where: str):
    if code == 0:
        return
    if code in _ARG_ERRORS:
        raise FaArgumentError(code, where)
    raise FaError(code, where)


def fa_status_string(code: int) -> str:
    return lib.fa_status_string(int(code)).decode()


def fa_version() -> int:
    return lib.fa_version()


def fa_unfused_workspace_bytes(B: int, H: int, N: int) -> int:
    return lib.fa_unfused_workspace_bytes(int(B), int(H), int(N))


def fa_select_blocks(d: int, N: int, B: int = 1, H: int = 1):
    br, bc, nw = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _raise(lib.fa_select_blocks(int(d), int(N), int(B), int(H), ctypes.byref(br), ctypes.byref(bc),
                                ctypes.byref(nw)), "fa_select_blocks")
    return br.value, bc.value, nw.value


def fa_check_args(q, k, v, o, lse, B, H, N, d, scale, need_workspace=0, workspace=None, workspace_bytes=0) -> int:
    """Raw pointer-level validation (integers or None for pointers); returns the status code."""
    return lib.fa_check_args(q, k, v, o, lse, int(B), int(H), int(N), int(d), float(scale),
                             int(need_workspace), workspace, int(workspace_bytes))


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device) -> int | None:
    """The hipStream_t to enqueue on: ``stream`` (a torch stream or a raw handle), or
    torch's current stream of ``device``. A torch stream must belong to ``device``."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        if getattr(stream, "device", device) != device:
            raise ValueError(f"stream is on {stream.device}, tensors are on {device}")
        return stream.cuda_stream
    return int(stream)


def _check_tensors(q, k, v, o, lse):
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("o", o, torch.bfloat16), ("lse", lse, torch.float32)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if len({t.device for t in (q, k, v, o, lse)}) != 1:
        raise ValueError("q, k, v, o and lse must be on the same GPU")


def _shape_of(q, k, v, o, lse):
    _check_tensors(q, k, v, o, lse)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or o.shape != q.shape:
        raise ValueError("q, k, v, o must all have shape [B, H, N, d]")
    if tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must have shape [B, H, N]")
    return tuple(int(x) for x in q.shape)


def fa_fwd(q, k, v, o, lse, scale=None, stream=None):
    """Fused forward into caller-provided ``o`` (bf16) and ``lse`` (fp32), enqueued on
    ``stream`` (default: torch's current stream). ``scale`` defaults to 1/sqrt(d)."""
    B, H, N, d = _shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):  # the library launches on the current device
        _raise(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                          _stream_handle(stream, q.device)), "fa_fwd")
    return o, lse


def fa_fwd_tile_order(q, k, v, o, lse, order, scale=None, stream=None):
    """fa_fwd with an explicit workgroup-to-tile order (0, 1, 2 or a TILE_ORDERS
    name), for traffic measurements; results are identical for every order."""
    B, H, N, d = _shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    order = TILE_ORDERS.get(order, order)
    with torch.cuda.device(q.device):
        _raise(lib.fa_fwd_tile_order(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                     int(order), _stream_handle(stream, q.device)), "fa_fwd_tile_order")
    return o, lse


def fa_fwd_blocks(q, k, v, o, lse, br, scale=None, stream=None):
    """fa_fwd with an explicit query-tile height ``br`` (256 or 128 rows per workgroup)
    instead of the selector's choice."""
    B, H, N, d = _shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        _raise(lib.fa_fwd_blocks(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                 int(br), _stream_handle(stream, q.device)), "fa_fwd_blocks")
    return o, lse


def fa_unfused_fwd(q, k, v, o, lse, workspace, scale=None, stream=None):
    """Three-kernel forward (S and P through ``workspace``, a uint8 GPU tensor of at
    least fa_unfused_workspace_bytes(B, H, N) bytes)."""
    B, H, N, d = _shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.device != q.device:
        raise ValueError("workspace must be on the same GPU as the tensors")
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _raise(lib.fa_unfused_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                  _ptr(workspace), nbytes, _stream_handle(stream, q.device)), "fa_unfused_fwd")
    return o, lse


def forward(q, k, v, scale=None, stream=None):
    """Allocate O and LSE with torch and run :func:`fa_fwd`. Returns (o, lse)."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    return fa_fwd(q, k, v, o, lse, scale=scale, stream=stream)


def unfused_forward(q, k, v, scale=None, stream=None):
    """Allocate O, LSE and the workspace and run :func:`fa_unfused_fwd`."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(fa_unfused_workspace_bytes(B, H, N), 256), dtype=torch.uint8, device=q.device)
    return fa_unfused_fwd(q, k, v, o, lse, ws, scale=scale, stream=stream)


def fa_decode_plan(B: int, H: int, Nq: int, Nk: int, d: int):
    """(splits, chunk, workspace_bytes) that fa_decode_fwd uses for this shape."""
    sp, ch, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _raise(lib.fa_decode_plan(int(B), int(H), int(Nq), int(Nk), int(d), ctypes.byref(sp), ctypes.byref(ch),
                              ctypes.byref(ws)), "fa_decode_plan")
    return sp.value, ch.value, ws.value


def fa_decode_check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, workspace=None, workspace_bytes=0) -> int:
    """Raw pointer-level validation of fa_decode_fwd (integers or None); returns the status code."""
    return lib.fa_decode_check_args(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
                                    workspace, int(workspace_bytes))


def _decode_shape_of(q, k, v, o, lse):
    _check_tensors(q, k, v, o, lse)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("q, o must have shape [B, H, Nq, d] and k, v shape [B, H, Nk, d]")
    if k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q and k must agree in B, H and d")
    if tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must have shape [B, H, Nq]")
    B, H, Nq, d = (int(x) for x in q.shape)
    return B, H, Nq, int(k.shape[2]), d


def fa_decode_fwd(q, k, v, o, lse, workspace, scale=None, stream=None):
    """Decode-shaped forward (Nq <= 16 query rows against Nk keys) into caller-provided
    ``o`` and ``lse``, with ``workspace`` a uint8 GPU tensor of at least the bytes
    fa_decode_plan reports."""
    B, H, Nq, Nk, d = _decode_shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.device != q.device:
        raise ValueError("workspace must be on the same GPU as the tensors")
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _raise(lib.fa_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                                 _ptr(workspace), nbytes, _stream_handle(stream, q.device)), "fa_decode_fwd")
    return o, lse


def fa_decode_fwd_noalloc(q, k, v, o, lse, scale=None, stream=None):
    """fa_decode_fwd into caller-provided ``o`` and ``lse`` without a workspace: the
    library's fixed per-GPU scratch array (DECODE_SCRATCH_BYTES) holds the partial
    results. Calls that can overlap in time on one GPU race on that array."""
    B, H, Nq, Nk, d = _decode_shape_of(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        _raise(lib.fa_decode_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                         float(scale), _stream_handle(stream, q.device)), "fa_decode_fwd_noalloc")
    return o, lse


def decode_forward(q, k, v, scale=None, stream=None):
    """Allocate O, LSE and the workspace and run :func:`fa_decode_fwd`. Returns (o, lse)."""
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _, _, ws_bytes = fa_decode_plan(B, H, Nq, k.shape[2], d)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    return fa_decode_fwd(q, k, v, o, lse, ws, scale=scale, stream=stream)


def fa_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return lib.fa_bwd_workspace_bytes(int(B), int(H), int(N))


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, scale=None, stream=None):
    """Backward into caller-provided dq, dk, dv (bf16, shaped like q) from the
    forward's o and lse and the upstream dO; workspace: uint8 GPU tensor of at least
    fa_bwd_workspace_bytes(B, H, N) bytes."""
    B, H, N, d = _shape_of(q, k, v, o, lse)
    _check_tensors(dO, dq, dk, dv, lse)
    for name, t in (("dO", dO), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must have q's shape and device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.device != q.device:
        raise ValueError("workspace must be on the same GPU as the tensors")
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _raise(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                          B, H, N, d, float(scale), _ptr(workspace), nbytes, _stream_handle(stream, q.device)),
               "fa_bwd")
    return dq, dk, dv


def backward(q, k, v, o, lse, dO, scale=None, stream=None):
    """Allocate dq, dk, dv and the workspace and run :func:`fa_bwd`. Returns (dq, dk, dv)."""
    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa_bwd_workspace_bytes(B, H, N), 256), dtype=torch.uint8, device=q.device)
    return fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws, scale=scale, stream=stream)

