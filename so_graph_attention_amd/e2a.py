"""Thin ctypes binding of libe2a (include/e2a.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device buffers and the current stream.  The library must be
built in-tree first (``python -m so_graph_attention_amd.build``); importing
this module without it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libe2a.so")

E2A_OK = 0
E2A_ERR_INVALID_ARG = 1
E2A_ERR_CAPACITY = 2
E2A_ERR_BOX_TOO_SMALL = 3
E2A_ERR_UNSUPPORTED = 4
E2A_ERR_HIP = 5
E2A_DTYPE_F32 = 0
E2A_DTYPE_BF16 = 1
VARIANTS = {"auto": 0, "reference": 1, "mfma": 2}

# Every symbol include/e2a.h declares.
EXPORTED = ["e2a_version", "e2a_status_string", "e2a_last_error_message", "e2a_neighbors_workspace_bytes",
            "e2a_build_neighbors", "e2a_so2_param_count", "e2a_attention_workspace_bytes", "e2a_attention_fwd",
            "e2a_conv_fwd", "e2a_attention_bwd_workspace_bytes", "e2a_attention_bwd",
            "e2a_attention_bwd_weights_workspace_bytes", "e2a_attention_bwd_weights", "e2a_attention_fwd_noalloc",
            "e2a_block_workspace_bytes", "e2a_block_fwd", "e2a_so2_packed_bytes", "e2a_pack_so2_weights",
            "e2a_destination_order_workspace_bytes", "e2a_destination_order"]
NOALLOC_SCRATCH_BYTES = 64 << 20


class E2AError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("pos", ctypes.c_void_p), ("box", ctypes.c_void_p), ("n_atoms", ctypes.c_int64),
        ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("n_edges", ctypes.c_int64),
        ("cutoff", ctypes.c_float), ("L", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
        ("n_rbf", ctypes.c_int), ("dtype", ctypes.c_int), ("variant", ctypes.c_int),
        ("feat", ctypes.c_void_p), ("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p),
        ("w_rad", ctypes.c_void_p), ("w_so2", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("out_lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("w_so2_packed", ctypes.c_void_p), ("order", ctypes.c_void_p),
    ]


class BlockArgs(ctypes.Structure):
    _fields_ = [
        ("pos", ctypes.c_void_p), ("box", ctypes.c_void_p), ("n_atoms", ctypes.c_int64),
        ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("n_edges", ctypes.c_int64),
        ("cutoff", ctypes.c_float), ("L", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
        ("n_rbf", ctypes.c_int), ("dtype", ctypes.c_int), ("variant", ctypes.c_int),
        ("h_in", ctypes.c_void_p), ("h_out", ctypes.c_void_p),
        ("norm1", ctypes.c_void_p), ("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p), ("w_rad", ctypes.c_void_p),
        ("w_so2", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("norm2", ctypes.c_void_p), ("w_1", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_2", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("w_so2_packed", ctypes.c_void_p), ("order", ctypes.c_void_p),
    ]


BLOCK_WEIGHTS = ("norm1", "w_q", "w_k", "w_rad", "w_so2", "w_o", "norm2", "w_1", "w_gate", "w_2")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libe2a.so not built at {_LIB_PATH}; run `python -m so_graph_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.e2a_version.restype = ctypes.c_int
    lib.e2a_status_string.restype = ctypes.c_char_p
    lib.e2a_status_string.argtypes = [ctypes.c_int32]
    lib.e2a_last_error_message.restype = ctypes.c_char_p
    lib.e2a_neighbors_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_neighbors_workspace_bytes.argtypes = [ctypes.c_int64]
    lib.e2a_build_neighbors.restype = ctypes.c_int32
    lib.e2a_build_neighbors.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
    lib.e2a_so2_param_count.restype = ctypes.c_int64
    lib.e2a_so2_param_count.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.e2a_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_attention_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]
    lib.e2a_attention_fwd.restype = ctypes.c_int32
    lib.e2a_attention_fwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.e2a_attention_fwd_noalloc.restype = ctypes.c_int32
    lib.e2a_attention_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.e2a_so2_packed_bytes.restype = ctypes.c_size_t
    lib.e2a_so2_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.e2a_pack_so2_weights.restype = ctypes.c_int32
    lib.e2a_pack_so2_weights.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.e2a_destination_order_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_destination_order_workspace_bytes.argtypes = [ctypes.c_int64]
    lib.e2a_destination_order.restype = ctypes.c_int32
    lib.e2a_destination_order.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
    lib.e2a_block_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_block_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int]
    lib.e2a_block_fwd.restype = ctypes.c_int32
    lib.e2a_block_fwd.argtypes = [ctypes.POINTER(BlockArgs), ctypes.c_void_p]
    lib.e2a_conv_fwd.restype = ctypes.c_int32
    lib.e2a_conv_fwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.e2a_attention_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_attention_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_int]
    lib.e2a_attention_bwd.restype = ctypes.c_int32
    lib.e2a_attention_bwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.e2a_attention_bwd_weights_workspace_bytes.restype = ctypes.c_size_t
    lib.e2a_attention_bwd_weights_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                              ctypes.c_int, ctypes.c_int]
    lib.e2a_attention_bwd_weights.restype = ctypes.c_int32
    lib.e2a_attention_bwd_weights.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def lib():
    return _lib


def e2a_version() -> int:
    return _lib.e2a_version()


def status_string(s: int) -> str:
    return _lib.e2a_status_string(int(s)).decode()


def last_error_message() -> str:
    return _lib.e2a_last_error_message().decode()


def e2a_so2_param_count(L: int, C: int) -> int:
    return int(_lib.e2a_so2_param_count(L, C))


def e2a_neighbors_workspace_bytes(n_atoms: int) -> int:
    return int(_lib.e2a_neighbors_workspace_bytes(n_atoms))


def e2a_attention_workspace_bytes(n_atoms: int, L: int, C: int, H: int, dtype: int) -> int:
    return int(_lib.e2a_attention_workspace_bytes(n_atoms, L, C, H, dtype))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return getattr(stream, "cuda_stream", stream)


def _check(status: int):
    if status != E2A_OK:
        raise E2AError(status, last_error_message())


def _box_arg(box):
    if box is None:
        return None, None
    arr = (ctypes.c_float * 3)(*[float(b) for b in box])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None, numel=None):
    """Raises unless t is a contiguous tensor of the given dtype, device and
    shape (or element count).  Runs before any library call, so a wrong
    argument never reaches a kernel as a bad pointer."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _gpu_device(pos: torch.Tensor) -> torch.device:
    if not isinstance(pos, torch.Tensor):
        raise TypeError("pos must be a torch.Tensor")
    if pos.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {pos.device}")
    return pos.device


def _storage_dtype(feat: torch.Tensor) -> int:
    if feat.dtype == torch.bfloat16:
        return E2A_DTYPE_BF16
    if feat.dtype == torch.float32:
        return E2A_DTYPE_F32
    raise TypeError("feat must be float32 or bfloat16")


def _fill_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, L, C, H, cutoff, box, variant,
               workspace, need_qk=True, w_so2_packed=None, order=None):
    """Checks the layer's inputs (device, dtype, shape) and fills the argument
    struct.  Returns (args, box array that must stay alive for the call)."""
    dev = _gpu_device(pos)
    dtype = _storage_dtype(feat)
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    n = pos.shape[0]
    K = (L + 1) ** 2
    _need(pos, "pos", torch.float32, dev, shape=(n, 3))
    _need(row_ptr, "row_ptr", torch.int64, dev, shape=(n + 1,))
    _need(col, "col", torch.int32, dev)
    if col.dim() != 1:
        raise ValueError("col must be one-dimensional")
    _need(feat, "feat", feat.dtype, dev, shape=(n, K, C))
    if need_qk:
        _need(w_q, "w_q", feat.dtype, dev, shape=(C, C))
        _need(w_k, "w_k", feat.dtype, dev, shape=(C, C))
    _need(w_rad, "w_rad", feat.dtype, dev, shape=(8, L + 1, C))
    _need(w_so2, "w_so2", feat.dtype, dev, numel=e2a_so2_param_count(L, C))
    if out is not None:
        _need(out, "out", torch.float32, dev, shape=(n, K, C))
    if out_lse is not None:
        _need(out_lse, "out_lse", torch.float32, dev, shape=(n, H))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if w_so2_packed is not None:
        _need(w_so2_packed, "w_so2_packed", torch.uint8, dev, numel=e2a_so2_packed_bytes(L, C, dtype))
    if order is not None:
        _need(order, "order", torch.int32, dev, shape=(n,))
    box_arr, box_p = _box_arg(box)
    a = AttnArgs()
    a.pos = _ptr(pos)
    a.box = box_p
    a.n_atoms = n
    a.row_ptr = _ptr(row_ptr)
    a.col = _ptr(col)
    a.n_edges = col.numel()
    a.cutoff = float(cutoff)
    a.L, a.C, a.H, a.n_rbf, a.dtype, a.variant = L, C, H, 8, dtype, VARIANTS[variant]
    a.feat, a.w_q, a.w_k, a.w_rad, a.w_so2 = (_ptr(feat), _ptr(w_q), _ptr(w_k), _ptr(w_rad), _ptr(w_so2))
    a.out = _ptr(out)
    a.out_lse = _ptr(out_lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel()
    a.w_so2_packed = _ptr(w_so2_packed)
    a.order = _ptr(order)
    return a, box_arr


def e2a_build_neighbors(pos: torch.Tensor, cutoff: float, box=None, batch: Optional[torch.Tensor] = None,
                        capacity: Optional[int] = None, stream=None):
    """CSR radius graph (row_ptr int64 [N+1], col int32 [E]) on pos.device."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    _need(pos, "pos", torch.float32, dev, shape=(n, 3))
    if batch is not None:
        _need(batch, "batch", torch.int32, dev, shape=(n,))
    row_ptr = torch.empty(n + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(1, e2a_neighbors_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    cap = int(capacity) if capacity is not None else max(64, 64 * n)
    box_arr, box_p = _box_arg(box)
    while True:
        col = torch.empty(max(1, cap), dtype=torch.int32, device=dev)
        ne = ctypes.c_int64(0)
        st = _lib.e2a_build_neighbors(_ptr(pos), n, _ptr(batch), box_p, ctypes.c_float(cutoff), _ptr(row_ptr),
                                      _ptr(col), cap, ctypes.byref(ne), _ptr(ws), ws.numel(), _stream(stream))
        if st == E2A_ERR_CAPACITY and capacity is None:
            cap = int(ne.value)
            continue
        _check(st)
        return row_ptr, col[: ne.value]


def _layer(fn, pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, box, variant, out, out_lse,
           workspace, stream, need_qk, w_so2_packed=None, order=None):
    dev = _gpu_device(pos)
    n = pos.shape[0]
    if out is None:
        out = torch.empty((n, (L + 1) ** 2, C), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, e2a_attention_workspace_bytes(n, L, C, H, _storage_dtype(feat))),
                                dtype=torch.uint8, device=dev)
    a, box_arr = _fill_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, L, C, H, cutoff, box,
                            variant, workspace, need_qk=need_qk, w_so2_packed=w_so2_packed, order=order)
    _check(fn(ctypes.byref(a), _stream(stream)))
    del box_arr
    return out


def e2a_attention_fwd(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, *, L: int, C: int, H: int,
                      cutoff: float, box=None, variant: str = "auto", out=None, out_lse=None,
                      workspace=None, stream=None, with_lse: bool = False, w_so2_packed=None, order=None):
    """Run the fused layer; returns out [N,(L+1)^2,C] fp32 (and lse [N,H] if requested).

    Storage dtype follows ``feat`` (float32 or bfloat16); all weights must match it."""
    if with_lse and out_lse is None:
        out_lse = torch.empty((pos.shape[0], H), dtype=torch.float32, device=pos.device)
    out = _layer(_lib.e2a_attention_fwd, pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, L, C, H, cutoff, box,
                 variant, out, out_lse, workspace, stream, True, w_so2_packed, order)
    return (out, out_lse) if with_lse else out


def e2a_attention_fwd_noalloc(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, *, L: int, C: int, H: int,
                              cutoff: float, box=None, variant: str = "auto", out=None, out_lse=None, stream=None,
                              with_lse: bool = False):
    """e2a_attention_fwd on the library's fixed per-GPU scratch (the C call
    allocates nothing; pass ``out`` and ``out_lse`` to allocate nothing here
    either).  Calls that overlap on one GPU race on that scratch."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    if out is None:
        out = torch.empty((n, (L + 1) ** 2, C), dtype=torch.float32, device=dev)
    if with_lse and out_lse is None:
        out_lse = torch.empty((n, H), dtype=torch.float32, device=dev)
    a, box_arr = _fill_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, L, C, H, cutoff, box,
                            variant, None)
    _check(_lib.e2a_attention_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    del box_arr
    return (out, out_lse) if with_lse else out


def e2a_conv_fwd(pos, row_ptr, col, feat, w_rad, w_so2, *, L: int, C: int, H: int = 8, cutoff: float, box=None,
                 variant: str = "auto", out=None, workspace=None, stream=None, w_so2_packed=None, order=None):
    """Sum of the same per-edge messages without attention weights (the EAAS
    convolution stage); returns out [N,(L+1)^2,C] fp32.  H only selects the
    build (the MFMA kernel is built for H = 8)."""
    return _layer(_lib.e2a_conv_fwd, pos, row_ptr, col, feat, None, None, w_rad, w_so2, L, C, H, cutoff, box,
                  variant, out, None, workspace, stream, False, w_so2_packed, order)


def e2a_attention_bwd_workspace_bytes(n_atoms: int, n_edges: int, L: int, C: int, H: int) -> int:
    return int(_lib.e2a_attention_bwd_workspace_bytes(n_atoms, n_edges, L, C, H))


def _bwd_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, grad_out, L, C, H, cutoff, box,
              variant, workspace):
    """Checks the backward calls' inputs and fills their argument struct;
    returns (args, box array to keep alive)."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    K = (L + 1) ** 2
    _need(out, "out", torch.float32, dev, shape=(n, K, C))
    _need(out_lse, "out_lse", torch.float32, dev, shape=(n, H))
    _need(grad_out, "grad_out", torch.float32, dev, shape=(n, K, C))
    return _fill_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, L, C, H, cutoff, box, variant,
                      workspace)


def e2a_attention_bwd_weights_workspace_bytes(n_atoms: int, n_edges: int, L: int, C: int, H: int) -> int:
    return int(_lib.e2a_attention_bwd_weights_workspace_bytes(n_atoms, n_edges, L, C, H))


def e2a_attention_bwd_weights(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, grad_out, *, L: int,
                              C: int, H: int, cutoff: float, box=None, variant: str = "auto", feat_grad: bool = True,
                              weights=("w_q", "w_k", "w_rad", "w_so2"), pos_grad: bool = False, workspace=None,
                              stream=None):
    """Gradients of the layer with respect to its weights (those named in
    ``weights``), with feat_grad its node features and with pos_grad the atom
    positions, for grad_out = dL/do.  Returns a dict of fp32 tensors: "feat"
    [N,(L+1)^2,C], "w_q", "w_k" [C,C], "w_rad" [8,L+1,C], "w_so2" (flat, the
    layout of w_so2), "pos" [N,3]."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    K = (L + 1) ** 2
    shapes = {"feat": (n, K, C), "w_q": (C, C), "w_k": (C, C), "w_rad": (8, L + 1, C),
              "w_so2": (e2a_so2_param_count(L, C),), "pos": (n, 3)}
    want = (["feat"] if feat_grad else []) + list(weights) + (["pos"] if pos_grad else [])
    for name in want:
        if name not in shapes:
            raise ValueError(f"unknown gradient {name!r}")
    res = {name: torch.empty(shapes[name], dtype=torch.float32, device=dev) for name in want}
    if workspace is None:
        workspace = torch.empty(max(1, e2a_attention_bwd_weights_workspace_bytes(n, col.numel(), L, C, H)),
                                dtype=torch.uint8, device=dev)
    a, box_arr = _bwd_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, grad_out, L, C, H, cutoff,
                           box, variant, workspace)
    outs = [_ptr(res[name]) if name in res else None for name in ("feat", "w_q", "w_k", "w_rad", "w_so2", "pos")]
    _check(_lib.e2a_attention_bwd_weights(ctypes.byref(a), _ptr(grad_out), *outs, _stream(stream)))
    del box_arr
    return res


def e2a_attention_bwd(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, grad_out, *, L: int, C: int,
                      H: int, cutoff: float, box=None, variant: str = "auto", grad_feat=None, workspace=None,
                      stream=None):
    """dL/dh of the layer for grad_out = dL/do, from the forward's output and
    log-normaliser; returns grad_feat [N,(L+1)^2,C] fp32."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    K = (L + 1) ** 2
    if grad_feat is None:
        grad_feat = torch.empty((n, K, C), dtype=torch.float32, device=dev)
    _need(grad_feat, "grad_feat", torch.float32, dev, shape=(n, K, C))
    if workspace is None:
        workspace = torch.empty(max(1, e2a_attention_bwd_workspace_bytes(n, col.numel(), L, C, H)),
                                dtype=torch.uint8, device=dev)
    a, box_arr = _bwd_args(pos, row_ptr, col, feat, w_q, w_k, w_rad, w_so2, out, out_lse, grad_out, L, C, H, cutoff,
                           box, variant, workspace)
    _check(_lib.e2a_attention_bwd(ctypes.byref(a), _ptr(grad_out), _ptr(grad_feat), _stream(stream)))
    del box_arr
    return grad_feat


def e2a_block_workspace_bytes(n_atoms: int, L: int, C: int, H: int, dtype: int) -> int:
    return int(_lib.e2a_block_workspace_bytes(n_atoms, L, C, H, dtype))


def e2a_block_fwd(pos, row_ptr, col, h, weights: dict, *, L: int, C: int, H: int, cutoff: float, box=None,
                  variant: str = "auto", out=None, workspace=None, stream=None, w_so2_packed=None, order=None):
    """One block around the layer (include/e2a.h, e2a_block_fwd): h fp32
    [N,(L+1)^2,C] in, the block's output out.  ``weights`` maps the names in
    BLOCK_WEIGHTS to tensors in the storage dtype (w_gate may be absent for
    L = 0); all on h's device."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    K = (L + 1) ** 2
    w0 = weights["w_o"]
    dtype = _storage_dtype(w0)
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    _need(pos, "pos", torch.float32, dev, shape=(n, 3))
    _need(row_ptr, "row_ptr", torch.int64, dev, shape=(n + 1,))
    _need(col, "col", torch.int32, dev)
    _need(h, "h", torch.float32, dev, shape=(n, K, C))
    shapes = {"norm1": (L + 1, C), "w_q": (C, C), "w_k": (C, C), "w_rad": (8, L + 1, C), "w_o": (L + 1, C, C),
              "norm2": (L + 1, C), "w_1": (L + 1, C, C), "w_gate": (C, L * C), "w_2": (L + 1, C, C)}
    for name in BLOCK_WEIGHTS:
        t = weights.get(name)
        if name == "w_gate" and L == 0 and t is None:
            continue
        if name == "w_so2":
            _need(t, name, w0.dtype, dev, numel=e2a_so2_param_count(L, C))
        else:
            _need(t, name, w0.dtype, dev, shape=shapes[name])
    if out is None:
        out = torch.empty_like(h)
    _need(out, "out", torch.float32, dev, shape=(n, K, C))
    if workspace is None:
        workspace = torch.empty(max(1, e2a_block_workspace_bytes(n, L, C, H, dtype)), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    box_arr, box_p = _box_arg(box)
    a = BlockArgs()
    a.pos, a.box, a.n_atoms = _ptr(pos), box_p, n
    a.row_ptr, a.col, a.n_edges = _ptr(row_ptr), _ptr(col), col.numel()
    a.cutoff = float(cutoff)
    a.L, a.C, a.H, a.n_rbf, a.dtype, a.variant = L, C, H, 8, dtype, VARIANTS[variant]
    a.h_in, a.h_out = _ptr(h), _ptr(out)
    for name in BLOCK_WEIGHTS:
        setattr(a, name, _ptr(weights.get(name)))
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    if w_so2_packed is not None:
        _need(w_so2_packed, "w_so2_packed", torch.uint8, dev, numel=e2a_so2_packed_bytes(L, C, dtype))
    if order is not None:
        _need(order, "order", torch.int32, dev, shape=(n,))
    a.w_so2_packed, a.order = _ptr(w_so2_packed), _ptr(order)
    _check(_lib.e2a_block_fwd(ctypes.byref(a), _stream(stream)))
    del box_arr
    return out


def e2a_so2_packed_bytes(L: int, C: int, dtype: int) -> int:
    return int(_lib.e2a_so2_packed_bytes(L, C, dtype))


def e2a_pack_so2_weights(w_so2, *, L: int, C: int, out=None, stream=None):
    """The matrix-core image of w_so2 (bf16), as a uint8 tensor on its device,
    for the forward's w_so2_packed argument."""
    dev = _gpu_device(w_so2)
    dtype = _storage_dtype(w_so2)
    _need(w_so2, "w_so2", w_so2.dtype, dev, numel=e2a_so2_param_count(L, C))
    nb = e2a_so2_packed_bytes(L, C, dtype)
    if out is None:
        out = torch.empty(max(1, nb), dtype=torch.uint8, device=dev)
    _need(out, "out", torch.uint8, dev)
    _check(_lib.e2a_pack_so2_weights(_ptr(w_so2), _ptr(out), L, C, dtype, _stream(stream)))
    return out


def e2a_destination_order_workspace_bytes(n_atoms: int) -> int:
    return int(_lib.e2a_destination_order_workspace_bytes(n_atoms))


def e2a_destination_order(pos, *, order=None, workspace=None, stream=None):
    """The layer's default spatial order of the destinations (int32 [N])."""
    dev = _gpu_device(pos)
    n = pos.shape[0]
    _need(pos, "pos", torch.float32, dev, shape=(n, 3))
    if order is None:
        order = torch.empty(n, dtype=torch.int32, device=dev)
    _need(order, "order", torch.int32, dev, shape=(n,))
    if workspace is None:
        workspace = torch.empty(max(1, e2a_destination_order_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    _check(_lib.e2a_destination_order(_ptr(pos), n, _ptr(order), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return order
