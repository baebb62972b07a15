"""Thin Python binding of libmoe_ep.so, the MI355X MoE dispatch/combine core.

The functions carry the names of the C entry points declared in
include/moe_ep.h and only marshal arguments: they check that tensors live
on the GPU with the dtype and contiguity the ABI expects, allocate missing
outputs with torch (PyTorch is used for device memory and streams only),
and pass raw pointers plus the current HIP stream to the library. Every
step of the path runs in the library's HIP kernels; there is no fallback.
Importing this package fails when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_EP_LIB points the binding at another build of the same sources (the
# host-sanitizer test loads one whose host code is built with AddressSanitizer)
LIB_PATH = os.environ.get("MOE_EP_LIB") or os.path.join(_PKG, "libmoe_ep.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_LAUNCH = 4
MOE_ROUTE_NORMALIZE = 1
MOE_COMBINE_OUT_FP32 = 1
MOE_FLOOR_NT_STORE = 1

EXPORTS = ("moe_route_topk", "moe_route_topk_grouped", "moe_layout_workspace_size", "moe_dispatch_layout",
           "moe_route_dispatch_layout_workspace_size", "moe_route_dispatch_layout", "moe_dispatch_layout_noalloc",
           "moe_dispatch_permute", "moe_combine_reduce", "moe_fp8_row_bytes",
           "moe_dispatch_permute_fp8", "moe_fp8_dequant", "moe_recv_regroup_workspace_size",
           "moe_recv_regroup_layout", "moe_recv_regroup", "moe_recv_ungroup",
           "moe_expert_linear_workspace_size", "moe_expert_linear", "moe_expert_linear_return",
           "moe_expert_return_slots", "moe_hbm_floor", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_string(status)}")
        self.status = status


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python combine_route_topk_amd/build.py` "
            "(hipcc, gfx950) before using the package")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    lib.moe_route_topk.argtypes = [P, P, i64, i32, i32, u32, P, P, P]
    lib.moe_route_topk_grouped.argtypes = [P, P, i64, i32, i32, i32, i32, u32, P, P, P]
    lib.moe_layout_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_dispatch_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                        ctypes.c_size_t, P]
    lib.moe_route_dispatch_layout_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_route_dispatch_layout.argtypes = [P, P, i64, i32, i32, u32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                              ctypes.c_size_t, P]
    lib.moe_dispatch_layout_noalloc.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
    lib.moe_dispatch_permute.argtypes = [P, P, i64, i32, i32, i32, i32, P, i64, P]
    lib.moe_combine_reduce.argtypes = [P, i64, P, P, P, P, i64, i32, i32, u32, P, P]
    lib.moe_fp8_row_bytes.argtypes = [i32, ctypes.POINTER(ctypes.c_int64)]
    lib.moe_dispatch_permute_fp8.argtypes = [P, P, i64, i32, i32, i32, i32, P, i64, P]
    lib.moe_fp8_dequant.argtypes = [P, P, i64, i32, P, P]
    lib.moe_recv_regroup_workspace_size.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_recv_regroup_layout.argtypes = [P, i32, i32, P, P, P, i64, P, ctypes.c_size_t, P]
    lib.moe_recv_regroup.argtypes = [P, P, P, i64, i32, P, P]
    lib.moe_recv_ungroup.argtypes = [P, P, P, i64, i32, P, P]
    lib.moe_expert_linear_workspace_size.argtypes = [i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_expert_linear.argtypes = [P, P, i32, i32, i32, i32, P, i64, P, P, ctypes.c_size_t, P]
    lib.moe_expert_linear_return.argtypes = [P, P, i32, i32, i32, i32, P, i64, i32, i32, i32, P, P, P,
                                             ctypes.c_size_t, P]
    lib.moe_expert_return_slots.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.moe_hbm_floor.argtypes = [P, i64, P, i64, u32, P]
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load_library()


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptr(t: Optional[torch.Tensor], dtypes, name: str, ndim: Optional[int] = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t.data_ptr() or None


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def moe_route_topk(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                   normalize: bool = True, topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None, stream=None):
    """Top-k experts per token and their gate weights (see moe_route_topk)."""
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib.moe_route_topk(
        _ptr(logits, _F32, "logits", 2), _ptr(bias, _F32, "bias", 1), T, E, k,
        MOE_ROUTE_NORMALIZE if normalize else 0, _ptr(topk_idx, _I32, "topk_idx"),
        _ptr(topk_w, _F32, "topk_w"), _stream(stream)))
    return topk_idx, topk_w


def moe_route_topk_grouped(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                           n_groups: int, topk_groups: int, normalize: bool = True,
                           topk_idx: Optional[torch.Tensor] = None,
                           topk_w: Optional[torch.Tensor] = None, stream=None):
    """Group-limited top-k: at most topk_groups of n_groups expert groups per
    token (see moe_route_topk_grouped)."""
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk_grouped", lib.moe_route_topk_grouped(
        _ptr(logits, _F32, "logits", 2), _ptr(bias, _F32, "bias", 1), T, E, k, n_groups,
        topk_groups, MOE_ROUTE_NORMALIZE if normalize else 0, _ptr(topk_idx, _I32, "topk_idx"),
        _ptr(topk_w, _F32, "topk_w"), _stream(stream)))
    return topk_idx, topk_w


def moe_layout_workspace_size(T: int, E: int, k: int, R: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_layout_workspace_size", lib.moe_layout_workspace_size(T, E, k, R, ctypes.byref(n)))
    return n.value


def moe_dispatch_layout(topk_idx: torch.Tensor, E: int, R: int, capacity: int = -1,
                        workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                        with_send_src: bool = True, stream=None) -> dict:
    """Counts, offsets, drops and send positions (see moe_dispatch_layout).

    Returns a dict of int32 GPU tensors: expert_demand [E], expert_counts [E],
    expert_offsets [E+1], dest_counts [R], dest_offsets [R+1], pos [T,k] and
    send_src [T*k] (or None). `out` may hold preallocated tensors by name.
    """
    T, k = topk_idx.shape
    dev = topk_idx.device
    o = dict(out or {})

    def get(name, shape):
        if o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
        return o[name]

    get("expert_demand", (E,)); get("expert_counts", (E,)); get("expert_offsets", (E + 1,))
    get("dest_counts", (R,)); get("dest_offsets", (R + 1,)); get("pos", (T, k))
    if with_send_src:
        get("send_src", (T * k,))
    else:
        o["send_src"] = None
    need = moe_layout_workspace_size(T, E, k, R)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("moe_dispatch_layout", lib.moe_dispatch_layout(
        _ptr(topk_idx, _I32, "topk_idx", 2), T, E, k, R, capacity,
        _ptr(o["expert_demand"], _I32, "expert_demand"), _ptr(o["expert_counts"], _I32, "expert_counts"),
        _ptr(o["expert_offsets"], _I32, "expert_offsets"), _ptr(o["dest_counts"], _I32, "dest_counts"),
        _ptr(o["dest_offsets"], _I32, "dest_offsets"), _ptr(o["pos"], _I32, "pos"),
        _ptr(o["send_src"], _I32, "send_src"), _ptr(workspace, (torch.uint8,), "workspace"),
        workspace.numel(), _stream(stream)))
    return o


def moe_route_dispatch_layout_workspace_size(T: int, E: int, k: int, R: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_route_dispatch_layout_workspace_size",
           lib.moe_route_dispatch_layout_workspace_size(T, E, k, R, ctypes.byref(n)))
    return n.value


def moe_route_dispatch_layout(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int, R: int,
                              capacity: int = -1, normalize: bool = True,
                              workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                              with_send_src: bool = True, stream=None) -> dict:
    """moe_route_topk then moe_dispatch_layout in one call (see
    moe_route_dispatch_layout). Returns the layout dict of moe_dispatch_layout
    plus topk_idx [T,k] and topk_w [T,k]; `out` may hold any of them."""
    T, E = logits.shape
    dev = logits.device
    o = dict(out or {})
    shapes = {"topk_idx": (T, k), "expert_demand": (E,), "expert_counts": (E,), "expert_offsets": (E + 1,),
              "dest_counts": (R,), "dest_offsets": (R + 1,), "pos": (T, k), "send_src": (T * k,)}
    for name, shape in shapes.items():
        if name == "send_src" and not with_send_src:
            o[name] = None
        elif o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
    if o.get("topk_w") is None:
        o["topk_w"] = torch.empty((T, k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_route_dispatch_layout_workspace_size(T, E, k, R), dtype=torch.uint8,
                                device=dev)
    lay = [_ptr(o[n], _I32, n) for n in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts",
                                         "dest_offsets", "pos", "send_src")]
    _check("moe_route_dispatch_layout", lib.moe_route_dispatch_layout(
        _ptr(logits, _F32, "logits", 2), _ptr(bias, _F32, "bias", 1), T, E, k,
        MOE_ROUTE_NORMALIZE if normalize else 0, R, capacity, _ptr(o["topk_idx"], _I32, "topk_idx"),
        _ptr(o["topk_w"], _F32, "topk_w"), *lay, _ptr(workspace, (torch.uint8,), "workspace"),
        workspace.numel(), _stream(stream)))
    return o


def moe_dispatch_layout_noalloc(topk_idx: torch.Tensor, E: int, R: int, capacity: int = -1,
                                out: Optional[dict] = None, with_send_src: bool = True,
                                stream=None) -> dict:
    """moe_dispatch_layout without a workspace (see moe_dispatch_layout_noalloc):
    the library's own per-GPU device array holds the tile histograms. Outputs
    as moe_dispatch_layout; missing ones are allocated here, by torch."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    o = dict(out or {})
    shapes = {"expert_demand": (E,), "expert_counts": (E,), "expert_offsets": (E + 1,),
              "dest_counts": (R,), "dest_offsets": (R + 1,), "pos": (T, k), "send_src": (T * k,)}
    for name, shape in shapes.items():
        if name == "send_src" and not with_send_src:
            o[name] = None
        elif o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
    _check("moe_dispatch_layout_noalloc", lib.moe_dispatch_layout_noalloc(
        _ptr(topk_idx, _I32, "topk_idx", 2), T, E, k, R, capacity,
        *[_ptr(o[n], _I32, n) for n in shapes], _stream(stream)))
    return o


def send_rows_bound(T: int, k: int, E: int, capacity: int = -1) -> int:
    """Rows a send buffer needs: T*k when dropless, else min(T*k, E*capacity)."""
    return T * k if capacity < 0 else min(T * k, E * capacity)


def moe_dispatch_permute(x: torch.Tensor, pos: torch.Tensor, E: int, capacity: int = -1,
                         send: Optional[torch.Tensor] = None, send_rows: Optional[int] = None,
                         stream=None) -> torch.Tensor:
    """send[pos[t, j]] = x[t] for every kept replica (see moe_dispatch_permute).
    E and capacity are the layout's; send (allocated with the bound's rows when
    not given) must hold at least send_rows_bound(T, k, E, capacity) rows."""
    T, H = x.shape
    k = pos.shape[1]
    if send_rows is None:
        send_rows = send.shape[0] if send is not None else send_rows_bound(T, k, E, capacity)
    if send is None:
        send = torch.empty((send_rows, H), dtype=x.dtype, device=x.device)
    if send.shape[0] < send_rows or (send.dim() == 2 and send.shape[1] != H):
        raise ValueError("send buffer smaller than send_rows x H")
    _check("moe_dispatch_permute", lib.moe_dispatch_permute(
        _ptr(x, _BF16, "x", 2), _ptr(pos, _I32, "pos", 2), T, H, k, E, capacity,
        _ptr(send, _BF16, "send"), send_rows, _stream(stream)))
    return send


def moe_combine_reduce(y: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor,
                       shared: Optional[torch.Tensor] = None,
                       residual: Optional[torch.Tensor] = None, out_fp32: bool = False,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gate-weighted sum of the kept expert rows + shared + residual
    (see moe_combine_reduce). Returns bf16 [T, H], or float32 with out_fp32."""
    T, k = pos.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32 if out_fp32 else torch.bfloat16,
                          device=pos.device)
    want = _F32 if out_fp32 else _BF16
    _check("moe_combine_reduce", lib.moe_combine_reduce(
        _ptr(y, _BF16, "y", 2), y.shape[0], _ptr(pos, _I32, "pos", 2),
        _ptr(topk_w, _F32, "topk_w"), _ptr(shared, _BF16, "shared", 2),
        _ptr(residual, _BF16, "residual", 2), T, H, k,
        MOE_COMBINE_OUT_FP32 if out_fp32 else 0, _ptr(out, want, "out"), _stream(stream)))
    return out


def moe_recv_regroup_workspace_size(S: int, E_l: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_recv_regroup_workspace_size", lib.moe_recv_regroup_workspace_size(S, E_l, ctypes.byref(n)))
    return n.value


def moe_recv_regroup_layout(recv_counts: torch.Tensor, max_rows: int, out: Optional[dict] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Expert-major layout of a source-major receive buffer (see
    moe_recv_regroup_layout). Returns int32 GPU tensors local_expert_offsets
    [E_l+1], source_offsets [S+1] and recv_pos [max_rows]."""
    S, El = recv_counts.shape
    dev = recv_counts.device
    o = dict(out or {})
    for name, n in (("local_expert_offsets", El + 1), ("source_offsets", S + 1), ("recv_pos", max_rows)):
        if o.get(name) is None:
            o[name] = torch.empty(n, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_recv_regroup_workspace_size(S, El), dtype=torch.uint8, device=dev)
    _check("moe_recv_regroup_layout", lib.moe_recv_regroup_layout(
        _ptr(recv_counts, _I32, "recv_counts", 2), S, El,
        _ptr(o["local_expert_offsets"], _I32, "local_expert_offsets"),
        _ptr(o["source_offsets"], _I32, "source_offsets"), _ptr(o["recv_pos"], _I32, "recv_pos"),
        max_rows, _ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), _stream(stream)))
    return o


def moe_recv_regroup(recv: torch.Tensor, recv_pos: torch.Tensor, n_rows: torch.Tensor,
                     grouped: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """grouped[recv_pos[i]] = recv[i] for i < n_rows (device scalar)."""
    rows, H = recv.shape
    if grouped is None:
        grouped = torch.empty_like(recv)
    _check("moe_recv_regroup", lib.moe_recv_regroup(
        _ptr(recv, _BF16, "recv", 2), _ptr(recv_pos, _I32, "recv_pos"), _ptr(n_rows, _I32, "n_rows"),
        rows, H, _ptr(grouped, _BF16, "grouped"), _stream(stream)))
    return grouped


def moe_recv_ungroup(grouped: torch.Tensor, recv_pos: torch.Tensor, n_rows: torch.Tensor,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[i] = grouped[recv_pos[i]] for i < n_rows (device scalar)."""
    rows, H = grouped.shape
    if out is None:
        out = torch.empty_like(grouped)
    _check("moe_recv_ungroup", lib.moe_recv_ungroup(
        _ptr(grouped, _BF16, "grouped", 2), _ptr(recv_pos, _I32, "recv_pos"), _ptr(n_rows, _I32, "n_rows"),
        rows, H, _ptr(out, _BF16, "out"), _stream(stream)))
    return out


def moe_fp8_row_bytes(H: int) -> int:
    n = ctypes.c_int64(0)
    _check("moe_fp8_row_bytes", lib.moe_fp8_row_bytes(H, ctypes.byref(n)))
    return n.value


def moe_dispatch_permute_fp8(x: torch.Tensor, pos: torch.Tensor, E: int, capacity: int = -1,
                             send: Optional[torch.Tensor] = None, send_rows: Optional[int] = None,
                             stream=None) -> torch.Tensor:
    """FP8 send buffer [send_rows, moe_fp8_row_bytes(H)] uint8: row pos[t][j]
    holds x[t]'s E4M3 codes then its scale bytes (see moe_dispatch_permute_fp8).
    Rows as in moe_dispatch_permute."""
    T, H = x.shape
    k = pos.shape[1]
    rb = moe_fp8_row_bytes(H)
    if send_rows is None:
        send_rows = send.shape[0] if send is not None else send_rows_bound(T, k, E, capacity)
    if send is None:
        send = torch.empty((send_rows, rb), dtype=torch.uint8, device=x.device)
    elif send.dim() != 2 or send.shape[1] != rb or send.shape[0] < send_rows:
        raise ValueError(f"send must be [>= {send_rows}, {rb}] bytes, got {tuple(send.shape)}")
    _check("moe_dispatch_permute_fp8", lib.moe_dispatch_permute_fp8(
        _ptr(x, _BF16, "x", 2), _ptr(pos, _I32, "pos", 2), T, H, k, E, capacity,
        _ptr(send, (torch.uint8,), "send", 2), send_rows, _stream(stream)))
    return send


def moe_fp8_dequant(rows: torch.Tensor, H: int, n_rows: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bf16 [max_rows, H] decoded from FP8 rows (rows past *n_rows untouched)."""
    max_rows = rows.shape[0]
    if rows.dim() != 2 or rows.shape[1] != moe_fp8_row_bytes(H):
        raise ValueError(f"rows must be [n, {moe_fp8_row_bytes(H)}] bytes, got {tuple(rows.shape)}")
    if out is None:
        out = torch.empty((max_rows, H), dtype=torch.bfloat16, device=rows.device)
    _check("moe_fp8_dequant", lib.moe_fp8_dequant(
        _ptr(rows, (torch.uint8,), "rows", 2), None if n_rows is None else _ptr(n_rows, _I32, "n_rows"),
        max_rows, H, _ptr(out, _BF16, "out", 2), _stream(stream)))
    return out


def moe_expert_linear_workspace_size(S: int, E_l: int, max_rows: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_expert_linear_workspace_size", lib.moe_expert_linear_workspace_size(S, E_l, max_rows, ctypes.byref(n)))
    return n.value


def moe_expert_return_slots() -> int:
    n = ctypes.c_int32(0)
    _check("moe_expert_return_slots", lib.moe_expert_return_slots(ctypes.byref(n)))
    return n.value


def _linear_args(recv, recv_counts, W, y, workspace):
    S, El = recv_counts.shape
    max_rows, H = recv.shape
    El_w, H_out, H_w = W.shape
    if El_w != El or H_w != H:
        raise ValueError(f"W must be [{El}, H_out, {H}], got {tuple(W.shape)}")
    if y is None:
        y = torch.empty((max_rows, H_out), dtype=torch.bfloat16, device=recv.device)
    if workspace is None:
        workspace = torch.empty(moe_expert_linear_workspace_size(S, El, max_rows), dtype=torch.uint8,
                                device=recv.device)
    return S, El, max_rows, H, H_out, y, workspace


def moe_expert_linear(recv: torch.Tensor, recv_counts: torch.Tensor, W: torch.Tensor,
                      y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """y [max_rows, H_out] bf16: each received row times its local expert's
    W[l]^T (see moe_expert_linear)."""
    S, El, max_rows, H, H_out, y, workspace = _linear_args(recv, recv_counts, W, y, workspace)
    _check("moe_expert_linear", lib.moe_expert_linear(
        _ptr(recv, _BF16, "recv", 2), _ptr(recv_counts, _I32, "recv_counts", 2), S, El, H, H_out,
        _ptr(W, _BF16, "W", 3), max_rows, _ptr(y, _BF16, "y", 2),
        _ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), _stream(stream)))
    return y


def moe_expert_linear_return(recv: torch.Tensor, recv_counts: torch.Tensor, W: torch.Tensor,
                             self_rank: int, consumer_blocks: int, band_group: int,
                             y: Optional[torch.Tensor] = None, ret: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None):
    """(y, ret, workspace): the expert output and the rows returned to their
    sources, produced tile by tile with per-band flags (see
    moe_expert_linear_return). workspace[:4] holds the status word."""
    S, El, max_rows, H, H_out, y, workspace = _linear_args(recv, recv_counts, W, y, workspace)
    if ret is None:
        ret = torch.empty((max_rows, H_out), dtype=torch.bfloat16, device=recv.device)
    _check("moe_expert_linear_return", lib.moe_expert_linear_return(
        _ptr(recv, _BF16, "recv", 2), _ptr(recv_counts, _I32, "recv_counts", 2), S, El, H, H_out,
        _ptr(W, _BF16, "W", 3), max_rows, self_rank, consumer_blocks, band_group,
        _ptr(y, _BF16, "y", 2), _ptr(ret, _BF16, "ret", 2),
        _ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), _stream(stream)))
    return y, ret, workspace


def moe_hbm_floor(src: torch.Tensor, read_bytes: int, dst: torch.Tensor, write_bytes: int,
                  nt_store: bool = True, stream=None) -> None:
    """The synthetic floor: a contiguous streaming read of read_bytes from src
    and write of write_bytes to dst (see moe_hbm_floor)."""
    if src.numel() * src.element_size() < read_bytes or dst.numel() * dst.element_size() < write_bytes:
        raise ValueError("floor buffers smaller than the bytes to move")
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _check("moe_hbm_floor", lib.moe_hbm_floor(
        src.data_ptr() or None, read_bytes, dst.data_ptr() or None, write_bytes,
        MOE_FLOOR_NT_STORE if nt_store else 0, _stream(stream)))
