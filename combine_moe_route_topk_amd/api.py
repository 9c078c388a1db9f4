"""Thin PyTorch binding of libmoe_dc: same names as the C ABI.

Each function checks that its tensors are contiguous device tensors of the
expected dtype, allocates any output that was not passed in (torch owns all
device memory), and calls the C function on the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; nothing here
computes.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import (MOE_BF16, MOE_F32, MOE_F8E4M3, MOE_SORT_AUTO, MoeError, check, lib)

__all__ = ["moe_route_topk", "moe_resolve_sorted", "default_sort_cutoff", "moe_dispatch_workspace_bytes", "moe_dispatch",
           "moe_combine", "moe_dequant_rows", "moe_scatter_rows", "moe_gather_rows",
           "moe_route_dispatch", "moe_route_dispatch_noalloc", "moe_route_dispatch_workspace_bytes", "moe_grouped_swiglu_workspace_bytes",
           "moe_grouped_swiglu", "moe_grouped_gemm_fp8", "moe_gather_swiglu_workspace_bytes",
           "moe_gather_swiglu", "moe_gather_swiglu_combine", "moe_abi_version", "DispatchResult",
           "MoeError"]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t: Optional[torch.Tensor], name: str, shape) -> None:
    """The kernels take raw pointers: every buffer must hold exactly the
    elements the C call will touch, so undersized tensors are rejected here,
    before any launch."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_dispatch_out(out: "DispatchResult", n: int, k: int, n_experts: int, n_segments: int,
                        x: Optional[torch.Tensor], x_scales: Optional[torch.Tensor], dev) -> None:
    nk = n * k
    for name, shape in (("expert_counts", (n_experts,)), ("expert_offsets", (n_experts + 1,)),
                        ("segment_offsets", (n_segments + 1,)), ("src_pair", (nk,)),
                        ("dst_pos", (nk,))):
        t = getattr(out, name)
        _need(t, f"out.{name}", (torch.int32,), dev)
        _shape(t, f"out.{name}", shape)
    if out.row_expert is not None:
        _need(out.row_expert, "out.row_expert", (torch.int32,), dev)
        _shape(out.row_expert, "out.row_expert", (nk,))
    if (x is None) != (out.rows is None):
        raise ValueError("out.rows must be given exactly when x is")
    if x is not None:
        _need(out.rows, "out.rows", (x.dtype,), dev)
        _shape(out.rows, "out.rows", (nk, x.shape[1]))
    if (x_scales is None) != (out.row_scales is None):
        raise ValueError("out.row_scales must be given exactly when x_scales is")
    if x_scales is not None:
        _need(out.row_scales, "out.row_scales", (torch.float32,), dev)
        _shape(out.row_scales, "out.row_scales", (nk, x_scales.shape[1]))


_PAYLOAD = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_F8E4M3,
            torch.float8_e4m3fn: MOE_F8E4M3}
_FLOAT_IO = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def _payload_args(x, x_scales, n: int, dev):
    """(dtype code, hidden) of a dispatch payload, with its shape checks."""
    if x is None:
        if x_scales is not None:
            raise ValueError("x_scales given without x")
        return MOE_BF16, 1
    _need(x, "x", tuple(_PAYLOAD), dev)
    if x.dim() != 2 or x.shape[0] != n:
        raise ValueError(f"x must be [N={n}, D]")
    hidden = x.shape[1]
    if x_scales is not None:
        _need(x_scales, "x_scales", (torch.float32,), dev)
        if hidden % 128:
            raise ValueError("an fp8 payload needs D % 128 == 0")
        _shape(x_scales, "x_scales", (n, hidden // 128))
    return _PAYLOAD[x.dtype], hidden


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_route_topk(logits: torch.Tensor, k: int, renormalize: bool = True,
                   topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                   stream=None):
    """logits [N, E] float32 -> (topk_idx [N, k] int32, topk_w [N, k] float32)."""
    _need(logits, "logits", (torch.float32,))
    if logits.dim() != 2:
        raise ValueError("logits must be [N, E]")
    n, e = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((n, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((n, k), dtype=torch.float32, device=logits.device)
    _need(topk_idx, "topk_idx", (torch.int32,), logits.device)
    _need(topk_w, "topk_w", (torch.float32,), logits.device)
    if topk_idx.numel() != n * k or topk_w.numel() != n * k:
        raise ValueError("topk_idx / topk_w must hold N*k elements")
    check("moe_route_topk", lib.moe_route_topk(_ptr(logits), n, e, k, int(bool(renormalize)),
                                               _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
    return topk_idx, topk_w


def default_sort_cutoff(n_experts: int, top_k: int) -> int:
    """Token count above which the automatic mode sorts: 24 routed rows per
    expert on average (N * k / E > 24).  Measured on MI355X with SwiGLU
    experts: the grouped FFN on the sorted layout overtakes the per-row-expert
    FFN on the unsorted one between 24 and 28 rows per expert at D=7168,
    E=256, top-8, F=2048 (768 and 896 tokens) and between 16 and 32 at
    D=4096, E=8, top-2, F=14336 (64 and 128 tokens)."""
    return max(1, 24 * n_experts // max(1, top_k))


def moe_resolve_sorted(sort: int, n_tokens: int, sort_cutoff: int) -> bool:
    out = ctypes.c_int32(-1)
    check("moe_resolve_sorted", lib.moe_resolve_sorted(sort, n_tokens, sort_cutoff, ctypes.byref(out)))
    return bool(out.value)


def moe_dispatch_workspace_bytes(n_tokens: int, n_experts: int, k: int, n_segments: int = 1) -> int:
    return int(lib.moe_dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments))


@dataclass
class DispatchResult:
    sorted: bool
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    segment_offsets: torch.Tensor
    src_pair: torch.Tensor
    dst_pos: torch.Tensor
    row_expert: Optional[torch.Tensor]
    rows: Optional[torch.Tensor]
    row_scales: Optional[torch.Tensor]


def moe_dispatch(x: Optional[torch.Tensor], topk_idx: torch.Tensor, n_experts: int,
                 n_segments: int = 1, sort: int = MOE_SORT_AUTO, sort_cutoff: Optional[int] = None,
                 x_scales: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 out: Optional[DispatchResult] = None, want_row_expert: bool = True,
                 stream=None) -> DispatchResult:
    """Stable expert-major (sorted) or segment-major (unsorted) dispatch.

    x [N, D] float32 / bfloat16 / uint8-or-float8_e4m3fn (then x_scales
    [N, D/128] float32), or None to compute the maps only.  ``out`` may carry
    preallocated outputs (reused in place)."""
    _need(topk_idx, "topk_idx", (torch.int32,))
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [N, k]")
    dev = topk_idx.device
    n, k = topk_idx.shape
    nk = n * k
    dtype, hidden = _payload_args(x, x_scales, n, dev)
    if sort_cutoff is None:
        sort_cutoff = default_sort_cutoff(n_experts, k)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        rows = None if x is None else torch.empty((nk, hidden), dtype=x.dtype, device=dev)
        rs = None if x_scales is None else torch.empty((nk, x_scales.shape[1]), dtype=torch.float32, device=dev)
        out = DispatchResult(False, torch.empty(n_experts, **i32), torch.empty(n_experts + 1, **i32),
                             torch.empty(n_segments + 1, **i32), torch.empty(nk, **i32),
                             torch.empty(nk, **i32),
                             torch.empty(nk, **i32) if want_row_expert else None, rows, rs)
    _check_dispatch_out(out, n, k, n_experts, n_segments, x, x_scales, dev)
    if workspace is None:
        wsb = moe_dispatch_workspace_bytes(n, n_experts, k, n_segments)
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), dev)
    used = ctypes.c_int32(-1)
    check("moe_dispatch", lib.moe_dispatch(
        _ptr(x), _ptr(x_scales), dtype, n, hidden, _ptr(topk_idx), n_experts, k, n_segments, sort,
        sort_cutoff, ctypes.byref(used), _ptr(out.rows), _ptr(out.row_scales),
        _ptr(out.expert_counts), _ptr(out.expert_offsets), _ptr(out.segment_offsets),
        _ptr(out.src_pair), _ptr(out.dst_pos), _ptr(out.row_expert), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    out.sorted = bool(used.value)
    return out


def moe_route_dispatch_workspace_bytes(n_tokens: int, n_experts: int, k: int,
                                       n_segments: int = 1) -> int:
    return int(lib.moe_route_dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments))


def _route_dispatch_prepare(logits, x, k, n_segments, x_scales, topk_idx, topk_w, out,
                            want_row_expert):
    """Shared checks and output allocation of the two route + dispatch calls."""
    _need(logits, "logits", (torch.float32,))
    if logits.dim() != 2:
        raise ValueError("logits must be [N, E]")
    dev = logits.device
    n, e = logits.shape
    nk = n * k
    if topk_idx is None:
        topk_idx = torch.empty((n, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((n, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", (torch.int32,), dev)
    _need(topk_w, "topk_w", (torch.float32,), dev)
    _shape(topk_idx, "topk_idx", (n, k))
    _shape(topk_w, "topk_w", (n, k))
    dtype, hidden = _payload_args(x, x_scales, n, dev)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        rows = None if x is None else torch.empty((nk, hidden), dtype=x.dtype, device=dev)
        rs = None if x_scales is None else torch.empty((nk, x_scales.shape[1]), dtype=torch.float32, device=dev)
        out = DispatchResult(False, torch.empty(e, **i32), torch.empty(e + 1, **i32),
                             torch.empty(n_segments + 1, **i32), torch.empty(nk, **i32),
                             torch.empty(nk, **i32),
                             torch.empty(nk, **i32) if want_row_expert else None, rows, rs)
    _check_dispatch_out(out, n, k, e, n_segments, x, x_scales, dev)
    return dev, n, e, dtype, hidden, topk_idx, topk_w, out


def moe_route_dispatch(logits: torch.Tensor, x: Optional[torch.Tensor], k: int,
                       n_segments: int = 1, renormalize: bool = True, sort: int = MOE_SORT_AUTO,
                       sort_cutoff: Optional[int] = None, x_scales: Optional[torch.Tensor] = None,
                       topk_idx: Optional[torch.Tensor] = None,
                       topk_w: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[DispatchResult] = None, want_row_expert: bool = True,
                       stream=None):
    """Routing and dispatch in one call -> (topk_idx, topk_w, DispatchResult)."""
    dev, n, e, dtype, hidden, topk_idx, topk_w, out = _route_dispatch_prepare(
        logits, x, k, n_segments, x_scales, topk_idx, topk_w, out, want_row_expert)
    if sort_cutoff is None:
        sort_cutoff = default_sort_cutoff(e, k)
    if workspace is None:
        wsb = moe_route_dispatch_workspace_bytes(n, e, k, n_segments)
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), dev)
    used = ctypes.c_int32(-1)
    check("moe_route_dispatch", lib.moe_route_dispatch(
        _ptr(logits), int(bool(renormalize)), _ptr(topk_idx), _ptr(topk_w), _ptr(x), _ptr(x_scales),
        dtype, n, hidden, e, k, n_segments, sort, sort_cutoff, ctypes.byref(used), _ptr(out.rows),
        _ptr(out.row_scales), _ptr(out.expert_counts), _ptr(out.expert_offsets),
        _ptr(out.segment_offsets), _ptr(out.src_pair), _ptr(out.dst_pos), _ptr(out.row_expert),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    out.sorted = bool(used.value)
    return topk_idx, topk_w, out


def moe_route_dispatch_noalloc(logits: torch.Tensor, x: Optional[torch.Tensor], k: int,
                               n_segments: int = 1, renormalize: bool = True,
                               sort: int = MOE_SORT_AUTO, sort_cutoff: Optional[int] = None,
                               x_scales: Optional[torch.Tensor] = None,
                               topk_idx: Optional[torch.Tensor] = None,
                               topk_w: Optional[torch.Tensor] = None,
                               out: Optional[DispatchResult] = None,
                               want_row_expert: bool = True, stream=None):
    """moe_route_dispatch without a workspace: the library's static per-GPU
    scratch array serves instead, and the C call allocates nothing.  A caller
    that cannot allocate passes every output (topk_idx, topk_w, out); calls
    that overlap on one GPU race on the shared scratch."""
    dev, n, e, dtype, hidden, topk_idx, topk_w, out = _route_dispatch_prepare(
        logits, x, k, n_segments, x_scales, topk_idx, topk_w, out, want_row_expert)
    if sort_cutoff is None:
        sort_cutoff = default_sort_cutoff(e, k)
    used = ctypes.c_int32(-1)
    check("moe_route_dispatch_noalloc", lib.moe_route_dispatch_noalloc(
        _ptr(logits), int(bool(renormalize)), _ptr(topk_idx), _ptr(topk_w), _ptr(x), _ptr(x_scales),
        dtype, n, hidden, e, k, n_segments, sort, sort_cutoff, ctypes.byref(used), _ptr(out.rows),
        _ptr(out.row_scales), _ptr(out.expert_counts), _ptr(out.expert_offsets),
        _ptr(out.segment_offsets), _ptr(out.src_pair), _ptr(out.dst_pos), _ptr(out.row_expert),
        _stream(stream)))
    out.sorted = bool(used.value)
    return topk_idx, topk_w, out


def moe_scatter_rows(x: torch.Tensor, dst_pos: torch.Tensor, k: int,
                     rows: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rows[dst_pos[t*k+j]] = x[t] (bytes copied unchanged).  x [N, ...] contiguous."""
    _need(x, "x", None)
    _need(dst_pos, "dst_pos", (torch.int32,), x.device)
    n = x.shape[0]
    row_bytes = x[0].numel() * x.element_size() if n else max(1, x.element_size())
    if rows is None:
        rows = torch.empty((n * k,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    _need(rows, "rows", (x.dtype,), x.device)
    if dst_pos.numel() != n * k or rows.shape[0] != n * k:
        raise ValueError("dst_pos and rows must hold N*k entries")
    if tuple(rows.shape[1:]) != tuple(x.shape[1:]):
        raise ValueError("rows must have the row shape of x")
    check("moe_scatter_rows", lib.moe_scatter_rows(_ptr(x), n, row_bytes, k, _ptr(dst_pos),
                                                   _ptr(rows), _stream(stream)))
    return rows


def moe_gather_rows(x: torch.Tensor, src_pair: torch.Tensor, k: int,
                    rows: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rows[p] = x[src_pair[p] // k] (bytes copied unchanged)."""
    _need(x, "x", None)
    _need(src_pair, "src_pair", (torch.int32,), x.device)
    n = x.shape[0]
    n_rows = src_pair.numel()
    row_bytes = x[0].numel() * x.element_size() if n else max(1, x.element_size())
    if rows is None:
        rows = torch.empty((n_rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    _need(rows, "rows", (x.dtype,), x.device)
    _shape(rows, "rows", (n_rows,) + tuple(x.shape[1:]))
    check("moe_gather_rows", lib.moe_gather_rows(_ptr(x), n, row_bytes, k, _ptr(src_pair), n_rows,
                                                 _ptr(rows), _stream(stream)))
    return rows


def moe_combine(y: torch.Tensor, dst_pos: torch.Tensor, topk_w: torch.Tensor,
                out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """y [N*k, D] float32/bfloat16, dst_pos [N*k] int32, topk_w [N, k] float32 -> out [N, D]."""
    _need(y, "y", tuple(_FLOAT_IO))
    dev = y.device
    _need(dst_pos, "dst_pos", (torch.int32,), dev)
    _need(topk_w, "topk_w", (torch.float32,), dev)
    if topk_w.dim() != 2 or y.dim() != 2:
        raise ValueError("topk_w must be [N, k] and y [N*k, D]")
    n, k = topk_w.shape
    hidden = y.shape[1]
    if dst_pos.numel() != n * k or y.shape[0] != n * k:
        raise ValueError("y / dst_pos must hold N*k rows")
    if out is None:
        out = torch.empty((n, hidden), dtype=out_dtype or y.dtype, device=dev)
    _need(out, "out", tuple(_FLOAT_IO), dev)
    _shape(out, "out", (n, hidden))
    check("moe_combine", lib.moe_combine(_ptr(y), _FLOAT_IO[y.dtype], n, hidden, k, _ptr(dst_pos),
                                         _ptr(topk_w), _ptr(out), _FLOAT_IO[out.dtype],
                                         _stream(stream)))
    return out


def moe_dequant_rows(rows: torch.Tensor, row_scales: torch.Tensor,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp8 E4M3FN rows [R, D] (uint8 or float8_e4m3fn) + scales [R, D/128] -> bf16 [R, D]."""
    _need(rows, "rows", (torch.uint8, torch.float8_e4m3fn))
    _need(row_scales, "row_scales", (torch.float32,), rows.device)
    if rows.dim() != 2 or rows.shape[1] % 128:
        raise ValueError("rows must be [R, D] with D % 128 == 0")
    r, d = rows.shape
    _shape(row_scales, "row_scales", (r, d // 128))
    if out is None:
        out = torch.empty((r, d), dtype=torch.bfloat16, device=rows.device)
    _need(out, "out", (torch.bfloat16,), rows.device)
    _shape(out, "out", (r, d))
    check("moe_dequant_rows", lib.moe_dequant_rows(_ptr(rows), _ptr(row_scales), r, d, _ptr(out),
                                                   _stream(stream)))
    return out


def moe_grouped_swiglu_workspace_bytes(n_rows: int, n_experts: int, hidden: int, ffn: int) -> int:
    return int(lib.moe_grouped_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn))


def moe_grouped_swiglu(rows: torch.Tensor, expert_offsets: torch.Tensor, w_gate: torch.Tensor,
                       w_up: torch.Tensor, w_down: torch.Tensor, y: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rows [R, D] bf16 grouped by expert; w_gate/w_up [E, F, D], w_down [E, D, F] bf16."""
    _need(rows, "rows", (torch.bfloat16,))
    dev = rows.device
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, name, (torch.bfloat16,), dev)
    _need(expert_offsets, "expert_offsets", (torch.int32,), dev)
    if rows.dim() != 2 or w_gate.dim() != 3:
        raise ValueError("moe_grouped_swiglu: rows must be [R, D] and w_gate [E, F, D]")
    r, d = rows.shape
    e, f, d2 = w_gate.shape
    if d2 != d or tuple(w_up.shape) != (e, f, d) or tuple(w_down.shape) != (e, d, f) or \
            expert_offsets.numel() != e + 1:
        raise ValueError("moe_grouped_swiglu: inconsistent shapes (w_gate, w_up [E, F, D], "
                         "w_down [E, D, F], expert_offsets [E+1])")
    if y is None:
        y = torch.empty_like(rows)
    _need(y, "y", (torch.bfloat16,), dev)
    if tuple(y.shape) != (r, d):
        raise ValueError("moe_grouped_swiglu: y must be [R, D]")
    if workspace is None:
        workspace = torch.empty(max(moe_grouped_swiglu_workspace_bytes(r, e, d, f), 256),
                                dtype=torch.uint8, device=dev)
    check("moe_grouped_swiglu", lib.moe_grouped_swiglu(
        _ptr(rows), r, d, _ptr(expert_offsets), e, _ptr(w_gate), _ptr(w_up), _ptr(w_down), f,
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def moe_gather_swiglu_workspace_bytes(n_rows: int, n_experts: int, hidden: int, ffn: int) -> int:
    return int(lib.moe_gather_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn))


def moe_gather_swiglu(rows: torch.Tensor, row_expert: torch.Tensor, w_gate: torch.Tensor,
                      w_up: torch.Tensor, w_down: torch.Tensor, y: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rows [R, D] bf16 in any order, row_expert [R] int32 (the expert of each
    row); w_gate/w_up [E, F, D], w_down [E, D, F] bf16 -> y [R, D] bf16, row r
    computed with expert row_expert[r] (rows with an id outside [0, E) keep
    what y held)."""
    _need(rows, "rows", (torch.bfloat16,))
    dev = rows.device
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, name, (torch.bfloat16,), dev)
    _need(row_expert, "row_expert", (torch.int32,), dev)
    r, d = rows.shape
    e, f, d2 = w_gate.shape
    if d2 != d or tuple(w_up.shape) != (e, f, d) or tuple(w_down.shape) != (e, d, f) or \
            row_expert.numel() != r:
        raise ValueError("moe_gather_swiglu: inconsistent shapes")
    if y is None:
        y = torch.empty_like(rows)
    _need(y, "y", (torch.bfloat16,), dev)
    if tuple(y.shape) != (r, d):
        raise ValueError("moe_gather_swiglu: y must be [R, D]")
    if workspace is None:
        workspace = torch.empty(max(moe_gather_swiglu_workspace_bytes(r, e, d, f), 256),
                                dtype=torch.uint8, device=dev)
    check("moe_gather_swiglu", lib.moe_gather_swiglu(
        _ptr(rows), r, d, _ptr(row_expert), e, _ptr(w_gate), _ptr(w_up), _ptr(w_down), f,
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def moe_gather_swiglu_combine(rows: torch.Tensor, row_expert: torch.Tensor,
                              topk_w: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                              w_down: torch.Tensor, row_pair: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_gather_swiglu with the combine fused in: out [N, D] float32 (zeros
    unless given) += sum over rows r of topk_w[q] * FFN(rows[r]) at token q // k,
    q = row_pair[r] (or r); topk_w [N, k] float32."""
    _need(rows, "rows", (torch.bfloat16,))
    dev = rows.device
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, name, (torch.bfloat16,), dev)
    _need(row_expert, "row_expert", (torch.int32,), dev)
    _need(topk_w, "topk_w", (torch.float32,), dev)
    r, d = rows.shape
    e, f, d2 = w_gate.shape
    n, k = topk_w.shape
    if d2 != d or tuple(w_up.shape) != (e, f, d) or tuple(w_down.shape) != (e, d, f) or \
            row_expert.numel() != r:
        raise ValueError("moe_gather_swiglu_combine: inconsistent shapes")
    if row_pair is not None:
        _need(row_pair, "row_pair", (torch.int32,), dev)
        if row_pair.numel() != r:
            raise ValueError("moe_gather_swiglu_combine: row_pair must have one entry per row")
    if out is None:
        out = torch.zeros((n, d), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    if tuple(out.shape) != (n, d):
        raise ValueError("moe_gather_swiglu_combine: out must be [N, D]")
    if workspace is None:
        workspace = torch.empty(max(moe_gather_swiglu_workspace_bytes(r, e, d, f), 256),
                                dtype=torch.uint8, device=dev)
    check("moe_gather_swiglu_combine", lib.moe_gather_swiglu_combine(
        _ptr(rows), r, d, _ptr(row_expert), _ptr(row_pair) if row_pair is not None else None,
        _ptr(topk_w), n, k, e, _ptr(w_gate), _ptr(w_up), _ptr(w_down), f, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def moe_grouped_gemm_fp8(rows: torch.Tensor, row_scales: torch.Tensor, expert_offsets: torch.Tensor,
                         w: torch.Tensor, w_scales: torch.Tensor, y: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """rows [R, K] E4M3FN codes (uint8) with row_scales [R, K/128] f32, grouped
    by expert through expert_offsets [E+1]; w [E, N, K] E4M3FN codes with
    w_scales [E, N/128, K/128] f32 -> y [R, N] bf16."""
    _need(rows, "rows", (torch.uint8,))
    dev = rows.device
    _need(row_scales, "row_scales", (torch.float32,), dev)
    _need(expert_offsets, "expert_offsets", (torch.int32,), dev)
    _need(w, "w", (torch.uint8,), dev)
    _need(w_scales, "w_scales", (torch.float32,), dev)
    r, k = rows.shape
    e, n, k2 = w.shape
    if k2 != k or tuple(row_scales.shape) != (r, k // 128) or \
            tuple(w_scales.shape) != (e, n // 128, k // 128) or expert_offsets.numel() != e + 1:
        raise ValueError("moe_grouped_gemm_fp8: inconsistent shapes")
    if y is None:
        y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
    _need(y, "y", (torch.bfloat16,), dev)
    if tuple(y.shape) != (r, n):
        raise ValueError("moe_grouped_gemm_fp8: y must be [R, N]")
    check("moe_grouped_gemm_fp8", lib.moe_grouped_gemm_fp8(
        _ptr(rows), _ptr(row_scales), r, k, _ptr(expert_offsets), e, _ptr(w), _ptr(w_scales), n,
        _ptr(y), _stream(stream)))
    return y
