"""Python binding of the RocketKV C ABI (include/rkv.h): same call names, torch tensors in and
out. Argument marshalling only: every step runs in the HIP kernels of librkv.so; torch provides
device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

F32, BF16 = 0, 1
POOL = {"avg": 0, "max": 1}


class RkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.load().rkv_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise RkvError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], name: str, shape: Tuple[int, ...]) -> None:
    """The kernels index every buffer by the sizes the call passes, so a tensor of another shape
    would be read or written past its end: refused here, before any pointer is handed over."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _size_query(fn: str, *args: int) -> int:
    out = ctypes.c_size_t(0)
    _check(fn, getattr(_lib.load(), fn)(*args, ctypes.byref(out)))
    return out.value


def _workspace(t: torch.Tensor, nbytes: int, ws: Optional[torch.Tensor]) -> Tuple[int, int]:
    if nbytes == 0:
        return 0, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=t.device)
    _dev(ws, "workspace")
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ----------------------------------------------------------------------------- workspace sizes

def snapkvpp_workspace_bytes(B, Hq, Hkv, L, D, W, keep, dtype) -> int:
    return _size_query("rkv_snapkvpp_workspace_bytes", B, Hq, Hkv, L, D, W, keep, dtype)


def topk_workspace_bytes(rows, n, k) -> int:
    return _size_query("rkv_topk_workspace_bytes", rows, n, k)


def sparse_attend_workspace_bytes(B, Hq, Hkv, D, page_size, n_pages, dtype) -> int:
    return _size_query("rkv_sparse_attend_workspace_bytes", B, Hq, Hkv, D, page_size, n_pages,
                       dtype)


# ----------------------------------------------------------------------------- calls

def rkv_snapkvpp_evict(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: int,
                       pool_kernel: int, pool_type: str = "avg", scale: Optional[float] = None, *,
                       kept_idx: Optional[torch.Tensor] = None,
                       k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                       pooled_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, indices_only: bool = False):
    """SnapKV++ eviction. q_win [B,Hq,W,D]; k, v [B,Hkv,L,D] -> (kept_idx, k_c, v_c)."""
    B, Hq, W, D = q_win.shape
    Hkv, L = k.shape[1], k.shape[2]
    dt = _dtype_code(k)
    Lc = min(keep, L)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _shape(k, "k", (B, Hkv, L, D))
    _shape(v, "v", (B, Hkv, L, D))
    _shape(kept_idx, "kept_idx", (B, Hkv, Lc))
    _shape(k_out, "k_out", (B, Hkv, Lc, D))
    _shape(v_out, "v_out", (B, Hkv, Lc, D))
    _shape(pooled_out, "pooled_out", (B, Hkv, max(L - W, 1)))
    if kept_idx is None:
        kept_idx = torch.empty((B, Hkv, Lc), dtype=torch.int32, device=k.device)
    if not indices_only:
        if k_out is None:
            k_out = torch.empty((B, Hkv, Lc, D), dtype=k.dtype, device=k.device)
        if v_out is None:
            v_out = torch.empty((B, Hkv, Lc, D), dtype=k.dtype, device=k.device)
    nbytes = snapkvpp_workspace_bytes(B, Hq, Hkv, L, D, W, keep, dt)
    ws, wsb = _workspace(k, nbytes, workspace)
    _check("rkv_snapkvpp_evict", _lib.load().rkv_snapkvpp_evict(
        _dev(q_win, "q_win", k.dtype), _dev(k, "k"), _dev(v, "v", k.dtype), B, Hq, Hkv, L, D, W,
        keep, pool_kernel, POOL[pool_type], scale, dt, _dev(kept_idx, "kept_idx", torch.int32),
        _dev(k_out, "k_out", k.dtype) if k_out is not None else None,
        _dev(v_out, "v_out", k.dtype) if v_out is not None else None,
        _dev(pooled_out, "pooled_out", torch.float32) if pooled_out is not None else None,
        ws, wsb, _stream(k)))
    return kept_idx, k_out, v_out


def rkv_build_page_summaries(k_c: torch.Tensor, page_size: int, *,
                             kmin_t: Optional[torch.Tensor] = None,
                             kmax_t: Optional[torch.Tensor] = None):
    """k_c [B,Hkv,Lc,D] -> (kmin_t, kmax_t) channel-major [B,Hkv,D,P]."""
    B, Hkv, Lc, D = k_c.shape
    P = -(-Lc // page_size)
    _shape(kmin_t, "kmin_t", (B, Hkv, D, P))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, P))
    if kmin_t is None:
        kmin_t = torch.empty((B, Hkv, D, P), dtype=k_c.dtype, device=k_c.device)
    if kmax_t is None:
        kmax_t = torch.empty((B, Hkv, D, P), dtype=k_c.dtype, device=k_c.device)
    _check("rkv_build_page_summaries", _lib.load().rkv_build_page_summaries(
        _dev(k_c, "k_c"), B, Hkv, Lc, D, page_size, _dtype_code(k_c),
        _dev(kmin_t, "kmin_t", k_c.dtype), _dev(kmax_t, "kmax_t", k_c.dtype), _stream(k_c)))
    return kmin_t, kmax_t


def rkv_hybrid_approx_scores(q: torch.Tensor, kmin_t: torch.Tensor, kmax_t: torch.Tensor, r: int,
                             *, chan_idx: Optional[torch.Tensor] = None,
                             page_scores: Optional[torch.Tensor] = None,
                             return_channels: bool = False):
    """q [B,Hq,D]; summaries [B,Hkv,D,P] -> page_scores [B,Hkv,P] (and chan_idx [B,Hkv,r])."""
    B, Hq, D = q.shape
    Hkv, P = kmin_t.shape[1], kmin_t.shape[3]
    _shape(kmin_t, "kmin_t", (B, Hkv, D, P))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, P))
    _shape(page_scores, "page_scores", (B, Hkv, P))
    _shape(chan_idx, "chan_idx", (B, Hkv, r))
    if page_scores is None:
        page_scores = torch.empty((B, Hkv, P), dtype=torch.float32, device=q.device)
    if return_channels and chan_idx is None:
        chan_idx = torch.empty((B, Hkv, r), dtype=torch.int32, device=q.device)
    _check("rkv_hybrid_approx_scores", _lib.load().rkv_hybrid_approx_scores(
        _dev(q, "q"), _dev(kmin_t, "kmin_t", q.dtype), _dev(kmax_t, "kmax_t", q.dtype), B, Hq, Hkv,
        D, P, r, _dtype_code(q),
        _dev(chan_idx, "chan_idx", torch.int32) if chan_idx is not None else None,
        _dev(page_scores, "page_scores", torch.float32), _stream(q)))
    return (page_scores, chan_idx) if return_channels else page_scores


def rkv_topk_select(scores: torch.Tensor, k: int, *, idx_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores [..., n] float32 -> int32 [..., min(k, n)] ascending indices of the top k."""
    n = scores.shape[-1]
    rows = scores.numel() // n
    kk = min(k, n)
    _shape(idx_out, "idx_out", (*scores.shape[:-1], kk))
    if idx_out is None:
        idx_out = torch.empty((*scores.shape[:-1], kk), dtype=torch.int32, device=scores.device)
    nbytes = topk_workspace_bytes(rows, n, k)
    ws, wsb = _workspace(scores, nbytes, workspace)
    _check("rkv_topk_select", _lib.load().rkv_topk_select(
        _dev(scores, "scores", torch.float32), rows, n, k, _dev(idx_out, "idx_out", torch.int32),
        ws, wsb, _stream(scores)))
    return idx_out


def rkv_sparse_attend_decode(q: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor,
                             page_idx: torch.Tensor, page_size: int,
                             scale: Optional[float] = None, *,
                             out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q [B,Hq,D]; k_c, v_c [B,Hkv,Lc,D]; page_idx [B,Hkv,n_pages] -> out [B,Hq,D]."""
    B, Hq, D = q.shape
    Hkv, Lc = k_c.shape[1], k_c.shape[2]
    n_pages = page_idx.shape[-1]
    _shape(k_c, "k_c", (B, Hkv, Lc, D))
    _shape(v_c, "v_c", (B, Hkv, Lc, D))
    _shape(page_idx, "page_idx", (B, Hkv, n_pages))
    _shape(out, "out", (B, Hq, D))
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    nbytes = sparse_attend_workspace_bytes(B, Hq, Hkv, D, page_size, n_pages, dt)
    ws, wsb = _workspace(q, nbytes, workspace)
    _check("rkv_sparse_attend_decode", _lib.load().rkv_sparse_attend_decode(
        _dev(q, "q"), _dev(k_c, "k_c", q.dtype), _dev(v_c, "v_c", q.dtype),
        _dev(page_idx, "page_idx", torch.int32), B, Hq, Hkv, Lc, D, page_size, n_pages, scale, dt,
        _dev(out, "out", q.dtype), ws, wsb, _stream(q)))
    return out


def hybrid_decode_workspace_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, dtype) -> int:
    return _size_query("rkv_hybrid_decode_workspace_bytes", B, Hq, Hkv, Lc, D, page_size, n_pages,
                       dtype)


def rkv_hybrid_decode_workspace(q: torch.Tensor, Hkv: int, Lc: int, page_size: int,
                                n_pages: int) -> torch.Tensor:
    """A prepared workspace for rkv_hybrid_decode_step with q's batch, heads and dtype."""
    B, Hq, D = q.shape
    nbytes = hybrid_decode_workspace_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, _dtype_code(q))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check("rkv_hybrid_decode_workspace_init", _lib.load().rkv_hybrid_decode_workspace_init(
        ws.data_ptr(), nbytes, _stream(q)))
    return ws


# Status bits of the fused step that make a call's output invalid (the others are informational:
# a block computed work whose owner had not delivered in time).
DECODE_STATUS_INVALID = 0xF


def decode_workspace_status(ws: torch.Tensor, clear: bool = False) -> int:
    """The fused step's status word through rkv_hybrid_decode_status (synchronises the current
    stream): every call on this workspace was valid when (status & DECODE_STATUS_INVALID) == 0."""
    val = ctypes.c_uint32(0)
    _check("rkv_hybrid_decode_status", _lib.load().rkv_hybrid_decode_status(
        ws.data_ptr(), ws.numel() * ws.element_size(), int(bool(clear)), ctypes.byref(val),
        _stream(ws)))
    return int(val.value)


def _step_shapes(q, kmin_t, kmax_t, Hkv, P_rows, P, r, n_pages, chan_idx, page_scores,
                 page_idx, out) -> None:
    """Shapes of a fused step's summaries (P_rows pages per channel row) and outputs (P valid)."""
    B, Hq, D = q.shape
    _shape(kmin_t, "kmin_t", (B, Hkv, D, P_rows))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, P_rows))
    _shape(chan_idx, "chan_idx", (B, Hkv, r))
    _shape(page_scores, "page_scores", (B, Hkv, P))
    _shape(page_idx, "page_idx", (B, Hkv, n_pages))
    _shape(out, "out", (B, Hq, D))


def rkv_hybrid_decode_step(q: torch.Tensor, kmin_t: torch.Tensor, kmax_t: torch.Tensor,
                           k_c: torch.Tensor, v_c: torch.Tensor, page_size: int, r: int,
                           n_pages: int, scale: Optional[float] = None, *,
                           chan_idx: Optional[torch.Tensor] = None,
                           page_scores: Optional[torch.Tensor] = None,
                           page_idx: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused decode step (one launch). q [B,Hq,D]; summaries [B,Hkv,D,P]; k_c, v_c
    [B,Hkv,Lc,D] -> out [B,Hq,D]. Optional outputs: chan_idx, page_scores, page_idx."""
    B, Hq, D = q.shape
    Hkv, Lc = k_c.shape[1], k_c.shape[2]
    P = -(-Lc // page_size)
    _shape(k_c, "k_c", (B, Hkv, Lc, D))
    _shape(v_c, "v_c", (B, Hkv, Lc, D))
    _step_shapes(q, kmin_t, kmax_t, Hkv, P, P, r, n_pages, chan_idx, page_scores, page_idx, out)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = rkv_hybrid_decode_workspace(q, Hkv, Lc, page_size, n_pages)
    ws, wsb = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    opt = lambda t, n, d: _dev(t, n, d) if t is not None else None  # noqa: E731
    _check("rkv_hybrid_decode_step", _lib.load().rkv_hybrid_decode_step(
        _dev(q, "q"), _dev(kmin_t, "kmin_t", q.dtype), _dev(kmax_t, "kmax_t", q.dtype),
        _dev(k_c, "k_c", q.dtype), _dev(v_c, "v_c", q.dtype), B, Hq, Hkv, Lc, D, page_size, r,
        n_pages, scale, dt, opt(chan_idx, "chan_idx", torch.int32),
        opt(page_scores, "page_scores", torch.float32), opt(page_idx, "page_idx", torch.int32),
        _dev(out, "out", q.dtype), ws, wsb, _stream(q)))
    return out


def rkv_hybrid_decode_step_noalloc(q: torch.Tensor, kmin_t: torch.Tensor, kmax_t: torch.Tensor,
                                   k_c: torch.Tensor, v_c: torch.Tensor, page_size: int, r: int,
                                   n_pages: int, scale: Optional[float] = None, *,
                                   chan_idx: Optional[torch.Tensor] = None,
                                   page_scores: Optional[torch.Tensor] = None,
                                   page_idx: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None,
                                   status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rkv_hybrid_decode_step on the library's own per-GPU scratch (no workspace; the C call
    allocates nothing). status: optional int32 GPU tensor of one element that receives the
    scratch's status word after the step. Calls that overlap in time on one GPU race."""
    B, Hq, D = q.shape
    Hkv, Lc = k_c.shape[1], k_c.shape[2]
    P = -(-Lc // page_size)
    _shape(k_c, "k_c", (B, Hkv, Lc, D))
    _shape(v_c, "v_c", (B, Hkv, Lc, D))
    _step_shapes(q, kmin_t, kmax_t, Hkv, P, P, r, n_pages, chan_idx, page_scores, page_idx, out)
    if status is not None and status.numel() != 1:
        raise ValueError("status must hold one element")
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    opt = lambda t, n, d: _dev(t, n, d) if t is not None else None  # noqa: E731
    _check("rkv_hybrid_decode_step_noalloc", _lib.load().rkv_hybrid_decode_step_noalloc(
        _dev(q, "q"), _dev(kmin_t, "kmin_t", q.dtype), _dev(kmax_t, "kmax_t", q.dtype),
        _dev(k_c, "k_c", q.dtype), _dev(v_c, "v_c", q.dtype), B, Hq, Hkv, Lc, D, page_size, r,
        n_pages, scale, dt, opt(chan_idx, "chan_idx", torch.int32),
        opt(page_scores, "page_scores", torch.float32), opt(page_idx, "page_idx", torch.int32),
        _dev(out, "out", q.dtype), opt(status, "status", torch.int32), _stream(q)))
    return out


# ----------------------------------------------------------------------------- growing caches
def _cap_shapes(k_c: torch.Tensor, kmin_t: torch.Tensor, page_size: int) -> Tuple[int, int]:
    cap = k_c.shape[2]
    pcap = -(-cap // page_size)
    if kmin_t.shape[-1] != pcap:
        raise ValueError(f"summaries must have ceil(cap/page_size) = {pcap} pages per row "
                         f"(got {kmin_t.shape[-1]})")
    return cap, pcap


def rkv_build_page_summaries_cap(k_c: torch.Tensor, Lc: int, page_size: int, *,
                                 kmin_t: Optional[torch.Tensor] = None,
                                 kmax_t: Optional[torch.Tensor] = None):
    """k_c [B,Hkv,cap,D] (first Lc slots valid) -> (kmin_t, kmax_t) [B,Hkv,D,ceil(cap/ps)]."""
    B, Hkv, cap, D = k_c.shape
    pcap = -(-cap // page_size)
    _shape(kmin_t, "kmin_t", (B, Hkv, D, pcap))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, pcap))
    if kmin_t is None:
        kmin_t = torch.empty((B, Hkv, D, pcap), dtype=k_c.dtype, device=k_c.device)
    if kmax_t is None:
        kmax_t = torch.empty((B, Hkv, D, pcap), dtype=k_c.dtype, device=k_c.device)
    _cap_shapes(k_c, kmin_t, page_size)
    _check("rkv_build_page_summaries_cap", _lib.load().rkv_build_page_summaries_cap(
        _dev(k_c, "k_c"), B, Hkv, Lc, cap, D, page_size, _dtype_code(k_c),
        _dev(kmin_t, "kmin_t", k_c.dtype), _dev(kmax_t, "kmax_t", k_c.dtype), _stream(k_c)))
    return kmin_t, kmax_t


def rkv_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor,
                  kmin_t: torch.Tensor, kmax_t: torch.Tensor, Lc: int, page_size: int) -> int:
    """Writes k_new, v_new [B,Hkv,D] to slot Lc of k_c, v_c [B,Hkv,cap,D] and folds k_new into
    its page summary (kmin_t, kmax_t [B,Hkv,D,ceil(cap/ps)]). Returns the new length Lc + 1."""
    B, Hkv, cap, D = k_c.shape
    _, pcap = _cap_shapes(k_c, kmin_t, page_size)
    _shape(v_c, "v_c", (B, Hkv, cap, D))
    _shape(kmin_t, "kmin_t", (B, Hkv, D, pcap))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, pcap))
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new, v_new must be [B, Hkv, D] of the caches")
    dt = k_c.dtype
    _check("rkv_kv_append", _lib.load().rkv_kv_append(
        _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt), B, Hkv, Lc, cap, D, page_size,
        _dtype_code(k_c), _dev(k_c, "k_c"), _dev(v_c, "v_c", dt), _dev(kmin_t, "kmin_t", dt),
        _dev(kmax_t, "kmax_t", dt), _stream(k_c)))
    return Lc + 1


def rkv_hybrid_decode_step_cap(q: torch.Tensor, kmin_t: torch.Tensor, kmax_t: torch.Tensor,
                               k_c: torch.Tensor, v_c: torch.Tensor, Lc: int, page_size: int,
                               r: int, n_pages: int, scale: Optional[float] = None, *,
                               chan_idx: Optional[torch.Tensor] = None,
                               page_scores: Optional[torch.Tensor] = None,
                               page_idx: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rkv_hybrid_decode_step over the first Lc slots of caches of capacity cap = k_c.shape[2]
    (summaries [B,Hkv,D,ceil(cap/ps)]); the workspace is rkv_hybrid_decode_workspace(q, Hkv,
    cap, page_size, n_pages)."""
    B, Hq, D = q.shape
    Hkv = k_c.shape[1]
    cap, pcap = _cap_shapes(k_c, kmin_t, page_size)
    _shape(k_c, "k_c", (B, Hkv, cap, D))
    _shape(v_c, "v_c", (B, Hkv, cap, D))
    _step_shapes(q, kmin_t, kmax_t, Hkv, pcap, -(-Lc // page_size), r, n_pages, chan_idx,
                 page_scores, page_idx, out)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = rkv_hybrid_decode_workspace(q, Hkv, cap, page_size, n_pages)
    ws, wsb = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    opt = lambda t, n, d: _dev(t, n, d) if t is not None else None  # noqa: E731
    _check("rkv_hybrid_decode_step_cap", _lib.load().rkv_hybrid_decode_step_cap(
        _dev(q, "q"), _dev(kmin_t, "kmin_t", q.dtype), _dev(kmax_t, "kmax_t", q.dtype),
        _dev(k_c, "k_c", q.dtype), _dev(v_c, "v_c", q.dtype), B, Hq, Hkv, Lc, cap, D, page_size,
        r, n_pages, scale, dt, opt(chan_idx, "chan_idx", torch.int32),
        opt(page_scores, "page_scores", torch.float32), opt(page_idx, "page_idx", torch.int32),
        _dev(out, "out", q.dtype), ws, wsb, _stream(q)))
    return out


# ----------------------------------------------------------------------------- budget planner
def rkv_plan_budget(L: int, D: int, W: int, token_budget: int) -> dict:
    """Settings of both stages for a token budget (host only): keep, page_size, r, topk,
    pool_kernel, approx_tokens."""
    outs = [ctypes.c_int(0) for _ in range(6)]
    _check("rkv_plan_budget", _lib.load().rkv_plan_budget(
        L, D, W, token_budget, *[ctypes.byref(o) for o in outs]))
    names = ("keep", "page_size", "r", "topk", "pool_kernel", "approx_tokens")
    return {n: o.value for n, o in zip(names, outs)}


# ----------------------------------------------------------------------------- multi-turn variant
def _kept_rows(k: torch.Tensor, kept_idx: torch.Tensor) -> int:
    B, Hkv, L, D = k.shape
    if kept_idx.dim() != 3 or tuple(kept_idx.shape[:2]) != (B, Hkv):
        raise ValueError("kept_idx must be [B, Hkv, Lc] of the cache")
    _dev(kept_idx, "kept_idx", torch.int32)
    return kept_idx.shape[2]


def rkv_build_page_summaries_indexed(k: torch.Tensor, kept_idx: torch.Tensor, page_size: int, *,
                                     kmin_t: Optional[torch.Tensor] = None,
                                     kmax_t: Optional[torch.Tensor] = None):
    """Summaries of the view k[b, h, kept_idx[b, h]] of the full cache k [B,Hkv,L,D]:
    (kmin_t, kmax_t) [B,Hkv,D,ceil(Lc/ps)]."""
    B, Hkv, L, D = k.shape
    Lc = _kept_rows(k, kept_idx)
    P = -(-Lc // page_size)
    _shape(kmin_t, "kmin_t", (B, Hkv, D, P))
    _shape(kmax_t, "kmax_t", (B, Hkv, D, P))
    if kmin_t is None:
        kmin_t = torch.empty((B, Hkv, D, P), dtype=k.dtype, device=k.device)
    if kmax_t is None:
        kmax_t = torch.empty((B, Hkv, D, P), dtype=k.dtype, device=k.device)
    _check("rkv_build_page_summaries_indexed", _lib.load().rkv_build_page_summaries_indexed(
        _dev(k, "k"), kept_idx.data_ptr(), B, Hkv, L, Lc, D, page_size, _dtype_code(k),
        _dev(kmin_t, "kmin_t", k.dtype), _dev(kmax_t, "kmax_t", k.dtype), _stream(k)))
    return kmin_t, kmax_t


def rkv_hybrid_decode_step_indexed(q: torch.Tensor, kmin_t: torch.Tensor, kmax_t: torch.Tensor,
                                   k: torch.Tensor, v: torch.Tensor, kept_idx: torch.Tensor,
                                   page_size: int, r: int, n_pages: int,
                                   scale: Optional[float] = None, *,
                                   chan_idx: Optional[torch.Tensor] = None,
                                   page_scores: Optional[torch.Tensor] = None,
                                   page_idx: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rkv_hybrid_decode_step over the view k[b, h, kept_idx[b, h]] (and v) of the full caches
    k, v [B,Hkv,L,D]; summaries from rkv_build_page_summaries_indexed."""
    B, Hq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    Lc = _kept_rows(k, kept_idx)
    P = -(-Lc // page_size)
    _shape(k, "k", (B, Hkv, L, D))
    _shape(v, "v", (B, Hkv, L, D))
    _step_shapes(q, kmin_t, kmax_t, Hkv, P, P, r, n_pages, chan_idx, page_scores, page_idx, out)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = rkv_hybrid_decode_workspace(q, Hkv, Lc, page_size, n_pages)
    ws, wsb = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    opt = lambda t, n, d: _dev(t, n, d) if t is not None else None  # noqa: E731
    _check("rkv_hybrid_decode_step_indexed", _lib.load().rkv_hybrid_decode_step_indexed(
        _dev(q, "q"), _dev(kmin_t, "kmin_t", q.dtype), _dev(kmax_t, "kmax_t", q.dtype),
        _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), kept_idx.data_ptr(), B, Hq, Hkv, L, Lc, D,
        page_size, r, n_pages, scale, dt, opt(chan_idx, "chan_idx", torch.int32),
        opt(page_scores, "page_scores", torch.float32), opt(page_idx, "page_idx", torch.int32),
        _dev(out, "out", q.dtype), ws, wsb, _stream(q)))
    return out


def hybrid_decode_step(q, k_c, v_c, kmin_t, kmax_t, page_size: int, r: int, topk: int,
                       scale: Optional[float] = None, *, scores=None, pages=None, out=None,
                       workspace=None):
    """One decode step as the three C-ABI calls in order: approx scores, page top-k, attention."""
    P = kmin_t.shape[-1]
    if topk % page_size:
        raise ValueError("topk must be a multiple of page_size")
    n_pages = min(topk // page_size, P)
    scores = rkv_hybrid_approx_scores(q, kmin_t, kmax_t, r, page_scores=scores)
    pages = rkv_topk_select(scores, n_pages, idx_out=pages)
    out = rkv_sparse_attend_decode(q, k_c, v_c, pages, page_size, scale, out=out,
                                   workspace=workspace)
    return out, pages, scores
