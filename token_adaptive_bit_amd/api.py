"""PyTorch-facing wrappers over the C ABI (include/mbq.h).

Tensors are plain CUDA (HIP) tensors; each call passes their device pointers and the
current stream to libmbq and returns without synchronizing.  No arithmetic happens here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MBQ_BF16, MBQ_F32, MbqDesc, MbqError, check, describe

__all__ = ["PackedLinear", "pack", "pack_bitplane", "pack_concat", "route", "route_from_logits", "regroup", "linear",
           "linear_workspace", "describe", "MbqError", "MlpRouter", "route_mlp",
           "route_mlp_from_scores", "route_mlp_workspace", "linear_lowrank",
           "linear_lowrank_workspace"]


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MBQ_F32
    if t.dtype == torch.bfloat16:
        return MBQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _p(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class PackedLinear:
    """One packed weight: geometry plus the slice-major blob (uint8 device tensor)."""
    desc: MbqDesc
    blob: torch.Tensor

    @property
    def n(self): return self.desc.n

    @property
    def k(self): return self.desc.k

    @property
    def group(self): return self.desc.group

    @property
    def slices(self): return self.desc.slices

    def slice_bytes(self) -> int:
        return int(self.desc.slice_stride)


def pack(w: torch.Tensor, group: int = 128, slices: int = 3, status: torch.Tensor | None = None,
         out: torch.Tensor | None = None) -> PackedLinear:
    """MoBiSlice pack of W [n, k] (float32 or bfloat16) into a new or given blob."""
    _dev(w, "w")
    n, k = w.shape
    d = describe(n, k, group, slices)
    if out is None:
        out = torch.empty(int(d.total_bytes), dtype=torch.uint8, device=w.device)
    if out.numel() < d.total_bytes:
        raise ValueError("out is smaller than the packed size")
    check(_lib.LIB.mbq_pack(ctypes.byref(d), _p(w), _dtype(w), _p(out), _p(status), _stream()),
          "mbq_pack")
    return PackedLinear(d, out)


def pack_bitplane(w: torch.Tensor, group: int = 128, slices: int = 3,
                  status: torch.Tensor | None = None, out: torch.Tensor | None = None) -> PackedLinear:
    """Bit-plane pack of W [n, k]: slice j is the j-th 2-bit plane of one uniform 2S-bit
    code; the routed linear reads it like any other blob."""
    _dev(w, "w")
    n, k = w.shape
    d = describe(n, k, group, slices)
    if out is None:
        out = torch.empty(int(d.total_bytes), dtype=torch.uint8, device=w.device)
    if out.numel() < d.total_bytes:
        raise ValueError("out is smaller than the packed size")
    check(_lib.LIB.mbq_pack_bitplane(ctypes.byref(d), _p(w), _dtype(w), _p(out), _p(status), _stream()),
          "mbq_pack_bitplane")
    return PackedLinear(d, out)


def pack_concat(ws, group: int = 128, slices: int = 3, status: torch.Tensor | None = None):
    """One blob for weights that read the same activations: W_i [n_i, k] packed as the row
    concatenation (every n_i but the last a multiple of 16).  Returns the PackedLinear and
    the first output column of each weight in the fused output."""
    k = ws[0].shape[1]
    n = sum(w.shape[0] for w in ws)
    d = describe(n, k, group, slices)
    out = torch.empty(int(d.total_bytes), dtype=torch.uint8, device=ws[0].device)
    starts, row0 = [], 0
    for w in ws:
        _dev(w, "w")
        if w.shape[1] != k:
            raise ValueError("all weights must have the same number of inputs")
        check(_lib.LIB.mbq_pack_rows(ctypes.byref(d), row0, w.shape[0], _p(w), _dtype(w), _p(out),
                                     _p(status), _stream()), "mbq_pack_rows")
        starts.append(row0)
        row0 += w.shape[0]
    return PackedLinear(d, out), starts


def route(x: torch.Tensor, wr: torch.Tensor, logits=None, budget=None, perm=None, offsets=None):
    """Router logits x . wr (float32), budgets 1 + first argmax, stable regroup."""
    _dev(x, "x")
    _dev(wr, "wr")
    t, k = x.shape
    s = wr.shape[1]
    dev = x.device
    logits = torch.empty((t, s), dtype=torch.float32, device=dev) if logits is None else logits
    budget = torch.empty(t, dtype=torch.int32, device=dev) if budget is None else budget
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    check(_lib.LIB.mbq_route(t, k, s, _p(x), _dtype(x), _p(wr), _p(logits), _p(budget), _p(perm),
                             _p(offsets), _stream()), "mbq_route")
    return logits, budget, perm, offsets


def route_from_logits(logits: torch.Tensor):
    """Route from given float32 logits [t, s] (the bit-exact route contract)."""
    _dev(logits, "logits")
    t, s = logits.shape
    dev = logits.device
    budget = torch.empty(t, dtype=torch.int32, device=dev)
    perm = torch.empty(t, dtype=torch.int32, device=dev)
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev)
    check(_lib.LIB.mbq_route(t, 0, s, None, MBQ_F32, None, _p(logits), _p(budget), _p(perm),
                             _p(offsets), _stream()), "mbq_route")
    return budget, perm, offsets


def regroup(budget: torch.Tensor, slices: int, perm=None, offsets=None):
    """Stable regroup of tokens with given budgets (int32 [t], values in 1..slices)."""
    _dev(budget, "budget")
    t = budget.shape[0]
    dev = budget.device
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(slices + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    check(_lib.LIB.mbq_regroup(t, slices, _p(budget), _p(perm), _p(offsets), _stream()),
          "mbq_regroup")
    return perm, offsets


@dataclass
class MlpRouter:
    """Weights of the 2-layer MLP router on the device.

    w1 [hidden, k] bfloat16, b1 [hidden] float32, w2 [hidden, slices - 1] float32,
    b2 [slices - 1] float32.
    """
    w1: torch.Tensor
    b1: torch.Tensor
    w2: torch.Tensor
    b2: torch.Tensor

    @property
    def hidden(self): return self.w1.shape[0]

    @property
    def k(self): return self.w1.shape[1]

    @property
    def slices(self): return self.w2.shape[1] + 1


def route_mlp_workspace(t: int, k: int, hidden: int) -> int:
    return _lib.route_mlp_workspace_bytes(t, k, hidden)


def _mlp_outputs(t, s, dev, scores, budget, perm, offsets):
    scores = torch.empty((t, s - 1), dtype=torch.float32, device=dev) if scores is None else scores
    budget = torch.empty(t, dtype=torch.int32, device=dev) if budget is None else budget
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    return scores, budget, perm, offsets


def route_mlp(x: torch.Tensor, r: MlpRouter, delta: float, scores=None, budget=None, perm=None,
              offsets=None, workspace: torch.Tensor | None = None):
    """MLP router scores, threshold-delta budgets and the stable regroup."""
    _dev(x, "x")
    for name in ("w1", "b1", "w2", "b2"):
        _dev(getattr(r, name), name)
    if r.w1.dtype != torch.bfloat16:
        raise TypeError("w1 must be bfloat16")
    t, k = x.shape
    s = r.slices
    scores, budget, perm, offsets = _mlp_outputs(t, s, x.device, scores, budget, perm, offsets)
    need = route_mlp_workspace(t, k, r.hidden)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_route_mlp(t, k, s, r.hidden, _p(x), _dtype(x), _p(r.w1), _p(r.b1),
                                 _p(r.w2), _p(r.b2), float(delta), _p(scores), _p(budget),
                                 _p(perm), _p(offsets), _p(workspace), ws_bytes, _stream()),
          "mbq_route_mlp")
    return scores, budget, perm, offsets


def route_mlp_from_scores(scores: torch.Tensor, delta: float, budget=None, perm=None,
                          offsets=None):
    """Threshold-delta budgets and regroup from given float32 scores [t, slices - 1]."""
    _dev(scores, "scores")
    t, r = scores.shape
    s = r + 1
    _, budget, perm, offsets = _mlp_outputs(t, s, scores.device, scores, budget, perm, offsets)
    check(_lib.LIB.mbq_route_mlp(t, 0, s, 0, None, MBQ_F32, None, None, None, None, float(delta),
                                 _p(scores), _p(budget), _p(perm), _p(offsets), None, 0,
                                 _stream()), "mbq_route_mlp")
    return budget, perm, offsets


def linear_workspace(p: PackedLinear, t: int, x_dtype=torch.bfloat16) -> int:
    return _lib.workspace_bytes(p.desc, t, MBQ_BF16 if x_dtype == torch.bfloat16 else MBQ_F32)


def linear(p: PackedLinear, x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
           out_dtype: torch.dtype | None = None, y: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Routed linear y = x . W^(b(t))^T, original token order."""
    _dev(x, "x")
    t = x.shape[0]
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=x.device)
    need = linear_workspace(p, t, x.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_linear(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(perm),
                              _p(offsets), _p(y), _dtype(y), _p(workspace), ws_bytes, _stream()),
          "mbq_linear")
    return y


def route_linear(p: PackedLinear, x: torch.Tensor, wr: torch.Tensor, out_dtype: torch.dtype | None = None,
                 y: torch.Tensor | None = None, logits=None, budget=None, perm=None, offsets=None,
                 workspace: torch.Tensor | None = None):
    """One decode step: route (logits x . wr, budgets, stable regroup) and the routed linear.
    Returns (y, logits, budget, perm, offsets); one launch for bfloat16 x and t <= 16 when
    K fits one workgroup, else route then linear."""
    _dev(x, "x")
    _dev(wr, "wr")
    t = x.shape[0]
    s = p.slices
    dev = x.device
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=dev)
    logits = torch.empty((t, s), dtype=torch.float32, device=dev) if logits is None else logits
    budget = torch.empty(t, dtype=torch.int32, device=dev) if budget is None else budget
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    need = linear_workspace(p, t, x.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_route_linear(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(wr),
                                    _p(logits), _p(budget), _p(perm), _p(offsets), _p(y), _dtype(y),
                                    _p(workspace), ws_bytes, _stream()), "mbq_route_linear")
    return y, logits, budget, perm, offsets


def linear_lowrank_workspace(p: PackedLinear, t: int, rank: int, x_dtype=torch.bfloat16) -> int:
    return _lib.lowrank_workspace_bytes(p.desc, t, MBQ_BF16 if x_dtype == torch.bfloat16 else MBQ_F32,
                                        rank)


def linear_lowrank(p: PackedLinear, x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
                   a: torch.Tensor, b: torch.Tensor, out_dtype: torch.dtype | None = None,
                   y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Routed linear plus the low-rank side path: y = x . W^(b(t))^T + (x . a^T) . b^T,
    a [rank, k] and b [n, rank] bfloat16."""
    _dev(x, "x")
    _dev(a, "a")
    _dev(b, "b")
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("a and b must be bfloat16")
    t = x.shape[0]
    rank = a.shape[0]
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=x.device)
    need = linear_lowrank_workspace(p, t, rank, x.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_linear_lowrank(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(perm),
                                      _p(offsets), _p(a), _p(b), rank, _p(y), _dtype(y), _p(workspace),
                                      ws_bytes, _stream()), "mbq_linear_lowrank")
    return y
