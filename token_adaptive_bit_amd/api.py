"""PyTorch-facing wrappers over the C ABI (include/mbq.h).

Tensors are plain CUDA (HIP) tensors; each call checks their shapes, dtypes and device
(the C ABI carries pointers, not sizes, so a mismatch would otherwise read or write past
an allocation), passes their device pointers and the current stream to libmbq and returns
without synchronizing.  No arithmetic happens here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (MBQ_BF16, MBQ_F32, MBQ_MUL_AUTO, MBQ_MUL_BF16, MBQ_MUL_FP8_FP4, MBQ_PATH_AUTO,
                   MBQ_PATH_GENERIC, MbqDesc, MbqError, MbqOpts, check, describe)

__all__ = ["PackedLinear", "pack", "pack_bitplane", "pack_concat", "route", "route_from_logits", "regroup", "linear",
           "linear_workspace", "describe", "MbqError", "MlpRouter", "route_mlp",
           "route_mlp_from_scores", "route_mlp_workspace", "linear_lowrank",
           "linear_lowrank_workspace", "route_linear", "route_linear_workspace", "linear_static", "opts",
           "route_prepare", "route_prepare_workspace", "route_linear_prepared"]

_FLOATS = (torch.float32, torch.bfloat16)


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
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _arg(t, name: str, shape, dtypes, device) -> None:
    """A tensor argument: on `device`, contiguous, of this shape and one of these dtypes."""
    _dev(t, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")


def _opt(t, name, shape, dtypes, device) -> None:
    if t is not None:
        _arg(t, name, shape, dtypes, device)


def _workspace(ws, name, need, device) -> None:
    if ws is None:
        return
    _dev(ws, name)
    if ws.device != device:
        raise ValueError(f"{name} is on {ws.device}, expected {device}")
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError(f"{name} must be a 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"{name} holds {ws.numel()} bytes, the call needs {need}")


_PATHS = {None: MBQ_PATH_AUTO, "auto": MBQ_PATH_AUTO, "generic": MBQ_PATH_GENERIC}
_MULS = {None: MBQ_MUL_AUTO, "auto": MBQ_MUL_AUTO, "bf16": MBQ_MUL_BF16, "fp8fp4": MBQ_MUL_FP8_FP4}


def opts(path: str | None = None, decode_mul: str | None = None, prefill_slots: int = 0,
         decode_launches: int = 0) -> MbqOpts:
    """Kernel choices (mbq_opts): path 'auto' | 'generic'; decode_mul 'auto' | 'bf16' |
    'fp8fp4' (the routed decode step's multiply); prefill_slots, the workgroups the MFMA
    prefill's tile plan assumes run at once (0: the device's compute units);
    decode_launches 0 (the plan's choice), 1 or 2 for the fp8 x fp4 decode step."""
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(k for k in _PATHS if k)}")
    if decode_mul not in _MULS:
        raise ValueError(f"decode_mul must be one of {sorted(k for k in _MULS if k)}")
    if int(prefill_slots) < 0:
        raise ValueError("prefill_slots must be >= 0")
    if int(decode_launches) not in (0, 1, 2):
        raise ValueError("decode_launches must be 0, 1 or 2")
    return MbqOpts(_PATHS[path], _MULS[decode_mul], int(prefill_slots), int(decode_launches))


def _optp(o: MbqOpts | None):
    return None if o is None else ctypes.byref(o)


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


def _blob(p: PackedLinear, device) -> None:
    _dev(p.blob, "packed blob")
    if p.blob.device != device:
        raise ValueError(f"packed blob is on {p.blob.device}, expected {device}")
    if p.blob.dtype != torch.uint8 or p.blob.numel() < p.desc.total_bytes:
        raise ValueError("packed blob must be uint8 holding at least desc.total_bytes")


def _pack_args(w, status, out, d):
    _dev(w, "w")
    if w.dim() != 2 or w.dtype not in _FLOATS:
        raise TypeError("w must be a 2-D float32 or bfloat16 tensor")
    _opt(status, "status", (1,), (torch.int32,), w.device)
    if out is None:
        out = torch.empty(int(d.total_bytes), dtype=torch.uint8, device=w.device)
    _workspace(out, "out", int(d.total_bytes), w.device)
    return out


def pack(w: torch.Tensor, group: int = 128, slices: int = 3, status: torch.Tensor | None = None,
         out: torch.Tensor | None = None) -> PackedLinear:
    """MoBiSlice pack of W [n, k] (float32 or bfloat16) into a new or given blob."""
    _dev(w, "w")
    n, k = w.shape
    d = describe(n, k, group, slices)
    out = _pack_args(w, status, out, d)
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
    out = _pack_args(w, status, out, d)
    check(_lib.LIB.mbq_pack_bitplane(ctypes.byref(d), _p(w), _dtype(w), _p(out), _p(status), _stream()),
          "mbq_pack_bitplane")
    return PackedLinear(d, out)


def pack_concat(ws, group: int = 128, slices: int = 3, status: torch.Tensor | None = None):
    """One blob for weights that read the same activations: W_i [n_i, k] packed as the row
    concatenation (every n_i but the last a multiple of 16).  Returns the PackedLinear and
    the first output column of each weight in the fused output."""
    for i, w in enumerate(ws):
        _dev(w, f"w[{i}]")
        if w.dim() != 2 or w.dtype not in _FLOATS:
            raise TypeError("every weight must be a 2-D float32 or bfloat16 tensor")
        if w.device != ws[0].device:
            raise ValueError("all weights must be on one device")
    k = ws[0].shape[1]
    n = sum(w.shape[0] for w in ws)
    d = describe(n, k, group, slices)
    _opt(status, "status", (1,), (torch.int32,), ws[0].device)
    out = torch.empty(int(d.total_bytes), dtype=torch.uint8, device=ws[0].device)
    starts, row0 = [], 0
    for w in ws:
        if w.shape[1] != k:
            raise ValueError("all weights must have the same number of inputs")
        check(_lib.LIB.mbq_pack_rows(ctypes.byref(d), row0, w.shape[0], _p(w), _dtype(w), _p(out),
                                     _p(status), _stream()), "mbq_pack_rows")
        starts.append(row0)
        row0 += w.shape[0]
    return PackedLinear(d, out), starts


def _route_outputs(t, s, dev, logits, budget, perm, offsets):
    _opt(logits, "logits", (t, s), (torch.float32,), dev)
    _opt(budget, "budget", (t,), (torch.int32,), dev)
    _opt(perm, "perm", (t,), (torch.int32,), dev)
    _opt(offsets, "offsets", (s + 1,), (torch.int32,), dev)
    logits = torch.empty((t, s), dtype=torch.float32, device=dev) if logits is None else logits
    budget = torch.empty(t, dtype=torch.int32, device=dev) if budget is None else budget
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    return logits, budget, perm, offsets


def route(x: torch.Tensor, wr: torch.Tensor, logits=None, budget=None, perm=None, offsets=None):
    """Router logits x . wr (float32), budgets 1 + first argmax, stable regroup."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [t, k]")
    t, k = x.shape
    _dev(wr, "wr")
    if wr.dim() != 2:
        raise ValueError("wr must be 2-D [k, s]")
    s = wr.shape[1]
    _arg(x, "x", (t, k), _FLOATS, x.device)
    _arg(wr, "wr", (k, s), (torch.float32,), x.device)
    logits, budget, perm, offsets = _route_outputs(t, s, x.device, logits, budget, perm, offsets)
    check(_lib.LIB.mbq_route(t, k, s, _p(x), _dtype(x), _p(wr), _p(logits), _p(budget), _p(perm),
                             _p(offsets), _stream()), "mbq_route")
    return logits, budget, perm, offsets


def route_from_logits(logits: torch.Tensor):
    """Route from given float32 logits [t, s] (the bit-exact route contract)."""
    _dev(logits, "logits")
    if logits.dim() != 2 or logits.dtype != torch.float32:
        raise TypeError("logits must be a 2-D float32 tensor")
    t, s = logits.shape
    _, budget, perm, offsets = _route_outputs(t, s, logits.device, None, None, None, None)
    check(_lib.LIB.mbq_route(t, 0, s, None, MBQ_F32, None, _p(logits), _p(budget), _p(perm),
                             _p(offsets), _stream()), "mbq_route")
    return budget, perm, offsets


def regroup(budget: torch.Tensor, slices: int, perm=None, offsets=None):
    """Stable regroup of tokens with given budgets (int32 [t], values in 1..slices)."""
    _dev(budget, "budget")
    if budget.dim() != 1 or budget.dtype != torch.int32:
        raise TypeError("budget must be a 1-D int32 tensor")
    t = budget.shape[0]
    dev = budget.device
    _opt(perm, "perm", (t,), (torch.int32,), dev)
    _opt(offsets, "offsets", (slices + 1,), (torch.int32,), dev)
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
    _opt(scores, "scores", (t, s - 1), (torch.float32,), dev)
    _opt(budget, "budget", (t,), (torch.int32,), dev)
    _opt(perm, "perm", (t,), (torch.int32,), dev)
    _opt(offsets, "offsets", (s + 1,), (torch.int32,), dev)
    scores = torch.empty((t, s - 1), dtype=torch.float32, device=dev) if scores is None else scores
    budget = torch.empty(t, dtype=torch.int32, device=dev) if budget is None else budget
    perm = torch.empty(t, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(s + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    return scores, budget, perm, offsets


def route_mlp(x: torch.Tensor, r: MlpRouter, delta: float, scores=None, budget=None, perm=None,
              offsets=None, workspace: torch.Tensor | None = None):
    """MLP router scores, threshold-delta budgets and the stable regroup."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [t, k]")
    t, k = x.shape
    dev = x.device
    _arg(x, "x", (t, k), _FLOATS, dev)
    h = r.w1.shape[0]
    s = r.slices
    _arg(r.w1, "w1", (h, k), (torch.bfloat16,), dev)
    _arg(r.b1, "b1", (h,), (torch.float32,), dev)
    _arg(r.w2, "w2", (h, s - 1), (torch.float32,), dev)
    _arg(r.b2, "b2", (s - 1,), (torch.float32,), dev)
    scores, budget, perm, offsets = _mlp_outputs(t, s, dev, scores, budget, perm, offsets)
    need = route_mlp_workspace(t, k, h)
    _workspace(workspace, "workspace", need, dev)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_route_mlp(t, k, s, h, _p(x), _dtype(x), _p(r.w1), _p(r.b1),
                                 _p(r.w2), _p(r.b2), float(delta), _p(scores), _p(budget),
                                 _p(perm), _p(offsets), _p(workspace), ws_bytes, _stream()),
          "mbq_route_mlp")
    return scores, budget, perm, offsets


def route_mlp_from_scores(scores: torch.Tensor, delta: float, budget=None, perm=None,
                          offsets=None):
    """Threshold-delta budgets and regroup from given float32 scores [t, slices - 1]."""
    _dev(scores, "scores")
    if scores.dim() != 2 or scores.dtype != torch.float32:
        raise TypeError("scores must be a 2-D float32 tensor")
    t, r = scores.shape
    s = r + 1
    _, budget, perm, offsets = _mlp_outputs(t, s, scores.device, scores, budget, perm, offsets)
    check(_lib.LIB.mbq_route_mlp(t, 0, s, 0, None, MBQ_F32, None, None, None, None, float(delta),
                                 _p(scores), _p(budget), _p(perm), _p(offsets), None, 0,
                                 _stream()), "mbq_route_mlp")
    return budget, perm, offsets


def linear_workspace(p: PackedLinear, t: int, x_dtype=torch.bfloat16) -> int:
    return _lib.workspace_bytes(p.desc, t, MBQ_BF16 if x_dtype == torch.bfloat16 else MBQ_F32)


def _linear_args(p, x, perm, offsets, out_dtype, y):
    """Checks the routed linear's tensors; returns (t, y)."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [t, k]")
    t = x.shape[0]
    dev = x.device
    _blob(p, dev)
    _arg(x, "x", (t, p.k), _FLOATS, dev)
    _arg(perm, "perm", (t,), (torch.int32,), dev)
    _arg(offsets, "offsets", (p.slices + 1,), (torch.int32,), dev)
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=dev)
    _arg(y, "y", (t, p.n), _FLOATS, dev)
    return t, y


def linear(p: PackedLinear, x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
           out_dtype: torch.dtype | None = None, y: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, options: MbqOpts | None = None) -> torch.Tensor:
    """Routed linear y = x . W^(b(t))^T, original token order."""
    t, y = _linear_args(p, x, perm, offsets, out_dtype, y)
    need = linear_workspace(p, t, x.dtype)
    _workspace(workspace, "workspace", need, x.device)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_linear(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(perm),
                              _p(offsets), _p(y), _dtype(y), _p(workspace), ws_bytes, _optp(options),
                              _stream()), "mbq_linear")
    return y


def linear_static(p: PackedLinear, x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
                  out_dtype: torch.dtype | None = None, y: torch.Tensor | None = None,
                  options: MbqOpts | None = None) -> torch.Tensor:
    """The routed linear without a workspace (mbq_linear_static): for callers that cannot
    allocate; y must then be given.  Calls that overlap on one GPU race (one shared buffer)."""
    t, y = _linear_args(p, x, perm, offsets, out_dtype, y)
    check(_lib.LIB.mbq_linear_static(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(perm),
                                     _p(offsets), _p(y), _dtype(y), _optp(options), _stream()),
          "mbq_linear_static")
    return y


def route_linear_workspace(p: PackedLinear, t: int, x_dtype=torch.bfloat16) -> int:
    return _lib.route_linear_workspace_bytes(p.desc, t, MBQ_BF16 if x_dtype == torch.bfloat16 else MBQ_F32)


def route_prepare_workspace(p: PackedLinear, t: int) -> int:
    n = ctypes.c_size_t(0)
    check(_lib.LIB.mbq_route_prepare_workspace(ctypes.byref(p.desc), t, ctypes.byref(n)),
          "mbq_route_prepare_workspace")
    return int(n.value)


def route_prepare(p: PackedLinear, x: torch.Tensor, wr: torch.Tensor, prep: torch.Tensor | None = None):
    """First launch of the fp8 x fp4 decode step: prepared operands and partial logits of
    x [t, k] (bfloat16, t <= 16) for weights shaped like p.  Returns the prepared buffer."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [t, k]")
    t = x.shape[0]
    _arg(x, "x", (t, p.k), (torch.bfloat16,), x.device)
    _arg(wr, "wr", (p.k, p.slices), (torch.float32,), x.device)
    need = route_prepare_workspace(p, t)
    if prep is None:
        prep = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _workspace(prep, "prep", need, x.device)
    check(_lib.LIB.mbq_route_prepare(ctypes.byref(p.desc), t, _p(x), _p(wr), _p(prep), prep.numel(), _stream()),
          "mbq_route_prepare")
    return prep


def route_linear_prepared(p: PackedLinear, t: int, prep: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                          y: torch.Tensor | None = None, logits=None, budget=None, perm=None, offsets=None):
    """Second launch: routing from the prepared partial logits and the routed linear on the
    prepared operands.  Returns (y, logits, budget, perm, offsets)."""
    dev = prep.device
    _blob(p, dev)
    _workspace(prep, "prep", route_prepare_workspace(p, t), dev)
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=dev)
    _arg(y, "y", (t, p.n), _FLOATS, dev)
    logits, budget, perm, offsets = _route_outputs(t, p.slices, dev, logits, budget, perm, offsets)
    check(_lib.LIB.mbq_route_linear_prepared(ctypes.byref(p.desc), _p(p.blob), t, _p(prep), prep.numel(),
                                             _p(logits), _p(budget), _p(perm), _p(offsets), _p(y), _dtype(y),
                                             _stream()), "mbq_route_linear_prepared")
    return y, logits, budget, perm, offsets


def route_linear(p: PackedLinear, x: torch.Tensor, wr: torch.Tensor, out_dtype: torch.dtype | None = None,
                 y: torch.Tensor | None = None, logits=None, budget=None, perm=None, offsets=None,
                 workspace: torch.Tensor | None = None, options: MbqOpts | None = None):
    """One decode step: route (logits x . wr, budgets, stable regroup) and the routed linear.
    Returns (y, logits, budget, perm, offsets).  For bfloat16 x, t <= 16 and K within one
    workgroup: one launch up to 8 tokens, two from 9 (the fp8 operands prepared once in the
    workspace); otherwise route, then linear."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [t, k]")
    t = x.shape[0]
    s = p.slices
    dev = x.device
    _blob(p, dev)
    _arg(x, "x", (t, p.k), _FLOATS, dev)
    _arg(wr, "wr", (p.k, s), (torch.float32,), dev)
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((t, p.n), dtype=out_dtype, device=dev)
    _arg(y, "y", (t, p.n), _FLOATS, dev)
    logits, budget, perm, offsets = _route_outputs(t, s, dev, logits, budget, perm, offsets)
    need = route_linear_workspace(p, t, x.dtype)
    _workspace(workspace, "workspace", need, dev)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_route_linear(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(wr),
                                    _p(logits), _p(budget), _p(perm), _p(offsets), _p(y), _dtype(y),
                                    _p(workspace), ws_bytes, _optp(options), _stream()),
          "mbq_route_linear")
    return y, logits, budget, perm, offsets


def linear_lowrank_workspace(p: PackedLinear, t: int, rank: int, x_dtype=torch.bfloat16) -> int:
    return _lib.lowrank_workspace_bytes(p.desc, t, MBQ_BF16 if x_dtype == torch.bfloat16 else MBQ_F32,
                                        rank)


def linear_lowrank(p: PackedLinear, x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
                   a: torch.Tensor, b: torch.Tensor, out_dtype: torch.dtype | None = None,
                   y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   options: MbqOpts | None = None) -> torch.Tensor:
    """Routed linear plus the low-rank side path: y = x . W^(b(t))^T + (x . a^T) . b^T,
    a [rank, k] and b [n, rank] bfloat16."""
    t, y = _linear_args(p, x, perm, offsets, out_dtype, y)
    _dev(a, "a")
    if a.dim() != 2:
        raise ValueError("a must be 2-D [rank, k]")
    rank = a.shape[0]
    _arg(a, "a", (rank, p.k), (torch.bfloat16,), x.device)
    _arg(b, "b", (p.n, rank), (torch.bfloat16,), x.device)
    need = linear_lowrank_workspace(p, t, rank, x.dtype)
    _workspace(workspace, "workspace", need, x.device)
    if need and workspace is None:  # zero-filled: the call state starts from zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(_lib.LIB.mbq_linear_lowrank(ctypes.byref(p.desc), _p(p.blob), t, _p(x), _dtype(x), _p(perm),
                                      _p(offsets), _p(a), _p(b), rank, _p(y), _dtype(y), _p(workspace),
                                      ws_bytes, _optp(options), _stream()), "mbq_linear_lowrank")
    return y
