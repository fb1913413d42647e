"""Centroid-scored 3D block-sparse attention for video DiTs on MI355X (gfx950).

Thin binding over the C ABI of libvsa.so (include/vsa.h).  Torch provides
device memory and the current stream; every step of the computation runs in
the library's HIP kernels.  There is no CPU fallback: without the built
library every call raises.

    index = plan(q, k, grid=(T, H, W), block=(bt, bh, bw), density=0.2)
    o = attn(q, k, v, index)

q, k, v: contiguous CUDA tensors [B, heads, T*H*W, D], bfloat16 or float32,
tokens in raster order (t*H + h)*W + w.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import torch

from . import _lib
from ._lib import VsaError, VsaHeadOption, VsaIndex, VsaSelect, VsaShape, check, load

__all__ = ["plan", "plan_noalloc", "plan_heads", "attn_heads", "select_scheme_means", "plan_schemes",
           "attn_schemes", "SchemeMeans", "SchemePlan", "plan_select", "plan_mixed", "attn", "query", "query_select", "permute", "unpermute",
           "centroids", "centroid_scores", "estimate", "sics", "select_scheme", "calib_mfma_bf16", "Index", "VsaError", "load"]

_DTYPES = {torch.bfloat16: _lib.VSA_BF16, torch.float32: _lib.VSA_F32}


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape_of(x: torch.Tensor, grid, block) -> VsaShape:
    if x.dim() != 4:
        raise ValueError("expected [B, heads, N, D]")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if not x.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    T, H, W = (int(a) for a in grid)
    bt, bh, bw = (int(a) for a in block)
    B, Hh, N, D = x.shape
    if N != T * H * W:
        raise ValueError(f"N={N} does not match grid {T}x{H}x{W}")
    return VsaShape(B, Hh, D, T, H, W, bt, bh, bw, _DTYPES[x.dtype])


def _densities(density, heads: int):
    if isinstance(density, (int, float)):
        vals = [float(density)]
    else:
        vals = [float(d) for d in density]
    return (ctypes.c_float * len(vals))(*vals), len(vals)


@dataclass
class Index:
    """CSR block index produced by plan(): row r = (b*heads + h)*nb + i."""
    shape: VsaShape
    nb: int
    window_t: int
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    capacity: int
    equal_heads: int = 0

    def c_index(self) -> VsaIndex:
        return VsaIndex(self.shape, self.nb, self.window_t, ctypes.c_void_p(self.row_ptr.data_ptr()),
                        ctypes.c_void_p(self.col_idx.data_ptr()), self.capacity, self.equal_heads)

    @property
    def grid(self) -> Tuple[int, int, int]:
        return (self.shape.T, self.shape.H, self.shape.W)

    @property
    def block(self) -> Tuple[int, int, int]:
        return (self.shape.bt, self.shape.bh, self.shape.bw)

    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())


def query(shape: VsaShape, density, window_t: int = -1):
    """(row_ptr_len, col_capacity, plan_ws_bytes, attn_ws_bytes)."""
    lib = load()
    dens, nd = _densities(density, shape.heads)
    rl, cap = ctypes.c_int64(), ctypes.c_int64()
    pws, aws = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib.vsa_query(ctypes.byref(shape), dens, nd, int(window_t), ctypes.byref(rl),
                        ctypes.byref(cap), ctypes.byref(pws), ctypes.byref(aws)), "vsa_query")
    return rl.value, cap.value, pws.value, aws.value


def plan(q: torch.Tensor, k: torch.Tensor, grid, block, density: Union[float, Sequence[float]],
         window_t: int = -1) -> Index:
    """Block means -> centroid scores -> per-row top-k (+ window) -> CSR."""
    lib = load()
    shape = _shape_of(q, grid, block)
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    rl, cap, pws, _ = query(shape, density, window_t)
    dev = q.device
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()),
                    ctypes.c_void_p(col_idx.data_ptr()), cap)
    dens, nd = _densities(density, shape.heads)
    check(lib.vsa_plan(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                       ctypes.byref(shape), dens, nd, int(window_t), ctypes.byref(cidx),
                       ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(q)), "vsa_plan")
    return Index(cidx.shape, cidx.nb, cidx.window_t, row_ptr, col_idx, cap, cidx.equal_heads)


def plan_noalloc(q: torch.Tensor, k: torch.Tensor, grid, block, density: Union[float, Sequence[float]],
                 window_t: int = -1, index: Optional[Index] = None) -> Index:
    """plan() through vsa_plan_noalloc: the plan workspace comes from the
    library's static per-GPU array, so the call allocates no workspace.
    With `index` (an Index of the same shape, e.g. from an earlier call)
    its arrays are reused and nothing at all is allocated."""
    lib = load()
    shape = _shape_of(q, grid, block)
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    rl, cap, _, _ = query(shape, density, window_t)
    if index is None:
        row_ptr = torch.empty(rl, dtype=torch.int32, device=q.device)
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=q.device)
    else:
        row_ptr, col_idx = index.row_ptr, index.col_idx
        if row_ptr.numel() < rl or col_idx.numel() < cap or row_ptr.device != q.device:
            raise ValueError("index arrays too small for this plan")
    cidx = VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()),
                    col_idx.numel())
    dens, nd = _densities(density, shape.heads)
    check(lib.vsa_plan_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                               ctypes.byref(shape), dens, nd, int(window_t), ctypes.byref(cidx), _stream(q)),
          "vsa_plan_noalloc")
    return Index(cidx.shape, cidx.nb, cidx.window_t, row_ptr, col_idx, cidx.capacity, cidx.equal_heads)


_MODES = {"topk": _lib.VSA_TOPK, "topp": _lib.VSA_TOPP}
_ESTIMATORS = {"mean": _lib.VSA_EST_MEAN, "dsa": _lib.VSA_EST_DSA, "dsa2": _lib.VSA_EST_DSA2}


def _estimator(name: str) -> int:
    if name not in _ESTIMATORS:
        raise ValueError(f"estimator must be one of {sorted(_ESTIMATORS)}")
    return _ESTIMATORS[name]


def _select(shape: VsaShape, mode: str, value, window_t: int, sink: int, scale: Optional[float],
            estimator: str = "mean"):
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    vals, n = _densities(value, shape.heads)
    sel = VsaSelect(_MODES[mode], n, ctypes.cast(vals, ctypes.POINTER(ctypes.c_float)), int(window_t),
                    int(sink), 0.0 if scale is None else float(scale), _estimator(estimator))
    return sel, vals   # keep vals alive with sel


def query_select(shape: VsaShape, mode: str, value, window_t: int = -1, sink: int = 0,
                 scale: Optional[float] = None, estimator: str = "mean"):
    """(row_ptr_len, col_capacity, plan_ws_bytes) for plan_select."""
    lib = load()
    sel, _vals = _select(shape, mode, value, window_t, sink, scale, estimator)
    rl, cap, pws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    check(lib.vsa_query_select(ctypes.byref(shape), ctypes.byref(sel), ctypes.byref(rl),
                               ctypes.byref(cap), ctypes.byref(pws)), "vsa_query_select")
    return rl.value, cap.value, pws.value


def plan_select(q: torch.Tensor, k: torch.Tensor, grid, block, mode: str,
                value: Union[float, Sequence[float]], window_t: int = -1, sink: int = 0,
                scale: Optional[float] = None, estimator: str = "mean") -> Index:
    """Block summaries -> estimator scores ("mean", "dsa" or "dsa2") ->
    per-row Top-K (value = keep rate) or Top-P (value = cumulative
    threshold p of softmax(scale * scores)), united with the temporal window
    and the first `sink` key blocks -> CSR."""
    lib = load()
    shape = _shape_of(q, grid, block)
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    rl, cap, pws = query_select(shape, mode, value, window_t, sink, scale, estimator)
    dev = q.device
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()),
                    ctypes.c_void_p(col_idx.data_ptr()), cap)
    sel, _vals = _select(shape, mode, value, window_t, sink, scale, estimator)
    check(lib.vsa_plan_select(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                              ctypes.byref(shape), ctypes.byref(sel), ctypes.byref(cidx),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(q)), "vsa_plan_select")
    return Index(cidx.shape, cidx.nb, cidx.window_t, row_ptr, col_idx, cap, cidx.equal_heads)


_KINDS = {"dynamic": _lib.VSA_HEAD_DYNAMIC, "static": _lib.VSA_HEAD_STATIC, "dense": _lib.VSA_HEAD_DENSE}


def _head_options(options):
    arr = (VsaHeadOption * len(options))()
    for h, o in enumerate(options):
        if o["kind"] not in _KINDS:
            raise ValueError(f"head kind must be one of {sorted(_KINDS)}")
        arr[h] = VsaHeadOption(_KINDS[o["kind"]], float(o.get("value", 1.0)), int(o.get("window_t", -1)))
    return arr


def query_mixed(shape: VsaShape, options, estimator: str = "mean"):
    """(row_ptr_len, col_capacity, plan_ws_bytes) for plan_mixed."""
    lib = load()
    opts = _head_options(options)
    rl, cap, pws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    check(lib.vsa_query_mixed(ctypes.byref(shape), opts, _estimator(estimator), ctypes.byref(rl),
                              ctypes.byref(cap), ctypes.byref(pws)), "vsa_query_mixed")
    return rl.value, cap.value, pws.value


def plan_mixed(q: Optional[torch.Tensor], k: Optional[torch.Tensor], grid, block, options,
               static_scores: Optional[torch.Tensor] = None, estimator: str = "mean",
               B: Optional[int] = None, D: Optional[int] = None, dtype=torch.bfloat16,
               device=None) -> Index:
    """Mixed per-head plan.  options: one dict per head, {"kind": "dynamic" |
    "static" | "dense", "value": keep rate, "window_t": r}.  static_scores:
    float32 [heads, NB, NB] on the device for static heads.  q and k may be
    None when no head is dynamic; then B, D, dtype and device describe the
    index (it depends on the table alone and can be reused)."""
    lib = load()
    if q is not None:
        shape = _shape_of(q, grid, block)
        if k is None or k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
            raise ValueError("k must match q")
        dev = q.device
    else:
        T, H, W = (int(a) for a in grid)
        shape = VsaShape(int(B), len(options), int(D), T, H, W, *(int(a) for a in block), _DTYPES[dtype])
        dev = torch.device(device) if device is not None else static_scores.device
    if len(options) != shape.heads:
        raise ValueError("one option per head")
    if static_scores is not None and (static_scores.dtype != torch.float32 or not static_scores.is_contiguous()):
        raise ValueError("static_scores must be contiguous float32 [heads, NB, NB]")
    rl, cap, pws = query_mixed(shape, options, estimator)
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()), cap)
    opts = _head_options(options)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    check(lib.vsa_plan_mixed(ptr(q), ptr(k), ctypes.byref(shape), opts, _estimator(estimator), ptr(static_scores),
                             ctypes.byref(cidx), ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream),
          "vsa_plan_mixed")
    return Index(cidx.shape, cidx.nb, cidx.window_t, row_ptr, col_idx, cap, cidx.equal_heads)


def _check_out(q: torch.Tensor, out: torch.Tensor) -> None:
    """The kernels write every valid token row of `out` in raster order, so
    it must be exactly q's shape, dtype and device, and contiguous."""
    if not isinstance(out, torch.Tensor):
        raise TypeError("out must be a tensor")
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must match q: shape {tuple(q.shape)}, dtype {q.dtype}, device {q.device}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: Index,
         scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-sparse attention over the kept blocks; output in raster order."""
    lib = load()
    shape = _shape_of(q, index.grid, index.block)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    if (shape.B, shape.heads, shape.D, shape.dtype) != (index.shape.B, index.shape.heads,
                                                         index.shape.D, index.shape.dtype):
        raise ValueError("index was planned for another shape")
    if out is not None:
        _check_out(q, out)
    o = torch.empty_like(q) if out is None else out
    cidx = index.c_index()
    check(lib.vsa_attn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                       ctypes.c_void_p(v.data_ptr()), ctypes.byref(cidx),
                       ctypes.c_float(0.0 if scale is None else float(scale)),
                       ctypes.c_void_p(o.data_ptr()), None, 0, _stream(q)), "vsa_attn")
    return o


def permute(x: torch.Tensor, grid, block) -> torch.Tensor:
    """Raster [B, heads, N, D] -> blocked [B, heads, NB, bt*bh*bw, D] (zero pad)."""
    lib = load()
    s = _shape_of(x, grid, block)
    nb = math.prod(-(-int(n) // int(b)) for n, b in zip(grid, block))
    P = s.bt * s.bh * s.bw
    xb = torch.empty((s.B, s.heads, nb, P, s.D), dtype=x.dtype, device=x.device)
    check(lib.vsa_permute(ctypes.c_void_p(x.data_ptr()), ctypes.byref(s),
                          ctypes.c_void_p(xb.data_ptr()), _stream(x)), "vsa_permute")
    return xb


def unpermute(xb: torch.Tensor, grid, block) -> torch.Tensor:
    """Blocked [B, heads, NB, P, D] -> raster [B, heads, N, D]."""
    lib = load()
    B, Hh, nb, P, D = xb.shape
    N = math.prod(int(a) for a in grid)
    x = torch.empty((B, Hh, N, D), dtype=xb.dtype, device=xb.device)
    s = _shape_of(x, grid, block)
    if not xb.is_contiguous() or P != s.bt * s.bh * s.bw:
        raise ValueError("blocked tensor does not match the block shape")
    check(lib.vsa_unpermute(ctypes.c_void_p(xb.data_ptr()), ctypes.byref(s),
                            ctypes.c_void_p(x.data_ptr()), _stream(x)), "vsa_unpermute")
    return x


def centroids(x: torch.Tensor, grid, block) -> torch.Tensor:
    """Block means in float32 [B, heads, NB, D] (the planning order)."""
    lib = load()
    s = _shape_of(x, grid, block)
    nb = math.prod(-(-int(n) // int(b)) for n, b in zip(grid, block))
    out = torch.empty((s.B, s.heads, nb, s.D), dtype=torch.float32, device=x.device)
    check(lib.vsa_centroids(ctypes.c_void_p(x.data_ptr()), ctypes.byref(s),
                            ctypes.c_void_p(out.data_ptr()), _stream(x)), "vsa_centroids")
    return out


def centroid_scores(qc: torch.Tensor, kc: torch.Tensor, grid, block, dtype=torch.bfloat16) -> torch.Tensor:
    """Score matrix [B, heads, NB, NB] from float32 block means."""
    lib = load()
    B, Hh, nb, D = qc.shape
    N = math.prod(int(a) for a in grid)
    s = VsaShape(B, Hh, D, *(int(a) for a in grid), *(int(a) for a in block), _DTYPES[dtype])
    if qc.dtype != torch.float32 or kc.shape != qc.shape or not qc.is_contiguous() or not kc.is_contiguous():
        raise ValueError("qc, kc must be contiguous float32 [B, heads, NB, D]")
    del N
    out = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=qc.device)
    check(lib.vsa_centroid_scores(ctypes.c_void_p(qc.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
                                  ctypes.byref(s), ctypes.c_void_p(out.data_ptr()), _stream(qc)),
          "vsa_centroid_scores")
    return out


def estimate(q: torch.Tensor, k: torch.Tensor, grid, block, estimator: str = "mean") -> torch.Tensor:
    """Inter-block importance matrix float32 [B, heads, NB, NB] of an
    estimator, as vsa_plan_select ranks it."""
    lib = load()
    s = _shape_of(q, grid, block)
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    _, _, pws = query_select(s, "topk", 1.0, estimator=estimator)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=q.device)
    nb = math.prod(-(-int(n) // int(b)) for n, b in zip(grid, block))
    out = torch.empty((s.B, s.heads, nb, nb), dtype=torch.float32, device=q.device)
    check(lib.vsa_estimate(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.byref(s),
                           _estimator(estimator), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                           ws.numel(), _stream(q)), "vsa_estimate")
    return out


def sics(x: torch.Tensor, grid, block) -> torch.Tensor:
    """Intra-block aggregation (sum of pairwise cosine similarities) of every
    block, float32 [B, heads, NB]."""
    lib = load()
    s = _shape_of(x, grid, block)
    nb = math.prod(-(-int(n) // int(b)) for n, b in zip(grid, block))
    out = torch.empty((s.B, s.heads, nb), dtype=torch.float32, device=x.device)
    check(lib.vsa_sics(ctypes.c_void_p(x.data_ptr()), ctypes.byref(s), ctypes.c_void_p(out.data_ptr()),
                       _stream(x)), "vsa_sics")
    return out


def select_scheme(q: torch.Tensor, k: torch.Tensor, grid, candidates: Sequence[Sequence[int]]):
    """Head-wise blocking-scheme selection: returns (scores float32
    [n_cand, B*heads] = AS(Q|c) + AS(K|c), choice int32 [B*heads])."""
    lib = load()
    s = _shape_of(q, grid, candidates[0])
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    flat = [int(a) for c in candidates for a in c]
    if len(flat) != 3 * len(candidates):
        raise ValueError("each candidate is a (bt, bh, bw) triple")
    cand = (ctypes.c_int32 * len(flat))(*flat)
    n = len(candidates)
    wsb = ctypes.c_size_t()
    check(lib.vsa_scheme_workspace(ctypes.byref(s), cand, n, ctypes.byref(wsb)), "vsa_scheme_workspace")
    ws = torch.empty(max(int(wsb.value), 1), dtype=torch.uint8, device=q.device)
    bh = s.B * s.heads
    scores = torch.empty((n, bh), dtype=torch.float32, device=q.device)
    choice = torch.empty((bh,), dtype=torch.int32, device=q.device)
    check(lib.vsa_select_scheme(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.byref(s),
                                cand, n, ctypes.c_void_p(scores.data_ptr()), ctypes.c_void_p(choice.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(q)), "vsa_select_scheme")
    return scores, choice


# ---------------------------------------------------------------------------
# Per-head blocking schemes: calls over a subset of the heads, and scheme
# selection that keeps each candidate's block means for the plans after it.
# ---------------------------------------------------------------------------

def _head_list(heads):
    hl = [int(h) for h in heads]
    return (ctypes.c_int32 * len(hl))(*hl), len(hl)


def plan_heads(q: Optional[torch.Tensor], k: Optional[torch.Tensor], grid, block, heads: Sequence[int],
               density: Union[float, Sequence[float]], window_t: int = -1,
               means: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, heads_total: Optional[int] = None,
               B: Optional[int] = None, D: Optional[int] = None, dtype=torch.bfloat16) -> Index:
    """Plan of the listed heads of q, k ([B, total, N, D]) under one
    blocking.  With means = (query means, key means) of every head (as
    select_scheme_means leaves them) q and k are not read; then heads_total,
    B, D and dtype describe the tensors when q is None.  density: one value
    or one per listed head."""
    lib = load()
    if q is not None:
        shape = _shape_of(q, grid, block)
        if k is None or k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
            raise ValueError("k must match q")
        dev = q.device
    else:
        if means is None:
            raise ValueError("q and k, or means, are needed")
        T, H, W = (int(a) for a in grid)
        shape = VsaShape(int(B), int(heads_total), int(D), T, H, W, *(int(a) for a in block), _DTYPES[dtype])
        dev = means[0].device
    hl, n = _head_list(heads)
    sub = VsaShape(shape.B, n, shape.D, shape.T, shape.H, shape.W, shape.bt, shape.bh, shape.bw, shape.dtype)
    rl, cap, pws, _ = query(sub, density, window_t)
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = VsaIndex(sub, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()), cap)
    dens, nd = _densities(density, n)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    qm, km = (None, None) if means is None else means
    if means is not None:
        for t in (qm, km):
            if t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev:
                raise ValueError("means must be contiguous float32 tensors on the device")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    check(lib.vsa_plan_heads(ptr(q), ptr(k), ptr(qm), ptr(km), ctypes.byref(shape), hl, n, dens, nd, int(window_t),
                             ctypes.byref(cidx), ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream),
          "vsa_plan_heads")
    return Index(cidx.shape, cidx.nb, cidx.window_t, row_ptr, col_idx, cap, cidx.equal_heads)


def attn_heads(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: Index, heads: Sequence[int],
               out: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> torch.Tensor:
    """Attention of the listed heads (the index's row order) into out (a
    zero tensor like q when None); the other heads of out are left as
    they are."""
    lib = load()
    _shape_of(q, index.grid, index.block)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    o = torch.zeros_like(q) if out is None else out
    if out is not None:
        _check_out(q, out)
    hl, n = _head_list(heads)
    if n != index.shape.heads:
        raise ValueError("the head list must have one entry per head of the index")
    cidx = index.c_index()
    check(lib.vsa_attn_heads(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                             ctypes.c_void_p(v.data_ptr()), ctypes.byref(cidx), hl, int(q.shape[1]),
                             ctypes.c_float(0.0 if scale is None else float(scale)), ctypes.c_void_p(o.data_ptr()),
                             None, 0, _stream(q)), "vsa_attn_heads")
    return o


@dataclass
class SchemeMeans:
    """Workspace of select_scheme_means: each candidate's block means of Q
    ([B*heads, NB_c, D]) and K ([B*heads, D, NB_c]) stay in it."""
    ws: torch.Tensor
    offsets: Tuple[int, ...]
    candidates: Tuple[Tuple[int, int, int], ...]
    grid: Tuple[int, int, int]
    B: int
    heads: int
    D: int

    def means(self, c: int) -> Tuple[torch.Tensor, torch.Tensor]:
        nb = math.prod(-(-int(n) // int(b)) for n, b in zip(self.grid, self.candidates[c]))
        cnt = self.B * self.heads * nb * self.D
        qm = self.ws[self.offsets[2 * c]: self.offsets[2 * c] + 4 * cnt].view(torch.float32)
        km = self.ws[self.offsets[2 * c + 1]: self.offsets[2 * c + 1] + 4 * cnt].view(torch.float32)
        return qm, km


def select_scheme_means(q: torch.Tensor, k: torch.Tensor, grid, candidates: Sequence[Sequence[int]]):
    """select_scheme that also keeps each candidate's block means: returns
    (scores [n_cand, B*heads], choice [B*heads], SchemeMeans)."""
    lib = load()
    s = _shape_of(q, grid, candidates[0])
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("k must match q")
    flat = [int(a) for c in candidates for a in c]
    if len(flat) != 3 * len(candidates):
        raise ValueError("each candidate is a (bt, bh, bw) triple")
    cand = (ctypes.c_int32 * len(flat))(*flat)
    n = len(candidates)
    wsb = ctypes.c_size_t()
    offs = (ctypes.c_size_t * (2 * n))()
    check(lib.vsa_scheme_means_workspace(ctypes.byref(s), cand, n, ctypes.byref(wsb), offs),
          "vsa_scheme_means_workspace")
    ws = torch.empty(max(int(wsb.value), 1), dtype=torch.uint8, device=q.device)
    bh = s.B * s.heads
    scores = torch.empty((n, bh), dtype=torch.float32, device=q.device)
    choice = torch.empty((bh,), dtype=torch.int32, device=q.device)
    check(lib.vsa_select_scheme_means(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      ctypes.byref(s), cand, n, ctypes.c_void_p(scores.data_ptr()),
                                      ctypes.c_void_p(choice.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                      _stream(q)), "vsa_select_scheme_means")
    sm = SchemeMeans(ws, tuple(int(x) for x in offs), tuple(tuple(int(a) for a in c) for c in candidates),
                     tuple(int(a) for a in grid), s.B, s.heads, s.D)
    return scores, choice, sm


@dataclass
class SchemePlan:
    """Per-head plan: for every candidate chosen by some head, the heads
    that chose it and their index under that blocking."""
    groups: list            # [(candidate index, block, [heads], Index)]
    scores: torch.Tensor
    choice: torch.Tensor


def plan_schemes(q: torch.Tensor, k: torch.Tensor, grid, candidates: Sequence[Sequence[int]],
                 density: float, window_t: int = -1) -> SchemePlan:
    """Head-wise blocking schemes end to end: select_scheme_means, then one
    plan per chosen candidate over the heads that chose it, from the means
    the selection left (Q and K are read once per candidate in all).  The
    heads' choices come back to the host to group them (one sync).  With
    B > 1 a head's scheme is taken from batch item 0."""
    scores, choice, sm = select_scheme_means(q, k, grid, candidates)
    ch = choice.cpu().tolist()[: q.shape[1]]
    groups = []
    for c in range(len(candidates)):
        hs = [h for h in range(q.shape[1]) if ch[h] == c]
        if not hs:
            continue
        idx = plan_heads(None, None, grid, candidates[c], hs, density, window_t, means=sm.means(c),
                         heads_total=q.shape[1], B=q.shape[0], D=q.shape[3], dtype=q.dtype)
        groups.append((c, tuple(int(a) for a in candidates[c]), hs, idx))
    return SchemePlan(groups, scores, choice)


def attn_schemes(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sp: SchemePlan,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention of every head under its own blocking scheme, one launch per
    group of heads that share a scheme, into one output."""
    o = torch.empty_like(q) if out is None else out
    for _, _, hs, idx in sp.groups:
        attn_heads(q, k, v, idx, hs, out=o)
    return o


def calib_mfma_bf16(pool: torch.Tensor, out: torch.Tensor, n_workgroups: int, iters: int) -> None:
    """Launch the sustained bf16 MFMA-rate kernel (a measurement aid, not a
    step of the method) on the current stream: pool is a device uint8
    tensor of at least VSA_CALIB_POOL_BYTES bytes of bf16 operands, out a
    device float32 tensor of n_workgroups * 256 entries.  Work per launch:
    n_workgroups * 4 * iters * 16 * 32768 FLOP."""
    lib = load()
    if pool.device.type != "cuda" or out.device.type != "cuda" or out.dtype != torch.float32:
        raise ValueError("pool and out must be device tensors, out float32")
    if not pool.is_contiguous() or not out.is_contiguous() or out.numel() < n_workgroups * 256:
        raise ValueError("out must be contiguous with n_workgroups * 256 entries")
    check(lib.vsa_calib_mfma_bf16(ctypes.c_void_p(pool.data_ptr()), pool.numel() * pool.element_size(),
                                  ctypes.c_void_p(out.data_ptr()), int(n_workgroups), int(iters),
                                  _stream(out)), "vsa_calib_mfma_bf16")
