"""Seeded synthetic workloads for centroid-scored 3D block-sparse attention.

This module is shared by the CPU oracle and the HIP path.  It holds the
workload shapes and the random draws only: nothing here blocks, pools,
scores, selects or attends.  Every tensor is produced once on the host and
handed unchanged to both sides, so both see identical bits.

Workloads (shapes of the pages' video DiT workloads; no dataset is needed,
the tensors stand in for post-RoPE Q/K/V of one attention layer):

* ``tiny_fp32``     - 4x8x8 latent grid, 2x4x8 blocks, 2 heads, d=64, fp32,
                      density 0.5 (``tiny_fp32_dense``: density 1.0).
* ``wan13b``        - Wan2.1-1.3B 480p/81f latent 21x30x52, block 4x4x8
                      (the Wan block shape in the DecoupAttn plans table),
                      12 heads, d=128, bf16, density 0.20 (the DecoupAttn
                      "Centroid" estimator density).
* ``hunyuan``       - HunyuanVideo 720p/61f latent 16x45x80, block 1x8x16
                      (HunyuanVideo row of the DecoupAttn plans table),
                      24 heads, d=128, bf16, density 0.15 (about the 85%
                      sparsity of SPADE Table 1).
* ``wan14b_mixed``  - Wan2.1-14B 480p latent 21x30x52, block 4x4x8, 40
                      heads, per-head density drawn from
                      {1.0, 0.30, 0.20, 0.10, 0.05} (Dense plus a subset of
                      the DecoupAttn Static_theta option set).
* ``long4x``        - 333-frame long-horizon Wan latent 84x30x52, block
                      4x4x8, 12 heads, density 0.0675, plus a local
                      temporal window of +-1 block.

Recipe (seed 0 everywhere):

* ``tiny_fp32``: ``rng = default_rng(0)``; q, k, v drawn in that order as
  ``standard_normal((1, 2, 256, 64))`` cast to float32.  Other ``iid``
  workloads draw the same way at their own shape and, when their dtype is
  bf16, are rounded to bfloat16 (RNE) like the smooth ones.
* others: ``SeedSequence(0).spawn(4)`` gives independent PCG64 streams for
  (Q, K, V, densities).  Q and K are smooth fields plus noise,
  X[b,h,t,y,x,c] = 0.5*eps + sum_{m<4} cos(2*pi*(ft*t + fh*y + fw*x) + phi),
  eps ~ N(0,1), ft, fh, fw ~ U[0, 0.25) cycles/token, phi ~ U[0, 2*pi),
  independent per (tensor, batch, head, channel, mode); V ~ N(0,1).  The
  field is evaluated in float64, rounded to float32 (RNE) and then to
  bfloat16 (RNE); arrays are returned as float32 holding bf16-exact values.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Tuple

import numpy as np

DENSITY_OPTIONS_MIXED = (1.0, 0.30, 0.20, 0.10, 0.05)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    D: int
    grid: Tuple[int, int, int]      # (T, H, W) latent grid
    block: Tuple[int, int, int]     # (bt, bh, bw) tokens per 3D block
    dtype: str                      # "f32" or "bf16"
    density: Optional[float]        # uniform density, or None for per-head draw
    window_t: int                   # -1: no window; r >= 0: +-r temporal blocks
    gen: str                        # "iid" or "smooth"

    @property
    def N(self) -> int:
        T, H, W = self.grid
        return T * H * W

    def describe(self) -> Dict:
        return dataclasses.asdict(self)


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
    "tiny_fp32_dense": Workload("tiny_fp32_dense", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 1.0, -1, "iid"),
    "wan13b": Workload("wan13b", 1, 12, 128, (21, 30, 52), (4, 4, 8), "bf16", 0.20, -1, "smooth"),
    "hunyuan": Workload("hunyuan", 1, 24, 128, (16, 45, 80), (1, 8, 16), "bf16", 0.15, -1, "smooth"),
    "wan14b_mixed": Workload("wan14b_mixed", 1, 40, 128, (21, 30, 52), (4, 4, 8), "bf16", None, -1, "smooth"),
    "long4x": Workload("long4x", 1, 12, 128, (84, 30, 52), (4, 4, 8), "bf16", 0.0675, 1, "smooth"),
}


def with_heads(w: Workload, heads: int) -> Workload:
    """A one-GPU share of a workload: the same grid and block, fewer heads."""
    return dataclasses.replace(w, name=f"{w.name}_h{heads}", heads=heads)


def custom(name: str, B: int, heads: int, D: int, grid, block, dtype: str,
           density: Optional[float], window_t: int = -1, gen: str = "smooth") -> Workload:
    return Workload(name, B, heads, D, tuple(grid), tuple(block), dtype, density, window_t, gen)


# --------------------------------------------------------------------------
# rounding helpers (input synthesis only)
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> float32 (RNE) -> bfloat16 (RNE), returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16 << 16
    return (u.astype(np.uint32)).view(np.float32).reshape(f.shape)


def _smooth_field(rng: np.random.Generator, B: int, heads: int, D: int, grid) -> np.ndarray:
    """0.5*N(0,1) + sum of 4 random 3D cosine fields per (b, head, channel)."""
    T, H, W = grid
    f = rng.uniform(0.0, 0.25, size=(B, heads, D, 4, 3))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(B, heads, D, 4))
    eps = rng.standard_normal((B, heads, T * H * W, D))
    out = 0.5 * eps
    t = np.arange(T, dtype=np.float64)
    y = np.arange(H, dtype=np.float64)
    xw = np.arange(W, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            ft = f[b, h, :, :, 0]  # (D, 4)
            fh = f[b, h, :, :, 1]
            fw = f[b, h, :, :, 2]
            e = np.exp(1j * phi[b, h])                                  # (D, 4)
            at = np.exp(2j * np.pi * t[:, None, None] * ft[None]) * e[None]  # (T, D, 4)
            ah = np.exp(2j * np.pi * y[:, None, None] * fh[None])          # (H, D, 4)
            aw = np.exp(2j * np.pi * xw[:, None, None] * fw[None])         # (W, D, 4)
            th = at[:, None] * ah[None]                                     # (T, H, D, 4)
            thr = np.ascontiguousarray(np.moveaxis(th.real, -1, 0))        # (4, T, H, D)
            thi = np.ascontiguousarray(np.moveaxis(th.imag, -1, 0))
            awr = np.ascontiguousarray(np.moveaxis(aw.real, -1, 0))        # (4, W, D)
            awi = np.ascontiguousarray(np.moveaxis(aw.imag, -1, 0))
            field = np.zeros((T, H, W, D))
            for m in range(4):
                # Re(th * aw) for mode m, broadcast over (T, H) x W
                field += thr[m][:, :, None, :] * awr[m][None, None]
                field -= thi[m][:, :, None, :] * awi[m][None, None]
            out[b, h] += field.reshape(T * H * W, D)
    return out


def generate(w: Workload, seed: int = 0) -> Dict[str, object]:
    """Inputs of workload ``w``: q, k, v as float32 arrays [B, heads, N, D]
    (bf16-exact for bf16 workloads) and the per-head densities."""
    shape = (w.B, w.heads, w.N, w.D)
    if w.gen == "iid":
        rng = np.random.default_rng(seed)
        q = rng.standard_normal(shape).astype(np.float32)
        k = rng.standard_normal(shape).astype(np.float32)
        v = rng.standard_normal(shape).astype(np.float32)
        dens = np.full(w.heads, w.density, dtype=np.float32)
        if w.dtype == "bf16":
            q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    else:
        sq, sk, sv, sd = np.random.SeedSequence(seed).spawn(4)
        q = _smooth_field(np.random.default_rng(sq), w.B, w.heads, w.D, w.grid)
        k = _smooth_field(np.random.default_rng(sk), w.B, w.heads, w.D, w.grid)
        v = np.random.default_rng(sv).standard_normal(shape)
        if w.density is None:
            dens = np.random.default_rng(sd).choice(
                np.array(DENSITY_OPTIONS_MIXED), size=w.heads).astype(np.float32)
        else:
            dens = np.full(w.heads, w.density, dtype=np.float32)
        if w.dtype == "bf16":
            q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
        else:
            q, k, v = (a.astype(np.float32) for a in (q, k, v))
    return {"q": q, "k": k, "v": v, "density": dens, "workload": w, "seed": seed}


def content_hash(arrs: List[np.ndarray]) -> str:
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
