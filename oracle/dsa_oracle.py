"""CPU oracle for the max/min summarizers and their inter-estimators
(DSA-SPADE and DSA2-SPADE).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module; the HIP library never
calls it and shares no code with it (NumPy only, plus the geometry and the
Top-K / Top-P selection of the same oracle package).

Source: "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
Diffusion Models Inference" (arXiv 2608.03335), 3.1 (vDiT-SSR, Summarizer
and Estimator Expressions, Fig. 4): the summarizer reduces a block's Q or K
tokens over sequence positions (max, min or mean) into vectors in R^d; the
inter-estimator combines the summaries of a query block and a key block
into one importance value, the dot product of two vectors built from them.
DSA-SPADE estimates with (k_max, k_min, (q_max + q_min)/2), DSA2-SPADE with
(k_max, k_min, q_max, q_min).  3.3: the summaries Q', K' feed the
inter-block importance matrix, which is filtered by Top-K or Top-P.

Readings where the pages are silent (also listed in the design notes):

* R25 the inter-estimator of DSA is the largest dot product between the
  query summary qm = (q_max + q_min)/2 and any vector of the key block's
  channel-wise box [k_min, k_max]:
      score = sum_c max(qm_c * k_max_c, qm_c * k_min_c),
  i.e. the dot product of qm with the box corner picked channel by channel.
  For DSA2 it is the largest dot product between any vector of the query
  box [q_min, q_max] and any of the key box:
      score = sum_c max(q_max_c k_max_c, q_max_c k_min_c,
                        q_min_c k_max_c, q_min_c k_min_c).
  Both are single dot products of vectors built from the listed summaries
  and upper bounds of every token-pair logit the boxes contain, which is
  what a block estimator built from extremes can promise.  (Fig. 4's own
  equations are not in the text.)
* R26 precision and order: max and min are exact; qm = fl(fl(q_max +
  q_min) * 0.5) in float32; a score is the sequential
  float32 sum over channels, from +0, of the largest separately rounded
  product, with no fused multiply-add (as R6), so the index is reproducible
  bit for bit.
* R27 a cut-short edge block's extremes run over its valid tokens (R3).
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

from . import select_oracle as P
from . import vsa_oracle as O

ESTIMATORS = ("mean", "dsa", "dsa2")


def _gather(x: np.ndarray, g: "O.Geometry"):
    """Block token rows and a validity mask: xb [B, Hh, NB, P, D] float32
    (pad rows zero) and valid [NB, P]."""
    B, Hh, N, D = x.shape
    P_ = g.max_block
    idx = np.zeros((g.NB, P_), dtype=np.int64)
    valid = np.zeros((g.NB, P_), dtype=bool)
    for j, ids in enumerate(g.tokens):
        idx[j, : len(ids)] = ids
        valid[j, : len(ids)] = True
    xf = np.ascontiguousarray(x, dtype=np.float32)
    return xf[:, :, idx, :], valid


def block_max(x: np.ndarray, g: "O.Geometry") -> np.ndarray:
    """Channel-wise max over each block's valid tokens (R27): [B, Hh, NB, D]."""
    xb, valid = _gather(x, g)
    m = np.where(valid[None, None, :, :, None], xb, -np.inf)
    return m.max(axis=3).astype(np.float32)


def block_min(x: np.ndarray, g: "O.Geometry") -> np.ndarray:
    """Channel-wise min over each block's valid tokens (R27): [B, Hh, NB, D]."""
    xb, valid = _gather(x, g)
    m = np.where(valid[None, None, :, :, None], xb, np.inf)
    return m.min(axis=3).astype(np.float32)


def summaries(q: np.ndarray, k: np.ndarray, g: "O.Geometry", estimator: str) -> Dict[str, np.ndarray]:
    """The summaries each estimator uses (SPADE 3.1, Fig. 4)."""
    if estimator == "mean":
        return {"q_mean": O.centroids(q, g), "k_mean": O.centroids(k, g)}
    qmax, qmin = block_max(q, g), block_min(q, g)
    out = {"k_max": block_max(k, g), "k_min": block_min(k, g)}
    if estimator == "dsa":
        out["q_mid"] = ((qmax + qmin) * np.float32(0.5)).astype(np.float32)   # R26
    elif estimator == "dsa2":
        out["q_max"], out["q_min"] = qmax, qmin
    else:
        raise ValueError(estimator)
    return out


def scores_dsa(qmid: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """R25/R26 for DSA: S[.., i, j] = sum_c max(qm_ic*kmax_jc, qm_ic*kmin_jc),
    float32, channels in order."""
    *lead, NB, D = qmid.shape
    S = np.zeros((*lead, NB, kmax.shape[-2]), dtype=np.float32)
    for d in range(D):
        a = qmid[..., :, d][..., :, None] * kmax[..., :, d][..., None, :]   # float32 products
        b = qmid[..., :, d][..., :, None] * kmin[..., :, d][..., None, :]
        S = S + np.maximum(a, b)
    return S


def scores_dsa2(qmax: np.ndarray, qmin: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """R25/R26 for DSA2: the largest of the four corner products per
    channel, summed in order in float32."""
    *lead, NB, D = qmax.shape
    S = np.zeros((*lead, NB, kmax.shape[-2]), dtype=np.float32)
    for d in range(D):
        qa, qb = qmax[..., :, d][..., :, None], qmin[..., :, d][..., :, None]
        ka, kb = kmax[..., :, d][..., None, :], kmin[..., :, d][..., None, :]
        S = S + np.maximum(np.maximum(qa * ka, qa * kb), np.maximum(qb * ka, qb * kb))
    return S


def estimate(q: np.ndarray, k: np.ndarray, g: "O.Geometry", estimator: str) -> np.ndarray:
    """Inter-block importance [B, Hh, NB, NB] for an estimator."""
    s = summaries(q, k, g, estimator)
    if estimator == "mean":
        return O.scores(s["q_mean"], s["k_mean"])
    if estimator == "dsa":
        return scores_dsa(s["q_mid"], s["k_max"], s["k_min"])
    return scores_dsa2(s["q_max"], s["q_min"], s["k_max"], s["k_min"])


def plan_estimate(q: np.ndarray, k: np.ndarray, grid, block, estimator: str, mode: str, values,
                  window_t: int = -1, sink: int = 0, scale: float = None):
    """Geometry -> summaries -> estimator -> Top-K or Top-P -> union with the
    window and the sinks -> CSR (SPADE 3.3).  Returns (row_ptr, col_idx,
    info) with the geometry, the scores and the Top-P scale."""
    g = O.geometry(grid, block)
    sc = 1.0 / math.sqrt(q.shape[-1]) if not scale else float(np.float32(scale))
    S = estimate(q, k, g, estimator)
    row_ptr, col_idx = P.select_rows(S, mode, values, g, window_t, sink, sc)
    return row_ptr, col_idx, {"geometry": g, "S": S, "scale": sc}
