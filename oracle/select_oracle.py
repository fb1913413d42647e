"""CPU oracle for the selection variants of the planning step: Top-P over a
query-block row of centroid scores, and attention-sink key blocks.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module; the HIP library never
calls it and shares no code with it (NumPy only, plus the geometry, scores
and Top-K of the same oracle package).

Source: "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
Diffusion Models Inference" (arXiv 2608.03335):
* 3.1 (vDiT-SSR): the utility parameters are an attention-sink length and a
  Top-K / Top-P mode; each head's scheme carries an inter-top value that is
  either a Top-P cumulative threshold or a Top-K keep count.
* 3.3 (Head-wise Sparse Attention): the inter-block importance matrix is
  filtered by Top-K or Top-P, and the result is united with the local-window
  and attention-sink masks into the binary block mask.

Readings where the pages are silent (also listed in the design notes):

* R21 Top-P normalizes a query-block row with a softmax of its centroid
  scores times the logit scale (1/sqrt(d) unless given):
  prob_j = exp(scale*s_j) / sum_l exp(scale*s_l).  It keeps the shortest
  prefix of the row, taken in (score descending, block id ascending) order,
  whose cumulative probability is at least p: at least one block.  p = 1
  keeps the whole row: every probability is positive in exact arithmetic,
  so no shorter prefix reaches 1 (a float64 cumulative sum can round to 1
  early when a block's probability is below its resolution); likewise the
  whole row if rounding leaves the total mass below p.
* R22 the scores are the float32 ones of R5/R6; the softmax and the
  cumulative sums here run in float64.  The GPU decides the prefix length in
  float32: where a prefix's float64 mass lies within the float32 error bound
  of p, either side of it is accepted by the tests.
* R23 an attention-sink length s counts key blocks: blocks 0 .. s-1 (the
  first blocks of the blocked key sequence, i.e. the first temporal slab's
  leading blocks) are kept by every query-block row; s = 0 means none.
* R24 the kept set of a row is the union of its Top-K or Top-P selection,
  its local window (R8) and the sink blocks, listed in ascending id (R9).
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from . import vsa_oracle as O


def rank_order(s: np.ndarray) -> np.ndarray:
    """Block ids of a score row in (score descending, id ascending) order.
    The float32 scores compare as numbers, so -0 and +0 tie (R7)."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    ids = np.arange(s.shape[0])
    return np.lexsort((ids, -s))


def row_probabilities(s: np.ndarray, scale: float) -> np.ndarray:
    """R21: softmax of scale * s over the row, in float64 (max subtracted
    first, which leaves the quotient unchanged)."""
    z = np.asarray(s, dtype=np.float32).astype(np.float64) * float(scale)
    e = np.exp(z - z.max())
    return e / e.sum()


def prefix_mass(s: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """(order, F): order = rank_order(s); F[c-1] = float64 probability mass
    of the first c blocks of that order."""
    order = rank_order(s)
    return order, np.cumsum(row_probabilities(s, scale)[order])


def topp_count(s: np.ndarray, p: float, scale: float) -> int:
    """R21: the length of the shortest prefix with mass >= p (>= 1), or the
    whole row when p = 1 or no prefix reaches p."""
    _, F = prefix_mass(s, scale)
    if float(p) >= 1.0:
        return int(F.shape[0])
    hit = np.nonzero(F >= float(p))[0]
    return int(hit[0]) + 1 if hit.size else int(F.shape[0])


def topp_row(s: np.ndarray, p: float, scale: float) -> np.ndarray:
    """Top-P selection of one row, in ascending block id."""
    order = rank_order(s)
    return np.sort(order[: topp_count(s, p, scale)])


def sink_blocks(NB: int, sink: int) -> np.ndarray:
    """R23: the first `sink` key blocks."""
    return np.arange(min(int(sink), int(NB)), dtype=np.int64)


def select_rows(S: np.ndarray, mode: str, values: Sequence[float], g: "O.Geometry",
                window_t: int = -1, sink: int = 0, scale: float = None):
    """Block index from scores S [B, Hh, NB, NB].

    mode "topk": values are per-head keep rates (k by R4); mode "topp":
    values are per-head cumulative thresholds p.  Every row is united with
    the window (R8) and the sink blocks (R23).  Returns (row_ptr, col_idx)
    in the CSR layout of R9."""
    B, Hh, NB, _ = S.shape
    vals = np.broadcast_to(np.asarray(values, dtype=np.float32), (Hh,))
    if scale is None:
        raise ValueError("scale is required for the selection oracle")
    sinks = sink_blocks(NB, sink)
    rows = []
    for b in range(B):
        for h in range(Hh):
            for i in range(NB):
                if mode == "topk":
                    kept = O.topk_row(S[b, h, i], O.k_rule(float(vals[h]), NB))
                elif mode == "topp":
                    kept = topp_row(S[b, h, i], float(vals[h]), scale)
                else:
                    raise ValueError(mode)
                if window_t >= 0:
                    kept = np.union1d(kept, O.window_blocks(g, i, window_t))
                if sinks.size:
                    kept = np.union1d(kept, sinks)
                rows.append(np.asarray(kept, dtype=np.int32))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int32)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def plan_select(q: np.ndarray, k: np.ndarray, grid, block, mode: str, values,
                window_t: int = -1, sink: int = 0, scale: float = None):
    """Geometry -> centroids -> scores (R5, R6) -> Top-K or Top-P -> union
    with the window and the sinks -> CSR.  scale defaults to 1/sqrt(d).
    Returns (row_ptr, col_idx, info) with the geometry, scores and scale."""
    g = O.geometry(grid, block)
    D = q.shape[-1]
    sc = 1.0 / math.sqrt(D) if not scale else float(np.float32(scale))
    S = O.scores(O.centroids(q, g), O.centroids(k, g))
    row_ptr, col_idx = select_rows(S, mode, values, g, window_t, sink, sc)
    return row_ptr, col_idx, {"geometry": g, "S": S, "scale": sc}
