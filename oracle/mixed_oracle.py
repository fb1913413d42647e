"""CPU oracle for mixed per-head plans: every head of a layer call takes its
own option (dense, static or dynamic) and its own temporal window.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module; the HIP library never
calls it and shares no code with it (NumPy only, plus the geometry, Top-K
and estimators of the same oracle package).

Sources:
* DecoupAttn Plans (dataset README), introduction: the plan compiled
  offline for a model assigns each (timestep, layer, head) unit a dense
  option, a static top-theta option over an offline ranking of key blocks
  (theta from a fixed menu of six keep rates, 0.05 to 0.45) or a
  computation-only option, and assigns each call an estimator (the full
  attention map or block centroids) that selects 20% of the blocks.
* SPADE (arXiv 2608.03335) 3.1: each head's sparsity scheme has a
  local-window length and a Top-K keep; 3.3: the selection is united with
  the local window.

Readings where the pages are silent (also listed in the design notes):

* R28 a head's option is one of
    dense:   every key block;
    static:  Top-K at keep rate theta over a block ranking supplied by the
             caller (D_u: a float32 score per (query block, key block) of
             the head, the same for every batch item), with R4's k rule and
             R7's tie rule -- it does not look at Q or K;
    dynamic: Top-K at keep rate rho over the scores of an estimator
             (mean / Centroid, DSA or DSA2) of this call's Q and K.
  CompOnly is not defined on the pages and is not built.
* R29 each head has its own temporal window (R8), united with its
  selection; a dense head's rows are full anyway.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import dsa_oracle as E
from . import vsa_oracle as O

KINDS = ("dynamic", "static", "dense")


def plan_mixed(q: Optional[np.ndarray], k: Optional[np.ndarray], grid, block, options: Sequence[dict],
               static_scores: Optional[np.ndarray] = None, estimator: str = "mean", B: int = None):
    """Per-head options [{"kind": ..., "value": ..., "window_t": ...}] ->
    CSR (R9 layout).  static_scores: float32 [heads, NB, NB] when a head is
    static.  q, k: [B, heads, N, D] when a head is dynamic (B is then taken
    from q; otherwise pass B).  Returns (row_ptr, col_idx, info)."""
    g = O.geometry(grid, block)
    Hh = len(options)
    dynamic = any(o["kind"] == "dynamic" for o in options)
    S = E.estimate(q, k, g, estimator) if dynamic else None
    if q is not None:
        B = q.shape[0]
    rows = []
    for b in range(B):
        for h, opt in enumerate(options):
            kind, val, win = opt["kind"], float(opt.get("value", 1.0)), int(opt.get("window_t", -1))
            for i in range(g.NB):
                if kind == "dense":
                    kept = np.arange(g.NB)
                elif kind == "static":
                    kept = O.topk_row(static_scores[h, i], O.k_rule(val, g.NB))
                elif kind == "dynamic":
                    kept = O.topk_row(S[b, h, i], O.k_rule(val, g.NB))
                else:
                    raise ValueError(kind)
                if win >= 0:
                    kept = np.union1d(kept, O.window_blocks(g, i, win))
                rows.append(np.asarray(kept, dtype=np.int32))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int32)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32), {"geometry": g, "S": S}
