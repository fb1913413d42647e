"""CPU oracle for centroid-scored 3D block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no
code with that path: it imports NumPy (and nothing from the package).

Sources (cited by page title and section):

* SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video Diffusion
  Models Inference (arXiv 2608.03335) -- "SPADE" below.
  - 2.1: the VAE latent (T/4+1, H/8, W/8) is flattened to a 1D sequence.
  - 2.2, Eq. 1 (dense attention) and Eq. 2 (block-sparse attention with a
    block-pair mask M).
  - 3.1, Fig. 3: 3D blocking schemes (T,H,W order), e.g. (2,4,8).
  - 3.1, Fig. 4(c): MEAN-SPADE summarizes a block by (q_mean, k_mean); the
    dot product of summaries gives inter-block importance.
  - 3.3: blocked layout -> summaries Q', K' of shape (N_blocks, d_head) ->
    N_Qblocks x N_Kblocks importance -> Top-K -> union with the local
    window -> block-sparse attention -> restore the original layout.
* DecoupAttn Plans (dataset README), Contents table: block shapes are
  frames x rows x cols of one key block; "Centroid" estimator at density 0.20.
* "Does sparse attention actually speed up video generation?", How this was
  measured: the keep rate is the fraction of key blocks each query block keeps.

Readings where the pages are silent (each one also listed in the design notes):

* R1 raster order n = (t*H + h)*W + w for the flattened latent.
* R2 block id (tb*nbh + hb)*nbw + wb; tokens inside a block in row-major
  (t, h, w) order.
* R3 ragged edges: a partial block is a block; its centroid averages its
  valid tokens only; it competes like any other block.
* R4 k = min(NB, max(1, floor(density*NB + 0.5))) in float64 from the
  float32 density.
* R5 score = raw dot product of the two means (no 1/sqrt(d), no softmax:
  neither changes the ranking in exact arithmetic).
* R6 plan arithmetic in float32: centroid = (sequential sum over the block's
  tokens in block order, starting from +0) / n, correctly rounded; score =
  sequential sum over channels of separately rounded products, no fused
  multiply-add.
* R7 ties: equal float32 scores (-0 == +0) go to the lower block id.
* R8 window: key blocks whose temporal block index is within +-window_t of
  the query block's are kept in addition to the top-k over all blocks.
* R9 a CSR row lists its kept key blocks in ascending id order; rows are
  ordered r = (b*heads + h)*NB + i.
* R10 scale 1/sqrt(d) by default; no token mask inside kept blocks.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# geometry (SPADE 2.1 and 3.1 Fig. 3; readings R1-R3)
# --------------------------------------------------------------------------

@dataclass
class Geometry:
    grid: Tuple[int, int, int]
    block: Tuple[int, int, int]
    nbt: int
    nbh: int
    nbw: int
    NB: int
    sizes: np.ndarray          # int64 [NB] tokens per block
    tokens: List[np.ndarray]   # raster indices of each block, in block order
    tblock: np.ndarray         # int64 [NB] temporal block index of each block

    @property
    def max_block(self) -> int:
        return int(self.sizes.max())


def geometry(grid: Sequence[int], block: Sequence[int]) -> Geometry:
    """Partition the T x H x W latent into bt x bh x bw boxes (SPADE 3.1,
    Fig. 3, order T,H,W).  Blocks at the far edge of a dimension that does
    not divide evenly are cut short (reading R3)."""
    T, H, W = (int(x) for x in grid)
    bt, bh, bw = (int(x) for x in block)
    nbt, nbh, nbw = -(-T // bt), -(-H // bh), -(-W // bw)
    sizes, tokens, tblock = [], [], []
    for tb in range(nbt):
        for hb in range(nbh):
            for wb in range(nbw):
                ts = range(tb * bt, min(T, (tb + 1) * bt))
                hs = range(hb * bh, min(H, (hb + 1) * bh))
                ws = range(wb * bw, min(W, (wb + 1) * bw))
                ids = [(t * H + h) * W + w for t in ts for h in hs for w in ws]
                tokens.append(np.array(ids, dtype=np.int64))
                sizes.append(len(ids))
                tblock.append(tb)
    return Geometry((T, H, W), (bt, bh, bw), nbt, nbh, nbw, nbt * nbh * nbw,
                    np.array(sizes, dtype=np.int64), tokens,
                    np.array(tblock, dtype=np.int64))


def k_rule(density: float, NB: int) -> int:
    """Key blocks kept per query block from a keep rate (the JEV comparison
    page, How this was measured: the fraction of key blocks each query block
    keeps).  Rounding is reading R4."""
    d = float(np.float32(density))
    return int(min(NB, max(1, math.floor(d * NB + 0.5))))


def window_blocks(g: Geometry, i: int, window_t: int) -> np.ndarray:
    """Key blocks within +-window_t temporal blocks of query block i (SPADE
    3.3, union with the local-window mask; reading R8)."""
    if window_t < 0:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero(np.abs(g.tblock - g.tblock[i]) <= window_t)[0]


# --------------------------------------------------------------------------
# layout transform (SPADE 3.3: rearrange into the blocked layout, restore)
# --------------------------------------------------------------------------

def permute(x: np.ndarray, g: Geometry, pad_to: Optional[int] = None) -> np.ndarray:
    """Raster [B, Hh, N, D] -> blocked [B, Hh, NB, P, D], P = pad_to or the
    largest block; rows past a block's size are zero."""
    B, Hh, N, D = x.shape
    P = pad_to or g.max_block
    out = np.zeros((B, Hh, g.NB, P, D), dtype=x.dtype)
    for j, ids in enumerate(g.tokens):
        out[:, :, j, : len(ids), :] = x[:, :, ids, :]
    return out


def unpermute(xb: np.ndarray, g: Geometry) -> np.ndarray:
    """Blocked [B, Hh, NB, P, D] -> raster [B, Hh, N, D], dropping pad rows."""
    B, Hh, NB, P, D = xb.shape
    N = int(g.sizes.sum())
    out = np.zeros((B, Hh, N, D), dtype=xb.dtype)
    for j, ids in enumerate(g.tokens):
        out[:, :, ids, :] = xb[:, :, j, : len(ids), :]
    return out


# --------------------------------------------------------------------------
# summarizer: block means (SPADE 3.1 Fig. 4(c), 3.3; reading R6)
# --------------------------------------------------------------------------

def centroids(x: np.ndarray, g: Geometry) -> np.ndarray:
    """Per-block mean of x [B, Hh, N, D] -> float32 [B, Hh, NB, D].

    float32 arithmetic: acc starts at +0; acc = acc + x_u for the block's
    tokens u in block order; mean = acc / n (each step correctly rounded).
    Vectorized over blocks and channels, sequential over the in-block index.
    """
    B, Hh, N, D = x.shape
    xf = np.ascontiguousarray(x, dtype=np.float32)
    P = g.max_block
    idx = np.zeros((g.NB, P), dtype=np.int64)
    valid = np.zeros((g.NB, P), dtype=bool)
    for j, ids in enumerate(g.tokens):
        idx[j, : len(ids)] = ids
        valid[j, : len(ids)] = True
    acc = np.zeros((B, Hh, g.NB, D), dtype=np.float32)
    for u in range(P):
        xu = xf[:, :, idx[:, u], :]                        # [B, Hh, NB, D]
        m = valid[:, u][None, None, :, None]
        acc = np.where(m, acc + xu, acc)                   # float32 add
    n = g.sizes.astype(np.float32)[None, None, :, None]
    return (acc / n).astype(np.float32)                    # float32 divide


# --------------------------------------------------------------------------
# inter-estimator: dot products of summaries (SPADE 3.1 Fig. 4(c), 3.3; R5, R6)
# --------------------------------------------------------------------------

def scores(qc: np.ndarray, kc: np.ndarray) -> np.ndarray:
    """Inter-block importance S[..., i, j] = <qc_i, kc_j> in float32:
    S = +0; for each channel d in order: S = S + qc_i[d] * kc_j[d], the
    product and the sum each rounded to float32 (no fused multiply-add)."""
    *lead, NB, D = qc.shape
    S = np.zeros((*lead, NB, kc.shape[-2]), dtype=np.float32)
    for d in range(D):
        prod = qc[..., :, d][..., :, None] * kc[..., :, d][..., None, :]   # float32 multiply
        S = S + prod                                                       # float32 add
    return S


# --------------------------------------------------------------------------
# selection: Top-K per query-block row, union with the window, CSR
# (SPADE 3.3; readings R4, R7-R9)
# --------------------------------------------------------------------------

def topk_row(s: np.ndarray, k: int) -> np.ndarray:
    """The k key blocks with the largest scores, ties to the lower id,
    returned in ascending id order.  Sorting on (score desc, id asc)."""
    s = np.asarray(s, dtype=np.float32)
    ids = np.arange(s.shape[0])
    # lexsort sorts by the last key first; float compare treats -0 == +0.
    order = np.lexsort((ids, -s.astype(np.float64)))
    return np.sort(order[:k])


def select(S: np.ndarray, ks: Sequence[int], g: Geometry, window_t: int = -1):
    """Block index from scores S [B, Hh, NB, NB] and per-head k.

    Returns (row_ptr int32 [B*Hh*NB + 1], col_idx int32 [nnz]); row
    r = (b*Hh + h)*NB + i lists kept key blocks in ascending id order."""
    B, Hh, NB, _ = S.shape
    rows = []
    for b in range(B):
        for h in range(Hh):
            for i in range(NB):
                kept = topk_row(S[b, h, i], int(ks[h]))
                if window_t >= 0:
                    kept = np.union1d(kept, window_blocks(g, i, window_t))
                rows.append(kept.astype(np.int32))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int32)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def plan(q: np.ndarray, k: np.ndarray, grid, block, density, window_t: int = -1):
    """Full planning step: geometry -> centroids -> scores -> top-k (+window).

    ``density`` is a scalar or one value per head.  Returns
    (row_ptr, col_idx, info) where info holds the geometry, per-head k,
    centroids and scores for inspection."""
    g = geometry(grid, block)
    B, Hh, N, D = q.shape
    dens = np.broadcast_to(np.asarray(density, dtype=np.float32), (Hh,))
    ks = [k_rule(float(d), g.NB) for d in dens]
    qc = centroids(q, g)
    kc = centroids(k, g)
    S = scores(qc, kc)
    row_ptr, col_idx = select(S, ks, g, window_t)
    return row_ptr, col_idx, {"geometry": g, "k": ks, "qc": qc, "kc": kc, "S": S}


# --------------------------------------------------------------------------
# attention (SPADE 2.2 Eq. 1 and Eq. 2; reading R10)
# --------------------------------------------------------------------------

def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_row(q, k, v, g: Geometry, row_ptr, col_idx, b: int, h: int, i: int,
                  scale: Optional[float] = None, return_weights: bool = False):
    """Output of query block i of head (b, h) in float64: every query token
    of the block attends to every token of the kept key blocks (Eq. 2 with M
    zero on kept block pairs and -inf elsewhere)."""
    D = q.shape[-1]
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    NB = g.NB
    r = (b * q.shape[1] + h) * NB + i
    kept = col_idx[row_ptr[r]: row_ptr[r + 1]]
    kid = np.concatenate([g.tokens[j] for j in kept])
    qi = q[b, h, g.tokens[i]].astype(np.float64)
    kk = k[b, h, kid].astype(np.float64)
    vv = v[b, h, kid].astype(np.float64)
    p = _softmax_rows((qi @ kk.T) * sc)
    o = p @ vv
    if return_weights:
        return o, p, kid
    return o


def attention(q, k, v, grid, block, row_ptr, col_idx, scale: Optional[float] = None,
              rows: Optional[Sequence[Tuple[int, int, int]]] = None) -> np.ndarray:
    """Block-sparse attention in float64, output in raster order
    [B, Hh, N, D] (SPADE 3.3: output blocks restored to the original
    layout).  With ``rows`` = [(b, h, i), ...] only those query blocks are
    computed and the rest of the output is NaN."""
    g = geometry(grid, block)
    B, Hh, N, D = q.shape
    out = np.full((B, Hh, N, v.shape[-1]), np.nan if rows is not None else 0.0)
    todo = rows if rows is not None else [(b, h, i) for b in range(B) for h in range(Hh)
                                          for i in range(g.NB)]
    for (b, h, i) in todo:
        out[b, h, g.tokens[i]] = attention_row(q, k, v, g, row_ptr, col_idx, b, h, i, scale)
    return out


# --------------------------------------------------------------------------
# accounting (SPADE 4.1 Metrics: sparsity is the fraction of pruned scores)
# --------------------------------------------------------------------------

def executed_flops(g: Geometry, row_ptr, col_idx, B: int, Hh: int, D: int) -> int:
    """4*D per valid (query token, kept key token) pair, summed over rows."""
    total = 0
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    n = g.sizes
    for r in range(B * Hh * g.NB):
        i = r % g.NB
        total += int(n[i]) * int(n[ci[rp[r]: rp[r + 1]]].sum())
    return 4 * D * total
