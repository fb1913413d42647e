"""CPU oracle for the intra-block aggregation score and head-wise blocking
scheme selection.

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module; the HIP
library never calls it and shares no code with it (NumPy only, plus the
geometry of the same oracle package).

Source: "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
Diffusion Models Inference" (arXiv 2608.03335), 3.2 Schemes Generation:
Eq. 3 (aggregation score of a blocking scheme = sum over its blocks of
SICS), Eq. 4 (SICS = sum of all pairwise cosine similarities inside a
block), Eq. 5 and Algorithm 1 (the online form: normalize each token, add
its inner product with the running sum of the previous normalized tokens to
sigma, add it to the running sum; SICS = 2*sigma + BS).  The head's selected
blocking scheme is the candidate with the highest aggregation score.

Readings where the pages are silent (also listed in the design notes):

* R17 ragged edges: a cut-short block's SICS runs over its valid tokens
  (BS = that block's token count).
* R18 a zero token vector normalizes to the zero vector: its cosine
  similarity with anything, itself included, is 0, so the diagonal term BS
  of Algorithm 1 counts the nonzero tokens only.
* R19 a head's scheme score is AS(Q | scheme) + AS(K | scheme) (the module
  aggregates "Q and K under each" candidate).
* R20 the selected scheme is the first candidate (lowest index) with the
  highest score.  The GPU decides in float32; where two candidates' float64
  scores lie within the float32 error bound of each other, either choice
  is accepted by the tests.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import vsa_oracle as O


def sics_online(xb: np.ndarray) -> float:
    """Algorithm 1 (SPADE 3.2) in float64 for one block's tokens xb [n, d],
    in token order: r holds the running sum of the normalized tokens seen so
    far, sigma the sum of their inner products with each new token."""
    xb = np.asarray(xb, dtype=np.float64)
    r = np.zeros(xb.shape[1], dtype=np.float64)
    sigma = 0.0
    nonzero = 0
    for x in xb:
        norm = float(np.sqrt(np.dot(x, x)))
        if norm == 0.0:      # R18
            continue
        xh = x / norm
        sigma += float(np.dot(r, xh))
        r += xh
        nonzero += 1
    return 2.0 * sigma + nonzero


def _sics_online_many(xb: np.ndarray) -> np.ndarray:
    """Algorithm 1 run side by side on many blocks of the same token count:
    xb [m, n, d] -> [m], each block with exactly the steps of sics_online."""
    xb = np.asarray(xb, dtype=np.float64)
    m, n, d = xb.shape
    r = np.zeros((m, d), dtype=np.float64)
    sigma = np.zeros(m, dtype=np.float64)
    nonzero = np.zeros(m, dtype=np.float64)
    for t in range(n):
        x = xb[:, t, :]
        norm = np.sqrt(np.einsum("md,md->m", x, x))
        ok = norm > 0.0
        xh = np.where(ok[:, None], x / np.where(ok, norm, 1.0)[:, None], 0.0)
        sigma += np.where(ok, np.einsum("md,md->m", r, xh), 0.0)
        r += xh
        nonzero += ok
    return 2.0 * sigma + nonzero


def block_sics(x: np.ndarray, g: "O.Geometry", heads: Sequence[int] = None) -> np.ndarray:
    """SICS of every block of x [B, heads, N, d] under the blocking of g:
    float64 [B, heads, NB], each block by Algorithm 1 over its tokens in
    block order (R17).  heads limits the work to some heads (the others
    stay zero)."""
    B, Hh = x.shape[:2]
    out = np.zeros((B, Hh, g.NB), dtype=np.float64)
    hs = range(Hh) if heads is None else heads
    for size in np.unique(g.sizes):
        js = np.nonzero(g.sizes == size)[0]
        idx = np.stack([g.tokens[j] for j in js])          # [m, size]
        for b in range(B):
            for h in hs:
                out[b, h, js] = _sics_online_many(x[b, h][idx])
    return out


def aggregation_score(x: np.ndarray, grid: Sequence[int], block: Sequence[int]) -> np.ndarray:
    """Eq. 3: AS(x | scheme) = sum over the scheme's blocks of SICS, per
    (batch, head): float64 [B, heads]."""
    g = O.geometry(grid, block)
    return block_sics(x, g).sum(axis=2)


def scheme_scores(q: np.ndarray, k: np.ndarray, grid: Sequence[int],
                  candidates: Sequence[Sequence[int]]) -> np.ndarray:
    """R19: score[c, b, h] = AS(Q | c) + AS(K | c), float64."""
    return np.stack([aggregation_score(q, grid, c) + aggregation_score(k, grid, c) for c in candidates])


def select_scheme(scores: np.ndarray) -> np.ndarray:
    """R20: per (batch, head), the first candidate with the highest score."""
    return np.argmax(scores, axis=0).astype(np.int32)
