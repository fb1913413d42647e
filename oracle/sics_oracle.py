"""CPU oracle for the intra-block aggregation score and head-wise blocking
scheme selection.

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module; the HIP
library never calls it and shares no code with it (NumPy only, plus the
geometry of the same oracle package).

Source: "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
Diffusion Models Inference" (arXiv 2608.03335), 3.2 Schemes Generation.
Eq. 4 defines SICS of a block as the sum of every entry of the cosine
similarity matrix of its tokens: with D the diagonal matrix of the token
norms, the sum of all entries of D^-1 X X^T D^-1.  Eq. 3 sums SICS over the
blocks of a scheme (the aggregation score AS), and the head keeps the
candidate scheme with the highest score.  This oracle evaluates Eq. 4 as
written, through the Gram matrix of the normalized tokens; the online
rewrite of Eq. 5 is what the GPU evaluates, and the tests pin this module
against the closed form ||sum of normalized tokens||^2 and SciPy's pairwise
cosine distances independently.

Readings where the pages are silent (also listed in the design notes):

* R17 ragged edges: a cut-short block's SICS runs over its valid tokens
  (BS = that block's token count).
* R18 a zero token vector normalizes to the zero vector: its cosine
  similarity with anything, itself included, is 0, so the diagonal of the
  Gram matrix counts the nonzero tokens only.
* R19 a head's scheme score is AS(Q | scheme) + AS(K | scheme): the module
  scores a candidate by aggregating both Q and K under it.
* R20 the selected scheme is the first candidate (lowest index) with the
  highest score.  The GPU decides in float32; where two candidates' float64
  scores lie within the float32 error bound of each other, either choice
  is accepted by the tests.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import vsa_oracle as O


def _normalized(x: np.ndarray) -> np.ndarray:
    """Rows of x (last axis = channels) divided by their Euclidean norm, in
    float64; a zero row stays zero (R18)."""
    x = np.asarray(x, dtype=np.float64)
    norm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, norm, out=np.zeros_like(x), where=norm > 0.0)


def sics(xb: np.ndarray) -> float:
    """Eq. 4 for one block's tokens xb [n, d]: the sum of all entries of the
    n x n cosine similarity matrix (normalized Gram matrix), float64."""
    xh = _normalized(xb)
    return float((xh @ xh.T).sum())


def _sics_many(xb: np.ndarray) -> np.ndarray:
    """Eq. 4 for many blocks of the same token count: xb [m, n, d] -> [m]."""
    xh = _normalized(xb)
    return np.matmul(xh, np.swapaxes(xh, 1, 2)).sum(axis=(1, 2))


def block_sics(x: np.ndarray, g: "O.Geometry", heads: Sequence[int] = None) -> np.ndarray:
    """SICS of every block of x [B, heads, N, d] under the blocking of g:
    float64 [B, heads, NB], each block by Eq. 4 over its valid tokens (R17).
    heads limits the work to some heads (the others stay zero)."""
    B, Hh = x.shape[:2]
    out = np.zeros((B, Hh, g.NB), dtype=np.float64)
    hs = range(Hh) if heads is None else heads
    for size in np.unique(g.sizes):
        js = np.nonzero(g.sizes == size)[0]
        idx = np.stack([g.tokens[j] for j in js])          # [m, size]
        for b in range(B):
            for h in hs:
                out[b, h, js] = _sics_many(x[b, h][idx])
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
