"""Pins for the SICS / aggregation-score oracle (SPADE 3.2, Eq. 3 and 4):
each checks the oracle against something other than its own formula -- the closed form ||sum of normalized tokens||^2, SciPy's cosine
distance, special cases with known values, a hand-worked example and a
constructed input whose best blocking scheme is known."""
import json
import math
import os

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import sics_oracle as S
from oracle import vsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _closed_form(xb):
    xb = np.asarray(xb, np.float64)
    n = np.linalg.norm(xb, axis=1, keepdims=True)
    xh = np.divide(xb, n, out=np.zeros_like(xb), where=n > 0)
    s = xh.sum(axis=0)
    return float(s @ s)


@pytest.mark.parametrize("n,d,seed", [(1, 4, 0), (7, 3, 1), (64, 128, 2), (128, 64, 3), (33, 128, 4)])
def test_sics_equals_closed_form(n, d, seed):
    xb = np.random.default_rng(seed).standard_normal((n, d))
    assert S.sics(xb) == pytest.approx(_closed_form(xb), rel=1e-12, abs=1e-9)


@pytest.mark.parametrize("n,d,seed", [(5, 3, 0), (40, 16, 1), (128, 128, 2)])
def test_sics_equals_scipy_pairwise_cosine(n, d, seed):
    xb = np.random.default_rng(seed).standard_normal((n, d)) + 0.3
    pairwise = 1.0 - cdist(xb, xb, metric="cosine")   # Eq. 4 via a library routine
    assert S.sics(xb) == pytest.approx(pairwise.sum(), rel=1e-10, abs=1e-8)


def test_special_cases():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(32)
    # identical tokens: every cosine is 1 -> BS^2
    assert S.sics(np.tile(v, (10, 1))) == pytest.approx(100.0, rel=1e-12)
    # orthonormal tokens: only the diagonal -> BS
    q, _ = np.linalg.qr(rng.standard_normal((32, 12)))
    assert S.sics(q.T * rng.uniform(0.5, 3.0, (12, 1))) == pytest.approx(12.0, abs=1e-9)
    # antipodal pairs: the normalized sum vanishes -> 0
    w = rng.standard_normal((6, 32))
    assert S.sics(np.concatenate([w, -2.0 * w])) == pytest.approx(0.0, abs=1e-9)
    # positive scaling of tokens and their order do not matter
    x = rng.standard_normal((20, 8))
    base = S.sics(x)
    assert S.sics(x * rng.uniform(0.1, 10.0, (20, 1))) == pytest.approx(base, rel=1e-12)
    assert S.sics(x[rng.permutation(20)]) == pytest.approx(base, rel=1e-12)
    # bounds: 0 <= SICS <= BS^2
    assert 0.0 <= base <= 400.0


def test_zero_token_reading():
    """R18: a zero token contributes nothing, not even its diagonal term."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((9, 5))
    with_zero = np.concatenate([x[:4], np.zeros((1, 5)), x[4:]])
    assert S.sics(with_zero) == pytest.approx(S.sics(x), rel=1e-12)
    assert S.sics(np.zeros((3, 5))) == 0.0


def test_hand_example():
    ex = json.load(open(os.path.join(HERE, "golden", "sics_hand_example.json")))
    assert S.sics(np.array(ex["block"])) == pytest.approx(ex["sics_value"], rel=1e-14)
    assert ex["sics_value"] == pytest.approx(3.0 + 2.0 * math.sqrt(2.0), rel=1e-14)


def test_block_sics_uses_block_tokens_and_ragged_edges():
    """Eq. 3 per block: each block's SICS is over exactly its own tokens
    (checked against the closed form on the raster tokens of its box);
    cut-short edge blocks use their valid tokens (R17)."""
    grid, block = (3, 5, 6), (2, 4, 4)
    g = O.geometry(grid, block)
    x = np.random.default_rng(7).standard_normal((1, 2, int(np.prod(grid)), 8))
    bs = S.block_sics(x, g)
    for h in range(2):
        for j in range(g.NB):
            t0, h0, w0 = np.unravel_index(j, (g.nbt, g.nbh, g.nbw))
            tt, hh, ww = np.meshgrid(np.arange(t0 * 2, min(3, t0 * 2 + 2)), np.arange(h0 * 4, min(5, h0 * 4 + 4)),
                                     np.arange(w0 * 4, min(6, w0 * 4 + 4)), indexing="ij")
            raster = ((tt * 5 + hh) * 6 + ww).reshape(-1)
            assert bs[0, h, j] == pytest.approx(_closed_form(x[0, h, raster]), rel=1e-10)
    assert S.aggregation_score(x, grid, block)[0, 1] == pytest.approx(bs[0, 1].sum(), rel=1e-12)


def test_one_block_scheme_is_sics_of_everything():
    grid = (2, 3, 4)
    x = np.random.default_rng(8).standard_normal((1, 1, 24, 6))
    assert S.aggregation_score(x, grid, grid)[0, 0] == pytest.approx(_closed_form(x[0, 0]), rel=1e-10)


def test_selection_prefers_the_scheme_that_follows_the_structure():
    """Tokens that vary only with (t, h) are identical along w: blocks that
    run along w (1, 1, 8) are all-identical (SICS = 64, the maximum for 8
    tokens each), so that candidate must win over (1, 8, 1) and (8, 1, 1),
    whose blocks mix different tokens."""
    T, H, W, d = 8, 8, 8, 16
    rng = np.random.default_rng(9)
    base = rng.standard_normal((T, H, 1, d))
    x = np.broadcast_to(base, (T, H, W, d)).reshape(1, 1, T * H * W, d).copy()
    cands = [(1, 8, 1), (8, 1, 1), (1, 1, 8)]
    sc = S.scheme_scores(x, x, (T, H, W), cands)
    assert S.select_scheme(sc)[0, 0] == 2
    assert sc[2, 0, 0] == pytest.approx(2 * 64 * 64, rel=1e-12)   # Q and K: 64 blocks of SICS 64
    assert sc[0, 0, 0] < sc[2, 0, 0] and sc[1, 0, 0] < sc[2, 0, 0]


def test_selection_ties_go_to_the_lowest_index():
    sc = np.array([[[1.0, 3.0]], [[2.0, 3.0]], [[2.0, 1.0]]])   # [cand, B, heads]
    assert S.select_scheme(sc).tolist() == [[1, 0]]


def test_vectorized_blocks_match_one_block_at_a_time():
    grid, block = (5, 6, 7), (2, 4, 4)
    g = O.geometry(grid, block)
    x = np.random.default_rng(10).standard_normal((1, 2, int(np.prod(grid)), 8))
    x[0, 1, 3] = 0.0
    bs = S.block_sics(x, g)
    for h in range(2):
        for j in range(g.NB):
            assert bs[0, h, j] == pytest.approx(S.sics(x[0, h, g.tokens[j]]), rel=1e-12, abs=1e-12)
