"""Pins for the max/min summarizers and the DSA / DSA2 inter-estimators
(SPADE 3.1, Fig. 4; readings R25-R27).  Each checks the oracle against
something other than its own formula: a hand-worked example, a linear
program and vertex enumeration of the summary boxes (the definition of the
largest dot product), the bound over every token pair, single-token blocks
that reduce to the mean estimator bit for bit, NumPy reductions per block,
and sign-flip invariance."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.optimize import linprog

import workloads as W
from oracle import dsa_oracle as E
from oracle import select_oracle as P
from oracle import vsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _hand():
    with open(os.path.join(HERE, "golden", "dsa_hand_example.json")) as f:
        gold = json.load(f)
    q = np.array(gold["q_tokens"], np.float32)[None, None]
    k = np.array(gold["k_tokens"], np.float32)[None, None]
    g = O.geometry(gold["grid"], gold["block"])
    return gold, q, k, g


def test_golden_hand_example():
    gold, q, k, g = _hand()
    s = E.summaries(q, k, g, "dsa")
    assert s["q_mid"][0, 0].tolist() == gold["q_mid"]
    assert s["k_max"][0, 0].tolist() == gold["k_max"]
    assert s["k_min"][0, 0].tolist() == gold["k_min"]
    s2 = E.summaries(q, k, g, "dsa2")
    assert s2["q_max"][0, 0].tolist() == gold["q_max"]
    assert s2["q_min"][0, 0].tolist() == gold["q_min"]
    assert E.estimate(q, k, g, "dsa")[0, 0].tolist() == gold["dsa_scores"]
    assert E.estimate(q, k, g, "dsa2")[0, 0].tolist() == gold["dsa2_scores"]
    assert E.estimate(q, k, g, "mean")[0, 0].tolist() == gold["mean_scores"]
    # both are upper bounds of the block pair's largest token logit
    L = np.array(gold["largest_token_logit"])
    assert np.all(np.array(gold["dsa2_scores"]) >= L)


@pytest.mark.parametrize("seed", range(6))
def test_dsa_is_the_box_maximum_linear_program(seed):
    """DSA = max of <qm, k> over k in [k_min, k_max] (R25), by scipy's LP."""
    rng = np.random.default_rng(seed)
    D = 16
    qm = rng.standard_normal((1, 1, 3, D)).astype(np.float32)
    lo = rng.standard_normal((1, 1, 4, D)).astype(np.float32)
    hi = (lo + rng.uniform(0, 2, (1, 1, 4, D))).astype(np.float32)
    S = E.scores_dsa(qm, hi, lo)
    for i in range(3):
        for j in range(4):
            res = linprog(-qm[0, 0, i].astype(np.float64), bounds=list(zip(lo[0, 0, j], hi[0, 0, j])),
                          method="highs")
            assert res.status == 0
            assert S[0, 0, i, j] == pytest.approx(-res.fun, rel=1e-5, abs=1e-5)


@pytest.mark.parametrize("seed", range(4))
def test_vertex_enumeration(seed):
    """DSA over the 2^D corners of the key box, DSA2 over every pair of
    corners of the two boxes, with whole dot products in float64."""
    rng = np.random.default_rng(10 + seed)
    D = 5
    qlo = rng.standard_normal(D)
    qhi = qlo + rng.uniform(0, 2, D)
    klo = rng.standard_normal(D)
    khi = klo + rng.uniform(0, 2, D)
    f = lambda a: np.asarray(a, np.float32)[None, None, None, :]
    qcorners = [np.where(bits, qhi, qlo) for bits in itertools.product([0, 1], repeat=D)]
    kcorners = [np.where(bits, khi, klo) for bits in itertools.product([0, 1], repeat=D)]
    qhi32, qlo32, khi32, klo32 = (np.float32(a).astype(np.float64) for a in (qhi, qlo, khi, klo))
    qmid = (qhi32 + qlo32) / 2
    best_dsa = max(float(qmid @ np.where(b, khi32, klo32)) for b in itertools.product([0, 1], repeat=D))
    s = E.scores_dsa(f((np.float32(qhi) + np.float32(qlo)) * np.float32(0.5)), f(khi), f(klo))
    assert float(s.ravel()[0]) == pytest.approx(best_dsa, rel=1e-5, abs=1e-5)
    best2 = max(float(np.float32(qc).astype(np.float64) @ np.float32(kc).astype(np.float64))
                for qc in qcorners for kc in kcorners)
    s2 = E.scores_dsa2(f(qhi), f(qlo), f(khi), f(klo))
    assert float(s2.ravel()[0]) == pytest.approx(best2, rel=1e-5, abs=1e-5)


def test_upper_bound_of_every_token_logit():
    """The boxes contain every token, so DSA2 >= the largest q.k over the
    block pair and DSA >= the largest qm.k over the key block's tokens."""
    w = W.custom("ub", 1, 2, 32, (3, 6, 8), (2, 4, 4), "f32", 0.5, -1, "iid")
    inp = W.generate(w, seed=1)
    g = O.geometry(w.grid, w.block)
    S1 = E.estimate(inp["q"], inp["k"], g, "dsa")
    S2 = E.estimate(inp["q"], inp["k"], g, "dsa2")
    qmid = E.summaries(inp["q"], inp["k"], g, "dsa")["q_mid"]
    slack = 1e-4
    for h in range(2):
        L = inp["q"][0, h].astype(np.float64) @ inp["k"][0, h].astype(np.float64).T
        for i in range(g.NB):
            for j in range(g.NB):
                top = L[np.ix_(g.tokens[i], g.tokens[j])].max()
                assert S2[0, h, i, j] >= top - slack
                assert S1[0, h, i, j] >= float((inp["k"][0, h, g.tokens[j]] @ qmid[0, h, i]).max()) - slack
                assert S2[0, h, i, j] >= S1[0, h, i, j] - slack   # the query box holds qm


def test_single_token_blocks_reduce_to_mean():
    """A one-token block's max, min, mid and mean are that token, so DSA and
    DSA2 equal the mean estimator bit for bit."""
    w = W.custom("one", 1, 2, 64, (2, 4, 6), (1, 1, 1), "bf16", 0.5, -1, "smooth")
    inp = W.generate(w, seed=2)
    g = O.geometry(w.grid, w.block)
    Sm = E.estimate(inp["q"], inp["k"], g, "mean")
    assert np.array_equal(E.estimate(inp["q"], inp["k"], g, "dsa"), Sm)
    assert np.array_equal(E.estimate(inp["q"], inp["k"], g, "dsa2"), Sm)


def test_extremes_match_numpy_per_block():
    w = W.custom("ext", 2, 2, 64, (5, 7, 9), (2, 4, 4), "bf16", 0.5, -1, "smooth")
    inp = W.generate(w, seed=3)
    g = O.geometry(w.grid, w.block)
    mx, mn = E.block_max(inp["k"], g), E.block_min(inp["k"], g)
    for j in range(g.NB):
        toks = inp["k"][:, :, g.tokens[j], :]
        assert np.array_equal(mx[:, :, j], toks.max(axis=2))
        assert np.array_equal(mn[:, :, j], toks.min(axis=2))
    assert len(set(g.sizes.tolist())) > 1     # ragged edges covered


def test_sign_flip_invariance():
    """Negating Q and K swaps max and min and negates both factors: the
    largest products are the same numbers, so the scores are identical."""
    w = W.custom("neg", 1, 2, 64, (4, 8, 8), (2, 4, 4), "bf16", 0.5, -1, "smooth")
    inp = W.generate(w, seed=4)
    g = O.geometry(w.grid, w.block)
    for est in ("dsa", "dsa2"):
        a = E.estimate(inp["q"], inp["k"], g, est)
        b = E.estimate(-inp["q"], -inp["k"], g, est)
        assert np.array_equal(a, b), est


def test_growing_the_key_box_never_lowers_dsa():
    rng = np.random.default_rng(5)
    qm = rng.standard_normal((1, 1, 6, 8)).astype(np.float32)
    lo = rng.standard_normal((1, 1, 6, 8)).astype(np.float32)
    hi = (lo + 1).astype(np.float32)
    base = E.scores_dsa(qm, hi, lo)
    grown = E.scores_dsa(qm, (hi + np.float32(0.5)).astype(np.float32), (lo - np.float32(0.5)).astype(np.float32))
    assert np.all(grown >= base)


def test_mean_estimator_plan_matches_select_oracle():
    w = W.custom("pm", 1, 2, 64, (4, 8, 8), (1, 4, 4), "f32", 0.5, -1, "iid")
    inp = W.generate(w, seed=5)
    a = E.plan_estimate(inp["q"], inp["k"], w.grid, w.block, "mean", "topp", [0.5], sink=1)
    b = P.plan_select(inp["q"], inp["k"], w.grid, w.block, "topp", [0.5], sink=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
