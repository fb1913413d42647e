"""Pins for the selection-variant oracle (SPADE 3.1 Top-K/Top-P mode and
attention-sink length, 3.3 Top-P filtering and union with the sink mask;
readings R21-R24).  Each checks the oracle against something other than its
own formula: a hand-worked example, brute force over all subsets of tiny
rows, closed forms of uniform and two-level rows, limits that reduce to
argmax or to the whole row, nesting in p, shift invariance of the softmax,
and constructed inputs whose kept sets are known."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import select_oracle as P
from oracle import vsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _hand_scores():
    return np.array([math.log(4.0), 0.0, math.log(2.0), math.log(2.0), 0.0], dtype=np.float32)


def test_golden_hand_example():
    with open(os.path.join(HERE, "golden", "topp_hand_example.json")) as f:
        gold = json.load(f)
    s = _hand_scores()
    probs = P.row_probabilities(s, 1.0)
    np.testing.assert_allclose(probs, gold["scale_1"]["prob"], rtol=1e-6)
    order, F = P.prefix_mass(s, 1.0)
    assert order.tolist() == gold["scale_1"]["order"]
    np.testing.assert_allclose(F, gold["scale_1"]["cumulative"], rtol=1e-6)
    for p, kept in gold["scale_1"]["cases"]:
        assert P.topp_row(s, p, 1.0).tolist() == kept, p
    for p, kept in gold["scale_0.5"]["cases"]:
        assert P.topp_row(s, p, 0.5).tolist() == kept, p
    # the exact half of the second table: (2 + sqrt 2) / (4 + 2 sqrt 2)
    _, F5 = P.prefix_mass(s, 0.5)
    assert F5[1] == pytest.approx(0.5, abs=1e-6)
    assert F5[0] == pytest.approx(2.0 / (4.0 + 2.0 * math.sqrt(2.0)), rel=1e-6)


def test_golden_sink_example():
    with open(os.path.join(HERE, "golden", "topp_hand_example.json")) as f:
        gold = json.load(f)["sink"]
    s = _hand_scores()
    g = O.geometry((1, 1, 5), (1, 1, 1))     # five blocks of one token
    S = np.zeros((1, 1, 5, 5), dtype=np.float32)
    S[0, 0, :, :] = s
    rp, ci = P.select_rows(S, "topp", [0.3], g, sink=2, scale=1.0)
    assert ci[rp[0]:rp[1]].tolist() == gold["topp_p0.3_sink2"]
    rp, ci = P.select_rows(S, "topk", [0.2], g, sink=3, scale=1.0)
    assert ci[rp[0]:rp[1]].tolist() == gold["topk_k1_sink3"]


def _subset_mass(prob, ids):
    return float(sum(prob[j] for j in ids))


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_smallest_covering_set(seed):
    """R21 as a set statement: the kept blocks form a smallest set whose
    probability reaches p, of the largest mass among sets of that size, and
    among those the one with the lowest ids."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    if seed % 3 == 0:
        s = rng.integers(-2, 3, n).astype(np.float32)      # ties
    else:
        s = rng.standard_normal(n).astype(np.float32)
    scale = float(rng.uniform(0.3, 3.0))
    prob = P.row_probabilities(s, scale)
    subsets = [c for r in range(1, n + 1) for c in itertools.combinations(range(n), r)]
    for p in rng.uniform(0.05, 1.0, 6):
        masses = {c: _subset_mass(prob, c) for c in subsets}
        if any(abs(m - p) < 1e-9 for m in masses.values()):
            continue                                       # boundary: not decidable
        covering = [c for c in subsets if masses[c] >= p]
        size = min(len(c) for c in covering) if covering else n
        same = [c for c in subsets if len(c) == size]
        best = max(masses[c] for c in same)
        top = sorted(c for c in same if masses[c] >= best - 1e-12)
        assert P.topp_row(s, p, scale).tolist() == list(top[0]), (s, p, scale)


@pytest.mark.parametrize("NB,p", [(10, 0.35), (336, 0.2), (336, 0.9), (7, 0.999)])
def test_uniform_row_closed_form(NB, p):
    s = np.full(NB, 0.75, dtype=np.float32)
    c = math.ceil(p * NB)
    assert P.topp_count(s, p, 0.125) == c
    assert P.topp_row(s, p, 0.125).tolist() == list(range(c))


@pytest.mark.parametrize("m,a,NB,p", [(3, 2.0, 20, 0.4), (5, 1.0, 50, 0.1), (8, 4.0, 64, 0.8)])
def test_two_level_row_closed_form(m, a, NB, p):
    """m blocks at score a (spread over the row), the rest at 0, scale 1:
    a prefix of c <= m blocks holds c*e^a / (m*e^a + NB - m)."""
    rng = np.random.default_rng(m)
    hi = np.sort(rng.choice(NB, m, replace=False))
    s = np.zeros(NB, dtype=np.float32)
    s[hi] = a
    ea = float(np.exp(np.float64(np.float32(a))))
    Z = m * ea + (NB - m)
    c = math.ceil(p * Z / ea)
    assert c <= m
    assert P.topp_count(s, p, 1.0) == c
    assert P.topp_row(s, p, 1.0).tolist() == hi[:c].tolist()


def test_limits():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(100).astype(np.float32)
    s[[17, 60]] = s.max() + 1.0                            # tied maximum at 17 and 60
    prob = P.row_probabilities(s, 1.0)
    # p at most the largest probability: the argmax alone, ties to the lower id
    assert P.topp_row(s, float(prob.max()) * 0.5, 1.0).tolist() == [int(np.argmax(s))] == [17]
    # p = 1: every block (rounding may leave the total just below 1)
    assert P.topp_count(s, 1.0, 1.0) == 100
    # p = 1 even where a probability underflows: exp(-1000) > 0 exactly
    assert P.topp_row(np.array([0.0, -1000.0, 3.0], np.float32), 1.0, 1.0).tolist() == [0, 1, 2]
    assert P.topp_row(np.array([0.0, -1000.0, 3.0], np.float32), 0.99, 1.0).tolist() == [0, 2]
    # a huge scale concentrates all the mass on the tied maxima
    assert P.topp_row(s, 0.4, 1e6).tolist() == [17]
    assert P.topp_row(s, 0.9, 1e6).tolist() == [17, 60]
    # a vanishing scale makes the row uniform: ceil(p*NB) blocks, the best-scored ones
    c = P.topp_count(s, 0.335, 1e-12)
    assert c == 34
    assert P.topp_row(s, 0.335, 1e-12).tolist() == sorted(np.argsort(-s.astype(np.float64), kind="stable")[:34].tolist())


def test_nested_in_p_and_at_least_one():
    rng = np.random.default_rng(11)
    for _ in range(20):
        s = rng.standard_normal(int(rng.integers(1, 400))).astype(np.float32)
        scale = float(rng.uniform(0.05, 2.0))
        prev = set()
        for p in np.linspace(1e-6, 1.0, 15):
            cur = set(P.topp_row(s, p, scale).tolist())
            assert len(cur) >= 1
            assert prev <= cur
            prev = cur


def test_shift_invariance():
    """The softmax does not see a common shift of the row's scores."""
    rng = np.random.default_rng(3)
    s = (rng.integers(-40, 40, 200) / 8.0).astype(np.float32)   # exact in float32, with ties
    for p in (0.1, 0.5, 0.77, 0.95):
        assert P.topp_row(s, p, 0.7).tolist() == P.topp_row(s + np.float32(4.0), p, 0.7).tolist()


def test_sink_blocks_and_union():
    """Scores that favour the last blocks: Top-K keeps the last k, the sink
    adds the first s, and the two sets are disjoint, so each row has k + s."""
    g = O.geometry((4, 4, 8), (1, 2, 2))                   # NB = 4*2*4 = 32
    NB = g.NB
    S = np.broadcast_to(np.arange(NB, dtype=np.float32), (2, 3, NB, NB)).copy()
    k = O.k_rule(0.25, NB)
    rp, ci = P.select_rows(S, "topk", [0.25], g, sink=5, scale=1.0)
    for r in range(len(rp) - 1):
        row = ci[rp[r]:rp[r + 1]].tolist()
        assert row == list(range(5)) + list(range(NB - k, NB))
    # sink = NB keeps everything; sink = 0 changes nothing
    rp, ci = P.select_rows(S, "topp", [0.5], g, sink=NB, scale=1.0)
    assert np.all(np.diff(rp) == NB)
    a = P.select_rows(S, "topp", [0.5], g, sink=0, scale=1.0)
    b = P.select_rows(S, "topp", [0.5], g, scale=1.0)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_window_sink_topp_union():
    """Temporal window, sink and Top-P together: the row is the union of the
    three sets built by hand for a constructed row."""
    g = O.geometry((6, 2, 2), (1, 2, 2))                   # one block per frame, NB = 6
    S = np.zeros((1, 1, 6, 6), dtype=np.float32)
    S[0, 0, :, 4] = 10.0                                   # block 4 dominates every row
    rp, ci = P.select_rows(S, "topp", [0.5], g, window_t=1, sink=1, scale=1.0)
    expect = {0: [0, 1, 4], 1: [0, 1, 2, 4], 2: [0, 1, 2, 3, 4], 3: [0, 2, 3, 4],
              4: [0, 3, 4, 5], 5: [0, 4, 5]}
    for i in range(6):
        assert ci[rp[i]:rp[i + 1]].tolist() == expect[i]


def test_topk_mode_matches_plan():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 4 * 8 * 8, 64)).astype(np.float32)
    k = rng.standard_normal((1, 2, 4 * 8 * 8, 64)).astype(np.float32)
    a = P.plan_select(q, k, (4, 8, 8), (1, 4, 4), "topk", [0.3, 0.6], window_t=0)
    b = O.plan(q, k, (4, 8, 8), (1, 4, 4), [0.3, 0.6], window_t=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
