"""Pins for the mixed per-head plan oracle (DecoupAttn Plans, introduction;
SPADE 3.1 / 3.3; readings R28-R29): a hand-worked three-head plan, a rank
count for static heads written independently of the sort, closed forms for
dense heads, independence of static plans from Q and K, dynamic heads equal
to the pinned single-head plan, and per-head windows."""
import json
import os

import numpy as np

import workloads as W
from oracle import mixed_oracle as M
from oracle import vsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows(rp, ci):
    return [ci[rp[r]:rp[r + 1]].tolist() for r in range(len(rp) - 1)]


def test_golden_hand_example():
    with open(os.path.join(HERE, "golden", "mixed_hand_example.json")) as f:
        gold = json.load(f)
    t0 = np.array(gold["static_scores_head0"], np.float32)
    table = np.stack([t0, np.zeros_like(t0), t0])
    rp, ci, _ = M.plan_mixed(None, None, gold["grid"], gold["block"], gold["options"], table, B=1)
    rows = _rows(rp, ci)
    assert rows[0:4] == gold["rows"]["head0"]
    assert rows[4:8] == gold["rows"]["head1"]
    assert rows[8:12] == gold["rows"]["head2"]


def _rank_count(s, j):
    """Blocks strictly ahead of j: a higher score, or the same score and a
    lower id (R7)."""
    return int(np.sum(s > s[j]) + np.sum((s == s[j]) & (np.arange(len(s)) < j)))


def test_static_heads_by_rank_count():
    rng = np.random.default_rng(0)
    g = O.geometry((6, 4, 8), (2, 2, 4))
    NB = g.NB
    table = rng.integers(-3, 4, (3, NB, NB)).astype(np.float32)     # many ties
    opts = [{"kind": "static", "value": v} for v in (0.1, 0.5, 0.8)]
    rp, ci, _ = M.plan_mixed(None, None, g.grid, g.block, opts, table, B=2)
    rows = _rows(rp, ci)
    for b in range(2):
        for h, v in enumerate((0.1, 0.5, 0.8)):
            kk = O.k_rule(v, NB)
            for i in range(NB):
                s = table[h, i]
                want = [j for j in range(NB) if _rank_count(s, j) < kk]
                assert rows[(b * 3 + h) * NB + i] == want


def test_dense_heads_and_static_independent_of_qk():
    w = W.custom("mx", 1, 3, 64, (4, 8, 8), (2, 4, 4), "f32", 0.5, -1, "iid")
    g = O.geometry(w.grid, w.block)
    rng = np.random.default_rng(1)
    table = rng.standard_normal((3, g.NB, g.NB)).astype(np.float32)
    opts = [{"kind": "dense"}, {"kind": "static", "value": 0.3, "window_t": 0}, {"kind": "dense", "window_t": 1}]
    a = M.plan_mixed(None, None, w.grid, w.block, opts, table, B=1)
    inp = W.generate(w, seed=2)
    b = M.plan_mixed(inp["q"], inp["k"], w.grid, w.block, opts, table)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    lens = np.diff(a[0]).reshape(3, g.NB)
    assert np.all(lens[0] == g.NB) and np.all(lens[2] == g.NB)


def test_dynamic_heads_equal_single_head_plans():
    w = W.custom("dy", 2, 3, 64, (5, 8, 12), (2, 4, 4), "bf16", 0.5, -1, "smooth")
    g = O.geometry(w.grid, w.block)
    inp = W.generate(w, seed=3)
    table = np.zeros((3, g.NB, g.NB), np.float32)
    opts = [{"kind": "dynamic", "value": 0.2, "window_t": 1}, {"kind": "static", "value": 0.4},
            {"kind": "dynamic", "value": 0.5}]
    rp, ci, _ = M.plan_mixed(inp["q"], inp["k"], w.grid, w.block, opts, table)
    rows = _rows(rp, ci)
    for h, (dens, win) in ((0, (0.2, 1)), (2, (0.5, -1))):
        hrp, hci, _ = O.plan(inp["q"][:, h:h + 1], inp["k"][:, h:h + 1], w.grid, w.block, dens, win)
        hrows = _rows(hrp, hci)
        for b in range(2):
            assert rows[(b * 3 + h) * g.NB:(b * 3 + h + 1) * g.NB] == hrows[b * g.NB:(b + 1) * g.NB]
    # the static head with an all-zero table keeps the lowest ids
    kk = O.k_rule(0.4, g.NB)
    assert all(rows[(b * 3 + 1) * g.NB + i] == list(range(kk)) for b in range(2) for i in range(g.NB))


def test_per_head_windows():
    g = O.geometry((6, 2, 2), (1, 2, 2))         # one block per frame
    table = np.zeros((2, 6, 6), np.float32)
    table[:, :, 5] = 1.0                          # block 5 ranks first everywhere
    opts = [{"kind": "static", "value": 0.1, "window_t": 0}, {"kind": "static", "value": 0.1, "window_t": 2}]
    rp, ci, _ = M.plan_mixed(None, None, g.grid, g.block, opts, table, B=1)
    rows = _rows(rp, ci)
    for i in range(6):
        assert rows[i] == sorted({5, i})
        assert rows[6 + i] == sorted({5} | set(range(max(0, i - 2), min(6, i + 3))))
