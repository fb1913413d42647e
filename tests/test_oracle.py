"""Pins of the CPU oracle against facts that do not come from the oracle
itself: closed forms, a hand-worked example, a library routine (torch SDPA
on the CPU), brute force over an N x N mask, and invariants.

Each test names the part of the method it pins (SPADE 2.2 Eq. 1/2 and 3.3;
the JEV keep-rate definition) and the plausible mistakes it would catch.
"""
import json
import math
import os
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import vsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- geometry

def _closed_form_hist(grid, block):
    """Block-size histogram as the product of per-dimension extent lists."""
    per_dim = []
    for n, b in zip(grid, block):
        ext = [b] * (n // b) + ([n % b] if n % b else [])
        per_dim.append(ext)
    c = Counter()
    for a in per_dim[0]:
        for bb in per_dim[1]:
            for cc in per_dim[2]:
                c[a * bb * cc] += 1
    return c


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_geometry_closed_form(name):
    w = W.WORKLOADS[name]
    g = O.geometry(w.grid, w.block)
    assert g.NB == math.prod(-(-n // b) for n, b in zip(w.grid, w.block))
    assert Counter(g.sizes.tolist()) == _closed_form_hist(w.grid, w.block)
    assert int(g.sizes.sum()) == w.N
    allt = np.concatenate(g.tokens)
    assert np.array_equal(np.sort(allt), np.arange(w.N))          # bijection


def test_geometry_wan_histogram_values():
    # 21x30x52 with 4x4x8 blocks: t extents 4x5 + 1, h 4x7 + 2, w 8x6 + 4.
    g = O.geometry((21, 30, 52), (4, 4, 8))
    assert g.NB == 336
    assert dict(Counter(g.sizes.tolist())) == {128: 210, 64: 65, 32: 47, 16: 13, 8: 1}
    g = O.geometry((84, 30, 52), (4, 4, 8))
    assert g.NB == 1176 and dict(Counter(g.sizes.tolist())) == {128: 882, 64: 273, 32: 21}
    g = O.geometry((16, 45, 80), (1, 8, 16))
    assert g.NB == 480 and dict(Counter(g.sizes.tolist())) == {128: 400, 80: 80}


@pytest.mark.parametrize("grid,block", [((3, 5, 7), (2, 2, 4)), ((21, 30, 52), (4, 4, 8)),
                                        ((5, 9, 11), (1, 8, 16)), ((4, 8, 8), (2, 4, 8))])
def test_block_tokens_are_their_box(grid, block):
    """Each block's tokens are exactly its 3D box, in row-major (t, h, w)
    order, with ids row-major over (tb, hb, wb)."""
    T, H, Wd = grid
    g = O.geometry(grid, block)
    for j, ids in enumerate(g.tokens):
        t, h, w = np.unravel_index(ids, (T, H, Wd))
        tb, hb, wb = np.unravel_index(j, (g.nbt, g.nbh, g.nbw))
        assert np.all(t // block[0] == tb) and np.all(h // block[1] == hb) and np.all(w // block[2] == wb)
        # row-major inside the box: sorting by (t, h, w) keeps the order
        assert np.all(np.diff(ids) > 0)
        assert len(ids) == len(set(ids.tolist()))
    assert g.tblock.tolist() == [j // (g.nbh * g.nbw) for j in range(g.NB)]


# ---------------------------------------------------------------- k rule

def test_k_rule_table():
    assert O.k_rule(0.5, 4) == 2 and O.k_rule(1.0, 4) == 4
    assert O.k_rule(0.20, 336) == 67
    assert O.k_rule(0.15, 480) == 72
    assert [O.k_rule(d, 336) for d in (1.0, 0.30, 0.20, 0.10, 0.05)] == [336, 101, 67, 34, 17]
    assert O.k_rule(0.0675, 1176) == 79
    assert O.k_rule(1e-6, 336) == 1 and O.k_rule(1.0, 7) == 7


# ---------------------------------------------------------------- layout

@pytest.mark.parametrize("grid,block", [((3, 5, 7), (2, 2, 4)), ((21, 30, 52), (4, 4, 8))])
def test_permute_unpermute_identity(grid, block):
    rng = np.random.default_rng(1)
    N = math.prod(grid)
    x = rng.standard_normal((1, 2, N, 8)).astype(np.float32)
    g = O.geometry(grid, block)
    xb = O.permute(x, g)
    assert np.array_equal(O.unpermute(xb, g), x)
    for j, ids in enumerate(g.tokens):
        assert np.all(xb[:, :, j, len(ids):] == 0)                # pad rows zero
        assert np.array_equal(xb[:, :, j, : len(ids)], x[:, :, ids])


# ---------------------------------------------------------------- centroids

def test_centroids_identical_rows_exact():
    """A block whose tokens are all the same bf16 row has that row as its
    mean exactly (n*x is exact in float32 for bf16 x and n <= 128)."""
    grid, block = (21, 30, 52), (4, 4, 8)
    g = O.geometry(grid, block)
    rng = np.random.default_rng(2)
    rows = W.round_to_bf16(rng.standard_normal((g.NB, 16)) * 3)
    x = np.zeros((1, 1, math.prod(grid), 16), dtype=np.float32)
    for j, ids in enumerate(g.tokens):
        x[0, 0, ids] = rows[j]
    assert np.array_equal(O.centroids(x, g)[0, 0], rows)


def test_centroids_small_integers_match_exact_mean():
    """Integer inputs: the float32 sum is exact, so the result is the
    correctly rounded exact mean.  Catches dividing by the padded size,
    summing pad rows or skipping tokens."""
    grid, block = (21, 30, 52), (4, 4, 8)
    g = O.geometry(grid, block)
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(1, 2, math.prod(grid), 4)).astype(np.float32)
    c = O.centroids(x, g)
    for j, ids in enumerate(g.tokens):
        for h in range(2):
            for d in range(4):
                exact = Fraction(int(x[0, h, ids, d].astype(np.int64).sum()), len(ids))
                got = Fraction(float(c[0, h, j, d]))
                ulp = Fraction(float(np.spacing(np.float32(abs(float(exact)) or 1e-30))))
                assert abs(got - exact) <= ulp / 2


def test_centroid_is_sequential_float32():
    """The float32 summation order is the in-block token order: with
    1 + 2^-24 (x 3) the sequential sum differs from pairwise/reordered sums."""
    g = O.geometry((1, 1, 4), (1, 1, 4))
    x = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], dtype=np.float32).reshape(1, 1, 4, 1)
    # sequential: 1 + e = 1 (tie to even) three times -> 1, /4 = 0.25
    assert O.centroids(x, g)[0, 0, 0, 0] == np.float32(0.25)
    x2 = x[:, :, ::-1].copy()   # e + e + e + 1 = 1 + 3e rounds to 1 + 4e
    assert O.centroids(x2, g)[0, 0, 0, 0] == np.float32((1.0 + 4 * 2.0 ** -24) / 4)


# ---------------------------------------------------------------- scores

def test_scores_exact_for_integers_and_close_otherwise():
    rng = np.random.default_rng(4)
    qi = rng.integers(-20, 21, size=(3, 40, 64)).astype(np.float32)
    ki = rng.integers(-20, 21, size=(3, 50, 64)).astype(np.float32)
    S = O.scores(qi, ki)
    assert np.array_equal(S.astype(np.float64), qi.astype(np.float64) @ np.swapaxes(ki, -1, -2).astype(np.float64))
    qf = rng.standard_normal((2, 30, 128)).astype(np.float32)
    kf = rng.standard_normal((2, 30, 128)).astype(np.float32)
    S = O.scores(qf, kf).astype(np.float64)
    ref = qf.astype(np.float64) @ np.swapaxes(kf, -1, -2).astype(np.float64)
    bound = 2 * 128 * 2.0 ** -24 * (np.abs(qf.astype(np.float64)) @ np.swapaxes(np.abs(kf), -1, -2))
    assert np.all(np.abs(S - ref) <= bound)


def test_scores_not_transposed():
    q = np.array([[[1, 0], [0, 0]]], dtype=np.float32)
    k = np.array([[[0, 0], [5, 0]]], dtype=np.float32)
    S = O.scores(q, k)
    assert S[0, 0, 1] == 5 and S[0, 1, 0] == 0   # row = query block, col = key block


# ---------------------------------------------------------------- selection

def _rank_count_select(s, k):
    """Independent top-k: keep j iff fewer than k ids beat it, where j'
    beats j if its score is larger, or equal with a lower id."""
    n = len(s)
    keep = []
    for j in range(n):
        rank = sum(1 for jj in range(n) if s[jj] > s[j] or (s[jj] == s[j] and jj < j))
        if rank < k:
            keep.append(j)
    return np.array(keep)


def test_topk_matches_rank_count_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 60))
        s = rng.integers(-3, 4, size=n).astype(np.float32)   # many ties
        if trial % 3 == 0:
            s[s == 0] = -0.0                                # signed zeros tie with +0
        k = int(rng.integers(1, n + 1))
        assert np.array_equal(O.topk_row(s, k), _rank_count_select(s, k))


def test_selection_special_cases():
    g = O.geometry((8, 8, 8), (2, 4, 4))    # NB = 16
    B, Hh, N, D = 1, 2, 512, 16
    rng = np.random.default_rng(6)
    q = rng.standard_normal((B, Hh, N, D)).astype(np.float32)
    k = rng.standard_normal((B, Hh, N, D)).astype(np.float32)
    # all-equal scores (Q == 0) -> the k lowest ids
    rp, ci, info = O.plan(np.zeros_like(q), k, g.grid, g.block, 0.25)
    assert info["k"] == [4, 4]
    assert np.array_equal(ci.reshape(-1, 4), np.tile(np.arange(4), (Hh * g.NB, 1)))
    # density 1 -> every block
    rp, ci, _ = O.plan(q, k, g.grid, g.block, 1.0)
    assert np.array_equal(ci.reshape(-1, g.NB), np.tile(np.arange(g.NB), (Hh * g.NB, 1)))
    # Q * 2 (exact power of two) -> identical index
    rp1, ci1, _ = O.plan(q, k, g.grid, g.block, 0.3)
    rp2, ci2, _ = O.plan(q * 2, k, g.grid, g.block, 0.3)
    assert np.array_equal(rp1, rp2) and np.array_equal(ci1, ci2)
    # rows are ascending, unique, and of length k
    for r in range(len(rp1) - 1):
        row = ci1[rp1[r]: rp1[r + 1]]
        assert len(row) == O.k_rule(0.3, g.NB) and np.all(np.diff(row) > 0)


def test_window_union():
    g = O.geometry((20, 8, 8), (4, 4, 8))    # nbt 5, nbh 2, nbw 1 -> NB 10
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 1280, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1280, 8)).astype(np.float32)
    rp, ci, info = O.plan(q, k, g.grid, g.block, 0.2, window_t=1)
    S = info["S"][0, 0]
    for i in range(g.NB):
        row = set(ci[rp[i]: rp[i + 1]].tolist())
        win = {j for j in range(g.NB) if abs(j // 2 - i // 2) <= 1}
        top = set(_rank_count_select(S[i], 2).tolist())
        assert row == win | top


def test_per_head_density():
    g = O.geometry((8, 8, 8), (2, 4, 4))
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 3, 512, 8)).astype(np.float32)
    k = rng.standard_normal((1, 3, 512, 8)).astype(np.float32)
    rp, ci, info = O.plan(q, k, g.grid, g.block, np.array([1.0, 0.5, 0.1], dtype=np.float32))
    assert info["k"] == [16, 8, 2]
    lens = np.diff(rp).reshape(3, g.NB)
    assert np.all(lens[0] == 16) and np.all(lens[1] == 8) and np.all(lens[2] == 2)


# ---------------------------------------------------------------- attention

def test_density_one_equals_dense_sdpa():
    """Eq. 1 special case: with every block kept, block-sparse attention is
    dense softmax attention (torch SDPA on the CPU in float64)."""
    w = W.WORKLOADS["tiny_fp32_dense"]
    inp = W.generate(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    rp, ci, _ = O.plan(q, k, w.grid, w.block, 1.0)
    o = O.attention(q, k, v, w.grid, w.block, rp, ci)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(), torch.from_numpy(v).double()).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def _brute_force_eq2(q, k, v, g, rp, ci, scale=None):
    """Eq. 2 with an N x N additive mask built from the block index."""
    B, Hh, N, D = q.shape
    sc = 1 / math.sqrt(D) if scale is None else scale
    blk = np.zeros(N, dtype=np.int64)
    for j, ids in enumerate(g.tokens):
        blk[ids] = j
    out = np.zeros((B, Hh, N, v.shape[-1]))
    for b in range(B):
        for h in range(Hh):
            keep = np.zeros((g.NB, g.NB), dtype=bool)
            for i in range(g.NB):
                r = (b * Hh + h) * g.NB + i
                keep[i, ci[rp[r]: rp[r + 1]]] = True
            M = np.where(keep[blk][:, blk], 0.0, -np.inf)
            L = q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T * sc + M
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[b, h] = P @ v[b, h].astype(np.float64)
    return out


@pytest.mark.parametrize("grid,block,dens,win", [
    ((4, 8, 8), (2, 4, 8), 0.5, -1),
    ((3, 5, 7), (2, 2, 4), 0.34, -1),
    ((5, 6, 9), (2, 4, 4), 0.2, 1),
    ((2, 9, 17), (1, 8, 16), 0.5, 0),
])
def test_matches_brute_force_eq2(grid, block, dens, win):
    rng = np.random.default_rng(9)
    N = math.prod(grid)
    q, k, v = (rng.standard_normal((2, 2, N, 16)).astype(np.float32) for _ in range(3))
    rp, ci, _ = O.plan(q, k, grid, block, dens, win)
    g = O.geometry(grid, block)
    o = O.attention(q, k, v, grid, block, rp, ci)
    assert np.max(np.abs(o - _brute_force_eq2(q, k, v, g, rp, ci))) < 1e-12


def test_softmax_weights_sum_to_one_and_vanish_elsewhere():
    grid, block = (3, 5, 7), (2, 2, 4)
    g = O.geometry(grid, block)
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((1, 1, 105, 8)).astype(np.float32) for _ in range(3))
    rp, ci, _ = O.plan(q, k, grid, block, 0.4)
    for i in range(g.NB):
        o, p, kid = O.attention_row(q, k, v, g, rp, ci, 0, 0, i, return_weights=True)
        assert np.max(np.abs(p.sum(axis=1) - 1)) < 1e-12
        kept = set(ci[rp[i]: rp[i + 1]].tolist())
        assert set(kid.tolist()) == set(np.concatenate([g.tokens[j] for j in kept]).tolist())


def test_constant_v_and_shift():
    grid, block = (3, 5, 7), (2, 2, 4)
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 2, 105, 8)).astype(np.float32) for _ in range(3))
    rp, ci, _ = O.plan(q, k, grid, block, 0.5)
    o1 = O.attention(q, k, np.ones_like(v), grid, block, rp, ci)
    assert np.max(np.abs(o1 - 1)) < 1e-12
    o = O.attention(q, k, v, grid, block, rp, ci)
    o_shift = O.attention(q, k, v.astype(np.float64) + 3.0, grid, block, rp, ci)
    assert np.max(np.abs(o_shift - o - 3.0)) < 1e-12


def test_equals_sdpa_over_gathered_tokens():
    grid, block = (4, 8, 8), (2, 4, 8)
    g = O.geometry(grid, block)
    inp = W.generate(W.WORKLOADS["tiny_fp32"])
    q, k, v = inp["q"], inp["k"], inp["v"]
    rp, ci, _ = O.plan(q, k, grid, block, 0.5)
    o = O.attention(q, k, v, grid, block, rp, ci)
    for h in range(2):
        for i in range(g.NB):
            kid = np.concatenate([g.tokens[j] for j in ci[rp[h * g.NB + i]: rp[h * g.NB + i + 1]]])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[0, h, g.tokens[i]]).double()[None],
                torch.from_numpy(k[0, h, kid]).double()[None],
                torch.from_numpy(v[0, h, kid]).double()[None])[0].numpy()
            assert np.max(np.abs(o[0, h, g.tokens[i]] - ref)) < 1e-12


# ---------------------------------------------------------------- hand example

def test_hand_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    grid, block, D = tuple(ex["grid"]), tuple(ex["block"]), ex["D"]
    N = math.prod(grid)
    q = np.zeros((1, 1, N, D), dtype=np.float32)
    k = np.zeros((1, 1, N, D), dtype=np.float32)
    for n, val in ex["q_tokens"].items():
        q[0, 0, int(n)] = val
    for n, val in ex["k_tokens"].items():
        k[0, 0, int(n)] = val
    v = np.array([[n, -n] for n in range(N)], dtype=np.float32)[None, None]
    rp, ci, info = O.plan(q, k, grid, block, ex["density"])
    assert np.array_equal(info["qc"][0, 0], np.array(ex["q_centroids"], dtype=np.float32))
    assert np.array_equal(info["kc"][0, 0], np.array(ex["k_centroids"], dtype=np.float32))
    assert np.array_equal(info["S"][0, 0], np.array(ex["scores"], dtype=np.float32))
    assert rp.tolist() == ex["row_ptr"] and ci.tolist() == ex["col_idx"]
    o = O.attention(q, k, v, grid, block, rp, ci)
    for n, val in ex["output_tokens"].items():
        assert np.allclose(o[0, 0, int(n)], val, atol=1e-12)


def test_executed_flops_dense_matches_4N2D():
    g = O.geometry((4, 8, 8), (2, 4, 8))
    rp = np.arange(0, 17, 4)
    ci = np.tile(np.arange(4), 4)
    assert O.executed_flops(g, rp, ci, 1, 1, 64) == 4 * 256 * 256 * 64
