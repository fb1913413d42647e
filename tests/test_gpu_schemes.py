"""GPU parity for scheme generation (SPADE 3.2): per-block SICS and the
head-wise blocking-scheme choice, through the C ABI, against the float64
oracle (Algorithm 1).

Bar: SICS and aggregation scores within rtol 1e-4 (atol 1e-3) of the
oracle -- the kernel accumulates unit vectors in float32, a relative error
near 1e-6 at these sizes; the chosen scheme must be an argmax of the
oracle's scores within that bound (a float32 decision, reading R20).
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sics_oracle as S
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import block_sparse_attention_centroids_amd as pkg
    pkg.load()
    return pkg


def _dev(a, w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dt).contiguous()


CASES = [
    W.custom("sics_fp32_d64", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
    W.custom("sics_fp32_d128_ragged", 1, 2, 128, (3, 5, 7), (2, 2, 4), "f32", 0.5, -1, "iid"),
    W.custom("sics_bf16_ragged", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, -1, "smooth"),
    W.custom("sics_bf16_d64", 2, 3, 64, (5, 9, 11), (1, 8, 16), "bf16", 0.5, -1, "smooth"),
    W.custom("sics_token_blocks", 1, 1, 128, (4, 4, 4), (1, 1, 1), "bf16", 0.5, -1, "smooth"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_sics_small(vsa, w):
    _say(f"[gpu] sics {w.name} grid={w.grid} block={w.block} D={w.D} {w.dtype}")
    inp = W.generate(w, seed=4)
    q = inp["q"].copy()
    q[0, 0, 5] = 0.0   # a zero token: adds nothing (reading R18)
    got = vsa.sics(_dev(q, w), w.grid, w.block).cpu().numpy()
    ref = S.block_sics(q, O.geometry(w.grid, w.block))
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_sics_special_values(vsa):
    """Identical tokens in every block -> BS^2; antipodal halves -> 0."""
    w = W.custom("sics_special", 1, 2, 128, (2, 4, 8), (2, 4, 8), "f32", 0.5, -1, "iid")
    v = np.random.default_rng(11).standard_normal(128).astype(np.float32)
    x = np.zeros((1, 2, 64, 128), dtype=np.float32)
    x[0, 0] = v
    x[0, 1, :32] = v
    x[0, 1, 32:] = -3.0 * v
    got = vsa.sics(_dev(x, w), w.grid, w.block).cpu().numpy()
    assert got[0, 0, 0] == pytest.approx(64.0 * 64.0, rel=1e-5)
    assert abs(got[0, 1, 0]) < 1e-2


def _check_selection(scores, choice, ref):
    n, BH = scores.shape
    np.testing.assert_allclose(scores, ref.reshape(n, BH), rtol=RTOL, atol=ATOL)
    refm = ref.reshape(n, BH)
    best = refm.max(axis=0)
    for bh in range(BH):
        c = int(choice[bh])
        assert 0 <= c < n
        assert refm[c, bh] >= best[bh] - RTOL * abs(best[bh]) - ATOL, (bh, c, refm[:, bh])


def test_select_scheme_small(vsa):
    w = W.custom("sel_small", 2, 3, 128, (8, 16, 16), (4, 4, 8), "bf16", 0.5, -1, "smooth")
    inp = W.generate(w, seed=6)
    cands = [(4, 4, 8), (1, 8, 16), (2, 8, 8), (8, 4, 4), (4, 4, 4)]
    scores, choice = vsa.select_scheme(_dev(inp["q"], w), _dev(inp["k"], w), w.grid, cands)
    ref = S.scheme_scores(inp["q"], inp["k"], w.grid, cands)
    _check_selection(scores.cpu().numpy(), choice.cpu().numpy(), ref)


def test_select_scheme_follows_structure(vsa):
    """Tokens constant along w: blocks along w are all-identical, so the
    (1, 1, 8) candidate has the largest score for every head."""
    T, H, Wd, d = 8, 8, 8, 64
    w = W.custom("sel_struct", 1, 2, d, (T, H, Wd), (1, 1, 8), "f32", 0.5, -1, "iid")
    base = np.random.default_rng(12).standard_normal((1, 2, T, H, 1, d)).astype(np.float32)
    x = np.broadcast_to(base, (1, 2, T, H, Wd, d)).reshape(1, 2, T * H * Wd, d).copy()
    scores, choice = vsa.select_scheme(_dev(x, w), _dev(x, w), w.grid, [(1, 8, 1), (8, 1, 1), (1, 1, 8)])
    assert choice.cpu().numpy().tolist() == [2, 2]
    assert scores.cpu().numpy()[2] == pytest.approx([2 * 64 * 64.0] * 2, rel=1e-5)


def test_select_scheme_repeatable(vsa):
    w = W.custom("sel_rep", 1, 4, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, -1, "smooth")
    inp = W.generate(w, seed=7)
    q, k = _dev(inp["q"], w), _dev(inp["k"], w)
    cands = [(4, 4, 8), (2, 8, 8), (1, 8, 16)]
    a = vsa.select_scheme(q, k, w.grid, cands)
    b = vsa.select_scheme(q, k, w.grid, cands)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.timeout(600)
def test_select_scheme_wan_shape(vsa):
    """Full Wan2.1-1.3B shape, three 128-token candidates; every head."""
    w = W.WORKLOADS["wan13b"]
    _say("[gpu] scheme selection at the Wan2.1-1.3B shape")
    inp = W.generate(w)
    cands = [(4, 4, 8), (1, 8, 16), (2, 8, 8)]
    scores, choice = vsa.select_scheme(_dev(inp["q"], w), _dev(inp["k"], w), w.grid, cands)
    ref = S.scheme_scores(inp["q"], inp["k"], w.grid, cands)
    _check_selection(scores.cpu().numpy(), choice.cpu().numpy(), ref)
    _say(f"[gpu]   choices {choice.cpu().numpy().tolist()}")
