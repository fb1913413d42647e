"""GPU parity of per-head blocking schemes (SPADE 3.2: a blocking scheme
per head; 3.3: heads that share one run in one launch), through the C ABI:

* planning and attention over a subset of the heads equal the oracle on
  those heads (index bit for bit, outputs within the bf16 bar) and leave
  the other heads of the output untouched;
* scheme selection that keeps each candidate's block means leaves exactly
  the planner's means (bit for bit against vsa_centroids), and a plan from
  them equals the plan that reads Q and K;
* end to end on an input whose heads prefer different blockings: every
  head is planned and attended under its own scheme, each head's index bit
  for bit and its output within the bar against the oracle at that head's
  blocking.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sics_oracle as S
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3


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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=torch.bfloat16).contiguous()


def _index_np(idx):
    rp = idx.row_ptr.cpu().numpy()
    return rp, idx.col_idx.cpu().numpy()[: int(rp[-1])]


@pytest.mark.parametrize("B,heads,window_t", [(1, [4, 1, 3], -1), (2, [2, 0], 1), (1, [0, 1, 2, 3, 4, 5], -1)])
def test_plan_and_attention_over_a_head_subset(vsa, B, heads, window_t):
    w = W.custom("heads_sub", B, 6, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, window_t, "smooth")
    _say(f"[gpu] head subset {heads} B={B} window={window_t}")
    inp = W.generate(w, seed=91)
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    idx = vsa.plan_heads(q, k, w.grid, w.block, heads, 0.3, window_t)
    sentinel = 7.0
    o = torch.full_like(q, sentinel)
    vsa.attn_heads(q, k, v, idx, heads, out=o)
    torch.cuda.synchronize()
    sub = lambda a: np.ascontiguousarray(a[:, heads])
    rp, ci, _ = O.plan(sub(inp["q"]), sub(inp["k"]), w.grid, w.block, np.float32(0.3), window_t)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    ref = O.attention(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), w.grid, w.block, rp, ci)
    og = o.float().cpu().numpy()
    err = np.abs(og[:, heads] - ref)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    others = [h for h in range(6) if h not in heads]
    assert np.all(og[:, others] == sentinel)


CANDS = [(4, 4, 8), (1, 8, 16), (2, 8, 8)]


@pytest.mark.parametrize("B", [1, 2])
def test_scheme_means_are_the_planner_means(vsa, B):
    w = W.custom("scheme_means", B, 4, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, -1, "smooth")
    _say(f"[gpu] scheme means against vsa_centroids and vsa_select_scheme, B={B}")
    inp = W.generate(w, seed=92)
    q, k = _dev(inp["q"]), _dev(inp["k"])
    scores, choice, sm = vsa.select_scheme_means(q, k, w.grid, CANDS)
    scores0, choice0 = vsa.select_scheme(q, k, w.grid, CANDS)
    torch.cuda.synchronize()
    np.testing.assert_allclose(scores.cpu().numpy(), scores0.cpu().numpy(), rtol=1e-5)
    ref = S.scheme_scores(inp["q"], inp["k"], w.grid, CANDS).reshape(len(CANDS), -1)
    np.testing.assert_allclose(scores.cpu().numpy(), ref, rtol=1e-4, atol=1e-3)
    for c, blk in enumerate(CANDS):
        qm, km = sm.means(c)
        g = O.geometry(w.grid, blk)
        cq = vsa.centroids(q, w.grid, blk).reshape(-1)
        ck = vsa.centroids(k, w.grid, blk).reshape(w.B * w.heads, g.NB, w.D).transpose(1, 2).contiguous()
        assert torch.equal(qm.view(torch.int32), cq.view(torch.int32))
        assert torch.equal(km.view(torch.int32), ck.reshape(-1).view(torch.int32))
        oq = O.centroids(inp["q"], g).astype(np.float32)
        assert np.array_equal(qm.cpu().numpy().reshape(oq.shape).view(np.uint32), oq.view(np.uint32))
        # a plan from the kept means equals the plan that reads Q and K
        heads = [3, 0]
        a = vsa.plan_heads(q, k, w.grid, blk, heads, 0.25)
        b = vsa.plan_heads(None, None, w.grid, blk, heads, 0.25, means=(qm, km), heads_total=w.heads, B=w.B,
                           D=w.D)
        torch.cuda.synchronize()
        ra, ca = _index_np(a)
        rb, cb = _index_np(b)
        assert np.array_equal(ra, rb) and np.array_equal(ca, cb)


def _structured_heads(rng, grid, D, nheads):
    """Head h's tokens vary only along one axis (t for h % 3 == 0, h for
    1, w for 2) plus small noise, so the blocking that keeps that axis
    fixed inside a block aggregates best (SPADE 3.2 Eq. 3 and 4)."""
    T, H, Wd = grid
    out = np.empty((1, nheads, T * H * Wd, D), np.float64)
    for h in range(nheads):
        ax = h % 3
        n_ax = grid[ax]
        base = rng.standard_normal((n_ax, D))
        shape = [1, 1, 1, D]
        shape[ax] = n_ax
        field = np.broadcast_to(base.reshape(shape), (T, H, Wd, D))
        out[0, h] = (field + 0.05 * rng.standard_normal((T, H, Wd, D))).reshape(-1, D)
    return W.round_to_bf16(out)


def test_per_head_schemes_end_to_end(vsa):
    grid = (8, 16, 16)
    cands = [(1, 16, 8), (8, 1, 16), (8, 16, 1)]   # each keeps one axis fixed inside a block
    rng = np.random.default_rng(93)
    nheads, D = 6, 128
    qn = _structured_heads(rng, grid, D, nheads)
    kn = _structured_heads(rng, grid, D, nheads)
    vn = W.round_to_bf16(rng.standard_normal(qn.shape))
    _say("[gpu] per-head schemes end to end")
    q, k, v = _dev(qn), _dev(kn), _dev(vn)
    sp = vsa.plan_schemes(q, k, grid, cands, 0.25)
    o = vsa.attn_schemes(q, k, v, sp)
    torch.cuda.synchronize()
    choice = sp.choice.cpu().numpy()
    assert choice.tolist() == [h % 3 for h in range(nheads)]
    ref_sc = S.scheme_scores(qn, kn, grid, cands).reshape(len(cands), -1)
    assert np.array_equal(S.select_scheme(ref_sc[:, None, :]).reshape(-1), choice)
    assert len(sp.groups) == 3
    og = o.float().cpu().numpy()
    for c, blk, hs, idx in sp.groups:
        sub = lambda a: np.ascontiguousarray(a[:, hs])
        rp, ci, _ = O.plan(sub(qn), sub(kn), grid, blk, np.float32(0.25), -1)
        grp, gci = _index_np(idx)
        assert np.array_equal(grp, rp) and np.array_equal(gci, ci), blk
        ref = O.attention(sub(qn), sub(kn), sub(vn), grid, blk, rp, ci)
        err = np.abs(og[:, hs] - ref)
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (blk, err.max(), err.mean())
