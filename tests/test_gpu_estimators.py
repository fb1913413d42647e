"""GPU parity of the max/min summarizers and the DSA / DSA2 inter-estimators
(SPADE 3.1, Fig. 4) through the C ABI, against the CPU oracle.

Bar: the estimator score matrices and Top-K indices are bit-exact (both
sides follow the same float32 order); Top-P indices are checked as in the
selection tests (prefixes of the oracle order within the float32 band);
attention over the planned index matches the oracle's attention within the
bf16 / fp32 bar on rows whose index matches.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dsa_oracle as E
from oracle import vsa_oracle as O
from select_check import check_index

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


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


def _to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype).contiguous()


def _tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _index_np(idx):
    rp = idx.row_ptr.cpu().numpy()
    return rp, idx.col_idx.cpu().numpy()[: int(rp[-1])]


SHAPES = [
    W.custom("e_tiny_f32", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
    W.custom("e_ragged_bf16", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, -1, "smooth"),
    W.custom("e_hy_bf16_d64", 2, 2, 64, (5, 9, 11), (1, 8, 16), "bf16", 0.3, -1, "smooth"),
    W.custom("e_ragged_f32_d128", 1, 1, 128, (3, 5, 7), (2, 2, 4), "f32", 0.4, -1, "iid"),
    W.custom("e_lds_rows", 1, 1, 64, (8, 32, 40), (1, 2, 2), "bf16", 0.05, -1, "smooth"),
]


@pytest.mark.parametrize("est", ["mean", "dsa", "dsa2"])
@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_estimator_scores_bitexact(vsa, w, est):
    _say(f"[gpu] estimate {est} {w.name} grid={w.grid} block={w.block} D={w.D} {w.dtype}")
    inp = W.generate(w, seed=11)
    dt = _tdtype(w)
    q, k = (_to_dev(inp[n], dt) for n in ("q", "k"))
    S = vsa.estimate(q, k, w.grid, w.block, est)
    torch.cuda.synchronize()
    g = O.geometry(w.grid, w.block)
    ref = E.estimate(inp["q"], inp["k"], g, est)
    assert np.array_equal(S.cpu().numpy(), ref)


CASES = [
    # workload, estimator, mode, values, window_t, sink, scale
    (SHAPES[1], "dsa", "topk", [0.3, 0.1], -1, 0, None),
    (SHAPES[1], "dsa2", "topk", [0.2], 1, 2, None),
    (SHAPES[2], "dsa", "topp", [0.6, 0.3], -1, 1, None),
    (SHAPES[2], "dsa2", "topp", [0.9], 0, 0, 0.5),
    (SHAPES[0], "dsa", "topk", [0.5], -1, 0, None),
    (SHAPES[3], "dsa2", "topk", [0.4], -1, 3, None),
    (SHAPES[4], "dsa", "topk", [0.05], -1, 2, None),
    (SHAPES[4], "dsa2", "topp", [0.5], -1, 0, 0.25),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0].name}_{c[1]}_{c[2]}" for c in CASES])
def test_estimator_plan_and_attention(vsa, case):
    w, est, mode, vals, window_t, sink, scale = case
    _say(f"[gpu] plan {est} {mode} {vals} window={window_t} sink={sink} on {w.name}")
    inp = W.generate(w, seed=12)
    dt = _tdtype(w)
    q, k, v = (_to_dev(inp[n], dt) for n in ("q", "k", "v"))
    idx = vsa.plan_select(q, k, w.grid, w.block, mode, vals, window_t, sink, scale, est)
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    g = O.geometry(w.grid, w.block)
    S = E.estimate(inp["q"], inp["k"], g, est)
    sc = 1.0 / math.sqrt(w.D) if scale is None else float(np.float32(scale))
    grp, gci = _index_np(idx)
    (rows, band, differ), (rp, ci) = check_index(grp, gci, S, g, mode, vals, window_t, sink, sc)
    ref = O.attention(inp["q"], inp["k"], inp["v"], w.grid, w.block, rp, ci)
    og = o.float().cpu().numpy()
    # A Top-P row inside the float32 band (its GPU cut was validated above)
    # is checked against the oracle's attention over the GPU's own row.
    own = {int(r) for r in differ}
    errs = []
    for r in range(rows):
        b, rem = divmod(r, w.heads * g.NB)
        h, i = divmod(rem, g.NB)
        if r in own:
            want = O.attention_row(inp["q"], inp["k"], inp["v"], g, grp, gci, b, h, i)
        else:
            want = ref[b, h, g.tokens[i]]
        errs.append(np.abs(og[b, h, g.tokens[i]] - want).ravel())
    err = np.concatenate(errs)
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    else:
        assert err.max() <= F32_MAX, err.max()
    _say(f"[gpu]   ok rows={rows} band={band} nnz={idx.nnz()} max-abs {err.max():.2e}")


def test_dsa_zero_queries_tie_to_low_ids(vsa):
    """Q == 0 makes every DSA / DSA2 score 0: the lowest ids are kept."""
    w = W.custom("z", 1, 2, 128, (8, 8, 16), (2, 4, 8), "bf16", 0.25, -1, "smooth")
    inp = W.generate(w, seed=4)
    q = torch.zeros((1, 2, w.N, 128), dtype=torch.bfloat16, device="cuda")
    k = _to_dev(inp["k"], torch.bfloat16)
    g = O.geometry(w.grid, w.block)
    kk = O.k_rule(0.25, g.NB)
    for est in ("dsa", "dsa2"):
        idx = vsa.plan_select(q, k, w.grid, w.block, "topk", 0.25, estimator=est)
        torch.cuda.synchronize()
        _, ci = _index_np(idx)
        assert np.array_equal(ci.reshape(-1, kk), np.tile(np.arange(kk), (2 * g.NB, 1))), est


FULL = [("wan13b", "dsa", 0.2), ("wan13b", "dsa2", 0.2), ("hunyuan", "dsa", 0.15)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", FULL, ids=[f"{c[0]}_{c[1]}" for c in FULL])
def test_full_estimator_index(vsa, case):
    name, est, dens = case
    w = W.WORKLOADS[name]
    _say(f"[gpu] full {est} {name}: generating")
    inp = W.generate(w)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    _say(f"[gpu] full {est} {name}: GPU plan")
    idx = vsa.plan_select(q, k, w.grid, w.block, "topk", dens, estimator=est)
    torch.cuda.synchronize()
    grp, gci = _index_np(idx)
    _say(f"[gpu] full {est} {name}: oracle plan")
    rp, ci, _ = E.plan_estimate(inp["q"], inp["k"], w.grid, w.block, est, "topk", [dens])
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    _say(f"[gpu]   ok nnz={len(ci)}")
