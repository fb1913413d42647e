"""GPU parity of the selection variants (Top-P and attention-sink blocks)
through the C ABI, against the CPU oracle.

Top-K rows (with sinks and windows) must equal the oracle's bit for bit.
A Top-P row must be the union of a prefix of the oracle's (score desc, id
asc) order -- the scores are bit-identical on both sides -- with the window
and the sinks, and the prefix length must be valid: the GPU decides it in
float32, so a length c is accepted when the float64 mass of the first c-1
blocks is below p + tol and that of the first c blocks is at least p - tol,
tol = 6 * NB * 2^-24 (weights e_j = expf(fl(fl(s_j - m) * scale)) carry a
relative error of at most about 2u(1 + |a_j|), so an absolute error below
2.8u each since e^-a * a <= 1/e; sums of NB non-negative terms add at most
(NB - 1)u of the total, and the total is at least 1).  Rows whose oracle
cut lies outside that band must match exactly; the test reports how many
rows fell inside it.  Attention after a Top-P plan is compared with the
oracle's attention on the rows whose index matches the oracle's.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import select_oracle as P
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


SMALL = [
    # name, workload, mode, values, window_t, sink, scale
    ("topp_tiny_fp32", W.custom("t1", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
     "topp", [0.5], -1, 0, None),
    ("topp_ragged_bf16", W.custom("t2", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, -1, "smooth"),
     "topp", [0.3, 0.8], -1, 0, None),
    ("topp_scale1_sink", W.custom("t3", 1, 3, 64, (5, 9, 11), (1, 8, 16), "bf16", 0.5, -1, "smooth"),
     "topp", [0.9, 0.5, 0.2], -1, 2, 1.0),
    ("topp_window_sink", W.custom("t4", 2, 2, 128, (12, 8, 8), (4, 4, 8), "bf16", 0.5, 1, "smooth"),
     "topp", [0.6], 1, 3, None),
    ("topp_p1_all", W.custom("t5", 1, 2, 128, (6, 8, 16), (2, 4, 8), "bf16", 0.5, -1, "smooth"),
     "topp", [1.0], -1, 0, 2.0),
    ("topp_tiny_p", W.custom("t6", 1, 2, 128, (6, 8, 16), (2, 4, 8), "bf16", 0.5, -1, "smooth"),
     "topp", [1e-6], -1, 1, 4.0),
    ("topp_single_block", W.custom("t7", 1, 2, 128, (2, 3, 5), (4, 4, 8), "bf16", 0.5, -1, "smooth"),
     "topp", [0.5], -1, 1, None),
    ("topp_lds_rows", W.custom("t8", 1, 2, 64, (8, 32, 40), (1, 2, 2), "bf16", 0.5, -1, "smooth"),
     "topp", [0.3, 0.9], -1, 2, 0.25),
    ("topk_sink", W.custom("k1", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, -1, "smooth"),
     "topk", [0.1, 0.3], -1, 4, None),
    ("topk_sink_window", W.custom("k2", 2, 2, 128, (12, 8, 8), (4, 4, 8), "bf16", 0.5, 0, "smooth"),
     "topk", [0.2], 0, 2, None),
    ("topk_sink_all", W.custom("k3", 1, 1, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
     "topk", [0.25], -1, 4, None),
    ("topk_lds_rows_sink", W.custom("k4", 1, 2, 64, (8, 32, 40), (1, 2, 2), "bf16", 0.5, -1, "smooth"),
     "topk", [0.05], 1, 7, None),
]


def _scale(w, scale):
    return 1.0 / math.sqrt(w.D) if scale is None else float(np.float32(scale))


def _plan_both(vsa, w, inp, mode, vals, window_t, sink, scale):
    dt = _tdtype(w)
    q, k, v = (_to_dev(inp[n], dt) for n in ("q", "k", "v"))
    idx = vsa.plan_select(q, k, w.grid, w.block, mode, vals, window_t, sink, scale)
    torch.cuda.synchronize()
    g = O.geometry(w.grid, w.block)
    S = O.scores(O.centroids(inp["q"], g), O.centroids(inp["k"], g))
    return (q, k, v), idx, g, S


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_select_parity(vsa, case):
    name, w, mode, vals, window_t, sink, scale = case
    _say(f"[gpu] select {name}: {mode} {vals} window={window_t} sink={sink} scale={scale} "
         f"grid={w.grid} block={w.block} {w.dtype}")
    inp = W.generate(w, seed=6)
    (q, k, v), idx, g, S = _plan_both(vsa, w, inp, mode, vals, window_t, sink, scale)
    grp, gci = _index_np(idx)
    (rows, band, differ), (rp, ci) = check_index(grp, gci, S, g, mode, vals, window_t, sink, _scale(w, scale))
    if mode == "topp" and float(np.max(vals)) >= 1.0:
        assert np.all(np.diff(grp) == g.NB)
    assert idx.nnz() <= idx.capacity
    # attention over the planned index on the rows that match the oracle's
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
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


# Rows of NB blocks keep their keys in 4, 6, 8, 12, 16 or 20 register chunks
# of 64 (the fewest that hold the row) and longer rows in LDS: each width at
# its edges.
WIDTHS = [(256, (1, 32, 32)), (257, (1, 2, 514)), (384, (1, 32, 48)), (385, (1, 10, 154)),
          (512, (1, 32, 64)), (513, (1, 54, 38)), (768, (1, 32, 96)), (769, (1, 2, 1538)),
          (1024, (1, 64, 64)), (1025, (1, 50, 82)), (1280, (1, 64, 80)), (1281, (1, 42, 122))]


@pytest.mark.parametrize("mode,val", [("topk", 0.3), ("topp", 0.5)])
@pytest.mark.parametrize("nb,grid", WIDTHS, ids=[f"nb{n}" for n, _ in WIDTHS])
def test_register_chunk_widths(vsa, nb, grid, mode, val):
    w = W.custom(f"cw{nb}", 1, 2, 64, grid, (1, 2, 2), "bf16", 0.5, -1, "smooth")
    _say(f"[gpu] select chunk widths NB={nb}: {mode} {val} grid={grid}")
    inp = W.generate(w, seed=12)
    _, idx, g, S = _plan_both(vsa, w, inp, mode, [val], -1, 1, None)
    assert g.NB == nb
    grp, gci = _index_np(idx)
    (rows, band, _), _ = check_index(grp, gci, S, g, mode, [val], -1, 1, _scale(w, None))
    _say(f"[gpu]   ok rows={rows} band={band} nnz={idx.nnz()}")


def test_topp_uniform_ties(vsa):
    """Q == 0 makes every score 0: Top-P keeps ceil(p * NB) blocks, the
    lowest ids (p * NB = 4.8 here, far from an integer)."""
    w = W.custom("ties", 1, 2, 128, (8, 8, 16), (2, 4, 8), "bf16", 0.5, -1, "smooth")
    _say("[gpu] select ties")
    inp = W.generate(w, seed=4)
    q = torch.zeros((1, 2, w.N, 128), dtype=torch.bfloat16, device="cuda")
    k = _to_dev(inp["k"], torch.bfloat16)
    idx = vsa.plan_select(q, k, w.grid, w.block, "topp", 0.3)
    torch.cuda.synchronize()
    g = O.geometry(w.grid, w.block)
    assert g.NB == 16
    rp, ci = _index_np(idx)
    assert np.array_equal(ci.reshape(-1, 5), np.tile(np.arange(5), (2 * g.NB, 1)))


def test_topk_mode_equals_plan(vsa):
    w = W.custom("eq", 1, 3, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, 1, "smooth")
    _say("[gpu] select topk == plan")
    inp = W.generate(w, seed=8)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    a = vsa.plan_select(q, k, w.grid, w.block, "topk", [0.3, 0.1, 0.6], 1, 0)
    b = vsa.plan(q, k, w.grid, w.block, [0.3, 0.1, 0.6], 1)
    torch.cuda.synchronize()
    assert torch.equal(a.row_ptr, b.row_ptr)
    assert torch.equal(a.col_idx[: a.nnz()], b.col_idx[: b.nnz()])


def test_topp_repeatable(vsa):
    w = W.custom("rep", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, 1, "smooth")
    _say("[gpu] select repeatable")
    inp = W.generate(w, seed=9)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    a = vsa.plan_select(q, k, w.grid, w.block, "topp", [0.7, 0.4], 1, 2)
    b = vsa.plan_select(q, k, w.grid, w.block, "topp", [0.7, 0.4], 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(a.row_ptr, b.row_ptr)
    assert torch.equal(a.col_idx[: a.nnz()], b.col_idx[: b.nnz()])


@functools.lru_cache(maxsize=1)
def _full_inputs(name):
    return W.generate(W.WORKLOADS[name])


FULL = [("wan13b", "topp", 0.25, -1, 2, None), ("wan13b", "topp", 0.9, -1, 0, 1.0),
        ("wan13b", "topk", 0.2, -1, 4, None), ("long4x", "topp", 0.1, 1, 2, None)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", FULL, ids=[f"{c[0]}_{c[1]}_{c[2]}_s{c[4]}" for c in FULL])
def test_full_select(vsa, case):
    name, mode, val, window_t, sink, scale = case
    w = W.WORKLOADS[name]
    _say(f"[gpu] full select {name} {mode} {val} window={window_t} sink={sink} scale={scale}: generating")
    inp = _full_inputs(name)
    _say(f"[gpu] full select {name}: GPU plan + oracle scores")
    (q, k, v), idx, g, S = _plan_both(vsa, w, inp, mode, [val], window_t, sink, scale)
    grp, gci = _index_np(idx)
    _say(f"[gpu] full select {name}: checking {len(grp) - 1} rows")
    (rows, band, differ), _ = check_index(grp, gci, S, g, mode, [val], window_t, sink, _scale(w, scale))
    assert idx.nnz() <= idx.capacity
    # Outputs: every row inside the float32 band and a seeded sample of 32
    # others, each against the oracle's attention over the GPU's own
    # (validated) row.
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    rng = np.random.default_rng(3)
    check = sorted({int(r) for r in differ} | {int(r) for r in rng.integers(0, rows, 32)})
    errs = []
    for r in check:
        b, rem = divmod(r, w.heads * g.NB)
        h, i = divmod(rem, g.NB)
        want = O.attention_row(inp["q"], inp["k"], inp["v"], g, grp, gci, b, h, i)
        errs.append(np.abs(og[b, h, g.tokens[i]] - want).ravel())
    err = np.concatenate(errs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    _say(f"[gpu]   ok rows={rows} band={band} nnz={idx.nnz()} density={idx.nnz() / (rows * g.NB):.3f} "
         f"outputs checked on {len(check)} rows, max-abs {err.max():.2e}")
