"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: block indices, centroids and centroid scores bit-exact; bf16 outputs
within max-abs 2e-2 and mean-abs 2e-3 of the float64 oracle; float32
outputs within max-abs 1e-4.  Small cases compare every output element;
the full-size workloads compare the whole index, and the outputs of every
query block (tiny, Wan2.1-1.3B and HunyuanVideo shapes) or of a stratified
sample of at least a tenth of them that covers every head, block-size
class and stretch of block ids (Wan2.1-14B mixed and long-video shapes).
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import vsa_oracle as O

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
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=dtype).contiguous()


def _tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _run(vsa, w, inp):
    dt = _tdtype(w)
    q, k, v = (_to_dev(inp[n], dt) for n in ("q", "k", "v"))
    dens = [float(d) for d in inp["density"]]
    idx = vsa.plan(q, k, w.grid, w.block, dens, w.window_t)
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    return q, k, v, idx, o


def _index_np(idx):
    rp = idx.row_ptr.cpu().numpy()
    return rp, idx.col_idx.cpu().numpy()[: int(rp[-1])]


def _check_out(w, got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX, f"max-abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN, f"mean-abs {err.mean():.3e}"
    else:
        assert err.max() <= F32_MAX, f"max-abs {err.max():.3e}"
    return float(err.max()), float(err.mean())


SMALL = [
    W.custom("s_tiny_fp32", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
    W.custom("s_tiny_fp32_dense", 1, 2, 64, (4, 8, 8), (2, 4, 8), "f32", 1.0, -1, "iid"),
    W.custom("s_ragged_fp32_d128", 1, 2, 128, (3, 5, 7), (2, 2, 4), "f32", 0.4, -1, "iid"),
    W.custom("s_ragged_bf16", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.25, -1, "smooth"),
    W.custom("s_hy_bf16_d64", 1, 3, 64, (5, 9, 11), (1, 8, 16), "bf16", 0.3, -1, "smooth"),
    W.custom("s_window_bf16", 1, 2, 128, (12, 8, 8), (4, 4, 8), "bf16", 0.1, 1, "smooth"),
    W.custom("s_window0_bf16", 1, 1, 128, (10, 9, 9), (2, 4, 4), "bf16", 0.05, 0, "smooth"),
    W.custom("s_batch2_bf16", 2, 3, 128, (6, 8, 16), (2, 4, 8), "bf16", None, -1, "smooth"),
    W.custom("s_single_block", 1, 2, 128, (2, 3, 5), (4, 4, 8), "bf16", 1.0, -1, "smooth"),
    W.custom("s_token_blocks", 1, 1, 128, (4, 4, 4), (1, 1, 1), "bf16", 0.25, -1, "smooth"),
    W.custom("s_dense_bf16", 1, 2, 128, (4, 8, 16), (2, 4, 8), "bf16", 1.0, -1, "smooth"),
    # batch 2 with query blocks of 128, 64, 32 and 16 tokens (the key split covers the short ones)
    W.custom("s_batch2_short_bf16", 2, 2, 128, (9, 10, 12), (4, 4, 8), "bf16", 0.4, -1, "smooth"),
    W.custom("s_batch2_short_d64", 2, 3, 64, (5, 6, 20), (2, 4, 8), "bf16", 0.5, 0, "smooth"),
]


def _gen_small(w):
    inp = W.generate(w, seed=3)
    if w.density is None:   # per-head mix including dense and very sparse heads
        inp["density"] = np.array([1.0, 0.3, 0.05][: w.heads], dtype=np.float32)
    return inp


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_full_parity(vsa, w):
    _say(f"[gpu] small parity {w.name} grid={w.grid} block={w.block} D={w.D} {w.dtype}")
    inp = _gen_small(w)
    q, k, v, idx, o = _run(vsa, w, inp)
    rp, ci, info = O.plan(inp["q"], inp["k"], w.grid, w.block, inp["density"], w.window_t)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    # summarizer and inter-estimator alone, bit for bit
    qc = vsa.centroids(q, w.grid, w.block)
    kc = vsa.centroids(k, w.grid, w.block)
    S = vsa.centroid_scores(qc, kc, w.grid, w.block)
    torch.cuda.synchronize()
    assert np.array_equal(qc.cpu().numpy().view(np.uint32), info["qc"].view(np.uint32))
    assert np.array_equal(kc.cpu().numpy().view(np.uint32), info["kc"].view(np.uint32))
    assert np.array_equal(S.cpu().numpy(), info["S"])
    ref = O.attention(inp["q"], inp["k"], inp["v"], w.grid, w.block, rp, ci)
    mx, mean = _check_out(w, o.float().cpu().numpy(), ref)
    _say(f"[gpu]   ok max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("grid,block", [((9, 14, 20), (4, 4, 8)), ((5, 9, 11), (1, 8, 16)),
                                        ((3, 3, 3), (2, 2, 2))])
def test_permute_unpermute(vsa, grid, block, dtype):
    _say(f"[gpu] permute {grid} {block} {dtype}")
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 2, math.prod(grid), 64)).astype(np.float32)
    xd = _to_dev(x, dtype)
    xb = vsa.permute(xd, grid, block)
    back = vsa.unpermute(xb, grid, block)
    torch.cuda.synchronize()
    g = O.geometry(grid, block)
    ref = O.permute(xd.cpu().float().numpy(), g, pad_to=block[0] * block[1] * block[2])
    assert np.array_equal(xb.cpu().float().numpy(), ref)
    assert torch.equal(back, xd)


def test_ties_and_constant_v(vsa):
    """Q == 0 gives all-equal scores (the lowest ids win); V == 1 gives O == 1."""
    w = W.custom("ties", 1, 2, 128, (8, 8, 16), (2, 4, 8), "bf16", 0.25, -1, "smooth")
    _say("[gpu] ties / constant V")
    inp = W.generate(w, seed=4)
    q = torch.zeros((1, 2, w.N, 128), dtype=torch.bfloat16, device="cuda")
    k = _to_dev(inp["k"], torch.bfloat16)
    v = torch.ones_like(q)
    idx = vsa.plan(q, k, w.grid, w.block, 0.25)
    o = vsa.attn(_to_dev(inp["q"], torch.bfloat16), k, v, idx)
    torch.cuda.synchronize()
    g = O.geometry(w.grid, w.block)
    kk = O.k_rule(0.25, g.NB)
    rp, ci = _index_np(idx)
    assert np.array_equal(ci.reshape(-1, kk), np.tile(np.arange(kk), (2 * g.NB, 1)))
    assert torch.all(o == 1)


def test_run_twice_bitwise(vsa):
    w = W.custom("det", 1, 2, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, 1, "smooth")
    _say("[gpu] determinism")
    inp = W.generate(w, seed=5)
    _, _, _, idx1, o1 = _run(vsa, w, inp)
    _, _, _, idx2, o2 = _run(vsa, w, inp)
    assert torch.equal(idx1.row_ptr, idx2.row_ptr)
    assert torch.equal(idx1.col_idx[: idx1.nnz()], idx2.col_idx[: idx2.nnz()])
    assert torch.equal(o1, o2)


def test_side_stream_matches_current_stream(vsa):
    """The calls enqueue on the caller's current stream: planning and
    attention issued on a second stream (default priority), after it waits
    for the inputs, give the same index and output bit for bit."""
    w = W.custom("strm", 1, 3, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.25, 1, "smooth")
    _say("[gpu] side stream")
    inp = W.generate(w, seed=15)
    q, k, v, idx1, o1 = _run(vsa, w, inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        idx2 = vsa.plan(q, k, w.grid, w.block, [float(d) for d in inp["density"]], w.window_t)
        o2 = vsa.attn(q, k, v, idx2)
    side.synchronize()
    assert torch.equal(idx1.row_ptr, idx2.row_ptr)
    assert torch.equal(idx1.col_idx[: idx1.nnz()], idx2.col_idx[: idx2.nnz()])
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------- full size

FULL = ["tiny_fp32", "tiny_fp32_dense", "wan13b", "hunyuan", "wan14b_mixed", "long4x"]


# Every query block of these is compared; the others are sampled.
COMPARE_ALL = {"tiny_fp32", "tiny_fp32_dense", "wan13b", "hunyuan"}


def _stratified_rows(g, heads, B, frac=0.1, seed=0):
    """At least `frac` of the query blocks of every (batch, head) and every
    block-size class: each class's blocks, in id order, are cut into runs
    of round(1/frac) and one block of every run (at a seeded offset) is
    taken, so every contiguous stretch of block ids -- the slices the
    attention kernel deals to one XCD -- holds sampled rows."""
    rng = np.random.default_rng(seed)
    step = max(1, int(round(1.0 / frac)))
    rows = []
    for b in range(B):
        for h in range(heads):
            for size in np.unique(g.sizes):
                ids = np.nonzero(g.sizes == size)[0]
                for start in range(0, len(ids), step):
                    run = ids[start:start + step]
                    rows.append((b, h, int(run[int(rng.integers(0, len(run)))])))
    return rows


def _oracle_rows(inp, g, rp, ci, rows, say=None):
    """Oracle float64 attention of the given query blocks, computed on a
    thread pool (NumPy releases the GIL in its kernels); BLAS runs one
    thread per task."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    out = [None] * len(rows)

    def one(n):
        b, h, i = rows[n]
        out[n] = O.attention_row(inp["q"], inp["k"], inp["v"], g, rp, ci, b, h, i)

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(workers) as ex:
            for n, _ in enumerate(ex.map(one, range(len(rows)))):
                if say is not None and n % 2000 == 1999:
                    say(f"[gpu]   oracle rows {n + 1}/{len(rows)}")
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_workload(vsa, name):
    w = W.WORKLOADS[name]
    _say(f"[gpu] full workload {name}: generating")
    inp = W.generate(w)
    _say(f"[gpu] full workload {name}: GPU plan+attn")
    q, k, v, idx, o = _run(vsa, w, inp)
    grp, gci = _index_np(idx)
    _say(f"[gpu] full workload {name}: oracle plan")
    rp, ci, info = O.plan(inp["q"], inp["k"], w.grid, w.block, inp["density"], w.window_t)
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    g = info["geometry"]
    if name in COMPARE_ALL:
        rows = [(b, h, i) for b in range(w.B) for h in range(w.heads) for i in range(g.NB)]
    else:
        rows = _stratified_rows(g, w.heads, w.B)
        assert len(rows) >= 0.1 * w.B * w.heads * g.NB
    _say(f"[gpu] full workload {name}: oracle attention on {len(rows)} of "
         f"{w.B * w.heads * g.NB} query blocks")
    og = o.float().cpu().numpy()
    refs = _oracle_rows(inp, g, rp, ci, rows, _say)
    err = np.concatenate([np.abs(og[b, h, g.tokens[i]] - ref).ravel() for (b, h, i), ref in zip(rows, refs)])
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    else:
        assert err.max() <= F32_MAX, err.max()
    assert np.all(np.isfinite(og))
    if name in COMPARE_ALL:
        # every raster token was written (no query block was skipped)
        assert sum(len(g.tokens[i]) for i in range(g.NB)) == og.shape[2]
    _say(f"[gpu]   ok nnz={len(ci)} rows={len(rows)} max-abs {err.max():.2e} mean-abs {err.mean():.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_hand_built_index_with_empty_rows(vsa, dtype):
    """An index built by hand may leave rows empty (the planners never do):
    those query tokens come out as zeros, on full rows and on the short rows
    whose waves split the key tiles; every other row matches the oracle."""
    w = W.custom("empty_rows", 1, 2, 128 if dtype == torch.bfloat16 else 64, (9, 10, 12), (4, 4, 8),
                 "bf16" if dtype == torch.bfloat16 else "f32", 0.4, -1, "smooth")
    _say(f"[gpu] hand-built index with empty rows, {dtype}")
    inp = W.generate(w, seed=61)
    g = O.geometry(w.grid, w.block)
    rp, ci, _ = O.plan(inp["q"], inp["k"], w.grid, w.block, 0.4, -1)
    rows = len(rp) - 1
    empty = {r for r in range(rows) if r % 3 == 1}
    lens = [0 if r in empty else rp[r + 1] - rp[r] for r in range(rows)]
    nrp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nci = np.concatenate([ci[rp[r]:rp[r + 1]] for r in range(rows) if r not in empty]).astype(np.int32)
    q, k, v = (_to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    idx = vsa.plan(q, k, w.grid, w.block, 0.4)
    hand = vsa.Index(idx.shape, idx.nb, -1, torch.from_numpy(nrp).cuda(), torch.from_numpy(nci).cuda(), len(nci), 0)
    o = vsa.attn(q, k, v, hand).float().cpu().numpy()
    torch.cuda.synchronize()
    ref = O.attention(inp["q"], inp["k"], inp["v"], w.grid, w.block, rp, ci)
    tol = BF16_MAX if dtype == torch.bfloat16 else F32_MAX
    for r in range(rows):
        h, i = divmod(r, g.NB)
        got = o[0, h, g.tokens[i]]
        if r in empty:
            assert np.all(got == 0.0), (r, g.sizes[i])
        else:
            assert np.abs(got - ref[0, h, g.tokens[i]]).max() <= tol, (r, g.sizes[i])
