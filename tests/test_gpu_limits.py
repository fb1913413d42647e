"""GPU parity at the size limits of the planning path, through the C ABI:
the largest head count (per-head keep rates, windows and options fill the
whole per-head argument table) and the largest block count (one score row
per workgroup, 64 KiB of keys in LDS), the latter checked on sampled rows
that the oracle scores one by one."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import mixed_oracle as M
from oracle import select_oracle as P
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu


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


def _index_np(idx):
    rp = idx.row_ptr.cpu().numpy()
    return rp, idx.col_idx.cpu().numpy()[: int(rp[-1])]


def test_max_heads_per_head_options(vsa):
    """256 heads, each with its own keep rate (and, in the mixed plan, its
    own option and window): every entry of the per-head tables is used."""
    w = W.custom("h256", 1, 256, 64, (4, 4, 8), (2, 2, 4), "bf16", 0.5, -1, "iid")
    _say("[gpu] 256 heads")
    inp = W.generate(w, seed=51)
    rng = np.random.default_rng(52)
    dens = rng.choice([1.0, 0.3, 0.2, 0.1, 0.05], size=256).astype(np.float32)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    idx = vsa.plan(q, k, w.grid, w.block, dens.tolist())
    torch.cuda.synchronize()
    rp, ci, _ = O.plan(inp["q"], inp["k"], w.grid, w.block, dens, -1)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    g = O.geometry(w.grid, w.block)
    kinds = ["dynamic", "static", "dense"]
    options = [{"kind": kinds[h % 3], "value": float(dens[h]), "window_t": int(h % 4) - 1} for h in range(256)]
    table = rng.standard_normal((256, g.NB, g.NB)).astype(np.float32)
    idx = vsa.plan_mixed(q, k, w.grid, w.block, options, _to_dev(table, torch.float32))
    torch.cuda.synchronize()
    rp, ci, _ = M.plan_mixed(inp["q"], inp["k"], w.grid, w.block, options, table)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    assert idx.equal_heads == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode,value", [("topk", 0.01), ("topp", 0.3)])
def test_max_blocks_sampled_rows(vsa, mode, value):
    """16384 one-token blocks (the largest block count): the GPU index of
    sampled rows equals the oracle's, each row scored on its own."""
    w = W.custom("nb16k", 1, 1, 64, (16, 32, 32), (1, 1, 1), "bf16", 0.5, -1, "smooth")
    _say(f"[gpu] 16384 blocks, {mode} {value}")
    inp = W.generate(w, seed=53)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    idx = vsa.plan_select(q, k, w.grid, w.block, mode, value)
    torch.cuda.synchronize()
    grp, gci = _index_np(idx)
    g = O.geometry(w.grid, w.block)
    assert g.NB == 16384 and len(grp) == g.NB + 1
    qc = O.centroids(inp["q"], g)[0, 0]
    kc = O.centroids(inp["k"], g)[0, 0]
    rows = sorted(set(np.random.default_rng(54).integers(0, g.NB, 24).tolist()) | {0, g.NB - 1})
    scale = 1.0 / np.sqrt(64)
    S = O.scores(qc[rows][None, None], kc[None, None])[0, 0]        # [len(rows), NB]
    tol = 6.0 * g.NB * 2.0 ** -24
    for n, i in enumerate(rows):
        got = gci[grp[i]:grp[i + 1]]
        if mode == "topk":
            want = O.topk_row(S[n], O.k_rule(value, g.NB))
            assert np.array_equal(got, want), i
        else:
            order, F = P.prefix_mass(S[n], scale)
            c = len(got)
            assert np.array_equal(got, np.sort(order[:c])), i
            assert (c == 1 or F[c - 2] < value + tol) and F[c - 1] >= value - tol, (i, c)


@pytest.mark.parametrize("window_t", [32767, 32768, 70000])
def test_window_radius_past_the_grid(vsa, window_t):
    """A window radius at or beyond nbt - 1 keeps every temporal block: the
    plan must equal the oracle's plan at that radius (every row holds every
    key block) and record nbt - 1 in the index; a radius that does not fit
    16 bits must not reach the selection kernel in a narrowed form."""
    w = W.custom("bigwin", 1, 2, 64, (9, 10, 12), (4, 4, 8), "bf16", 0.2, -1, "smooth")
    _say(f"[gpu] window radius {window_t}")
    inp = W.generate(w, seed=71)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    g = O.geometry(w.grid, w.block)
    idx = vsa.plan(q, k, w.grid, w.block, 0.2, window_t)
    torch.cuda.synchronize()
    rp, ci, _ = O.plan(inp["q"], inp["k"], w.grid, w.block, np.float32(0.2), window_t)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    assert np.all(np.diff(grp) == g.NB)
    assert idx.window_t == g.nbt - 1
