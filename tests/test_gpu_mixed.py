"""GPU parity of mixed per-head plans (dense, static and dynamic heads with
per-head windows) through the C ABI, against the CPU oracle.

Bar: indices bit-exact (every head selects by Top-K on float32 scores that
both sides compute, or read, identically); attention over the index within
the bf16 / fp32 bar.  A plan of static and dense heads is built once without
Q/K and reused for attention calls on different inputs.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import mixed_oracle as M
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
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype).contiguous()


def _index_np(idx):
    rp = idx.row_ptr.cpu().numpy()
    return rp, idx.col_idx.cpu().numpy()[: int(rp[-1])]


def _table(heads, NB, seed):
    """Seeded static ranking (stands in for an offline block ranking): a
    smooth preference for near blocks plus noise, with some exact ties."""
    rng = np.random.default_rng(seed)
    i = np.arange(NB)
    near = -np.abs(i[:, None] - i[None, :]).astype(np.float64) / NB
    t = near[None] + 0.3 * rng.standard_normal((heads, NB, NB))
    t = np.round(t * 64) / 64                                  # ties
    return t.astype(np.float32)


def _check_attention(w, inp, o, rp, ci):
    ref = O.attention(inp["q"], inp["k"], inp["v"], w.grid, w.block, rp, ci)
    err = np.abs(o.float().cpu().numpy() - ref)
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    else:
        assert err.max() <= F32_MAX, err.max()
    return float(err.max())


CASES = [
    ("mix_bf16", W.custom("m1", 1, 4, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.5, -1, "smooth"),
     [{"kind": "dynamic", "value": 0.2, "window_t": 1}, {"kind": "static", "value": 0.3},
      {"kind": "dense"}, {"kind": "dynamic", "value": 0.5}], "mean"),
    ("mix_f32_batch2", W.custom("m2", 2, 3, 64, (4, 8, 8), (2, 4, 8), "f32", 0.5, -1, "iid"),
     [{"kind": "static", "value": 0.5, "window_t": 0}, {"kind": "dynamic", "value": 0.25},
      {"kind": "dense", "window_t": 1}], "mean"),
    ("mix_dsa_no_window", W.custom("m3", 1, 3, 64, (5, 9, 11), (1, 8, 16), "bf16", 0.5, -1, "smooth"),
     [{"kind": "dynamic", "value": 0.3}, {"kind": "static", "value": 0.1}, {"kind": "dynamic", "value": 0.6}],
     "dsa"),
    ("mix_lds_rows", W.custom("m4", 1, 2, 64, (8, 32, 40), (1, 2, 2), "bf16", 0.5, -1, "smooth"),
     [{"kind": "static", "value": 0.02, "window_t": 0}, {"kind": "dynamic", "value": 0.05}], "dsa2"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mixed_plan_parity(vsa, case):
    name, w, options, est = case
    _say(f"[gpu] mixed {name}: {options} estimator={est} grid={w.grid} block={w.block} {w.dtype}")
    inp = W.generate(w, seed=21)
    g = O.geometry(w.grid, w.block)
    table = _table(w.heads, g.NB, seed=22)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (_to_dev(inp[n], dt) for n in ("q", "k", "v"))
    idx = vsa.plan_mixed(q, k, w.grid, w.block, options, _to_dev(table, torch.float32), est)
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    rp, ci, _ = M.plan_mixed(inp["q"], inp["k"], w.grid, w.block, options, table, est)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    assert idx.window_t == max(o.get("window_t", -1) for o in options)
    if g.NB <= 64:
        mx = _check_attention(w, inp, o, rp, ci)
        _say(f"[gpu]   ok nnz={len(ci)} max-abs {mx:.2e}")
    else:
        _say(f"[gpu]   ok nnz={len(ci)}")


def test_static_plan_built_once_and_reused(vsa):
    """Static and dense heads only: the plan needs no Q/K; one index serves
    attention calls on two different inputs."""
    w = W.custom("st", 1, 3, 128, (6, 8, 16), (2, 4, 8), "bf16", 0.5, -1, "smooth")
    g = O.geometry(w.grid, w.block)
    options = [{"kind": "static", "value": 0.25, "window_t": 0}, {"kind": "dense"},
               {"kind": "static", "value": 0.5}]
    table = _table(3, g.NB, seed=23)
    _say("[gpu] static plan, built once")
    idx = vsa.plan_mixed(None, None, w.grid, w.block, options, _to_dev(table, torch.float32), B=1, D=128,
                         dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    rp, ci, _ = M.plan_mixed(None, None, w.grid, w.block, options, table, B=1)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    for seed in (31, 32):
        inp = W.generate(w, seed=seed)
        q, k, v = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
        o = vsa.attn(q, k, v, idx)
        torch.cuda.synchronize()
        mx = _check_attention(w, inp, o, rp, ci)
        _say(f"[gpu]   reuse seed {seed}: max-abs {mx:.2e}")


@pytest.mark.timeout(900)
def test_full_wan_mixed_heads(vsa):
    """The Wan2.1-1.3B shape with a mix of every option across its 12 heads."""
    w = W.WORKLOADS["wan13b"]
    g = O.geometry(w.grid, w.block)
    pattern = [{"kind": "dense"}, {"kind": "static", "value": 0.2}, {"kind": "dynamic", "value": 0.2, "window_t": 1},
               {"kind": "dynamic", "value": 0.1}, {"kind": "static", "value": 0.05, "window_t": 0},
               {"kind": "dynamic", "value": 0.3}]
    options = (pattern * 2)[: w.heads]
    _say("[gpu] full mixed wan13b: generating")
    inp = W.generate(w)
    table = _table(w.heads, g.NB, seed=24)
    q, k = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k"))
    idx = vsa.plan_mixed(q, k, w.grid, w.block, options, _to_dev(table, torch.float32))
    torch.cuda.synchronize()
    _say("[gpu] full mixed wan13b: oracle plan")
    rp, ci, _ = M.plan_mixed(inp["q"], inp["k"], w.grid, w.block, options, table)
    grp, gci = _index_np(idx)
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    _say(f"[gpu]   ok nnz={len(ci)} density={len(ci) / ((len(rp) - 1) * g.NB):.3f}")


def test_schedule_hint_does_not_change_results(vsa):
    """The equal-heads hint only changes which XCD runs a row: attention is
    bit-identical with either value, on an index of equal and of unequal
    heads."""
    import dataclasses
    w = W.custom("hint", 1, 4, 128, (9, 14, 20), (4, 4, 8), "bf16", 0.3, -1, "smooth")
    inp = W.generate(w, seed=41)
    q, k, v = (_to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    for dens in (0.3, [1.0, 0.3, 0.05, 0.2]):
        idx = vsa.plan(q, k, w.grid, w.block, dens)
        assert idx.equal_heads == (1 if isinstance(dens, float) else 0)
        flipped = dataclasses.replace(idx, equal_heads=1 - idx.equal_heads)
        o1 = vsa.attn(q, k, v, idx)
        o2 = vsa.attn(q, k, v, flipped)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
