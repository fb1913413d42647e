"""Seeded random configurations through the C ABI against the CPU oracle:
selection plans (plan_select), mixed per-head plans (plan_mixed) and
head-wise blocking-scheme selection (select_scheme).

Each case draws a grid, a block (at most 128 tokens, often not dividing the
grid), d, dtype, heads, batch, selection mode, estimator, window, sink
length (at most NB), per-head values, an optional Top-P scale and an input
generator, from its own seed.  The index must equal the oracle's (Top-P
rows within the float32 band of select_check), and every output row must
be within the bf16 / fp32 bar.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dsa_oracle as E
from oracle import mixed_oracle as M
from oracle import sics_oracle as SC
from oracle import vsa_oracle as O
from select_check import check_index

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4
N_CASES = 32


def _case(seed):
    rng = np.random.default_rng(seed)
    while True:
        block = tuple(int(x) for x in rng.integers(1, 9, size=3))
        if math.prod(block) <= 128:
            break
    while True:
        grid = tuple(int(x) for x in (rng.integers(1, 9), rng.integers(1, 25), rng.integers(1, 33)))
        if math.prod(grid) <= 2000:
            break
    nb = math.prod(-(-g // b) for g, b in zip(grid, block))
    heads = int(rng.integers(1, 4))
    return dict(
        grid=grid, block=block, D=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
        heads=heads, B=int(rng.integers(1, 3)), mode=str(rng.choice(["topk", "topp"])),
        est=str(rng.choice(["mean", "dsa", "dsa2"])), window=int(rng.choice([-1, -1, 0, 1, 2])),
        sink=min(int(rng.choice([0, 0, 1, 3])), nb),
        vals=[float(np.float32(rng.uniform(0.02, 1.0))) for _ in range(heads)],
        scale=None if rng.random() < 0.7 else float(np.float32(rng.uniform(0.1, 4.0))),
        gen=str(rng.choice(["smooth", "iid"])))


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import block_sparse_attention_centroids_amd as pkg
    pkg.load()
    return pkg


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(vsa, seed):
    c = _case(7000 + seed)
    print(f"[gpu] random case {seed}: {c}", flush=True)
    sys.stdout.flush()
    w = W.custom(f"r{seed}", c["B"], c["heads"], c["D"], c["grid"], c["block"], c["dtype"], 0.5,
                 c["window"], c["gen"])
    inp = W.generate(w, seed=9000 + seed)
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[n])).to(device="cuda", dtype=dt).contiguous()
               for n in ("q", "k", "v"))
    idx = vsa.plan_select(q, k, c["grid"], c["block"], c["mode"], c["vals"], c["window"], c["sink"],
                          c["scale"], c["est"])
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    g = O.geometry(c["grid"], c["block"])
    S = E.estimate(inp["q"], inp["k"], g, c["est"])
    rp = idx.row_ptr.cpu().numpy()
    ci = idx.col_idx.cpu().numpy()[: int(rp[-1])]
    scale = 1.0 / math.sqrt(c["D"]) if c["scale"] is None else c["scale"]
    check_index(rp, ci, S, g, c["mode"], c["vals"], c["window"], c["sink"], scale)
    ref = O.attention(inp["q"], inp["k"], inp["v"], c["grid"], c["block"], rp, ci)
    err = np.abs(o.float().cpu().numpy().astype(np.float64) - ref)
    if c["dtype"] == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    else:
        assert err.max() <= F32_MAX, err.max()


N_MIXED = 16


def _mixed_case(seed):
    rng = np.random.default_rng(seed)
    while True:
        block = tuple(int(x) for x in rng.integers(1, 9, size=3))
        if math.prod(block) <= 128:
            break
    while True:
        grid = tuple(int(x) for x in (rng.integers(1, 9), rng.integers(1, 25), rng.integers(1, 33)))
        if math.prod(grid) <= 2000:
            break
    heads = int(rng.integers(1, 5))
    options = []
    for _ in range(heads):
        kind = str(rng.choice(["dynamic", "static", "dense"]))
        o = {"kind": kind}
        if kind != "dense":
            o["value"] = float(np.float32(rng.uniform(0.02, 1.0)))
        wt = int(rng.choice([-1, -1, 0, 1]))
        if wt >= 0:
            o["window_t"] = wt
        options.append(o)
    return dict(grid=grid, block=block, D=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                heads=heads, B=int(rng.integers(1, 3)), est=str(rng.choice(["mean", "dsa", "dsa2"])),
                options=options, gen=str(rng.choice(["smooth", "iid"])), table_seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("seed", range(N_MIXED))
def test_random_mixed_plan(vsa, seed):
    c = _mixed_case(8000 + seed)
    print(f"[gpu] random mixed case {seed}: {c}", flush=True)
    sys.stdout.flush()
    w = W.custom(f"rm{seed}", c["B"], c["heads"], c["D"], c["grid"], c["block"], c["dtype"], 0.5, -1, c["gen"])
    g = O.geometry(c["grid"], c["block"])
    inp = W.generate(w, seed=9500 + seed)
    trng = np.random.default_rng(c["table_seed"])
    table = (np.round(trng.standard_normal((c["heads"], g.NB, g.NB)) * 8) / 8).astype(np.float32)   # ties
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[n])).to(device="cuda", dtype=dt).contiguous()
               for n in ("q", "k", "v"))
    idx = vsa.plan_mixed(q, k, c["grid"], c["block"], c["options"], torch.from_numpy(table).cuda(), c["est"])
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    rp, ci, _ = M.plan_mixed(inp["q"], inp["k"], c["grid"], c["block"], c["options"], table, c["est"])
    grp = idx.row_ptr.cpu().numpy()
    gci = idx.col_idx.cpu().numpy()[: int(grp[-1])]
    assert np.array_equal(grp, rp), "row_ptr differs"
    assert np.array_equal(gci, ci), "col_idx differs"
    ref = O.attention(inp["q"], inp["k"], inp["v"], c["grid"], c["block"], rp, ci)
    err = np.abs(o.float().cpu().numpy().astype(np.float64) - ref)
    if c["dtype"] == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    else:
        assert err.max() <= F32_MAX, err.max()


N_SCHEME = 8
SCHEME_RTOL, SCHEME_ATOL = 1e-4, 1e-3   # the scheme tests' bar: float32 sums of unit vectors


@pytest.mark.parametrize("seed", range(N_SCHEME))
def test_random_scheme_selection(vsa, seed):
    rng = np.random.default_rng(8500 + seed)
    while True:
        grid = tuple(int(x) for x in (rng.integers(1, 9), rng.integers(1, 25), rng.integers(1, 33)))
        if math.prod(grid) <= 2000:
            break
    cands = []
    while len(cands) < int(rng.integers(1, 6)):
        b = tuple(int(x) for x in rng.integers(1, 9, size=3))
        if math.prod(b) <= 128 and b not in cands:
            cands.append(b)
    D, dtype = int(rng.choice([64, 128])), str(rng.choice(["bf16", "f32"]))
    heads, B = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    print(f"[gpu] random scheme case {seed}: grid={grid} D={D} {dtype} heads={heads} B={B} cands={cands}",
          flush=True)
    sys.stdout.flush()
    w = W.custom(f"rs{seed}", B, heads, D, grid, cands[0], dtype, 0.5, -1, str(rng.choice(["smooth", "iid"])))
    inp = W.generate(w, seed=9700 + seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k = (torch.from_numpy(np.ascontiguousarray(inp[n])).to(device="cuda", dtype=dt).contiguous()
            for n in ("q", "k"))
    scores, choice = vsa.select_scheme(q, k, grid, cands)
    torch.cuda.synchronize()
    ref = SC.scheme_scores(inp["q"], inp["k"], grid, cands).reshape(len(cands), B * heads)
    got = scores.cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=SCHEME_RTOL, atol=SCHEME_ATOL)
    best = ref.max(axis=0)
    for bh, c in enumerate(choice.cpu().numpy().tolist()):
        assert 0 <= c < len(cands)
        assert ref[c, bh] >= best[bh] - SCHEME_RTOL * abs(best[bh]) - SCHEME_ATOL, (bh, c, ref[:, bh])
