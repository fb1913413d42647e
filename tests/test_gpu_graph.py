"""The plan and the attention captured in a HIP graph.

Every entry point only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronization), and vsa_plan_noalloc takes
its workspace from the library's static array, so vsa_plan_noalloc +
vsa_attn into preallocated index and output buffers can be captured with
torch.cuda.graph and replayed.  Each replay follows eager work of the
program (an unrelated plan and attention) and a synchronization; before it,
new Q, K and V are copied into the captured buffers and the index and
output are poisoned.  Every replay must equal the eager calls on the same
data bit for bit (the same kernels on the same inputs).
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

GRID, BLOCK, DENSITY, WINDOW = (9, 14, 20), (4, 4, 8), 0.25, 1


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


def _eager(vsa, inp):
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    idx = vsa.plan_noalloc(q, k, GRID, BLOCK, DENSITY, WINDOW)
    o = vsa.attn(q, k, v, idx)
    torch.cuda.synchronize()
    nnz = idx.nnz()
    return idx.row_ptr.clone(), idx.col_idx[:nnz].clone(), o.clone()


def test_graph_replays_match_eager(vsa):
    w = W.custom("graph", 1, 2, 128, GRID, BLOCK, "bf16", DENSITY, WINDOW, "smooth")
    inputs = [W.generate(w, seed=s) for s in (31, 32, 33)]
    refs = [_eager(vsa, inp) for inp in inputs]
    _say(f"[gpu] graph: eager references nnz={[int(r[0][-1]) for r in refs]}")

    q, k, v = (_dev(inputs[0][n]) for n in ("q", "k", "v"))
    idx = vsa.plan_noalloc(q, k, GRID, BLOCK, DENSITY, WINDOW)
    o = torch.empty_like(q)
    vsa.attn(q, k, v, idx, out=o)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vsa.plan_noalloc(q, k, GRID, BLOCK, DENSITY, WINDOW, index=idx)
        vsa.attn(q, k, v, idx, out=o)
    torch.cuda.synchronize()
    _say("[gpu] graph: captured")

    for rep in range(6):
        which = rep % 3
        _eager(vsa, inputs[(rep + 1) % 3])                 # the program's own eager work
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            t.copy_(_dev(inputs[which][name]))
        idx.row_ptr.fill_(-7)
        idx.col_idx.fill_(-7)
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rp, ci, oref = refs[which]
        assert torch.equal(idx.row_ptr, rp), f"replay {rep}: row_ptr"
        assert torch.equal(idx.col_idx[: ci.numel()], ci), f"replay {rep}: col_idx"
        assert torch.equal(o, oref), f"replay {rep}: output"
        _say(f"[gpu] graph: replay {rep} on input set {which} equals the eager calls")
