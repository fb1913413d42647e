"""vsa_plan_noalloc through the C ABI: the plan with its workspace in the
library's static per-GPU array equals vsa_plan with a caller workspace, bit
for bit, on two calls in a row (the second on a smaller input, so it reads
the array after a larger plan left its contents there), with and without a
temporal window (the windowed plan also keeps per-row counts and bitmaps in
the array); a plan whose workspace exceeds the array is refused before
anything is enqueued."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W
from block_sparse_attention_centroids_amd import _lib
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return _lib.load()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=torch.bfloat16).contiguous()


def _plan_both(lib, w, inp, density, window_t):
    """(vsa_plan index, vsa_plan_noalloc index) as numpy (row_ptr, col_idx)."""
    q, k = _dev(inp["q"]), _dev(inp["k"])
    shape = _lib.VsaShape(w.B, w.heads, w.D, *w.grid, *w.block, _lib.VSA_BF16)
    dens = (ctypes.c_float * 1)(density)
    rl, cap, pws, aws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.vsa_query(ctypes.byref(shape), dens, 1, window_t, ctypes.byref(rl), ctypes.byref(cap),
                         ctypes.byref(pws), ctypes.byref(aws)) == 0
    assert pws.value <= _lib.VSA_PLAN_NOALLOC_MAX_WS
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (False, True):
        # Poison the index arrays so that stale entries cannot pass.
        row_ptr = torch.full((rl.value,), -7, dtype=torch.int32, device="cuda")
        col_idx = torch.full((max(cap.value, 1),), -7, dtype=torch.int32, device="cuda")
        idx = _lib.VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()),
                            ctypes.c_void_p(col_idx.data_ptr()), cap.value)
        if noalloc:
            st = lib.vsa_plan_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      ctypes.byref(shape), dens, 1, window_t, ctypes.byref(idx), stream)
        else:
            ws = torch.empty(max(pws.value, 1), dtype=torch.uint8, device="cuda")
            st = lib.vsa_plan(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.byref(shape),
                              dens, 1, window_t, ctypes.byref(idx), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                              stream)
        assert st == 0, _lib.status_str(st)
        torch.cuda.synchronize()
        rp = row_ptr.cpu().numpy()
        out.append((rp, col_idx.cpu().numpy()[: int(rp[-1])], idx.window_t, idx.equal_heads))
    return out


@pytest.mark.parametrize("window_t", [-1, 1])
def test_noalloc_plan_equals_plan_twice(lib, window_t):
    big = W.custom("na_big", 1, 6, 128, (21, 30, 52), (4, 4, 8), "bf16", 0.2, window_t, "smooth")
    small = W.custom("na_small", 1, 2, 64, (9, 14, 20), (4, 4, 8), "bf16", 0.3, window_t, "smooth")
    for w, dens, seed in ((big, 0.2, 81), (small, 0.3, 82)):
        _say(f"[gpu] noalloc plan {w.name} window={window_t}")
        inp = W.generate(w, seed=seed)
        (rp_a, ci_a, win_a, eq_a), (rp_b, ci_b, win_b, eq_b) = _plan_both(lib, w, inp, dens, window_t)
        assert np.array_equal(rp_a, rp_b) and np.array_equal(ci_a, ci_b)
        assert (win_a, eq_a) == (win_b, eq_b)
        if w is small:   # the small case is cheap enough for the oracle too
            rp, ci, _ = O.plan(inp["q"], inp["k"], w.grid, w.block, np.float32(dens), window_t)
            assert np.array_equal(rp_b, rp) and np.array_equal(ci_b, ci)


def test_noalloc_refuses_oversized_workspace(lib):
    """256 heads at the long-video shape need far more than the array: the
    call returns VSA_ERR_WORKSPACE and enqueues nothing."""
    shape = _lib.VsaShape(1, 256, 128, 84, 30, 52, 4, 4, 8, _lib.VSA_BF16)
    dens = (ctypes.c_float * 1)(0.1)
    rl, cap, pws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    assert lib.vsa_query(ctypes.byref(shape), dens, 1, -1, ctypes.byref(rl), ctypes.byref(cap),
                         ctypes.byref(pws), None) == 0
    assert pws.value > _lib.VSA_PLAN_NOALLOC_MAX_WS
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")   # never read: the call is refused first
    idx = _lib.VsaIndex(shape, 0, 0, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), cap.value)
    st = lib.vsa_plan_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), ctypes.byref(shape),
                              dens, 1, -1, ctypes.byref(idx), None)
    assert st == _lib.VSA_ERR_WORKSPACE
