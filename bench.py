#!/usr/bin/env python3
"""Benchmark of centroid-scored 3D block-sparse attention on one MI355X.

One step = one attention call of the method: vsa_plan (block means,
centroid scores, per-row top-k, CSR) followed by vsa_attn (block-sparse
flash attention with the gather from raster order and the layout restore
fused in), on the Wan2.1-1.3B 480p/81f shape: B=1, 12 heads, d=128, latent
21x30x52 (32,760 tokens), 4x4x8 blocks, density 0.20, bf16, synthetic
smooth-field Q/K and N(0,1) V, resident in HBM before timing starts.

Prints one JSON line.  `value` is executed TFLOP/s of the step (valid
query-key token pairs of the produced index x 4*d, the convention of
SPADE Table 2), `ms_per_step` is the time per attention call.

    python bench.py [--steps K] [--warmup W] [--workload wan13b]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/attn call + executed TFLOP/s (% bf16 MFMA peak), Wan-1.3B shape, density 0.2"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
# fp32 vector peak without packed-fp32 instructions (the library is built
# with them disabled): 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP (FMA) x 2.4 GHz.
# The published 157.3 TFLOP/s counts packed fp32, which this build never issues.
PEAK_F32_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_wan13b_traffic.txt")


def block_sizes(grid, block):
    """Tokens per block in block-id order (edge blocks cut short)."""
    ext = []
    for n, b in zip(grid, block):
        e = [b] * (n // b) + ([n % b] if n % b else [])
        ext.append(np.array(e, dtype=np.int64))
    return (ext[0][:, None, None] * ext[1][None, :, None] * ext[2][None, None, :]).reshape(-1)


def executed_flops(row_ptr, col_idx, sizes, D):
    """4*D per valid (query token, kept key token) pair."""
    NB = len(sizes)
    lens = np.diff(row_ptr)
    rows = np.arange(len(lens)) % NB
    per_entry_q = np.repeat(sizes[rows], lens)
    return int(4 * D * np.sum(per_entry_q * sizes[col_idx[: row_ptr[-1]]]))


def padded_flops(row_ptr, col_idx, sizes, D, q_tile=32, k_tile=32):
    """Work the attention kernel issues: query rows rounded up to 32 per wave,
    keys rounded up to 32 per stage half."""
    NB = len(sizes)
    lens = np.diff(row_ptr)
    rows = np.arange(len(lens)) % NB
    qp = -(-sizes // q_tile) * q_tile
    kp = -(-sizes // k_tile) * k_tile
    return int(4 * D * np.sum(np.repeat(qp[rows], lens) * kp[col_idx[: row_ptr[-1]]]))


def read_traffic(src_hash):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current attention kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_source_hash():
    import hashlib
    p = os.path.join(ROOT, "block_sparse_attention_centroids_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()


def cpu_baseline(inp, w, row_ptr, col_idx, sizes, step_flops, budget_s=20.0):
    """The CPU oracle timed on the host: its full plan, plus its float64
    attention on a seeded sample of query blocks, scaled to a whole step."""
    from oracle import vsa_oracle as O
    host_cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=host_cores)   # BLAS threads = every core this process may use
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    t0 = time.perf_counter()
    rp, ci, info = O.plan(inp["q"], inp["k"], w.grid, w.block, inp["density"], w.window_t)
    t_plan = time.perf_counter() - t0
    g = info["geometry"]
    rng = np.random.default_rng(0)
    t_attn, f_attn, n_rows = 0.0, 0, 0
    while t_attn < budget_s and n_rows < 12 * g.NB:
        b, h, i = int(rng.integers(0, w.B)), int(rng.integers(0, w.heads)), int(rng.integers(0, g.NB))
        r = (b * w.heads + h) * g.NB + i
        t0 = time.perf_counter()
        O.attention_row(inp["q"], inp["k"], inp["v"], g, rp, ci, b, h, i)
        t_attn += time.perf_counter() - t0
        f_attn += 4 * w.D * int(sizes[i]) * int(sizes[ci[rp[r]: rp[r + 1]]].sum())
        n_rows += 1
    t_step = t_plan + t_attn * (step_flops / max(f_attn, 1))
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": step_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "host_cores": host_cores, "cpu_model": cpu_model,
            "sample": (f"full oracle plan ({t_plan:.2f} s) + float64 oracle attention on {n_rows} "
                       f"seeded query blocks ({t_attn:.1f} s, {f_attn / 1e9:.1f} GFLOP), scaled to "
                       f"the step's {step_flops / 1e12:.3f} TFLOP"),
            "seconds_per_step": t_step}


def time_select(vsa, lib, _lib, q, k, v, o, w, mode, val, sink, stream, sizes, estimator="mean", reps=20):
    """Mean plan time of vsa_plan_select for one selection, and attention
    over the index it produces (both timed with events on the stream)."""
    import ctypes

    import torch
    shape = vsa._shape_of(q, w.grid, w.block)
    rl, cap, pws = vsa.query_select(shape, mode, [val], w.window_t, sink, None, estimator)
    dev = q.device
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = _lib.VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()), cap)
    sel, _vals = vsa._select(shape, mode, [val], w.window_t, sink, None, estimator)
    sp = ctypes.c_void_p(stream.cuda_stream)
    qp, kp, vp, op = (ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o))

    def plan_call():
        _lib.check(lib.vsa_plan_select(qp, kp, ctypes.byref(shape), ctypes.byref(sel), ctypes.byref(cidx),
                                       ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp), "vsa_plan_select")

    def attn_call():
        _lib.check(lib.vsa_attn(qp, kp, vp, ctypes.byref(cidx), ctypes.c_float(0.0), op, None, 0, sp), "vsa_attn")

    for _ in range(2):
        plan_call(); attn_call()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        plan_call()
    e[1].record(stream)
    for _ in range(reps // 2):
        attn_call()
    e[2].record(stream)
    torch.cuda.synchronize()
    plan_ms = e[0].elapsed_time(e[1]) / reps
    attn_ms = e[1].elapsed_time(e[2]) / (reps // 2)
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)[: int(rp[-1])]
    flops = executed_flops(rp, ci, sizes, w.D)
    lens = np.diff(rp)
    return {"estimator": estimator, "mode": mode, "value": val, "sink": sink, "window_t": w.window_t,
            "plan_ms": round(plan_ms, 4), "attn_ms": round(attn_ms, 4),
            "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2),
            "nnz_blocks": int(rp[-1]), "density": round(float(rp[-1]) / (len(lens) * len(sizes)), 4),
            "row_len_min_max": [int(lens.min()), int(lens.max())]}


def time_layout(vsa, lib, _lib, x, w, stream, reps=20):
    """Standalone permute (raster -> blocked, zero pad rows) and unpermute of
    one tensor into preallocated buffers, timed with events on the stream;
    algorithmic bytes = one read of the source and one write of the
    destination (raster N*D plus blocked NB*bt*bh*bw*D elements)."""
    import ctypes

    import torch
    s = vsa._shape_of(x, w.grid, w.block)
    nb = int(np.prod([-(-int(n) // int(b)) for n, b in zip(w.grid, w.block)]))
    P = s.bt * s.bh * s.bw
    xb = torch.empty((s.B, s.heads, nb, P, s.D), dtype=x.dtype, device=x.device)
    xr = torch.empty_like(x)
    sp = ctypes.c_void_p(stream.cuda_stream)
    xp, bp, rp = (ctypes.c_void_p(t.data_ptr()) for t in (x, xb, xr))

    def perm():
        _lib.check(lib.vsa_permute(xp, ctypes.byref(s), bp, sp), "vsa_permute")

    def unperm():
        _lib.check(lib.vsa_unpermute(bp, ctypes.byref(s), rp, sp), "vsa_unpermute")

    for _ in range(3):
        perm(); unperm()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        perm()
    e[1].record(stream)
    for _ in range(reps):
        unperm()
    e[2].record(stream)
    torch.cuda.synchronize()
    pm, um = e[0].elapsed_time(e[1]) / reps, e[1].elapsed_time(e[2]) / reps
    nbytes = (x.numel() + xb.numel()) * x.element_size()
    return {"tensor": "k", "permute_ms": round(pm, 4), "unpermute_ms": round(um, 4),
            "algorithmic_bytes": int(nbytes),
            "permute_GB_per_s": round(nbytes / (pm * 1e-3) / 1e9, 1),
            "unpermute_GB_per_s": round(nbytes / (um * 1e-3) / 1e9, 1),
            "hbm_frac_permute": round(nbytes / (pm * 1e-3) / 8e12, 4),
            "hbm_frac_unpermute": round(nbytes / (um * 1e-3) / 8e12, 4),
            "roundtrip_identical": bool(torch.equal(xr, x))}


def time_mixed(vsa, lib, _lib, q, k, v, o, w, stream, sizes, reps=20):
    """A mixed per-head plan on the bench shape (dense, static, dynamic heads
    with windows; a seeded static ranking table), timed like time_select."""
    import ctypes

    import torch
    shape = vsa._shape_of(q, w.grid, w.block)
    nb = len(sizes)
    pattern = [{"kind": "dense"}, {"kind": "static", "value": 0.2}, {"kind": "dynamic", "value": 0.2, "window_t": 1},
               {"kind": "dynamic", "value": 0.1}, {"kind": "static", "value": 0.05, "window_t": 0},
               {"kind": "dynamic", "value": 0.3}]
    options = [pattern[h % len(pattern)] for h in range(w.heads)]
    table = torch.from_numpy(np.random.default_rng(24).standard_normal((w.heads, nb, nb)).astype(np.float32))
    table = table.to(q.device).contiguous()
    rl, cap, pws = vsa.query_mixed(shape, options)
    dev = q.device
    row_ptr = torch.empty(rl, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    cidx = _lib.VsaIndex(shape, 0, 0, ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()), cap)
    opts = vsa._head_options(options)
    sp = ctypes.c_void_p(stream.cuda_stream)
    qp, kp, vp, op, tp = (ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, table))

    def plan_call():
        _lib.check(lib.vsa_plan_mixed(qp, kp, ctypes.byref(shape), opts, 0, tp, ctypes.byref(cidx),
                                      ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp), "vsa_plan_mixed")

    def attn_call():
        _lib.check(lib.vsa_attn(qp, kp, vp, ctypes.byref(cidx), ctypes.c_float(0.0), op, None, 0, sp), "vsa_attn")

    for _ in range(2):
        plan_call(); attn_call()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        plan_call()
    e[1].record(stream)
    for _ in range(reps // 2):
        attn_call()
    e[2].record(stream)
    torch.cuda.synchronize()
    plan_ms = e[0].elapsed_time(e[1]) / reps
    attn_ms = e[1].elapsed_time(e[2]) / (reps // 2)
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)[: int(rp[-1])]
    flops = executed_flops(rp, ci, sizes, w.D)
    return {"heads": [o["kind"] + (f" {o['value']}" if "value" in o else "") +
                      (f" w{o['window_t']}" if o.get("window_t", -1) >= 0 else "") for o in options],
            "plan_ms": round(plan_ms, 4), "attn_ms": round(attn_ms, 4),
            "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2),
            "nnz_blocks": int(rp[-1]), "density": round(float(rp[-1]) / ((len(rp) - 1) * nb), 4)}


def time_scheme_flow(vsa, q, k, w, cands, dens, stream, plan_ms, reps=10):
    """Scheme selection that keeps each candidate's block means, then the
    plan of every head at the chosen candidate from those means (Q and K
    are read once per candidate in all), against selection plus a plan that
    reads Q and K again."""
    import torch
    for _ in range(2):
        _, choice, sm = vsa.select_scheme_means(q, k, w.grid, cands)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        _, choice, sm = vsa.select_scheme_means(q, k, w.grid, cands)
    e1.record(stream)
    torch.cuda.synchronize()
    sel_ms = e0.elapsed_time(e1) / reps
    c = int(choice[0].item())
    heads = list(range(w.heads))
    qm, km = sm.means(c)
    for _ in range(2):
        vsa.plan_heads(None, None, w.grid, cands[c], heads, dens[0], w.window_t, means=(qm, km),
                       heads_total=w.heads, B=w.B, D=w.D)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        vsa.plan_heads(None, None, w.grid, cands[c], heads, dens[0], w.window_t, means=(qm, km),
                       heads_total=w.heads, B=w.B, D=w.D)
    e1.record(stream)
    torch.cuda.synchronize()
    plan_means_ms = e0.elapsed_time(e1) / reps
    tensor_bytes = 2 * q.numel() * q.element_size()
    return {"select_with_means_ms": round(sel_ms, 4), "plan_from_means_ms": round(plan_means_ms, 4),
            "plan_reading_qk_ms": round(float(plan_ms), 4),
            "bytes_select_then_plan": (len(cands) + 1) * tensor_bytes,
            "bytes_with_means": len(cands) * tensor_bytes}


def time_cold(attn_call, stream, reps=10, scratch_mib=512):
    """Attention with cold caches: before every timed call a 512 MiB scratch
    buffer is overwritten, which evicts K/V from L2 and the 256 MB Infinity
    Cache; only the attention call sits between the events."""
    import torch
    scratch = torch.empty(scratch_mib << 20, dtype=torch.uint8, device="cuda")
    ms = []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        attn_call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(ms))


def mfma_sustained(vsa, stream, seconds=3.0, n_wg=4096, iters=2000):
    """Sustained bf16 MFMA rate of this card on N(0,1) operands held in
    registers (vsa_calib_mfma_bf16): the practical matrix-core ceiling
    under the card's power limit, timed with HIP events on `stream` until
    `seconds` of launches have run; the median rate over the second half
    of the launches (after the clock has settled) is reported."""
    import torch
    from block_sparse_attention_centroids_amd import _lib
    g = torch.Generator().manual_seed(0)
    pool = torch.randn(_lib.VSA_CALIB_POOL_BYTES // 2, generator=g).to(torch.bfloat16).view(torch.uint8).to("cuda")
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    flop = n_wg * 4 * iters * 16 * 32768
    vsa.calib_mfma_bf16(pool, out, n_wg, 10)
    torch.cuda.synchronize()
    ms, t0 = [], time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        vsa.calib_mfma_bf16(pool, out, n_wg, iters)
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    half = np.array(ms[len(ms) // 2:])
    med = float(np.median(half))
    return {"tflops": round(flop / (med * 1e-3) / 1e12, 1), "launch_ms_median": round(med, 3),
            "launches": len(ms), "seconds": round(time.perf_counter() - t0, 2),
            "data": "N(0,1) bf16 operands in registers, 32x32x16 MFMAs only",
            "kernel": f"vsa_calib_mfma_bf16 ({n_wg} workgroups x 4 waves x {iters} x 16 MFMAs)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the scheme-selection, selection-variant and mixed-plan timings "
                         "(profiled runs: only the step's own launches)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calib-seconds", type=float, default=3.0,
                    help="seconds of the sustained-MFMA measurement after the timed steps (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run one plain device-to-device copy of MIB MiB (HBM counter scale)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the method would shard by head with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import block_sparse_attention_centroids_amd as vsa

    vsa.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}))
        return
    w = W.WORKLOADS[a.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = W.generate(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda", 0)
    q, k, v = (torch.from_numpy(inp[n]).to(dev, dt).contiguous() for n in ("q", "k", "v"))
    dens = [float(d) for d in inp["density"]]
    torch.cuda.synchronize()

    def step():
        idx = vsa.plan(q, k, w.grid, w.block, dens, w.window_t)
        return idx, vsa.attn(q, k, v, idx)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        idx, o = step()
    torch.cuda.synchronize()

    # Pre-allocate the plan's buffers so the timed loop does not allocate:
    # the same index is re-planned in place every step.
    import ctypes
    from block_sparse_attention_centroids_amd import _lib
    lib = _lib.load()
    shape = idx.shape
    rl, cap, pws, _ = vsa.query(shape, dens, w.window_t)
    ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    darr = (ctypes.c_float * len(dens))(*dens)
    cidx = idx.c_index()
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    qp, kp, vp, op = (ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o))

    def plan_call():
        _lib.check(lib.vsa_plan(qp, kp, ctypes.byref(shape), darr, len(dens), w.window_t,
                                ctypes.byref(cidx), ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp), "vsa_plan")

    def attn_call():
        _lib.check(lib.vsa_attn(qp, kp, vp, ctypes.byref(cidx), ctypes.c_float(0.0), op, None, 0, sp), "vsa_attn")

    for _ in range(2):
        plan_call(); attn_call()
    torch.cuda.synchronize()

    K = a.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        plan_call()
        ev[s][1].record(stream)
        attn_call()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plan_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(K)])
    attn_ms = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(K)])
    step_ms = np.array([ev[s][0].elapsed_time(ev[s][2]) for s in range(K)])
    ms_per_step = wall * 1e3 / K

    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    ci = idx.col_idx.cpu().numpy().astype(np.int64)
    sizes = block_sizes(w.grid, w.block)
    flops = executed_flops(rp, ci, sizes, w.D)
    pflops = padded_flops(rp, ci, sizes, w.D)
    attn_tflops = flops / (attn_ms.mean() * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = read_traffic(kernel_source_hash())
    result = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded smooth-field Q/K, N(0,1) V; no dataset or weights)",
        "config": {"workload": w.name, "B": w.B, "heads": w.heads, "D": w.D, "grid": list(w.grid),
                   "block": list(w.block), "density": dens[0] if len(set(dens)) == 1 else dens,
                   "window_t": w.window_t},
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu",
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": traffic},
        "attn_ms": round(float(attn_ms.mean()), 4),
        "attn_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(attn_ms, [10, 50, 90])],
        "plan_ms": round(float(plan_ms.mean()), 4),
        "step_ms_events": round(float(step_ms.mean()), 4),
        "attn_tflops": round(attn_tflops, 2),
        "pct_bf16_peak_attn": round(100 * attn_tflops / peak, 2),
        "pct_bf16_peak_step": round(100 * step_tflops / peak, 2),
        "executed_tflop": round(flops / 1e12, 4),
        "issued_tflop_32x32_tiles": round(pflops / 1e12, 4),
        "nnz_blocks": int(rp[-1]),
        "gpu": torch.cuda.get_device_name(0) or torch.cuda.get_device_properties(0).gcnArchName,
    }
    # Scheme generation (outside the timed step): head-wise blocking-scheme
    # selection over three 128-token candidates; it reads Q and K once per
    # candidate, so it is reported against the HBM roofline.
    if w.dtype == "bf16" and w.D == 128 and w.name == "wan13b" and not a.no_extras:
        cands = [(4, 4, 8), (1, 8, 16), (2, 8, 8)]
        for _ in range(3):
            vsa.select_scheme(q, k, w.grid, cands)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            _, choice = vsa.select_scheme(q, k, w.grid, cands)
        e1.record(stream)
        torch.cuda.synchronize()
        sel_ms = e0.elapsed_time(e1) / 10
        sel_bytes = len(cands) * 2 * q.numel() * q.element_size()
        result["scheme_select"] = {
            "candidates": [list(c) for c in cands], "ms": round(sel_ms, 4),
            "algorithmic_bytes": sel_bytes, "GB_per_s": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(sel_bytes / (sel_ms * 1e-3) / 8e12, 4),
            "choices": choice.cpu().tolist()}
        result["scheme_means_flow"] = time_scheme_flow(vsa, q, k, w, cands, dens, stream, plan_ms.mean())
    # Selection variants (outside the timed step): Top-P and Top-K with
    # attention-sink blocks, each planned in place into preallocated buffers
    # and followed by attention over the index it produced.
    if w.dtype == "bf16" and w.name == "wan13b" and not a.no_extras:
        result["select_variants"] = [
            time_select(vsa, lib, _lib, q, k, v, o, w, mode, val, sink, stream, sizes, est)
            for est, mode, val, sink in (("mean", "topp", 0.25, 2), ("mean", "topk", 0.2, 2),
                                         ("dsa", "topk", 0.2, 0), ("dsa2", "topk", 0.2, 0))]
        result["mixed_plan"] = time_mixed(vsa, lib, _lib, q, k, v, o, w, stream, sizes)
        # Standalone layout kernels (the attention kernel gathers from and
        # stores to raster order itself; these serve callers that want the
        # blocked layout), against the HBM roofline.
        result["layout"] = time_layout(vsa, lib, _lib, k, w, stream)
    if not a.no_extras:
        cold = time_cold(attn_call, stream)
        result["attn_cold"] = {"scratch_MiB_between_calls": 512, "attn_ms_median": round(cold, 4),
                               "attn_tflops": round(flops / (cold * 1e-3) / 1e12, 2),
                               "warm_attn_ms": result["attn_ms"]}
    if a.calib_seconds > 0 and w.dtype == "bf16":
        print("[bench] sustained MFMA rate", file=sys.stderr, flush=True)
        ms_ = mfma_sustained(vsa, stream, a.calib_seconds)
        ms_["attn_frac_of_sustained"] = round(attn_tflops / ms_["tflops"], 4)
        result["mfma_sustained"] = ms_
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, w, rp, ci, sizes, flops, a.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
