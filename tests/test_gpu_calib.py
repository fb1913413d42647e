"""The sustained-MFMA measurement kernel (vsa_calib_mfma_bf16) computes the
products it claims: for each wave, the sum of its 64 output values equals
the sum of every entry of the bf16 fragment products the header assigns to
it, recomputed here in float64 from the same pool with the operand layout
of v_mfma_f32_32x32x16_bf16 (A lane l: row l mod 32, B lane l: column
l mod 32, inner indices 8*(l/32) .. 8*(l/32)+7)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import block_sparse_attention_centroids_amd as pkg
    pkg.load()
    return pkg


def _pool(seed):
    from block_sparse_attention_centroids_amd import _lib
    g = torch.Generator().manual_seed(seed)
    vals = torch.randn(_lib.VSA_CALIB_POOL_BYTES // 2, generator=g).to(torch.bfloat16)
    return vals


def _fragments(vals):
    # [4096 fragments][64 lanes][8 bf16] as float64
    return vals.float().numpy().astype(np.float64).reshape(4096, 64, 8)


def _a_matrix(frag):
    A = np.zeros((32, 16))
    for l in range(64):
        A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = frag[l]
    return A


def _b_matrix(frag):
    B = np.zeros((16, 32))
    for l in range(64):
        B[8 * (l // 32): 8 * (l // 32) + 8, l % 32] = frag[l]
    return B


def _wave_reference(F, g, w, iters):
    base = 16 * (4 * g + w)
    A = [_a_matrix(F[(base + j) % 4096]) for j in range(8)]
    B = [_b_matrix(F[(base + 8 + j) % 4096]) for j in range(8)]
    tot, mag = 0.0, 0.0
    for j in range(8):
        for P in (A[j] @ B[(j + 3) % 8], A[(j + 5) % 8] @ B[j]):
            tot += P.sum()
            mag += np.abs(P).sum()
    return iters * tot, iters * mag


@pytest.mark.parametrize("nwg,iters", [(3, 1), (70, 2), (1030, 5)])
def test_wave_sums_match_products(vsa, nwg, iters):
    print(f"[gpu] calib nwg={nwg} iters={iters}", flush=True)
    sys.stdout.flush()
    vals = _pool(nwg)
    pool = vals.view(torch.uint8).to("cuda")
    out = torch.full((nwg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    vsa.calib_mfma_bf16(pool, out, nwg, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(nwg, 4, 64).sum(axis=2)
    F = _fragments(vals)
    for g in sorted({0, 1, nwg // 2, nwg - 1}):
        for w in range(4):
            want, mag = _wave_reference(F, g, w, iters)
            assert abs(got[g, w] - want) <= 1e-5 * mag + 1e-6, (g, w, got[g, w], want)
    assert np.isfinite(got).all()


def test_zero_pool_and_repeat(vsa):
    from block_sparse_attention_centroids_amd import _lib
    pool = torch.zeros(_lib.VSA_CALIB_POOL_BYTES, dtype=torch.uint8, device="cuda")
    out = torch.full((64 * 256,), 1.0, dtype=torch.float32, device="cuda")
    vsa.calib_mfma_bf16(pool, out, 64, 3)
    torch.cuda.synchronize()
    assert (out == 0).all()
    vals = _pool(7)
    pool = vals.view(torch.uint8).to("cuda")
    o1 = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    vsa.calib_mfma_bf16(pool, o1, 64, 4)
    vsa.calib_mfma_bf16(pool, o2, 64, 4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
