"""CPU checks of the benchmark's FLOP accounting against the oracle.

The roofline figure divides the executed FLOPs of the produced index by the
measured time, so bench.py's vectorized count must equal the oracle's
row-by-row definition (4*D per valid query-key token pair), and its block
sizes must be the oracle's geometry.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from oracle import vsa_oracle as O  # noqa: E402

GRIDS = [((4, 8, 8), (2, 4, 8)), ((21, 30, 52), (4, 4, 8)), ((16, 45, 80), (1, 8, 16)),
         ((3, 5, 7), (2, 2, 4)), ((1, 1, 1), (4, 4, 8)), ((7, 23, 8), (8, 1, 2))]


@pytest.mark.parametrize("grid,block", GRIDS)
def test_block_sizes_match_oracle_geometry(grid, block):
    assert np.array_equal(bench.block_sizes(grid, block), O.geometry(grid, block).sizes)


@pytest.mark.parametrize("grid,block", GRIDS)
@pytest.mark.parametrize("D", [64, 128])
def test_executed_flops_match_oracle(grid, block, D):
    g = O.geometry(grid, block)
    rng = np.random.default_rng(len(grid) * 31 + D + g.NB)
    B, Hh = 2, 3
    rows = B * Hh * g.NB
    lens = rng.integers(0, g.NB + 1, size=rows)          # empty rows included
    row_ptr = np.zeros(rows + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col_idx = np.concatenate([np.sort(rng.choice(g.NB, size=n, replace=False)) for n in lens] +
                             [np.zeros(0, dtype=np.int64)]).astype(np.int64)
    got = bench.executed_flops(row_ptr, col_idx, bench.block_sizes(grid, block), D)
    assert got == O.executed_flops(g, row_ptr, col_idx, B, Hh, D)


def test_padded_flops_bound_executed():
    g = O.geometry((21, 30, 52), (4, 4, 8))
    rp = np.arange(g.NB + 1, dtype=np.int64) * g.NB     # dense: every row keeps every block
    ci = np.tile(np.arange(g.NB, dtype=np.int64), g.NB)
    sizes = bench.block_sizes((21, 30, 52), (4, 4, 8))
    ex = bench.executed_flops(rp, ci, sizes, 128)
    assert ex == 4 * 128 * int(sizes.sum()) ** 2        # dense: 4 N^2 D
    assert bench.padded_flops(rp, ci, sizes, 128) >= ex
