"""Index check shared by the GPU selection tests: a GPU CSR index against
the oracle's, row by row.  Top-K rows must be equal; a Top-P row must be
the union of a prefix of the oracle's (score desc, id asc) order with the
window and sink blocks, of a length inside the float32 band around p (see
tests/test_gpu_select.py for the bound)."""
import numpy as np

from oracle import select_oracle as P
from oracle import vsa_oracle as O


def topp_tol(NB):
    return 6.0 * NB * 2.0 ** -24


def check_index(grp, gci, S, g, mode, vals, window_t, sink, scale):
    """Row-by-row check of a GPU index against the oracle (see the module
    docstring).  Returns (rows, rows inside the Top-P band, differing rows)
    and the oracle's own index."""
    B, Hh, NB, _ = S.shape
    vals = np.broadcast_to(np.asarray(vals, dtype=np.float32), (Hh,))
    rp, ci = P.select_rows(S, mode, vals, g, window_t, sink, scale)
    assert len(grp) == len(rp)
    if mode == "topk":
        assert np.array_equal(grp, rp), "row_ptr differs"
        assert np.array_equal(gci, ci), "col_idx differs"
        return (len(rp) - 1, 0, np.zeros(0, dtype=np.int64)), (rp, ci)
    extra_all = P.sink_blocks(NB, sink)
    band, differ = 0, []
    tol = topp_tol(NB)
    for r in range(len(rp) - 1):
        b, rem = divmod(r, Hh * NB)
        h, i = divmod(rem, NB)
        got = gci[grp[r]:grp[r + 1]]
        assert np.all(np.diff(got) > 0), f"row {r} not strictly ascending"
        want = ci[rp[r]:rp[r + 1]]
        if np.array_equal(got, want):
            continue
        p = float(vals[h])
        order, F = P.prefix_mass(S[b, h, i], scale)
        extra = extra_all
        if window_t >= 0:
            extra = np.union1d(extra, O.window_blocks(g, i, window_t))
        cstar = P.topp_count(S[b, h, i], p, scale)
        ok = False
        for c in range(max(1, cstar - 4), min(NB, cstar + 4) + 1):
            lower_ok = c == 1 or F[c - 2] < p + tol
            upper_ok = c == NB or F[c - 1] >= p - tol
            if lower_ok and upper_ok and np.array_equal(got, np.union1d(order[:c], extra)):
                ok = True
                break
        assert ok, f"row {r} (b={b} h={h} i={i}): GPU kept {len(got)}, oracle {len(want)}, p={p}"
        band += 1
        differ.append(r)
    return (len(rp) - 1, band, np.array(differ, dtype=np.int64)), (rp, ci)
