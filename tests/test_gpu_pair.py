"""Rows of R shared by an edge and its reverse (spec.pair_radial).

The map Rrow that the forward writes is checked against the reverse index on
the host: every edge whose reverse lies in the chunk reads the row of the
lower-indexed of the two, every other edge keeps a row of its own, rows are
numbered in chunk order, and Rrow[E_chunk] counts them.  The rows it reads
hold the oracle's radial weights of that edge, and the whole step equals the
one-row-per-edge layout bit for bit."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
from _gpu import TOL, Case, rel, row_bounds, say, torch

pytestmark = pytest.mark.gpu


def _expected_map(rev, e0, e1):
    """Chunk-relative row of each edge of [e0, e1), written out edge by edge."""
    ne = e1 - e0
    rows = np.full(ne, -1, dtype=np.int64)
    n = 0
    for k in range(ne):
        r = int(rev[e0 + k]) - e0
        if r < 0 or r >= ne or k < r:
            rows[k] = n
            n += 1
    for k in range(ne):
        if rows[k] < 0:
            rows[k] = rows[int(rev[e0 + k]) - e0]
    return rows, n


@pytest.mark.parametrize("chunks", [1, 3])
def test_row_map_and_rows(chunks):
    t = torch()
    case = Case(1, pair=True)
    assert case.ctx.pair_radial
    nl = case.nbr()
    rp = nl.row_ptr.cpu().numpy()
    rev = nl.rev.cpu().numpy()
    s = case.scale(nl)
    flat = tpc.Context(tpc.spec_for(case.cfg))
    assert not flat.pair_radial
    out = t.empty((case.N, case.ctx.d_out, case.cfg["C"]), dtype=case.ctx.dtype, device="cuda")
    for a, b in row_bounds(rp, chunks):
        e0, e1 = int(rp[a]), int(rp[b])
        say(f"[gpu] pair forward cfg=1 rows=[{a},{b}) edges=[{e0},{e1})")
        _, eb = case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=out, rows=(a, b),
                                  edges=(e0, e1))
        _, ref = flat.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=t.empty_like(out), rows=(a, b),
                               edges=(e0, e1))
        t.cuda.synchronize()
        rows, n = _expected_map(rev, e0, e1)
        got = eb.Rrow.cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(got[:e1 - e0], rows)
        assert got[e1 - e0] == n
        if chunks == 1:
            assert 2 * n == e1 - e0          # a symmetric list: one row per pair
        else:
            assert 2 * n > e1 - e0           # pairs cut by the chunk boundary keep two rows
        # each edge reads exactly its own weights
        assert t.equal(eb.R_per_edge(), ref.R)


def test_rows_against_the_oracle():
    import workloads
    # the tiny geometry in float64 at 64 channels (shared rows take the
    # unmasked kernels, 64 or 128 channels)
    case = Case(0, data=workloads.variant(0, 64, 1, 2, 1, [16], "float64", 4242), pair=True)
    assert case.ctx.pair_radial
    nl = case.nbr()
    out, eb = case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, case.scale(nl))
    torch().cuda.synchronize()
    ref = case.oracle_csr()
    for a, b in zip((nl.row_ptr.cpu().numpy(), nl.src.cpu().numpy(), nl.shift.cpu().numpy()), ref):
        np.testing.assert_array_equal(a, b)
    prob = case.oracle(ref)
    _, _, _, _, R = prob.edge_terms(np.arange(nl.n_edges))
    assert rel(eb.R_per_edge().cpu().numpy(), R) < TOL["float64"]
    assert rel(out.cpu().numpy(), prob.forward()) < TOL["float64"]
    assert int(eb.Rrow[nl.n_edges].item()) * 2 == nl.n_edges


def test_fused_and_table_contexts_keep_one_row_per_edge():
    import workloads
    cfg = workloads.config(3)
    assert not tpc.Context(tpc.spec_for(cfg, fuse_radial=True, pair_radial=True)).pair_radial
    assert not tpc.Context(tpc.spec_for(cfg, table=(32, 8), pair_radial=True)).pair_radial
