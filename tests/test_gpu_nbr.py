"""GPU neighbour build against the oracle: bit-exact CSR, reverse index, the
capacity protocol, preconditions and edge cases."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import Case, np_csr, say, torch
from oracle import nbr

pytestmark = pytest.mark.gpu


def _check_invariants(rp, src, shift, rev, N):
    E = len(src)
    assert rp[0] == 0 and rp[-1] == E and np.all(np.diff(rp) >= 0)
    recv = np.repeat(np.arange(N), np.diff(rp))
    assert (rev >= 0).all()
    np.testing.assert_array_equal(rev[rev], np.arange(E))
    np.testing.assert_array_equal(src[rev], recv)
    np.testing.assert_array_equal(shift[rev], -shift)
    key = ((src.astype(np.int64) << 24) | ((shift[:, 0].astype(np.int64) + 128) << 16)
           | ((shift[:, 1].astype(np.int64) + 128) << 8) | (shift[:, 2].astype(np.int64) + 128))
    same_row = recv[1:] == recv[:-1]
    assert np.all(key[1:][same_row] > key[:-1][same_row])


@pytest.mark.parametrize("k", [0, 1, 2])
def test_csr_bit_exact(k):
    case = Case(k, with_grad=False)
    nl = case.nbr()
    rp, src, shift, rev = np_csr(nl)
    ref = nbr.brute_force(case.d["pos"], case.cell, case.cfg["r_cut"]) if k < 2 else \
        nbr.binned(case.d["pos"], case.cell, case.cfg["r_cut"])
    np.testing.assert_array_equal(rp, ref[0])
    np.testing.assert_array_equal(src, ref[1])
    np.testing.assert_array_equal(shift, ref[2])
    np.testing.assert_array_equal(rev, nbr.reverse_index(*ref))
    _check_invariants(rp, src, shift, rev, case.N)


def test_csr_large_sampled_rows_and_invariants():
    case = Case(4, with_grad=False)
    nl = case.nbr()
    rp, src, shift, rev = np_csr(nl)
    _check_invariants(rp, src, shift, rev, case.N)
    rows = np.concatenate([[0, case.N - 1], np.random.default_rng(7).choice(case.N, 6, replace=False)])
    for i, (s_bf, sh_bf) in zip(rows, nbr.brute_force_rows(case.d["pos"], case.cell, case.cfg["r_cut"], rows)):
        np.testing.assert_array_equal(src[rp[i]:rp[i + 1]], s_bf)
        np.testing.assert_array_equal(shift[rp[i]:rp[i + 1]], sh_bf)
    deg = nl.n_edges / case.N
    assert 70 < deg < 80


def test_capacity_protocol():
    case = Case(1, with_grad=False)
    full = case.nbr()
    E = full.n_edges
    with pytest.raises(tpc.TpcError) as ei:
        case.nbr(edge_cap=E - 1)
    assert ei.value.status == 3 and str(E) in ei.value.message
    again = case.nbr(edge_cap=E)
    for a, b in zip(np_csr(full), np_csr(again)):
        np.testing.assert_array_equal(a, b)


def test_deterministic():
    case = Case(2, with_grad=False)
    a = np_csr(case.nbr())
    b = np_csr(case.nbr())
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_unwrapped_positions_are_refused():
    case = Case(0, with_grad=False)
    p = case.pos.clone()
    p[3, 0] = -0.5
    say("[gpu] nbr_build unwrapped")
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.nbr_build(p, case.cell)
    assert ei.value.status == 4 and "wrapped" in ei.value.message


def test_species_out_of_range_is_refused():
    case = Case(0, with_grad=False)
    s = case.species.clone()
    s[5] = 1000
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.nbr_build(case.pos, case.cell, s)
    assert "species" in ei.value.message


def test_edge_cases_empty_and_isolated():
    t = torch()
    ctx = tpc.Context(tpc.spec_for(workloads.config(0)))
    cell = np.eye(3) * 50.0
    say("[gpu] nbr_build N=0")
    nl = ctx.nbr_build(t.zeros((0, 3), dtype=t.float64, device="cuda"), cell)
    assert nl.n_edges == 0 and nl.row_ptr.cpu().tolist() == [0]
    # two far-apart atoms: empty rows
    pos = t.tensor([[1.0, 1.0, 1.0], [25.0, 25.0, 25.0]], dtype=t.float64, device="cuda")
    nl = ctx.nbr_build(pos, cell)
    assert nl.n_edges == 0 and nl.row_ptr.cpu().tolist() == [0, 0, 0]
    # one atom alone in a small cell sees its own images
    pos = t.tensor([[0.5, 1.0, 2.0]], dtype=t.float64, device="cuda")
    nl = ctx.nbr_build(pos, np.eye(3) * 3.0)
    ref = nbr.brute_force(pos.cpu().numpy(), np.eye(3) * 3.0, 4.0)
    for a, b in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b)


def test_triclinic_cell():
    t = torch()
    rng = np.random.default_rng(3)
    cell = np.array([[9.0, 0.0, 0.0], [2.5, 8.5, 0.0], [-1.5, 1.2, 8.0]])
    f = rng.uniform(0.0, 1.0, (60, 3))
    pos = f @ cell
    ctx = tpc.Context(tpc.spec_for(workloads.config(0)))
    nl = ctx.nbr_build(t.from_numpy(pos).to("cuda"), cell)
    ref = nbr.brute_force(pos, cell, 4.0)
    for a, b in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b)
