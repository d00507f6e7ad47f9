"""GPU convolution forward and backward against the oracle, element by element
on full outputs (tiny, small) or sampled rows (medium, large), plus
determinism, chunking, preconditions and invariants that hold at any size."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
from _gpu import TOL, Case, np_csr, rel, run_chunked, say, torch
from oracle import conv, nbr

pytestmark = pytest.mark.gpu


def _prob(case, nl):
    """Oracle problem on the oracle's own neighbour list.  Per-edge outputs
    are compared edge by edge, so the GPU list must be the same arrays."""
    ref = case.oracle_csr()
    for a, b in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b)
    return case.oracle(ref)


# 0 tiny (float64), 1 small; 5-7 are the small system at other channel and
# hidden widths (the narrower-channel tensor-product kernels, the float32
# radial kernels that the wider networks do not take, and in 7 a radial
# width of 17 column steps of 32: a half-filled last weight tile forward and
# the float32 fallback backward); 8 is the small system with path-summed
# outputs (one block per output rank); 9 and 10 are dense systems whose rows
# hold 114-176 edges (the loops for rows longer than 128 edges)
@pytest.mark.timeout(300)
@pytest.mark.parametrize("k", [0, 1, 5, 6, 7, 8, 9, 10])
def test_full_parity(k):
    case = Case(k)
    nl = case.nbr()
    tol = TOL[case.cfg["dtype"]]
    res = run_chunked(case, nl, chunks=1, keep_edges=np.arange(nl.n_edges))
    prob = _prob(case, nl)
    say(f"[cpu] oracle cfg={k}")
    out_ref = prob.forward()
    b = prob.backward()
    assert rel(res["out"].cpu().numpy(), out_ref) < tol
    assert rel(res["dh"].cpu().numpy(), b["dh"]) < tol
    dR = np.stack([res["dR"][e] for e in range(nl.n_edges)])
    assert rel(dR, b["dR"]) < tol
    assert rel(res["g_edge"].cpu().numpy(), b["g"]) < tol
    assert rel(res["forces"].cpu().numpy(), b["F"]) < tol
    # per-edge intermediates
    _, _, Y, ef, R = prob.edge_terms(np.arange(nl.n_edges))
    assert rel(res["eb"].Y.cpu().numpy(), Y) < tol
    assert rel(res["eb"].ef.cpu().numpy(), ef) < tol
    assert rel(res["eb"].R_per_edge().cpu().numpy(), R) < tol


def _sampled_check(case, nl, res, rows, atoms, edges):
    prob = _prob(case, nl)
    tol = TOL[case.cfg["dtype"]]
    say(f"[cpu] oracle sampled cfg={case.k}: {len(rows)} rows, {len(atoms)} atoms, {len(edges)} edges")
    out_ref = prob.forward_rows(rows)
    assert rel(res["out"][rows].cpu().numpy(), out_ref) < tol
    b = prob.edge_backward(edges)
    dR = np.stack([res["dR"][int(e)] for e in edges])
    assert rel(dR, b["dR"]) < tol
    assert rel(res["g_edge"][edges].cpu().numpy(), b["g"]) < tol
    assert rel(res["dh"][atoms].cpu().numpy(), prob.dh_atoms(atoms)) < tol
    assert rel(res["forces"][atoms].cpu().numpy(), prob.forces_atoms(atoms)) < tol


def _spread(sorted_rows, k):
    """k entries of a sorted sample, evenly spaced over it, so the checks
    see every part of the row range (each XCD's share of the grid)."""
    idx = np.unique(np.linspace(0, len(sorted_rows) - 1, k).round().astype(int))
    return sorted_rows[idx]


def _samples(case, n_rows, seed, n_edge_rows=16):
    rp, N = case.oracle_csr()[0], case.N
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, n_rows, replace=False)]))
    edges = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in _spread(rows, n_edge_rows)])
    return rows, edges


def _both_row_layouts(case, nl, chunks, rows, atoms, edges):
    """The sampled check with one row of R per edge, then with the rows
    shared by edge pairs (the layout bench.py times); the second must equal
    the first bit for bit, since each row comes from the same arithmetic."""
    t = torch()
    res = run_chunked(case, nl, chunks=chunks, keep_edges=edges)
    _sampled_check(case, nl, res, rows, atoms, edges)
    keep = {k: res[k] for k in ("out", "dh", "forces", "g_edge")}
    kept_dR = res["dR"]
    del res
    case.ctx = tpc.Context(tpc.spec_for(case.cfg, pair_radial=True))
    assert case.ctx.pair_radial
    res = run_chunked(case, nl, chunks=chunks, keep_edges=edges)
    _sampled_check(case, nl, res, rows, atoms, edges)
    for k, v in keep.items():
        assert t.equal(res[k], v), k
    for e in edges:
        np.testing.assert_array_equal(res["dR"][int(e)], kept_dR[int(e)])


def test_medium_parity_sampled():
    case = Case(3)
    nl = case.nbr()
    rows, edges = _samples(case, 96, 11)
    atoms = np.unique(np.concatenate([np.arange(64), _spread(rows, 32)]))   # includes the 0-63 slice
    _both_row_layouts(case, nl, 1, rows, atoms, edges)


@pytest.mark.timeout(300)   # the oracle's own 19.6 M-edge list takes about 40 s
def test_large_parity_sampled_chunked():
    case = Case(4)
    nl = case.nbr()
    rows, edges = _samples(case, 40, 12)
    # the 2 receiver chunks bench.py times
    _both_row_layouts(case, nl, 2, rows, _spread(rows, 24), edges)


@pytest.mark.parametrize("pair", [False, True])
def test_chunked_equals_unchunked(pair):
    case = Case(1)
    nl = case.nbr()
    a = run_chunked(case, nl, chunks=1)
    case.ctx = tpc.Context(tpc.spec_for(case.cfg, pair_radial=pair))
    b = run_chunked(case, nl, chunks=5)
    for key in ("out", "dh", "forces", "g_edge"):
        assert torch().equal(a[key], b[key]), key


def test_chunked_dh_over_chunks_without_edges():
    """dh continues over every chunk's call: chunks that hold no edges (an
    isolated atom) still carry the running sums through, and the chunk of the
    last row scales them; the result equals the single call bit for bit."""
    t = torch()
    case = Case(0)
    ctx = case.ctx
    pos = t.tensor([[1.0, 1.0, 1.0], [1.5, 1.0, 1.0], [7.0, 7.0, 7.0], [1.0, 1.8, 1.0]], dtype=t.float64,
                   device="cuda")
    cell = np.eye(3) * 20.0
    nl = ctx.nbr_build(pos, cell)
    rp = nl.row_ptr.cpu().tolist()
    assert rp[3] == rp[2]    # atom 2 has no neighbours
    h = case.h[:4].contiguous()
    G = case.G[:4].contiguous()
    out, eb = ctx.conv_fwd(pos, cell, nl, h, case.W, 0.5)
    dh_ref, _, F_ref, _ = ctx.conv_bwd(nl, h, case.W, 0.5, G, eb)
    dh = t.full_like(h, float("nan"))       # every entry must be written
    g_edge = t.empty((nl.n_edges, 3), dtype=ctx.dtype, device="cuda")
    for a, b in [(0, 1), (1, 2), (2, 3), (3, 4)]:
        e0, e1 = rp[a], rp[b]
        ebc = ctx.alloc_edge_buffers(max(e1 - e0, 1), "cuda")
        ctx.conv_fwd(pos, cell, nl, h, case.W, 0.5, out=t.empty_like(out), eb=ebc, rows=(a, b), edges=(e0, e1))
        _, _, F, _ = ctx.conv_bwd(nl, h, case.W, 0.5, G, ebc, dh=dh, g_edge=g_edge, want_forces=b == 4)
    t.cuda.synchronize()
    assert t.equal(dh, dh_ref) and t.equal(F, F_ref)
    prob = conv.Problem(case.layout, pos.cpu().numpy(), cell, *np_csr(nl)[:3], case.d["h"][:4], case.d["W"],
                        case.cfg["r_cut"], 0.5, case.d["G"][:4])
    b = prob.backward()
    assert rel(dh.cpu().numpy(), b["dh"]) < 1e-10
    assert rel(F.cpu().numpy(), b["F"]) < 1e-10


def test_bitwise_deterministic():
    case = Case(2)
    nl = case.nbr()
    a = run_chunked(case, nl, keep_edges=np.arange(0, nl.n_edges, 997))
    b = run_chunked(case, nl, keep_edges=np.arange(0, nl.n_edges, 997))
    for key in ("out", "dh", "forces", "g_edge"):
        assert torch().equal(a[key], b[key]), key
    for e in a["dR"]:
        np.testing.assert_array_equal(a["dR"][e], b["dR"][e])


def test_invariants_at_medium_size():
    """Sum of forces vanishes; L is linear in h: <dh, h> = L."""
    case = Case(3)
    nl = case.nbr()
    res = run_chunked(case, nl)
    t = torch()
    F = res["forces"].double()
    assert float(F.sum(0).abs().max()) < 1e-4 * float(F.abs().max()) * np.sqrt(case.N)
    GO = case.G.double() * res["out"].double()
    L = float(GO.sum())
    hdh = float((case.h.double() * res["dh"].double()).sum())
    assert abs(L - hdh) <= 1e-4 * float(GO.abs().sum())


def test_validation_refuses_an_unsorted_csr():
    case = Case(0, validate=True)
    nl = case.nbr()
    rp = nl.row_ptr.cpu().numpy()
    i = int(np.argmax(np.diff(rp) >= 2))
    bad = nl.src.clone()
    a, b = int(rp[i]), int(rp[i]) + 1
    bad[a], bad[b] = nl.src[b].item(), nl.src[a].item()
    if int(bad[a]) == int(bad[b]):            # same sender: swap shifts instead
        pytest.skip("first multi-edge row has a repeated sender")
    bad_nl = tpc.NeighbourList(nl.row_ptr, bad, nl.shift, nl.rev, nl.n_edges)
    say("[gpu] conv_fwd with validate on an unsorted row")
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.conv_fwd(case.pos, case.cell, bad_nl, case.h, case.W, 1.0)
    assert ei.value.status == 4
    # the sorted list passes
    out, _ = case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, 1.0)
    torch().cuda.synchronize()


@pytest.mark.parametrize("k", [0, 1])
def test_virial_parity(k):
    """The virial kernel on the oracle's own edge gradients (same inputs), and
    end to end from the GPU's edge gradients."""
    t = torch()
    case = Case(k)
    nl = case.nbr()
    tol = TOL[case.cfg["dtype"]]
    res = run_chunked(case, nl, chunks=1)
    prob = _prob(case, nl)
    say(f"[cpu] oracle backward cfg={k}")
    b = prob.backward()
    g_in = t.tensor(b["g"], dtype=case.ctx.dtype, device="cuda")
    say(f"[gpu] virial cfg={k} on the oracle's edge gradients")
    W1 = case.ctx.virial(case.pos, case.cell, nl, g_in)
    ref1 = conv.virial(prob.rvec(np.arange(nl.n_edges)), g_in.cpu().double().numpy())
    assert rel(W1.cpu().numpy(), ref1) < tol
    say(f"[gpu] virial cfg={k} on its own edge gradients")
    W2 = case.ctx.virial(case.pos, case.cell, nl, res["g_edge"])
    assert rel(W2.cpu().numpy(), prob.virial_from(b["g"])) < tol


def test_virial_medium_size():
    """Full-size virial on seeded edge gradients (its only input besides the
    list and positions) against the oracle's sum over its own edge vectors."""
    t = torch()
    case = Case(3, with_grad=False)
    nl = case.nbr()
    rp, src, shift = case.oracle_csr()
    for a, b in zip(np_csr(nl)[:3], (rp, src, shift)):
        np.testing.assert_array_equal(a, b)
    g = t.tensor(np.random.default_rng(31).standard_normal((len(src), 3)), dtype=case.ctx.dtype,
                 device="cuda")
    say("[gpu] virial medium")
    W = case.ctx.virial(case.pos, case.cell, nl, g).cpu().numpy()
    vec = nbr.edge_vectors(case.d["pos"], case.cell, nbr.receivers_of(rp), src, shift)
    assert rel(W, conv.virial(vec, g.cpu().double().numpy())) < TOL[case.cfg["dtype"]]


def test_empty_rows_and_zero_edges():
    t = torch()
    case = Case(0)
    ctx = case.ctx
    pos = t.tensor([[1.0, 1.0, 1.0], [7.0, 7.0, 7.0], [1.5, 1.0, 1.0]], dtype=t.float64, device="cuda")
    cell = np.eye(3) * 20.0
    nl = ctx.nbr_build(pos, cell)
    assert nl.row_ptr.cpu().tolist() == [0, 1, 1, 2]
    h = case.h[:3].contiguous()
    G = case.G[:3].contiguous()
    out, eb = ctx.conv_fwd(pos, cell, nl, h, case.W, 1.0)
    dh, dR, F, g = ctx.conv_bwd(nl, h, case.W, 1.0, G, eb)
    t.cuda.synchronize()
    assert float(out[1].abs().max()) == 0.0 and float(dh[1].abs().max()) == 0.0
    assert float(F[1].abs().max()) == 0.0
    pos_np = np.array([[1.0, 1.0, 1.0], [7.0, 7.0, 7.0], [1.5, 1.0, 1.0]])
    ref = nbr.brute_force(pos_np, cell, 4.0)
    for a, b_ in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b_)
    prob = conv.Problem(case.layout, pos_np, cell, *ref, case.d["h"][:3], case.d["W"], 4.0, 1.0,
                        case.d["G"][:3])
    assert rel(out.cpu().numpy(), prob.forward()) < 1e-10
    b = prob.backward()
    assert rel(F.cpu().numpy(), b["F"]) < 1e-10
    W = ctx.virial(pos, cell, nl, g)
    assert rel(W.cpu().numpy(), prob.virial_from(b["g"])) < 1e-10
    # no edges at all
    pos2 = t.tensor([[1.0, 1.0, 1.0], [9.0, 9.0, 9.0]], dtype=t.float64, device="cuda")
    nl2 = ctx.nbr_build(pos2, cell)
    assert nl2.n_edges == 0
    out2, eb2 = ctx.conv_fwd(pos2, cell, nl2, h[:2].contiguous(), case.W, 1.0)
    dh2, _, F2, _ = ctx.conv_bwd(nl2, h[:2].contiguous(), case.W, 1.0, G[:2].contiguous(), eb2)
    t.cuda.synchronize()
    assert float(out2.abs().max()) == 0.0 and float(dh2.abs().max()) == 0.0
    assert float(F2.abs().max()) == 0.0
    W2 = ctx.virial(pos2, cell, nl2, t.empty((0, 3), dtype=ctx.dtype, device="cuda"))
    t.cuda.synchronize()
    assert float(W2.abs().max()) == 0.0


def test_validation_refuses_unwrapped_positions_and_a_broken_reverse_index():
    """With spec.validate, conv_fwd refuses positions outside the cell and
    conv_bwd refuses a reverse index that does not pair every edge with its
    reverse (the backward gathers sender gradients through that symmetry)."""
    t = torch()
    case = Case(0, validate=True)
    nl = case.nbr()
    out, eb = case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, 1.0)
    t.cuda.synchronize()
    bad_pos = case.pos.clone()
    bad_pos[3, 0] += float(case.cell[0, 0])            # one atom moved out by a cell vector
    say("[gpu] conv_fwd with validate on unwrapped positions")
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.conv_fwd(bad_pos, case.cell, nl, case.h, case.W, 1.0)
    assert ei.value.status == 4 and "wrapped" in ei.value.message
    bad_rev = nl.rev.clone()
    bad_rev[0], bad_rev[1] = nl.rev[1].item(), nl.rev[0].item()
    bad_nl = tpc.NeighbourList(nl.row_ptr, nl.src, nl.shift, bad_rev, nl.n_edges)
    say("[gpu] conv_bwd with validate on a broken reverse index")
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.conv_bwd(bad_nl, case.h, case.W, 1.0, case.G, eb)
    assert ei.value.status == 4 and "reverse" in ei.value.message
    dh, _, F, _ = case.ctx.conv_bwd(nl, case.h, case.W, 1.0, case.G, eb)
    t.cuda.synchronize()
