"""The VJP-of-VJP (double backward) on the GPU against the oracle: element by
element on every output of the tiny, small and dense systems, on sampled
receivers, atoms and edges of the medium system, chunked against unchunked,
and bitwise run to run."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
from _gpu import TOL, Case, cotangents, np_csr, rel, run_double, say, torch

pytestmark = pytest.mark.gpu


def _prob(case, nl):
    ref = case.oracle_csr()
    for a, b in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b)
    return case.oracle(ref)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("k", [0, 1, 9])
def test_double_backward_full_parity(k):
    case = Case(k)
    nl = case.nbr()
    u = cotangents(case, nl.n_edges, 40 + k)
    res = run_double(case, nl, u, keep_edges=np.arange(nl.n_edges))
    prob = _prob(case, nl)
    say(f"[cpu] oracle double backward cfg={k}")
    ref = prob.double_backward(*u)
    tol = TOL[case.cfg["dtype"]]
    errs = {"g_hat": rel(res["g_hat"].cpu().numpy(), ref["g_hat"]),
            "h_hat": rel(res["h_hat"].cpu().numpy(), ref["x_hat"]),
            "Y_hat": rel(np.stack([res["Y_hat"][e] for e in range(nl.n_edges)]), ref["y_hat"]),
            "R_hat": rel(np.stack([res["R_hat"][e] for e in range(nl.n_edges)]), ref["w_hat"])}
    say(f"[cmp] {errs}")
    assert all(v < tol for v in errs.values()), errs


def test_double_backward_medium_sampled():
    case = Case(3)
    nl = case.nbr()
    rp = case.oracle_csr()[0]
    u = cotangents(case, nl.n_edges, 43)
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, case.N - 1], rng.choice(case.N, 30, replace=False)]))
    erow = rows[np.unique(np.linspace(0, len(rows) - 1, 12).round().astype(int))]
    edges = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in erow])
    res = run_double(case, nl, u, keep_edges=edges)
    prob = _prob(case, nl)
    say(f"[cpu] oracle double backward, medium sample ({len(rows)} rows, {len(edges)} edges)")
    g, x = prob.double_backward_rows(rows, *u)
    b = prob.double_backward_edges(edges, *u)
    tol = TOL[case.cfg["dtype"]]
    assert rel(res["g_hat"][rows].cpu().numpy(), g) < tol
    assert rel(res["h_hat"][rows].cpu().numpy(), x) < tol
    assert rel(np.stack([res["Y_hat"][int(e)] for e in edges]), b["y_hat"]) < tol
    assert rel(np.stack([res["R_hat"][int(e)] for e in edges]), b["w_hat"]) < tol


def test_double_backward_chunked_and_deterministic():
    case = Case(1)
    nl = case.nbr()
    u = cotangents(case, nl.n_edges, 44)
    a = run_double(case, nl, u, chunks=1, keep_edges=np.arange(0, nl.n_edges, 101))
    b = run_double(case, nl, u, chunks=4, keep_edges=np.arange(0, nl.n_edges, 101))
    c = run_double(case, nl, u, chunks=1, keep_edges=np.arange(0, nl.n_edges, 101))
    # rows of R shared by edge pairs, in 4 chunks: the same bits
    case.ctx = tpc.Context(tpc.spec_for(case.cfg, pair_radial=True))
    d = run_double(case, nl, u, chunks=4, keep_edges=np.arange(0, nl.n_edges, 101))
    for key in ("g_hat", "h_hat"):
        assert torch().equal(a[key], b[key]), key
        assert torch().equal(a[key], c[key]), key
        assert torch().equal(a[key], d[key]), key
    for e in a["Y_hat"]:
        np.testing.assert_array_equal(a["Y_hat"][e], b["Y_hat"][e])
        np.testing.assert_array_equal(a["R_hat"][e], c["R_hat"][e])
        np.testing.assert_array_equal(a["Y_hat"][e], d["Y_hat"][e])
        np.testing.assert_array_equal(a["R_hat"][e], d["R_hat"][e])


def test_double_backward_refuses_summed_outputs():
    case = Case(8)
    nl = case.nbr()
    u = cotangents(case, nl.n_edges, 45)
    t = torch()
    out, eb = case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, 1.0)
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.conv_double_bwd(nl, case.h, 1.0, case.G, eb, *[t.from_numpy(x).cuda() for x in u])
    assert ei.value.status == 2
