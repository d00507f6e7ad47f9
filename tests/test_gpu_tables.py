"""Piecewise Chebyshev radial tables on the GPU (FastMACE page "Rewrites and
precision options", section "Radial network", radial_tables): the fitted
table against the oracle's float64 fit, the certificate, refusal of an
uncertified table, and the convolution with the table against the oracle
built on the same table (and on the radial network it stands in for)."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import TOL, Case, rel, run_chunked, say, torch
from oracle import radial

pytestmark = pytest.mark.gpu

PIECES, DEGREE = 32, 8


def _table_case(k, pieces=PIECES, degree=DEGREE):
    case = Case(k)
    case.ctx = tpc.Context(tpc.spec_for(case.cfg, table=(pieces, degree)))
    return case


@pytest.mark.parametrize("k", [1, 3])
def test_fit_is_certified_and_matches_the_oracle_fit(k):
    case = _table_case(k)
    say(f"[gpu] radial_table_fit cfg={k} pieces={PIECES} degree={DEGREE}")
    table, cert = case.ctx.radial_table_fit(case.W)
    torch().cuda.synchronize()
    say(f"[cmp] certificate ratios {cert}")
    assert cert[0] <= 1.0 and cert[1] <= 1.0
    pc = case.ctx.r_width
    got = table.cpu().numpy().astype(np.float64).reshape(PIECES, 2 * DEGREE + 1, pc)
    ref = radial.chebyshev_table(case.d["W"], case.cfg["r_cut"], PIECES, DEGREE)
    # value coefficients: float32 rounding of the same float64 fit
    assert rel(got[:, :DEGREE + 1], ref) < 1e-6
    # derivative series: values of the derivative at sample points
    r = np.random.default_rng(9).uniform(0.0, case.cfg["r_cut"], 200)
    _, dref = radial.chebyshev_eval(ref, r, case.cfg["r_cut"])
    h = case.cfg["r_cut"] / PIECES
    q = np.minimum((r / h).astype(int), PIECES - 1)
    x = 2 * (r - q * h) / h - 1
    T = np.polynomial.chebyshev.chebvander(x, DEGREE - 1)            # [n_r, DEGREE]
    dgot = np.einsum("ek,ekm->em", T, got[q, DEGREE + 1:])
    assert rel(dgot, dref) < 1e-6


def test_uncertified_table_is_refused():
    case = _table_case(1, pieces=2, degree=3)
    with pytest.raises(tpc.TpcError) as ei:
        case.ctx.radial_table_fit(case.W)
    assert ei.value.status == 4 and "not certified" in ei.value.message
    _, cert = case.ctx.radial_table_fit(case.W, check=False)
    assert cert[0] > 1.0


def test_float64_tables_are_held_to_float64_rounding():
    # the tiny float64 system: no table of this size reaches float64 rounding,
    # so the certificate refuses it
    case = _table_case(0, pieces=256, degree=12)
    _, cert = case.ctx.radial_table_fit(case.W, check=False)
    say(f"[cmp] float64 certificate {cert}")
    assert cert[0] > 1.0 or cert[1] > 1.0


@pytest.mark.parametrize("k", [1])
def test_convolution_with_the_table(k):
    case = _table_case(k)
    table, cert = case.ctx.radial_table_fit(case.W)
    W_net = case.W
    case.W = [table]                       # the table context takes one weights pointer
    nl = case.nbr()
    res = run_chunked(case, nl, chunks=1, keep_edges=np.arange(nl.n_edges))
    ref_csr = case.oracle_csr()
    prob = case.oracle(ref_csr)
    # the oracle on the same table (its own float64 fit)
    prob.table = radial.chebyshev_table(case.d["W"], case.cfg["r_cut"], PIECES, DEGREE)
    say(f"[cpu] oracle with the table cfg={k}")
    out_ref = prob.forward()
    b = prob.backward()
    tol = TOL[case.cfg["dtype"]]
    errs = {"out": rel(res["out"].cpu().numpy(), out_ref), "dh": rel(res["dh"].cpu().numpy(), b["dh"]),
            "dR": rel(np.stack([res["dR"][e] for e in range(nl.n_edges)]), b["dR"]),
            "g_edge": rel(res["g_edge"].cpu().numpy(), b["g"]),
            "forces": rel(res["forces"].cpu().numpy(), b["F"])}
    # and against the radial network the table stands in for
    prob.table = None
    b_net = prob.backward()
    errs["forces_vs_network"] = rel(res["forces"].cpu().numpy(), b_net["F"])
    say(f"[cmp] {errs}")
    assert all(v < tol for v in errs.values()), errs
    case.W = W_net
