"""Pins of the oracle's piecewise Chebyshev radial tables (FastMACE page
"Rewrites and precision options", section "Radial network", radial_tables):
the fit against numpy's Chebyshev interpolation, exact reproduction of
polynomials, the interpolation property, the derivative series against
differences, convergence to the radial MLP, and the convolution with a table
(forces by finite differences of the table-built forward)."""
import numpy as np
import pytest

import workloads
from oracle import conv, fd, nbr, paths, radial


@pytest.fixture(scope="module")
def small_weights():
    d = workloads.generate(1)
    return d["W"], d["cfg"]["r_cut"]


def test_fit_matches_numpy_chebinterpolate(small_weights):
    W, rc = small_weights
    a, b, deg = 1.5, 2.0, 7
    cols = [0, 17, 500, 1279]
    f = lambda r: radial.radial_weights(r, W, rc)[:, cols]
    c = radial.chebyshev_fit(f, a, b, deg)
    for k, col in enumerate(cols):
        ref = np.polynomial.chebyshev.chebinterpolate(
            lambda x: radial.radial_weights(a + (b - a) * (np.asarray(x) + 1) / 2, W, rc)[:, col], deg)
        np.testing.assert_allclose(c[:, k], ref, rtol=0, atol=1e-13 * np.abs(ref).max())


def test_polynomials_are_reproduced_with_their_derivatives():
    rng = np.random.default_rng(3)
    coef = rng.standard_normal((6, 2))                    # degree 5, two columns
    rc, pieces, deg = 4.0, 3, 5
    f = lambda r: np.stack([np.polynomial.polynomial.polyval(r, coef[:, m]) for m in range(2)], -1)
    df = lambda r: np.stack([np.polynomial.polynomial.polyval(
        r, np.polynomial.polynomial.polyder(coef[:, m])) for m in range(2)], -1)
    h = rc / pieces
    table = np.stack([radial.chebyshev_fit(f, q * h, (q + 1) * h, deg) for q in range(pieces)])
    r = np.concatenate([np.linspace(0.0, rc, 101), [h, 2 * h]])
    val, der = radial.chebyshev_eval(table, r, rc)
    np.testing.assert_allclose(val, f(r), rtol=0, atol=1e-11 * np.abs(f(r)).max())
    np.testing.assert_allclose(der, df(r), rtol=0, atol=1e-10 * np.abs(df(r)).max())


def test_interpolation_property_at_the_nodes(small_weights):
    W, rc = small_weights
    pieces, deg = 8, 6
    table = radial.chebyshev_table(W, rc, pieces, deg)
    h = rc / pieces
    n = deg + 1
    x = np.cos(np.pi * (np.arange(n) + 0.5) / n)
    for q in (0, 3, 7):
        r = q * h + h * (x + 1) / 2
        val, _ = radial.chebyshev_eval(table, r, rc)
        ref = radial.radial_weights(r, W, rc)
        np.testing.assert_allclose(val, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_radial_derivative_by_differences(small_weights):
    W, rc = small_weights
    r = np.linspace(0.7, 5.8, 9)
    d = 1e-3
    f = lambda x: radial.radial_weights(x, W, rc)
    fd5 = (-f(r + 2 * d) + 8 * f(r + d) - 8 * f(r - d) + f(r - 2 * d)) / (12 * d)
    der = radial.radial_weights_dr(r, W, rc)
    np.testing.assert_allclose(der, fd5, rtol=0, atol=1e-8 * np.abs(der).max())


def test_tables_converge_to_the_radial_network(small_weights):
    W, rc = small_weights
    r = np.random.default_rng(4).uniform(0.0, rc, 400)
    ref = radial.radial_weights(r, W, rc)
    dref = radial.radial_weights_dr(r, W, rc)
    errs = []
    for pieces in (8, 32, 128):
        table = radial.chebyshev_table(W, rc, pieces, 8)
        val, der = radial.chebyshev_eval(table, r, rc)
        errs.append((np.abs(val - ref).max() / np.abs(ref).max(), np.abs(der - dref).max() / np.abs(dref).max()))
    assert errs[0][0] > errs[1][0] > errs[2][0]
    assert errs[2][0] < 1e-9 and errs[2][1] < 1e-7


def test_table_convolution_forces_by_differences():
    """With a table standing in for the radial network, the backward's forces
    (dL/dr from the table's derivative series) equal 5-point differences of
    the table-built forward."""
    d = workloads.generate(0)
    c = d["cfg"]
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"])
    rp, src, shift = nbr.binned(d["pos"], d["cell"], c["r_cut"])
    # fine enough that the derivative jumps at piece ends stay below the
    # stencil's own error when a stencil crosses one
    table = radial.chebyshev_table(d["W"], c["r_cut"], 64, 10)
    prob = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"], 1.0, d["G"],
                        radial_table=table)
    b = prob.backward()
    F = fd.fd_forces(prob, np.arange(len(d["pos"])), delta=1e-3)
    assert np.abs(F - b["F"]).max() / np.abs(b["F"]).max() < 1e-7
    # and it is close to the network's forces (the table is accurate)
    prob_mlp = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"], 1.0, d["G"])
    assert np.abs(prob_mlp.backward()["F"] - b["F"]).max() / np.abs(b["F"]).max() < 1e-5
