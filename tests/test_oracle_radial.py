"""Pins of the oracle's radial pieces: closed forms, a library routine,
boundary conditions and derivatives."""
import numpy as np
import scipy.special as sps

from oracle import radial


def test_envelope_boundary_conditions():
    assert radial.envelope(0.0) == 1.0
    assert abs(radial.envelope(1.0)) < 1e-15
    assert abs(radial.envelope_dx(1.0)) < 1e-13
    # second derivative at 1 by the analytic polynomial: 2nd derivative of
    # 1 - 21 x^5 + 35 x^6 - 15 x^7
    d2 = -21 * 20 + 35 * 30 - 15 * 42
    assert d2 == 0
    x = np.linspace(0.0, 1.0, 11)
    np.testing.assert_allclose(radial.envelope(x), 1 - 21 * x**5 + 35 * x**6 - 15 * x**7, atol=1e-15)


def test_bessel_is_scaled_spherical_j0():
    rc = 5.0
    r = np.linspace(0.3, 4.99, 37)
    b = radial.bessel(r, rc)
    for n in range(1, 9):
        k = n * np.pi / rc
        ref = np.sqrt(2.0 / rc) * k * sps.spherical_jn(0, k * r)
        np.testing.assert_allclose(b[:, n - 1], ref, rtol=1e-13)


def test_derivatives_by_central_differences():
    rc = 6.0
    r = np.linspace(0.8, 5.9, 23)
    e = 1e-6
    np.testing.assert_allclose(radial.bessel_dr(r, rc),
                               (radial.bessel(r + e, rc) - radial.bessel(r - e, rc)) / (2 * e), atol=1e-7)
    np.testing.assert_allclose(radial.edge_features_dr(r, rc),
                               (radial.edge_features(r + e, rc) - radial.edge_features(r - e, rc)) / (2 * e),
                               atol=1e-7)
    z = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(radial.silu_dz(z), (radial.silu(z + e) - radial.silu(z - e)) / (2 * e), atol=1e-8)


def test_weights_vanish_at_the_cutoff():
    # bias-free MLP with SiLU(0) = 0 and ef(r_c) = 0  =>  R(r_c) = 0
    rng = np.random.default_rng(0)
    W = [rng.standard_normal((8, 16)), rng.standard_normal((16, 16)), rng.standard_normal((16, 40))]
    R, _ = radial.mlp_forward(radial.edge_features(np.array([4.0]), 4.0), W)
    assert np.abs(R).max() < 1e-13


def test_mlp_input_gradient_by_differences():
    rng = np.random.default_rng(1)
    W = [rng.standard_normal((8, 16)) / 3, rng.standard_normal((16, 16)) / 4, rng.standard_normal((16, 40)) / 4]
    ef = rng.standard_normal((5, 8))
    dR = rng.standard_normal((5, 40))
    g = radial.mlp_input_grad(dR, ef, W)
    e = 1e-6
    for k in range(8):
        d = np.zeros(8)
        d[k] = e
        fp = (radial.mlp_forward(ef + d, W)[0] * dR).sum(1)
        fm = (radial.mlp_forward(ef - d, W)[0] * dR).sum(1)
        np.testing.assert_allclose(g[:, k], (fp - fm) / (2 * e), atol=1e-7)


def test_envelope_factored_form_is_the_polynomial():
    """The envelope in the form (1-x)^3 sum_{k<p} C(k+2,2) x^k equals the
    polynomial 1 - (p+1)(p+2)/2 x^p + p(p+2) x^(p+1) - p(p+1)/2 x^(p+2) exactly
    (rational arithmetic), its derivative is -p(p+1)(p+2)/2 x^(p-1) (1-x)^2,
    and near x = 1 it keeps the relative accuracy the expanded sum loses."""
    from fractions import Fraction
    from math import comb
    for p in (3, 5, 6):
        for xq in (Fraction(0), Fraction(1, 3), Fraction(5, 7), Fraction(99, 100), Fraction(1)):
            expanded = 1 - Fraction((p + 1) * (p + 2), 2) * xq ** p + p * (p + 2) * xq ** (p + 1) \
                - Fraction(p * (p + 1), 2) * xq ** (p + 2)
            factored = (1 - xq) ** 3 * sum(comb(k + 2, 2) * xq ** k for k in range(p))
            assert expanded == factored
            assert abs(radial.envelope(float(xq), p) - float(expanded)) <= 1e-15
            dexp = -Fraction((p + 1) * (p + 2) * p, 2) * xq ** (p - 1) + p * (p + 2) * (p + 1) * xq ** p \
                - Fraction(p * (p + 1) * (p + 2), 2) * xq ** (p + 1)
            assert abs(radial.envelope_dx(float(xq), p) - float(dexp)) <= 1e-13
    # relative accuracy near the cutoff: exact value from rationals
    x = 1 - 2.0 ** -20
    exact = float((1 - Fraction(x)) ** 3 * sum(comb(k + 2, 2) * Fraction(x) ** k for k in range(5)))
    assert abs(radial.envelope(x) - exact) <= 1e-14 * abs(exact)
    assert abs(radial.envelope_expanded(x) - exact) > 0.5 * abs(exact)   # all relative accuracy lost
