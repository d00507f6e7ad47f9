"""Pins of the oracle's real spherical harmonics against a library and closed forms."""
import math

import numpy as np
import pytest
import scipy.special as sps

from oracle import sh

LMAX = 4


def _dirs(n, seed=0):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def _scipy_real(l, m, v):
    """Component-normalised real harmonic from scipy's complex Y_l^m (which has
    the Condon-Shortley phase); the sign (-1)^m removes it."""
    theta = np.arccos(np.clip(v[:, 2], -1, 1))
    phi = np.arctan2(v[:, 1], v[:, 0])
    am = abs(m)
    y = sps.sph_harm_y(l, am, theta, phi)
    c = math.sqrt(4 * math.pi)
    if m == 0:
        return c * y.real
    if m > 0:
        return c * math.sqrt(2) * (-1) ** am * y.real
    return c * math.sqrt(2) * (-1) ** am * y.imag


def test_matches_scipy():
    v = _dirs(500)
    Y = sh.sh(v * 2.7, LMAX)          # non-unit input: only the direction matters
    for l in range(LMAX + 1):
        for m in range(-l, l + 1):
            ref = _scipy_real(l, m, v)
            np.testing.assert_allclose(Y[:, l * l + m + l], ref, atol=1e-12, rtol=0)


def test_component_normalisation():
    Y = sh.sh(_dirs(300, 1), LMAX)
    for l in range(LMAX + 1):
        np.testing.assert_allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1), 2 * l + 1, rtol=1e-13)


def test_l1_closed_form_and_pole():
    v = _dirs(50, 2)
    Y = sh.sh(v, 3)
    np.testing.assert_allclose(Y[:, 0], 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Y[:, 1:4], math.sqrt(3) * v[:, [1, 2, 0]], atol=1e-14)
    z = sh.sh(np.array([[0.0, 0.0, 1.0]]), 3)[0]
    for l in range(4):
        np.testing.assert_allclose(z[l * l + l], math.sqrt(2 * l + 1), rtol=1e-14)


def test_parity():
    v = _dirs(100, 3)
    Yp, Ym = sh.sh(v, LMAX), sh.sh(-v, LMAX)
    for l in range(LMAX + 1):
        s = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose(Ym[:, s], (-1) ** l * Yp[:, s], atol=1e-13)


def test_orthogonality_by_lebedev_free_quadrature():
    # product Gauss-Legendre x trapezoid grid, different sizes from the oracle's
    t, wt = np.polynomial.legendre.leggauss(12)
    phi = 2 * np.pi * np.arange(25) / 25
    T, P = np.meshgrid(t, phi, indexing="ij")
    s = np.sqrt(1 - T * T)
    pts = np.stack([s * np.cos(P), s * np.sin(P), T], -1).reshape(-1, 3)
    w = (wt[:, None] * np.full(25, 2 * np.pi / 25)[None, :]).reshape(-1)
    Y = sh.sh(pts, LMAX)
    gram = np.einsum("q,qa,qb->ab", w, Y, Y)
    np.testing.assert_allclose(gram, 4 * np.pi * np.eye(len(gram)), atol=1e-12)


def test_gradient_against_central_differences():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((40, 3)) * 2.0
    g = sh.sh_grad(v, LMAX)
    eps = 1e-6
    for k in range(3):
        dv = np.zeros(3)
        dv[k] = eps
        fd = (sh.sh(v + dv, LMAX) - sh.sh(v - dv, LMAX)) / (2 * eps)
        np.testing.assert_allclose(g[..., k], fd, atol=1e-7)
    # Y depends on the direction only: the radial derivative vanishes
    np.testing.assert_allclose(np.einsum("elk,ek->el", g, v), 0.0, atol=1e-12)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_rotation_acts_linearly_within_l(l):
    # Y_l(Q r) = D_l(Q) Y_l(r) with an orthogonal D_l
    rng = np.random.default_rng(10 + l)
    q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    v = _dirs(60, 5)
    s = slice(l * l, (l + 1) ** 2)
    A, B = sh.sh(v, l)[:, s], sh.sh(v @ q.T, l)[:, s]
    D, *_ = np.linalg.lstsq(A, B, rcond=None)
    np.testing.assert_allclose(A @ D, B, atol=1e-12)
    np.testing.assert_allclose(D.T @ D, np.eye(2 * l + 1), atol=1e-12)
