"""Real coupling coefficients of an admissible path, from Gaunt integrals.

FlashCart paper, §2 "Irreducible Cartesian tensors": for an admissible path
(l1, l2) -> l3 the equivariant bilinear maps V_l1 x V_l2 -> V_l3 form a
one-dimensional space.  Any non-zero equivariant coupling therefore fixes the
path's coefficients up to one scale.  The real Gaunt integral

    G_{m1 m2 m3} = integral over the sphere of Y_{l1 m1} Y_{l2 m2} Y_{l3 m3}

is such a coupling (it is invariant under rotations acting on all three
indices) and it is non-zero exactly when l1 + l2 + l3 is even.  The reading
used here normalises it to unit Frobenius norm per path,

    C^p = G / ||G||_F ,

with the sign fixed by the integral itself and no further path weight, so
that (1,1) -> 0 gives delta_{m1 m2} / sqrt(3).

The integral is evaluated by quadrature that is exact for the integrand:
Gauss-Legendre nodes in cos(theta) (the integrand is a polynomial of degree
<= l1+l2+l3 in cos(theta) once the phi integral is non-zero) times a uniform
grid in phi (exact for trigonometric polynomials of degree < n_phi).
"""
from __future__ import annotations

import functools

import numpy as np

from .sh import sh

ZERO_TOL = 1e-14


@functools.lru_cache(maxsize=64)
def _quadrature(n_theta=16, n_phi=32):
    t, wt = np.polynomial.legendre.leggauss(n_theta)
    phi = 2.0 * np.pi * np.arange(n_phi) / n_phi
    wp = np.full(n_phi, 2.0 * np.pi / n_phi)
    T, P = np.meshgrid(t, phi, indexing="ij")
    s = np.sqrt(1.0 - T * T)
    pts = np.stack([s * np.cos(P), s * np.sin(P), T], axis=-1).reshape(-1, 3)
    w = (wt[:, None] * wp[None, :]).reshape(-1)
    return pts, w


def gaunt(l1, l2, l3):
    """Real Gaunt integral G[m1, m2, m3] (component-normalised harmonics)."""
    pts, w = _quadrature()
    lmax = max(l1, l2, l3)
    Y = sh(pts, lmax)
    a = Y[:, l1 * l1:(l1 + 1) ** 2]
    b = Y[:, l2 * l2:(l2 + 1) ** 2]
    c = Y[:, l3 * l3:(l3 + 1) ** 2]
    return np.einsum("q,qi,qj,qk->ijk", w, a, b, c)


@functools.lru_cache(maxsize=128)
def coupling(l1, l2, l3):
    """C^p[m1, m2, m3] for an admissible path: unit-norm real Gaunt tensor."""
    g = gaunt(l1, l2, l3)
    g = g / np.linalg.norm(g)
    g[np.abs(g) < ZERO_TOL] = 0.0
    g.setflags(write=False)
    return g


def tables(layout):
    """Coupling tensors of every path of ``layout``, in path order."""
    return [coupling(*p) for p in layout.paths]
