"""Radial basis, envelope and radial MLP: edge length -> per-path weights.

Each edge's length is mapped by a small MLP to one weight per coupling path
and channel for that edge's product (FastMACE page "Rewrites and precision
options", section "Radial network"; FlashCart §2 writes these weights as
W_{l1 l2 l}(r_uv)).

Readings (the pages name the pieces but print no formulas):
  * Bessel basis, n = 1..8:  b_n(r) = sqrt(2/r_c) sin(n pi r / r_c) / r
  * polynomial envelope with p = 5, x = r / r_c:
        u(x) = 1 - (p+1)(p+2)/2 x^p + p(p+2) x^(p+1) - p(p+1)/2 x^(p+2)
    so that u(1) = u'(1) = u''(1) = 0
  * MLP input ef_n = u(r/r_c) b_n(r); hidden layers a_k = SiLU(a_{k-1} W_k)
    with SiLU(z) = z sigmoid(z); no biases; the last layer is linear:
        R = a_{L-1} W_L,  R[e, p*C + u]
  * weights arrive already scaled (their 1/sqrt(fan_in) lives in the values)
"""
from __future__ import annotations

import numpy as np

P_ENVELOPE = 5
N_BESSEL = 8


def bessel(r, r_cut, n=N_BESSEL):
    k = np.arange(1, n + 1) * np.pi / r_cut
    r = np.asarray(r, dtype=np.float64)[..., None]
    return np.sqrt(2.0 / r_cut) * np.sin(k * r) / r


def bessel_dr(r, r_cut, n=N_BESSEL):
    k = np.arange(1, n + 1) * np.pi / r_cut
    r = np.asarray(r, dtype=np.float64)[..., None]
    return np.sqrt(2.0 / r_cut) * (k * np.cos(k * r) / r - np.sin(k * r) / (r * r))


def envelope_expanded(x, p=P_ENVELOPE):
    """u(x) = 1 - (p+1)(p+2)/2 x^p + p(p+2) x^(p+1) - p(p+1)/2 x^(p+2)."""
    x = np.asarray(x, dtype=np.float64)
    return (1.0 - (p + 1) * (p + 2) / 2.0 * x ** p + p * (p + 2) * x ** (p + 1)
            - p * (p + 1) / 2.0 * x ** (p + 2))


def envelope(x, p=P_ENVELOPE):
    """The same polynomial in the form (1-x)^3 sum_{k<p} C(k+2, 2) x^k (for
    p = 5: (1-x)^3 (1 + 3x + 6x^2 + 10x^3 + 15x^4)): u has a triple zero at
    x = 1, and this form keeps its relative accuracy there, where the
    expanded terms of size ~ p^2 cancel to a value of size (1-x)^3."""
    x = np.asarray(x, dtype=np.float64)
    q = np.zeros_like(x)
    for k in range(p - 1, -1, -1):
        q = q * x + (k + 2) * (k + 1) / 2.0
    return (1.0 - x) ** 3 * q


def envelope_dx(x, p=P_ENVELOPE):
    """u'(x) = -p(p+1)(p+2)/2 x^(p-1) (1-x)^2."""
    x = np.asarray(x, dtype=np.float64)
    return -p * (p + 1) * (p + 2) / 2.0 * x ** (p - 1) * (1.0 - x) ** 2


def edge_features(r, r_cut):
    """ef[e, n] = u(r/r_c) b_n(r)."""
    return envelope(np.asarray(r) / r_cut)[..., None] * bessel(r, r_cut)


def edge_features_dr(r, r_cut):
    x = np.asarray(r) / r_cut
    return (envelope_dx(x)[..., None] / r_cut * bessel(r, r_cut)
            + envelope(x)[..., None] * bessel_dr(r, r_cut))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def silu_dz(z):
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def mlp_forward(ef, W):
    """R = a_{L-1} W_L; returns (R, list of hidden pre-activations z_k)."""
    a = np.asarray(ef, dtype=np.float64)
    zs = []
    for Wk in W[:-1]:
        z = a @ np.asarray(Wk, dtype=np.float64)
        zs.append(z)
        a = silu(z)
    return a @ np.asarray(W[-1], dtype=np.float64), zs


def mlp_input_grad(dR, ef, W):
    """d(sum dR * R)/d ef: the chain back through W_L, SiLU', ..., W_1."""
    _, zs = mlp_forward(ef, W)
    d = np.asarray(dR, dtype=np.float64) @ np.asarray(W[-1], dtype=np.float64).T
    for Wk, z in zip(reversed(W[:-1]), reversed(zs)):
        d = (d * silu_dz(z)) @ np.asarray(Wk, dtype=np.float64).T
    return d


# ---- piecewise Chebyshev tables of the radial chain -------------------------
# FastMACE page "Rewrites and precision options", section "Radial network",
# option radial_tables: the chain distance -> edge weights is replaced by
# piecewise Chebyshev tables fitted when the plan is built, certified against
# a float64 evaluation of the same weights (values and first derivatives; see
# the "certified" class in the section on rewrite classes).  Here the pieces
# split [0, r_cut] into equal intervals; on each, the radial weights R(r) are
# interpolated at the n = degree + 1 Chebyshev-Gauss points.

def radial_weights(r, W, r_cut):
    """R(r) [len(r), P*C] in float64 through the basis, envelope and MLP."""
    R, _ = mlp_forward(edge_features(np.asarray(r, dtype=np.float64), r_cut), W)
    return R


def chebyshev_fit(f, a, b, degree):
    """Coefficients c_0..c_d of the degree-d interpolant of f on [a, b] at the
    Chebyshev-Gauss points x_j = cos(pi (j + 1/2) / n), j = 0..n-1, n = d + 1
    (mapped to r = a + (b - a)(x + 1) / 2):
        c_k = (2 - [k = 0]) / n * sum_j f(r_j) cos(pi k (j + 1/2) / n).
    f maps an array of r to an array [len(r), m]; returns [n, m]."""
    n = degree + 1
    j = np.arange(n)
    x = np.cos(np.pi * (j + 0.5) / n)
    r = a + (b - a) * (x + 1.0) / 2.0
    fv = np.asarray(f(r), dtype=np.float64)                    # [n, m]
    k = np.arange(n)
    T = np.cos(np.pi * np.outer(k, j + 0.5) / n)               # T_k(x_j)
    c = (2.0 / n) * (T @ fv)
    c[0] /= 2.0
    return c


def chebyshev_table(W, r_cut, pieces, degree):
    """[pieces, degree + 1, P*C] coefficients of R(r) on the equal pieces of
    [0, r_cut]."""
    h = r_cut / pieces
    return np.stack([chebyshev_fit(lambda r: radial_weights(r, W, r_cut), q * h, (q + 1) * h, degree)
                     for q in range(pieces)])


def chebyshev_eval(table, r, r_cut):
    """Values and r-derivatives [len(r), P*C] of a table at r in [0, r_cut]:
    the piece q = floor(r / h) (the last piece also takes r = r_cut), local
    x = 2 (r - q h) / h - 1, value sum_k c_k T_k(x), derivative
    (2 / h) sum_k c_k T_k'(x), with T_k(cos t) = cos(k t) and
    T_k'(x) = k U_{k-1}(x) (U_{k-1}(cos t) = sin(k t) / sin t)."""
    table = np.asarray(table, dtype=np.float64)
    P, n, m = table.shape
    r = np.asarray(r, dtype=np.float64)
    h = r_cut / P
    q = np.minimum(np.floor(r / h).astype(np.int64), P - 1)
    x = np.clip(2.0 * (r - q * h) / h - 1.0, -1.0, 1.0)
    # T_k and T_k' by the three-term recurrences
    Tk = np.zeros((len(r), n))
    dTk = np.zeros((len(r), n))
    Tk[:, 0] = 1.0
    if n > 1:
        Tk[:, 1] = x
        dTk[:, 1] = 1.0
    for k in range(2, n):
        Tk[:, k] = 2.0 * x * Tk[:, k - 1] - Tk[:, k - 2]
        dTk[:, k] = 2.0 * Tk[:, k - 1] + 2.0 * x * dTk[:, k - 1] - dTk[:, k - 2]
    c = table[q]                                               # [len(r), n, m]
    val = np.einsum("ek,ekm->em", Tk, c)
    der = np.einsum("ek,ekm->em", dTk, c) * (2.0 / h)
    return val, der


def radial_weights_dr(r, W, r_cut):
    """dR/dr [len(r), P*C] in float64 (chain rule through the MLP)."""
    ef = edge_features(np.asarray(r, dtype=np.float64), r_cut)
    def_dr = edge_features_dr(np.asarray(r, dtype=np.float64), r_cut)
    a, da = ef, def_dr
    for Wk in W[:-1]:
        z = a @ np.asarray(Wk, dtype=np.float64)
        dz = da @ np.asarray(Wk, dtype=np.float64)
        a, da = silu(z), silu_dz(z) * dz
    return da @ np.asarray(W[-1], dtype=np.float64)
