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


def envelope(x, p=P_ENVELOPE):
    x = np.asarray(x, dtype=np.float64)
    return (1.0 - (p + 1) * (p + 2) / 2.0 * x ** p + p * (p + 2) * x ** (p + 1)
            - p * (p + 1) / 2.0 * x ** (p + 2))


def envelope_dx(x, p=P_ENVELOPE):
    x = np.asarray(x, dtype=np.float64)
    return (-(p + 1) * (p + 2) / 2.0 * p * x ** (p - 1) + p * (p + 2) * (p + 1) * x ** p
            - p * (p + 1) / 2.0 * (p + 2) * x ** (p + 1))


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
