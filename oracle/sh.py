"""Real spherical harmonics of an edge direction, component normalised.

The direction tensor T_l(r_hat) of an edge (FlashCart paper, §2 "Equivariant
convolution and many-body correlations") is taken in its real spherical form
(FlashCart §2 "Irreducible Cartesian tensors": real spherical tensors and STF
tensors of rank l carry the same O(3) irrep).  The pages fix no convention;
the reading used here is

    Y_lm(r_hat) = sqrt(4 pi) N_lm P_l^{|m|}(cos theta) * { sqrt2 cos(m phi)   m > 0
                                                        { 1                 m = 0
                                                        { sqrt2 sin(|m| phi) m < 0
    N_lm = sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!)

with z the polar axis, m = -l..l, no Condon-Shortley phase, and component
normalisation sum_m Y_lm^2 = 2l+1 (so Y_00 = 1 and Y_1 = sqrt3 (y, z, x)).

The associated Legendre function is written as sin^m(theta) times the m-th
derivative of the Legendre polynomial P_l, and sin^m(theta) e^{i m phi} as
(x + i y)^m / r^m expanded into its real and imaginary polynomials.  Every
step is an analytic function of the Cartesian edge vector, so the gradient is
taken by complex-step differentiation, exact to rounding.
"""
from __future__ import annotations

import math

import numpy as np
from numpy.polynomial import legendre as _leg


def _re_im_power(x, y, m):
    """Real and imaginary parts of (x + i y)^m as real polynomials in x, y."""
    a = np.zeros_like(x)
    b = np.zeros_like(x)
    for k in range(m + 1):
        term = math.comb(m, k) * x ** (m - k) * y ** k
        if k % 4 == 0:
            a = a + term
        elif k % 4 == 1:
            b = b + term
        elif k % 4 == 2:
            a = a - term
        else:
            b = b - term
    return a, b


def sh(vec, lmax):
    """Y_lm(vec / |vec|) for l = 0..lmax, flattened as index l*l + (m + l).

    ``vec`` has shape [..., 3] and may be complex (complex-step derivative).
    """
    vec = np.asarray(vec)
    x, y, z = vec[..., 0], vec[..., 1], vec[..., 2]
    r = np.sqrt(x * x + y * y + z * z)
    t = z / r
    out = []
    for l in range(lmax + 1):
        coef = np.zeros(l + 1)
        coef[l] = 1.0                        # Legendre series of P_l
        for m in range(-l, l + 1):
            am = abs(m)
            d = _leg.legder(coef, am) if am else coef
            p = _leg.legval(t, d)           # d^|m| P_l / dt^|m| at cos(theta)
            norm = math.sqrt((2 * l + 1) * math.factorial(l - am) / math.factorial(l + am))
            if m == 0:
                ang = 1.0
            else:
                re, im = _re_im_power(x, y, am)
                ang = math.sqrt(2.0) * (re if m > 0 else im) / r ** am
            out.append(norm * p * ang)
    return np.stack(out, axis=-1)


def sh_grad(vec, lmax, step=1e-30):
    """d Y_lm / d vec, shape [..., (lmax+1)^2, 3], by complex-step differentiation."""
    vec = np.asarray(vec, dtype=np.float64)
    cols = []
    for k in range(3):
        v = vec.astype(np.complex128)
        v[..., k] += 1j * step
        cols.append(np.imag(sh(v, lmax)) / step)
    return np.stack(cols, axis=-1)
