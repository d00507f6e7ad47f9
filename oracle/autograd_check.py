"""A second, independently written forward in torch-CPU float64, for autograd.

FlashCart verifies its hand-derived derivatives against a separately
generated PyTorch forward differentiated by automatic differentiation
(FlashCart paper, §3 "Symbolic derivatives").  The same check is applied to
this oracle: the forward below is built from torch primitives (index_add for
the receiver sum, einsum for the path contraction), the radial MLP and the
edge geometry are rebuilt from the page-level definitions, and torch.autograd
produces dL/dh, dL/dR, dL/dY and dL/dpos for comparison with the hand-written
backward in ``conv``.  The coupling tensors and harmonics come from the oracle
(they are inputs of the product here, pinned separately).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import cg
from .paths import Layout


def _sh_torch(v, lmax):
    """Component-normalised real harmonics via the same Legendre recipe."""
    x, y, z = v[:, 0], v[:, 1], v[:, 2]
    r = torch.sqrt(x * x + y * y + z * z)
    t = z / r
    cols = []
    for l in range(lmax + 1):
        coef = np.zeros(l + 1)
        coef[l] = 1.0
        for m in range(-l, l + 1):
            am = abs(m)
            d = np.polynomial.legendre.legder(coef, am) if am else coef
            pc = np.polynomial.legendre.leg2poly(d)       # power-series coefficients
            p = torch.zeros_like(t)
            for k in range(len(pc) - 1, -1, -1):
                p = p * t + float(pc[k])
            norm = math.sqrt((2 * l + 1) * math.factorial(l - am) / math.factorial(l + am))
            if m == 0:
                ang = torch.ones_like(t)
            else:
                re = torch.zeros_like(t)
                im = torch.zeros_like(t)
                for k in range(am + 1):
                    term = math.comb(am, k) * x ** (am - k) * y ** k
                    if k % 4 == 0:
                        re = re + term
                    elif k % 4 == 1:
                        im = im + term
                    elif k % 4 == 2:
                        re = re - term
                    else:
                        im = im - term
                ang = math.sqrt(2.0) * (re if m > 0 else im) / r ** am
            cols.append(norm * p * ang)
    return torch.stack(cols, dim=-1)


def forward_torch(layout: Layout, pos, cell, recv, src, shift, h, W, r_cut, scale):
    """L-ready forward: returns (out, Y, R) with autograd graph to pos, h, R, Y."""
    a1, a2, a3 = cell[0], cell[1], cell[2]
    sf = shift.to(torch.float64)
    v = (pos[src] - pos[recv]) + ((sf[:, 0:1] * a1 + sf[:, 1:2] * a2) + sf[:, 2:3] * a3)
    r = torch.sqrt((v * v).sum(-1))
    Y = _sh_torch(v, layout.sh_lmax)
    n = torch.arange(1, 9, dtype=torch.float64) * math.pi / r_cut
    b = math.sqrt(2.0 / r_cut) * torch.sin(n * r[:, None]) / r[:, None]
    x = r / r_cut
    u = 1 - 21 * x ** 5 + 35 * x ** 6 - 15 * x ** 7
    a = u[:, None] * b
    for Wk in W[:-1]:
        a = torch.nn.functional.silu(a @ Wk)
    R = a @ W[-1]
    return v, Y, R


def convolve_torch(layout: Layout, Y, R, h, recv, src, N, scale):
    Cn = layout.C
    out = torch.zeros((N, layout.d_out, Cn), dtype=torch.float64)
    hs = h[src]
    for p, (l1, l2, l3) in enumerate(layout.paths):
        C = torch.from_numpy(np.array(cg.coupling(l1, l2, l3)))
        T = torch.einsum("abk,eau,eb->eku", C, hs[:, l1 * l1:(l1 + 1) ** 2],
                         Y[:, l2 * l2:(l2 + 1) ** 2])
        msg = R[:, None, p * Cn:(p + 1) * Cn] * T
        rows = torch.tensor(layout.out_rows(p))
        part = torch.zeros((N, 2 * l3 + 1, Cn), dtype=torch.float64).index_add(0, recv, msg)
        out[:, rows, :] = out[:, rows, :] + scale * part
    return out


def grads(layout: Layout, pos, cell, row_ptr, src, shift, h, W, G, r_cut, scale):
    """Autograd dL/dh, dL/dR, dL/dY, forces for L = sum(G * out)."""
    N = len(pos)
    recv = torch.from_numpy(np.repeat(np.arange(N), np.diff(row_ptr)).astype(np.int64))
    src_t = torch.from_numpy(np.asarray(src, dtype=np.int64))
    sh_t = torch.from_numpy(np.asarray(shift, dtype=np.int64))
    pos_t = torch.tensor(np.asarray(pos, dtype=np.float64), requires_grad=True)
    cell_t = torch.tensor(np.asarray(cell, dtype=np.float64))
    h_t = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    W_t = [torch.tensor(np.asarray(w, dtype=np.float64)) for w in W]
    G_t = torch.tensor(np.asarray(G, dtype=np.float64))
    v, Y, R = forward_torch(layout, pos_t, cell_t, recv, src_t, sh_t, h_t, W_t, r_cut, scale)
    Y.retain_grad()
    R.retain_grad()
    out = convolve_torch(layout, Y, R, h_t, recv, src_t, N, scale)
    L = (G_t * out).sum()
    L.backward()
    return dict(out=out.detach().numpy(), dh=h_t.grad.numpy(), dR=R.grad.numpy(),
                dY=Y.grad.numpy(), F=-pos_t.grad.numpy(), L=float(L.detach()))


def double_grads(layout: Layout, pos, cell, row_ptr, src, shift, h, W, G, r_cut, scale, uh, uY, uR):
    """Autograd of the VJP (FlashCart paper, section 3 "Symbolic
    derivatives": the VJP itself is differentiated for training on forces).
    The VJP (dh, dY, dR) of L = sum(G * out) is taken with create_graph, then
    Lam = <uh, dh> + <uY, dY> + <uR, dR> is differentiated with respect to G,
    h, Y and R, all four treated as independent inputs of the product (Y and R
    are leaves here, computed once from the geometry)."""
    N = len(pos)
    recv = torch.from_numpy(np.repeat(np.arange(N), np.diff(row_ptr)).astype(np.int64))
    src_t = torch.from_numpy(np.asarray(src, dtype=np.int64))
    sh_t = torch.from_numpy(np.asarray(shift, dtype=np.int64))
    pos_t = torch.tensor(np.asarray(pos, dtype=np.float64))
    cell_t = torch.tensor(np.asarray(cell, dtype=np.float64))
    W_t = [torch.tensor(np.asarray(w, dtype=np.float64)) for w in W]
    with torch.no_grad():
        _, Y0, R0 = forward_torch(layout, pos_t, cell_t, recv, src_t, sh_t, None, W_t, r_cut, scale)
    Y = Y0.clone().requires_grad_(True)
    R = R0.clone().requires_grad_(True)
    h_t = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    G_t = torch.tensor(np.asarray(G, dtype=np.float64), requires_grad=True)
    out = convolve_torch(layout, Y, R, h_t, recv, src_t, N, scale)
    L = (G_t * out).sum()
    dh, dY, dR = torch.autograd.grad(L, (h_t, Y, R), create_graph=True)
    lam = ((torch.tensor(np.asarray(uh, dtype=np.float64)) * dh).sum()
           + (torch.tensor(np.asarray(uY, dtype=np.float64)) * dY).sum()
           + (torch.tensor(np.asarray(uR, dtype=np.float64)) * dR).sum())
    gG, gh, gY, gR = torch.autograd.grad(lam, (G_t, h_t, Y, R))
    return dict(g_hat=gG.numpy(), x_hat=gh.numpy(), y_hat=gY.numpy(), w_hat=gR.numpy(),
                dh=dh.detach().numpy(), dY=dY.detach().numpy(), dR=dR.detach().numpy(),
                lam=float(lam.detach()))
