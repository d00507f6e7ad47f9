"""Finite-difference forces and virial of the surrogate scalar L = sum(G * out).

Forces are the negative position gradient of a scalar (FlashCart paper, §2
"Machine-learned interatomic potentials").  With the neighbour list held
fixed, moving atom k changes only the edges incident to it -- its own row and
the edges whose sender it is (the Frost model card measures exactly this
edge locality on a real model) -- so the change of L is evaluated on those
edges alone, which keeps round-off low.  A 5-point central stencil is used:

    dL/dx ~ (L(x-2d) - 8 L(x-d) + 8 L(x+d) - L(x+2d)) / (12 d)
"""
from __future__ import annotations

import numpy as np

from .conv import Problem, edges_of_rows


def _local_L(prob: Problem, e, n_copies):
    """L restricted to edges ``e`` (n_copies stacked position variants)."""
    L, Cn, s = prob.L, prob.L.C, prob.scale
    _, _, Y, _, R = prob.edge_terms(e)
    _, T = prob.products(e, Y)
    Gr = np.asarray(prob.G[prob.recv[e]], dtype=np.float64)
    tot = np.zeros(len(e))
    for p in range(L.n_paths):
        Rp = R[:, p * Cn:(p + 1) * Cn]
        tot += s * np.einsum("eku,eu,eku->e", Gr[:, L.out_rows(p), :], Rp, T[p], optimize=True)
    return tot.reshape(n_copies, -1).sum(1)


def fd_forces(prob: Problem, atoms, delta=1e-3):
    """F[k, d] = -dL/dx_{k,d} for each atom in ``atoms`` (CSR fixed)."""
    atoms = np.asarray(atoms, dtype=np.int64)
    F = np.zeros((len(atoms), 3))
    base = prob.pos.copy()
    for n, k in enumerate(atoms):
        e_in, _ = edges_of_rows(prob.row_ptr, [k])
        e_out = np.nonzero(prob.src == k)[0]
        e = np.unique(np.concatenate([e_in, e_out]))
        for d in range(3):
            vals = []
            for c in (-2, -1, 1, 2):
                prob.pos = base.copy()
                prob.pos[k, d] += c * delta
                vals.append(_local_L(prob, e, 1)[0])
            prob.pos = base
            F[n, d] = -(vals[0] - 8 * vals[1] + 8 * vals[2] - vals[3]) / (12 * delta)
    prob.pos = base
    return F


def fd_virial(prob: Problem, delta=1e-4):
    """W[a, b] = dL/d(eps_ab) by a 5-point central stencil in each strain
    component.  The strain x -> (I + eps) x moves the positions and the cell
    rows together (pet-jax README, "Conventions"); the CSR is held fixed and L
    is summed over every edge."""
    e = np.arange(len(prob.src))
    pos0, cell0 = prob.pos.copy(), prob.cell.copy()
    W = np.zeros((3, 3))
    for a in range(3):
        for b in range(3):
            vals = []
            for c in (-2, -1, 1, 2):
                F = np.eye(3)
                F[a, b] += c * delta
                prob.pos = pos0 @ F.T
                prob.cell = cell0 @ F.T
                vals.append(_local_L(prob, e, 1)[0])
            W[a, b] = (vals[0] - 8 * vals[1] + 8 * vals[2] - vals[3]) / (12 * delta)
    prob.pos, prob.cell = pos0, cell0
    return W
