"""The equivariant interaction convolution, its backward pass, and forces.

Forward (FlashCart paper, §2 "Equivariant convolution and many-body
correlations"): couple the sender's features h_{v l1} with the edge's
direction tensor along every admissible path (l1, l2) -> l3, weight the result
by the edge's radial weight for that path and channel, and sum over the
receiver's neighbourhood.  Written out, with s the neighbour normalisation
(s = 1, or 1/avg_num_neighbors where a configuration asks for it):

    out[i, (p,m3), u] = s * sum_{e in row i} R[e, p*C+u] *
                        sum_{m1,m2} C^p[m1,m2,m3] h[src_e, (l1,m1), u] Y[e, (l2,m2)]

This is the channelwise ("uvu") product: one weight per path and channel.

Backward of the surrogate scalar L = sum(G * out), G = dL/dout: since each
path's product is bilinear and the weight enters linearly, the input
gradients are the other factors contracted with G and the weight gradient is
the inner product of G with the unweighted product (FlashCart §3 "Symbolic
derivatives"):

    dR[e, p*C+u]   = s * sum_m3 G[i,(p,m3),u] * T[e,p,m3,u],
                     T[e,p,m3,u] = sum_{m1,m2} C^p h[src_e,m1,u] Y[e,m2]
    dY[e, (l2,m2)] = s * sum_p sum_u R[e,p,u] sum_{m1,m3} C^p h[src_e,m1,u] G[i,(p,m3),u]
    dh[j, (l1,m1), u] = s * sum_{e: src_e = j} sum_p R[e,p,u]
                            sum_{m2,m3} C^p Y[e,m2] G[recv_e,(p,m3),u]

Forces: F_u = -dL/dx_u (FlashCart §2 "Machine-learned interatomic
potentials").  With r_e = x_src - x_recv + shift (§2 neighbourhood
definition), g_e = dL/dr_e gives  F_k = sum_{e: recv_e = k} g_e
- sum_{e: src_e = k} g_e.  The edge gradient is
    g_e = sum_{lm} dY[e,lm] dY_lm/dr_e + (sum_n d(ef)[e,n] d ef_n/dr) r_hat_e,
with d(ef) from the radial MLP's input gradient.
"""
from __future__ import annotations

import numpy as np

from . import cg, nbr, radial, sh
from .paths import Layout


def row_chunks(row_ptr, rows, max_edges=8192):
    """Split a list of receivers into groups whose rows hold <= max_edges."""
    rows = np.asarray(rows, dtype=np.int64)
    deg = (row_ptr[rows + 1] - row_ptr[rows]).astype(np.int64)
    groups, cur, tot = [], [], 0
    for r, d in zip(rows, deg):
        if cur and tot + d > max_edges:
            groups.append(np.array(cur))
            cur, tot = [], 0
        cur.append(r)
        tot += d
    if cur:
        groups.append(np.array(cur))
    return groups


def edges_of_rows(row_ptr, rows):
    rows = np.asarray(rows, dtype=np.int64)
    if len(rows) == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    lo = row_ptr[rows].astype(np.int64)
    deg = (row_ptr[rows + 1] - row_ptr[rows]).astype(np.int64)
    e = np.concatenate([np.arange(a, a + d) for a, d in zip(lo, deg)]) if deg.sum() else np.zeros(0, np.int64)
    owner = np.repeat(np.arange(len(rows)), deg)
    return e.astype(np.int64), owner


class Problem:
    """Inputs of one convolution call, with per-edge quantities on demand."""

    def __init__(self, layout: Layout, pos, cell, row_ptr, src, shift, h, W,
                 r_cut, scale=1.0, G=None, radial_table=None):
        self.L = layout
        self.pos = np.asarray(pos, dtype=np.float64)
        self.cell = np.asarray(cell, dtype=np.float64)
        self.row_ptr = np.asarray(row_ptr, dtype=np.int64)
        self.src = np.asarray(src, dtype=np.int64)
        self.shift = np.asarray(shift, dtype=np.int64)
        self.h = h
        self.W = [np.asarray(w, dtype=np.float64) for w in W]
        self.r_cut = float(r_cut)
        self.scale = float(scale)
        self.G = G
        self.recv = nbr.receivers_of(self.row_ptr)
        self.C = cg.tables(layout)
        # optional piecewise Chebyshev table [pieces, degree+1, P*C] standing
        # in for the radial MLP (``radial.chebyshev_table``)
        self.table = None if radial_table is None else np.asarray(radial_table, dtype=np.float64)

    # ---- per-edge geometry and weights (FlashCart §2; radial module) -------
    def rvec(self, e):
        return nbr.edge_vectors(self.pos, self.cell, self.recv[e], self.src[e], self.shift[e])

    def edge_terms(self, e):
        v = self.rvec(e)
        r = np.sqrt((v * v).sum(-1))
        Y = sh.sh(v, self.L.sh_lmax)
        ef = radial.edge_features(r, self.r_cut)
        if self.table is not None:
            R, _ = radial.chebyshev_eval(self.table, r, self.r_cut)
        else:
            R, _ = radial.mlp_forward(ef, self.W)
        return v, r, Y, ef, R

    # ---- the unweighted path products T ------------------------------------
    def products(self, e, Y):
        hs = np.asarray(self.h[self.src[e]], dtype=np.float64)     # [E, d_in, C]
        T = []
        for p, (l1, l2, l3) in enumerate(self.L.paths):
            T.append(np.einsum("abk,eau,eb->eku", self.C[p], hs[:, self.L.in_slice(l1)],
                               Y[:, self.L.sh_slice(l2)], optimize=True))
        return hs, T

    # ---- forward ------------------------------------------------------------
    def forward_rows(self, rows, max_edges=8192):
        """out[rows] (float64) by the definition, one receiver group at a time."""
        L, Cn = self.L, self.L.C
        rows = np.asarray(rows, dtype=np.int64)
        out = np.zeros((len(rows), L.d_out, Cn))
        where = {int(r): k for k, r in enumerate(rows)}
        for grp in row_chunks(self.row_ptr, rows, max_edges):
            e, owner = edges_of_rows(self.row_ptr, grp)
            if len(e) == 0:
                continue
            _, _, Y, _, R = self.edge_terms(e)
            _, T = self.products(e, Y)
            for p in range(L.n_paths):
                msg = R[:, None, p * Cn:(p + 1) * Cn] * T[p]      # [E, 2l3+1, C]
                acc = np.zeros((len(grp),) + msg.shape[1:])
                np.add.at(acc, owner, msg)
                idx = [where[int(r)] for r in grp]
                out[np.ix_(idx, L.out_rows(p), np.arange(Cn))] += self.scale * acc
        return out

    def forward(self, max_edges=8192):
        return self.forward_rows(np.arange(len(self.pos)), max_edges)

    # ---- backward, per edge ------------------------------------------------
    def edge_backward(self, e):
        """dR, dY, d(ef), g and the edge's contribution to dh of its sender."""
        L, Cn, s = self.L, self.L.C, self.scale
        v, r, Y, ef, R = self.edge_terms(e)
        hs, T = self.products(e, Y)
        Gr = np.asarray(self.G[self.recv[e]], dtype=np.float64)      # [E, d_out, C]
        dR = np.zeros_like(R)
        dY = np.zeros_like(Y)
        dh_c = np.zeros_like(hs)
        for p, (l1, l2, l3) in enumerate(L.paths):
            Gp = Gr[:, L.out_rows(p), :]                               # [E, 2l3+1, C]
            Rp = R[:, p * Cn:(p + 1) * Cn]                             # [E, C]
            dR[:, p * Cn:(p + 1) * Cn] = s * np.einsum("eku,eku->eu", Gp, T[p])
            dY[:, L.sh_slice(l2)] += s * np.einsum("abk,eau,eku,eu->eb", self.C[p],
                                                   hs[:, L.in_slice(l1)], Gp, Rp, optimize=True)
            dh_c[:, L.in_slice(l1)] += s * Rp[:, None, :] * np.einsum(
                "abk,eb,eku->eau", self.C[p], Y[:, L.sh_slice(l2)], Gp, optimize=True)
        rhat = v / r[:, None]
        g = np.einsum("el,elk->ek", dY, sh.sh_grad(v, L.sh_lmax))
        if self.table is not None:
            # dL/dr through the table's own derivative series
            _, dRdr = radial.chebyshev_eval(self.table, r, self.r_cut)
            d_ef = None
            g += (dR * dRdr).sum(-1)[:, None] * rhat
        else:
            d_ef = radial.mlp_input_grad(dR, ef, self.W)
            g += (d_ef * radial.edge_features_dr(r, self.r_cut)).sum(-1)[:, None] * rhat
        return dict(dR=dR, dY=dY, d_ef=d_ef, g=g, dh_contrib=dh_c)

    def backward(self, max_edges=4096):
        """Full dR [E, P*C], dY [E, d_sh], dh [N, d_in, C], g [E, 3], F [N, 3]."""
        L = self.L
        E = len(self.src)
        N = len(self.pos)
        dR = np.zeros((E, L.n_paths * L.C))
        dY = np.zeros((E, L.d_sh))
        g = np.zeros((E, 3))
        dh = np.zeros((N, L.d_in, L.C))
        for lo in range(0, E, max_edges):
            e = np.arange(lo, min(E, lo + max_edges))
            b = self.edge_backward(e)
            dR[e], dY[e], g[e] = b["dR"], b["dY"], b["g"]
            np.add.at(dh, self.src[e], b["dh_contrib"])
        return dict(dR=dR, dY=dY, dh=dh, g=g, F=self.forces_from(g))

    # ---- VJP-of-VJP (double backward) ---------------------------------------
    def double_backward_edges(self, e, uh, uY, uR):
        """The VJP-of-VJP terms of edges ``e`` (FlashCart paper, §3 "Symbolic
        derivatives": training on forces differentiates through the VJP; §4
        "Receiver-sorted derivatives": the VJP-of-VJP runs over the same
        receiver-sorted edges).

        The VJP maps (h, Y, R, G) to (dh, dY, dR) above.  Given cotangents
        uh [N, d_in, C], uY [E, d_sh] and uR [E, P*C] of those three outputs,
        the scalar Lam = <uh, dh> + <uY, dY> + <uR, dR> is differentiated with
        respect to each VJP input.  Every output of the VJP is linear in G and
        in each of h, Y, R it depends on, so with the unweighted product
        T(a, y)[p, m3, u] = sum_{m1,m2} C^p a[m1,u] y[m2] (and i = recv_e,
        j = src_e):

          g_hat[i,(p,m3),u]  = s sum_{e in row i} ( uR[e,p,u] T(h_j, Y_e)
                                 + R[e,p,u] (T(h_j, uY_e) + T(uh_j, Y_e)) )
          w_hat[e,p,u]       = s sum_m3 G[i,(p,m3),u] (T(h_j,uY_e) + T(uh_j,Y_e))
          y_hat[e,(l2,m2)]   = s sum_p sum_u sum_{m1,m3} C^p G[i,(p,m3),u]
                                 ( uR[e,p,u] h[j,m1,u] + R[e,p,u] uh[j,m1,u] )
          x_hat[j,(l1,m1),u] = s sum_{e: src_e = j} sum_p sum_{m2,m3} C^p G[i,(p,m3),u]
                                 ( uR[e,p,u] Y[e,m2] + R[e,p,u] uY[e,m2] )

        (dh does not depend on h, dY not on Y, dR not on R.)  Returns the
        per-edge w_hat, y_hat, the per-edge message to g_hat of the receiver
        and the per-edge contribution to x_hat of the sender."""
        L, Cn, s = self.L, self.L.C, self.scale
        _, _, Y, _, R = self.edge_terms(e)
        hs = np.asarray(self.h[self.src[e]], dtype=np.float64)
        uhs = np.asarray(uh[self.src[e]], dtype=np.float64)
        uYe = np.asarray(uY[e], dtype=np.float64)
        uRe = np.asarray(uR[e], dtype=np.float64)
        Gr = np.asarray(self.G[self.recv[e]], dtype=np.float64)
        w_hat = np.zeros_like(R)
        y_hat = np.zeros_like(Y)
        g_msg = np.zeros((len(e), L.d_out, Cn))
        x_c = np.zeros_like(hs)
        for p, (l1, l2, l3) in enumerate(L.paths):
            Cp = self.C[p]
            a1, a2, rows = L.in_slice(l1), L.sh_slice(l2), L.out_rows(p)
            Rp, uRp = R[:, p * Cn:(p + 1) * Cn], uRe[:, p * Cn:(p + 1) * Cn]
            Gp = Gr[:, rows, :]
            T_hY = np.einsum("abk,eau,eb->eku", Cp, hs[:, a1], Y[:, a2], optimize=True)
            T_huY = np.einsum("abk,eau,eb->eku", Cp, hs[:, a1], uYe[:, a2], optimize=True)
            T_uhY = np.einsum("abk,eau,eb->eku", Cp, uhs[:, a1], Y[:, a2], optimize=True)
            g_msg[:, rows, :] += s * (uRp[:, None, :] * T_hY + Rp[:, None, :] * (T_huY + T_uhY))
            w_hat[:, p * Cn:(p + 1) * Cn] = s * np.einsum("eku,eku->eu", Gp, T_huY + T_uhY)
            y_hat[:, a2] += s * np.einsum("abk,eku,eau->eb", Cp, Gp,
                                          uRp[:, None, :] * hs[:, a1] + Rp[:, None, :] * uhs[:, a1],
                                          optimize=True)
            x_c[:, a1] += s * np.einsum("abk,eku,ebu->eau", Cp, Gp,
                                        uRp[:, None, :] * Y[:, a2, None] + Rp[:, None, :] * uYe[:, a2, None],
                                        optimize=True)
        return dict(w_hat=w_hat, y_hat=y_hat, g_msg=g_msg, x_contrib=x_c)

    def double_backward(self, uh, uY, uR, max_edges=4096):
        """g_hat [N, d_out, C], x_hat [N, d_in, C], y_hat [E, d_sh],
        w_hat [E, P*C] for the cotangents uh, uY, uR (see
        ``double_backward_edges``)."""
        L = self.L
        E, N = len(self.src), len(self.pos)
        g_hat = np.zeros((N, L.d_out, L.C))
        x_hat = np.zeros((N, L.d_in, L.C))
        y_hat = np.zeros((E, L.d_sh))
        w_hat = np.zeros((E, L.n_paths * L.C))
        for lo in range(0, E, max_edges):
            e = np.arange(lo, min(E, lo + max_edges))
            b = self.double_backward_edges(e, uh, uY, uR)
            w_hat[e], y_hat[e] = b["w_hat"], b["y_hat"]
            np.add.at(g_hat, self.recv[e], b["g_msg"])
            np.add.at(x_hat, self.src[e], b["x_contrib"])
        return dict(g_hat=g_hat, x_hat=x_hat, y_hat=y_hat, w_hat=w_hat)

    def double_backward_rows(self, rows, uh, uY, uR):
        """g_hat of receivers ``rows`` and x_hat of the atoms ``rows``
        (sampled pieces for large systems)."""
        rows = np.asarray(rows, dtype=np.int64)
        where = {int(r): k for k, r in enumerate(rows)}
        e_in, owner = edges_of_rows(self.row_ptr, rows)
        g = np.zeros((len(rows), self.L.d_out, self.L.C))
        if len(e_in):
            np.add.at(g, owner, self.double_backward_edges(e_in, uh, uY, uR)["g_msg"])
        e_out = self.edges_with_sender(rows)
        x = np.zeros((len(rows), self.L.d_in, self.L.C))
        if len(e_out):
            np.add.at(x, [where[int(j)] for j in self.src[e_out]],
                      self.double_backward_edges(e_out, uh, uY, uR)["x_contrib"])
        return g, x

    def forces_from(self, g):
        N = len(self.pos)
        F = np.zeros((N, 3))
        np.add.at(F, self.recv, g)
        np.add.at(F, self.src, -g)
        return F

    def virial_from(self, g):
        """Strain derivative of L from the edge gradients (see ``virial``)."""
        return virial(self.rvec(np.arange(len(self.src))), g)

    # ---- sampled pieces for large systems ---------------------------------
    def edges_with_sender(self, atoms):
        atoms = np.asarray(atoms, dtype=np.int64)
        return np.nonzero(np.isin(self.src, atoms))[0]

    def dh_atoms(self, atoms):
        """dh[atoms] from every edge whose sender is one of ``atoms``."""
        atoms = np.asarray(atoms, dtype=np.int64)
        e = self.edges_with_sender(atoms)
        where = {int(a): k for k, a in enumerate(atoms)}
        out = np.zeros((len(atoms), self.L.d_in, self.L.C))
        for lo in range(0, len(e), 4096):
            ee = e[lo:lo + 4096]
            b = self.edge_backward(ee)
            np.add.at(out, [where[int(j)] for j in self.src[ee]], b["dh_contrib"])
        return out

    def forces_atoms(self, atoms):
        atoms = np.asarray(atoms, dtype=np.int64)
        e_in, owner = edges_of_rows(self.row_ptr, atoms)
        e_out = self.edges_with_sender(atoms)
        where = {int(a): k for k, a in enumerate(atoms)}
        F = np.zeros((len(atoms), 3))
        if len(e_in):
            F_in = self.edge_backward(e_in)["g"]
            np.add.at(F, owner, F_in)
        if len(e_out):
            g_out = self.edge_backward(e_out)["g"]
            np.add.at(F, [where[int(j)] for j in self.src[e_out]], -g_out)
        return F


def virial(vec, g):
    """W[a, b] = dL/d(eps_ab) for a homogeneous strain x -> (I + eps) x applied
    to the positions and the cell rows together (the pet-jax README,
    "Conventions": the virial is the strain derivative of the energy; the
    FastMACE page, "Rewrites and precision options", Stress: one structure's
    strained cell).  With the neighbour list fixed, every edge vector becomes
    (I + eps) r_e, so by the chain rule through g_e = dL/dr_e

        W[a, b] = sum_e g_e[a] * r_e[b].

    ``vec`` [E, 3] are the edge vectors, ``g`` [E, 3] the edge gradients."""
    return np.einsum("ea,eb->ab", np.asarray(g, dtype=np.float64),
                     np.asarray(vec, dtype=np.float64))


def scale_for(cfg, n_atoms, n_edges):
    """s = 1, or N/E (= 1/avg_num_neighbors) where the configuration says so."""
    if cfg.get("scale") == "inv_avg_neighbors":
        return float(n_atoms) / float(n_edges)
    return 1.0
