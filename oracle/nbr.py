"""Periodic neighbour list as receiver-sorted CSR, and the reverse-edge index.

Definition (FlashCart paper, §2 "Equivariant convolution and many-body
correlations"): the neighbourhood of atom u holds every atom and periodic
image within the cutoff, except u itself in the reference cell; the edge
vector r_uv points from u to its neighbour v and includes the periodic
translation.  Edges are stored in receiver order with a row-pointer array and
a sender array (FlashCart §4 "Data layout"); an edge's identity is (receiver,
sender, image shift), as the Frost model card's edge keys are.

Readings fixed where the pages are silent:
  * an image shift S = (s1, s2, s3) translates the sender by s1 a1 + s2 a2 +
    s3 a3, the cell rows being a1, a2, a3;
  * the edge vector is evaluated in float64, component by component, in the
    order  (x_j - x_i) + ((s1 a1 + s2 a2) + s3 a3),  with no fused
    multiply-add, and d2 = (rx rx + ry ry) + rz rz;
  * an edge exists iff d2 < r_c * r_c (strict);
  * rows are in atom order; a row is sorted by (sender, s1, s2, s3).
"""
from __future__ import annotations

import math

import numpy as np


def heights(cell):
    """Perpendicular heights of the cell along each lattice direction."""
    a = np.asarray(cell, dtype=np.float64)
    vol = abs(np.linalg.det(a))
    return np.array([vol / np.linalg.norm(np.cross(a[(k + 1) % 3], a[(k + 2) % 3]))
                     for k in range(3)])


def shift_range(cell, r_cut):
    """Largest |s_k| any edge can have for wrapped positions (|df_k| <= 1)."""
    h = heights(cell)
    return [int(math.floor(r_cut / h[k] + 1.0 + 1e-9)) for k in range(3)]


def _vec(pos_i, pos_j, cell, S):
    """Edge vector with the fixed float64 operation order (no FMA in NumPy)."""
    a1, a2, a3 = cell[0], cell[1], cell[2]
    s1 = S[..., 0].astype(np.float64)[..., None]
    s2 = S[..., 1].astype(np.float64)[..., None]
    s3 = S[..., 2].astype(np.float64)[..., None]
    return (pos_j - pos_i) + ((s1 * a1 + s2 * a2) + s3 * a3)


def _d2(v):
    return (v[..., 0] * v[..., 0] + v[..., 1] * v[..., 1]) + v[..., 2] * v[..., 2]


def edge_vectors(pos, cell, recv, src, shift):
    return _vec(pos[recv], pos[src], np.asarray(cell, dtype=np.float64), shift)


def brute_force_rows(pos, cell, r_cut, receivers, block=None):
    """Edges of the given receivers by exhaustive search over atoms and shifts.

    Returns a list of (src [k], shift [k,3]) per receiver, each sorted by
    (src, s1, s2, s3).  Receivers are evaluated a few at a time only to bound
    memory; every candidate gets the same float64 test.
    """
    pos = np.asarray(pos, dtype=np.float64)
    cell = np.asarray(cell, dtype=np.float64)
    N = len(pos)
    K = shift_range(cell, r_cut)
    S = np.stack(np.meshgrid(*[np.arange(-k, k + 1) for k in K], indexing="ij"),
                 -1).reshape(-1, 3).astype(np.int64)
    rc2 = r_cut * r_cut
    js = np.repeat(np.arange(N), len(S))
    Ss = np.tile(S, (N, 1))
    receivers = np.asarray(list(receivers), dtype=np.int64)
    if block is None:
        block = max(1, 4_000_000 // max(1, len(js)))
    out = []
    for b0 in range(0, len(receivers), block):
        rb = receivers[b0:b0 + block]
        v = _vec(pos[rb][:, None, :], pos[js][None, :, :], cell, Ss[None, :, :])
        keep = _d2(v) < rc2
        keep &= ~((js[None, :] == rb[:, None]) & np.all(Ss == 0, axis=1)[None, :])
        for n in range(len(rb)):
            j_k, s_k = js[keep[n]], Ss[keep[n]]
            order = np.lexsort((s_k[:, 2], s_k[:, 1], s_k[:, 0], j_k))
            out.append((j_k[order].astype(np.int32), s_k[order].astype(np.int32)))
    return out


def brute_force(pos, cell, r_cut):
    """Full receiver-sorted CSR by exhaustive search (small systems only)."""
    rows = brute_force_rows(pos, cell, r_cut, range(len(pos)))
    return _to_csr(rows)


def _to_csr(rows):
    counts = np.array([len(r[0]) for r in rows], dtype=np.int64)
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    src = np.concatenate([r[0] for r in rows]) if rows else np.zeros(0, np.int32)
    shift = np.concatenate([r[1] for r in rows]) if rows else np.zeros((0, 3), np.int32)
    return row_ptr.astype(np.int32), src.astype(np.int32), shift.astype(np.int32)


def binned(pos, cell, r_cut, margin=1e-6):
    """Same edge set as brute_force, found through cell bins.

    Bins are at least r_cut * (1 + margin) wide in every lattice direction, so
    every edge joins bins that are at most one bin apart (images included);
    the edge test itself is the same float64 expression as brute_force.
    """
    pos = np.asarray(pos, dtype=np.float64)
    cell = np.asarray(cell, dtype=np.float64)
    N = len(pos)
    h = heights(cell)
    nb = np.maximum(1, np.floor(h / (r_cut * (1.0 + margin))).astype(np.int64))
    K = np.ceil(r_cut * (1.0 + margin) * nb / h).astype(np.int64)
    f = pos @ np.linalg.inv(cell)
    b = np.minimum(np.maximum(np.floor(f * nb).astype(np.int64), 0), nb - 1)
    flat = (b[:, 0] * nb[1] + b[:, 1]) * nb[2] + b[:, 2]
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=int(np.prod(nb)))
    cap = int(counts.max()) if N else 0
    nbin = int(np.prod(nb))
    start = np.zeros(nbin + 1, dtype=np.int64)
    np.cumsum(counts, out=start[1:])
    table = np.full((nbin, cap), -1, dtype=np.int64)
    slot = np.arange(N) - start[flat[order]]
    table[flat[order], slot] = order
    bins = np.stack(np.unravel_index(np.arange(nbin), tuple(nb)), -1)
    rc2 = r_cut * r_cut
    recv_l, src_l, sh_l = [], [], []
    offs = np.stack(np.meshgrid(*[np.arange(-k, k + 1) for k in K], indexing="ij"),
                    -1).reshape(-1, 3)
    for d in offs:
        tgt = bins + d
        S = np.floor_divide(tgt, nb)
        tb = tgt - S * nb
        tflat = (tb[:, 0] * nb[1] + tb[:, 1]) * nb[2] + tb[:, 2]
        I = table[:, :, None]                         # receivers [nbin, cap, 1]
        J = table[tflat][:, None, :]                  # candidates [nbin, 1, cap]
        ok = (I >= 0) & (J >= 0)
        I_b, J_b = np.broadcast_arrays(I, J)
        sel = np.nonzero(ok)
        ii, jj = I_b[sel], J_b[sel]
        SS = np.broadcast_to(S[:, None, None, :], ok.shape + (3,))[sel]
        v = _vec(pos[ii], pos[jj], cell, SS)
        keep = _d2(v) < rc2
        keep &= ~((ii == jj) & np.all(SS == 0, axis=1))
        recv_l.append(ii[keep])
        src_l.append(jj[keep])
        sh_l.append(SS[keep])
    recv = np.concatenate(recv_l)
    src = np.concatenate(src_l)
    shift = np.concatenate(sh_l).astype(np.int64)
    o = np.lexsort((shift[:, 2], shift[:, 1], shift[:, 0], src, recv))
    recv, src, shift = recv[o], src[o], shift[o]
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(np.bincount(recv, minlength=N), out=row_ptr[1:])
    return row_ptr.astype(np.int32), src.astype(np.int32), shift.astype(np.int32)


def receivers_of(row_ptr):
    return np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr)).astype(np.int64)


def _keys(recv, src, shift, N):
    s = shift.astype(np.int64) + 128
    return (((recv.astype(np.int64) * N + src) * 256 + s[:, 0]) * 256 + s[:, 1]) * 256 + s[:, 2]


def reverse_index(row_ptr, src, shift):
    """rev[e] = index of the edge (j <- i, -S) for e = (i <- j, S); -1 if absent."""
    N = len(row_ptr) - 1
    recv = receivers_of(row_ptr)
    k = _keys(recv, src.astype(np.int64), shift, N)
    q = _keys(src.astype(np.int64), recv, -shift.astype(np.int64), N)
    pos = np.searchsorted(k, q)
    pos_c = np.minimum(pos, len(k) - 1)
    found = (len(k) > 0) & (k[pos_c] == q) if len(k) else np.zeros(0, bool)
    return np.where(found, pos_c, -1).astype(np.int32)
