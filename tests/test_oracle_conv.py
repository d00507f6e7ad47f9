"""Pins of the oracle's convolution, backward and forces: autograd of an
independent forward, finite differences, linearity identities, closed forms on
two-atom systems, and O(3), translation and permutation symmetry."""
import math

import numpy as np
import pytest

import workloads
from oracle import conv, fd, nbr, paths, sh


def _problem(k, csr=None, **over):
    d = workloads.generate(k)
    c = d["cfg"]
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"])
    pos, cell = over.get("pos", d["pos"]), over.get("cell", d["cell"])
    rp, src, shift = csr if csr is not None else nbr.binned(d["pos"], d["cell"], c["r_cut"])
    s = conv.scale_for(c, len(pos), rp[-1])
    return conv.Problem(L, pos, cell, rp, src, shift, over.get("h", d["h"]), d["W"],
                        c["r_cut"], s, d["G"]), d


@pytest.fixture(scope="module")
def tiny():
    prob, d = _problem(0)
    return prob, d, prob.forward(), prob.backward()


def test_backward_matches_autograd(tiny):
    from oracle import autograd_check as ag
    prob, d, out, b = tiny
    a = ag.grads(prob.L, prob.pos, prob.cell, prob.row_ptr, prob.src, prob.shift,
                 d["h"], d["W"], d["G"], prob.r_cut, prob.scale)
    np.testing.assert_allclose(out, a["out"], rtol=0, atol=1e-13 * np.abs(out).max())
    for k in ("dh", "dR", "dY", "F"):
        np.testing.assert_allclose(b[k], a[k], rtol=0, atol=1e-12 * np.abs(a[k]).max())


def test_forces_by_finite_differences(tiny):
    prob, d, out, b = tiny
    F = fd.fd_forces(prob, np.arange(len(prob.pos)), delta=1e-3)
    assert np.abs(F - b["F"]).max() / np.abs(b["F"]).max() < 1e-7


def test_virial_by_strain_differences(tiny):
    """Virial from the edge gradients against differences of L under a
    homogeneous strain of positions and cell (an independent route: only the
    forward is evaluated)."""
    prob, d, out, b = tiny
    W = prob.virial_from(b["g"])
    Wfd = fd.fd_virial(prob, delta=1e-4)
    assert np.abs(W - Wfd).max() / np.abs(W).max() < 1e-7
    # the surrogate is not rotation invariant, so W need not be symmetric;
    # a dropped transpose would show here
    assert np.abs(W - W.T).max() > 1e-3 * np.abs(W).max()


def test_virial_two_atom_closed_form():
    """Two atoms, l = 0 only: L = s R(r) (G_0 h_1 + G_1 h_0) summed over
    channels for the pair, so W = (dL/dr) r_hat r^T summed over both edges,
    each edge vector seen from its own receiver."""
    L = paths.Layout(0, 0, 0, 3)
    h = np.random.default_rng(6).standard_normal((2, 1, 3))
    prob, pos = _two_atoms(L, h)
    prob.G = np.random.default_rng(7).standard_normal((2, 1, 3))
    b = prob.backward()
    W = prob.virial_from(b["g"])
    # both edge vectors are +-(x1 - x0); g_e is parallel to r_e for l = 0, so
    # W = sum_e |g_e| |r_e| rhat rhat^T: symmetric, rank one along the bond
    rhat = (pos[1] - pos[0]) / np.linalg.norm(pos[1] - pos[0])
    mag = sum(float(np.dot(b["g"][e], prob.rvec(np.array([e]))[0])) for e in range(2))
    np.testing.assert_allclose(W, mag * np.outer(rhat, rhat), rtol=0, atol=1e-13 * abs(mag))
    Wfd = fd.fd_virial(prob, delta=1e-4)
    np.testing.assert_allclose(W, Wfd, rtol=0, atol=1e-8 * abs(mag))


@pytest.fixture(scope="module")
def tiny_summed():
    """The tiny system with path-summed outputs and its own upstream gradient."""
    d = workloads.generate(0)
    c = d["cfg"]
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"], sum_paths=True)
    rp, src, shift = nbr.binned(d["pos"], d["cell"], c["r_cut"])
    G = np.random.default_rng(8).standard_normal((c["N"], L.d_out, c["C"]))
    prob = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"], 1.0, G)
    return prob, d


def test_summed_layout_sums_the_paths_of_each_rank(tiny_summed):
    """Each l3 block of the summed output is the sum of that rank's path
    blocks of the separate output (whose layout the closed forms pin)."""
    prob, d = tiny_summed
    Ls = prob.L
    assert Ls.d_out == sum(2 * l + 1 for l in sorted({p[2] for p in Ls.paths}))
    sep = conv.Problem(paths.Layout(Ls.l1max, Ls.sh_lmax, Ls.out_lmax, Ls.C), prob.pos, prob.cell,
                       prob.row_ptr, prob.src, prob.shift, d["h"], d["W"], prob.r_cut, 1.0)
    out_sep, out_sum = sep.forward(), prob.forward()
    ref = np.zeros_like(out_sum)
    for p in range(Ls.n_paths):
        ref[:, Ls.out_rows(p)] += out_sep[:, sep.L.out_rows(p)]
    np.testing.assert_allclose(out_sum, ref, rtol=0, atol=1e-13 * np.abs(ref).max())


def test_summed_layout_backward(tiny_summed):
    """Backward with summed outputs: autograd of the independent torch
    forward, 5-point difference forces, and <dh, h> = L."""
    from oracle import autograd_check as ag
    prob, d = tiny_summed
    b = prob.backward()
    a = ag.grads(prob.L, prob.pos, prob.cell, prob.row_ptr, prob.src, prob.shift, d["h"], d["W"],
                 prob.G, prob.r_cut, prob.scale)
    for k in ("dh", "dR", "dY", "F"):
        np.testing.assert_allclose(b[k], a[k], rtol=0, atol=1e-12 * np.abs(a[k]).max())
    F = fd.fd_forces(prob, np.arange(len(prob.pos)), delta=1e-3)
    assert np.abs(F - b["F"]).max() / np.abs(b["F"]).max() < 1e-7
    L = float((prob.G * prob.forward()).sum())
    assert abs(float((b["dh"] * d["h"]).sum()) - L) < 1e-10 * abs(L)


def test_linearity_identities(tiny):
    # L is linear in each of h, R and Y separately
    prob, d, out, b = tiny
    Lval = float((d["G"] * out).sum())
    _, _, Y, _, R = prob.edge_terms(np.arange(len(prob.src)))
    assert abs(float((b["dh"] * d["h"]).sum()) - Lval) < 1e-12 * abs(Lval)
    assert abs(float((b["dR"] * R).sum()) - Lval) < 1e-12 * abs(Lval)
    assert abs(float((b["dY"] * Y).sum()) - Lval) < 1e-12 * abs(Lval)
    np.testing.assert_allclose(b["F"].sum(0), 0.0, atol=1e-12 * np.abs(b["F"]).max())


def _wigner_D(l, q):
    v = np.random.default_rng(11).standard_normal((60, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    s = slice(l * l, (l + 1) ** 2)
    D, *_ = np.linalg.lstsq(sh.sh(v, l)[:, s], sh.sh(v @ q.T, l)[:, s], rcond=None)
    return D.T


def _rotate_feats(x, D_of_l, blocks):
    y = x.copy()
    for l, rows in blocks:
        y[:, rows, :] = np.einsum("ab,nbu->nau", D_of_l(l), x[:, rows, :])
    return y


@pytest.mark.parametrize("improper", [False, True])
def test_o3_equivariance(tiny, improper):
    prob, d, out, _ = tiny
    L = prob.L
    q, _ = np.linalg.qr(np.random.default_rng(21).standard_normal((3, 3)))
    q *= np.sign(np.linalg.det(q))
    if improper:
        q = -q                                   # includes the inversion
    D = {l: _wigner_D(l, q) for l in range(4)}
    if improper:                                 # natural parity: inversion acts as (-1)^l
        for l in D:
            np.testing.assert_allclose(_wigner_D(l, -np.eye(3)), (-1) ** l * np.eye(2 * l + 1), atol=1e-12)
    in_blocks = [(l, list(range(l * l, (l + 1) ** 2))) for l in range(L.l1max + 1)]
    h2 = _rotate_feats(d["h"], D.get, in_blocks)
    csr = (prob.row_ptr, prob.src, prob.shift)
    p2, _ = _problem(0, csr=csr, pos=d["pos"] @ q.T, cell=d["cell"] @ q.T, h=h2)
    out2 = p2.forward()
    # rotate the reference output block by block: rows of path p are (p, m3)
    want = out.copy()
    for p, (_, _, l3) in enumerate(L.paths):
        rows = L.out_rows(p)
        want[:, rows, :] = np.einsum("ab,nbu->nau", D[l3], out[:, rows, :])
    np.testing.assert_allclose(out2, want, atol=1e-11 * np.abs(out).max())


def test_translation_and_permutation(tiny):
    prob, d, out, _ = tiny
    csr = (prob.row_ptr, prob.src, prob.shift)
    p_t, _ = _problem(0, csr=csr, pos=d["pos"] + np.array([0.3, -0.2, 0.1]))
    np.testing.assert_allclose(p_t.forward(), out, atol=1e-12 * np.abs(out).max())
    perm = np.random.default_rng(2).permutation(len(d["pos"]))
    inv = np.argsort(perm)
    csr_p = nbr.binned(d["pos"][perm], d["cell"], prob.r_cut)
    p_p, _ = _problem(0, csr=csr_p, pos=d["pos"][perm], h=d["h"][perm])
    np.testing.assert_allclose(p_p.forward()[inv], out, atol=1e-12 * np.abs(out).max())


def _two_atoms(layout, h, d=1.7, rc=4.0):
    pos = np.array([[10.0, 10.0, 10.0], [10.0 + d * 0.6, 10.0 - d * 0.8, 10.0]])
    cell = np.eye(3) * 30.0
    rp, src, shift = nbr.brute_force(pos, cell, rc)
    rng = np.random.default_rng(3)
    W = [rng.standard_normal((8, 16)) / math.sqrt(8), rng.standard_normal((16, layout.n_paths * layout.C)) / 4]
    return conv.Problem(layout, pos, cell, rp, src, shift, h, W, rc, 1.0), pos


def test_scalar_path_closed_form():
    L = paths.Layout(0, 0, 0, 5)
    h = np.random.default_rng(4).standard_normal((2, 1, 5))
    prob, pos = _two_atoms(L, h)
    out = prob.forward()
    _, _, _, _, R = prob.edge_terms(np.arange(2))
    # out_i = R_e h_j (Y_00 = 1, C^{000} = 1)
    np.testing.assert_allclose(out[0, 0], R[0] * h[1, 0], rtol=1e-14)
    np.testing.assert_allclose(out[1, 0], R[1] * h[0, 0], rtol=1e-14)
    np.testing.assert_allclose(R[0], R[1], rtol=0, atol=0)


def test_dot_product_path_closed_form():
    L = paths.Layout(1, 1, 0, 4)
    assert L.paths == [(0, 0, 0), (1, 1, 0)]
    h = np.random.default_rng(5).standard_normal((2, 4, 4))
    h[:, 0, :] = 0.0                              # only the 1o part
    prob, pos = _two_atoms(L, h)
    out = prob.forward()
    _, _, _, _, R = prob.edge_terms(np.arange(2))
    rhat = (pos[1] - pos[0]) / np.linalg.norm(pos[1] - pos[0])
    rs = rhat[[1, 2, 0]]                           # (y, z, x) component order
    row = L.out_rows(1)[0]
    np.testing.assert_allclose(out[0, row], R[0, 4:8] * np.einsum("a,au->u", rs, h[1, 1:4]), rtol=1e-13)
    np.testing.assert_allclose(out[1, row], R[1, 4:8] * np.einsum("a,au->u", -rs, h[0, 1:4]), rtol=1e-13)


@pytest.mark.slow
def test_medium_slice_finite_differences():
    """Forces on atoms 0-63 of the medium system against 5-point differences."""
    prob, d = _problem(3)
    atoms = np.arange(64)
    F = prob.forces_atoms(atoms)
    Ffd = fd.fd_forces(prob, atoms, delta=1e-3)
    assert np.abs(F - Ffd).max() / np.abs(F).max() < 1e-7


@pytest.mark.parametrize("summed", [False, True])
def test_dh_atoms_matches_autograd(summed):
    """The sampled sender gradient (dh of chosen atoms, summed over the edges
    whose sender they are) against torch autograd of the independent forward,
    on every atom of the tiny system, with separate and path-summed outputs
    (FlashCart paper, section 3 "Symbolic derivatives": the input VJP)."""
    from oracle import autograd_check as ag
    d = workloads.generate(0)
    c = d["cfg"]
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"], summed)
    rp, src, shift = nbr.binned(d["pos"], d["cell"], c["r_cut"])
    G = d["G"] if not summed else np.random.default_rng(5).standard_normal((c["N"], L.d_out, c["C"]))
    prob = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"], 1.0, G)
    a = ag.grads(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], G, c["r_cut"], 1.0)
    atoms = np.arange(c["N"])
    dh = prob.dh_atoms(atoms)
    np.testing.assert_allclose(dh, a["dh"], rtol=0, atol=1e-12 * np.abs(a["dh"]).max())
    # a subset in shuffled order gives the same rows
    sub = np.random.default_rng(1).permutation(c["N"])[:9]
    np.testing.assert_allclose(prob.dh_atoms(sub), a["dh"][sub], rtol=0, atol=1e-12 * np.abs(a["dh"]).max())
    # the test separates sender from receiver grouping: the same per-edge
    # contributions summed by receiver are far from the gradient
    e = np.arange(len(src))
    by_recv = np.zeros_like(dh)
    np.add.at(by_recv, nbr.receivers_of(rp), prob.edge_backward(e)["dh_contrib"])
    assert np.abs(by_recv - a["dh"]).max() > 1e-3 * np.abs(a["dh"]).max()


def test_dh_atoms_small_sample_matches_full_backward():
    """On the small system (C = 128), dh of a spread sample of atoms from the
    sampled routine equals the rows of the full backward's dh (itself pinned to
    autograd on the tiny system above), so the per-atom edge selection and
    grouping hold on a large list too."""
    d = workloads.generate(1)
    c = d["cfg"]
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"])
    rp, src, shift = nbr.binned(d["pos"], d["cell"], c["r_cut"])
    prob = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"], 1.0, d["G"])
    atoms = np.unique(np.concatenate([[0, c["N"] - 1], np.random.default_rng(3).choice(c["N"], 14, replace=False)]))
    # the reference: every edge whose sender is in the sample, through the
    # full backward's edge routine, scattered by sender
    e = np.nonzero(np.isin(src, atoms))[0]
    contrib = prob.edge_backward(e)["dh_contrib"]
    ref = np.zeros((c["N"], L.d_in, c["C"]))
    np.add.at(ref, src[e], contrib)
    got = prob.dh_atoms(atoms)
    np.testing.assert_allclose(got, ref[atoms], rtol=0, atol=1e-13 * np.abs(ref).max())
    # <dh, h> over all atoms equals L (linearity in h) for the sampled rows' share:
    # sum over the sample of <dh_a, h_a> equals the L of the messages those
    # atoms send
    hs = np.asarray(d["h"], dtype=np.float64)
    lhs = float((got * hs[atoms]).sum())
    out_part = np.zeros((c["N"], L.d_out, c["C"]))
    _, _, Y, _, R = prob.edge_terms(e)
    _, T = prob.products(e, Y)
    recv = nbr.receivers_of(rp)[e]
    for p in range(L.n_paths):
        msg = R[:, None, p * c["C"]:(p + 1) * c["C"]] * T[p]
        acc = np.zeros((c["N"], msg.shape[1], c["C"]))
        np.add.at(acc, recv, msg)
        out_part[:, L.out_rows(p), :] += acc
    rhs = float((np.asarray(d["G"], dtype=np.float64) * out_part).sum())
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(rhs))


def _cotangents(prob, seed):
    rng = np.random.default_rng(seed)
    N, E, L = len(prob.pos), len(prob.src), prob.L
    return (rng.standard_normal((N, L.d_in, L.C)), rng.standard_normal((E, L.d_sh)),
            rng.standard_normal((E, L.n_paths * L.C)))


@pytest.fixture(scope="module")
def tiny_double(tiny):
    prob, d, out, b = tiny
    uh, uY, uR = _cotangents(prob, 21)
    return prob, d, b, (uh, uY, uR), prob.double_backward(uh, uY, uR)


def test_double_backward_matches_double_autograd(tiny_double):
    """VJP-of-VJP against torch autograd of the independent forward's VJP
    (FlashCart paper, section 3 "Symbolic derivatives")."""
    from oracle import autograd_check as ag
    prob, d, b, (uh, uY, uR), db = tiny_double
    a = ag.double_grads(prob.L, prob.pos, prob.cell, prob.row_ptr, prob.src, prob.shift, d["h"],
                        d["W"], d["G"], prob.r_cut, prob.scale, uh, uY, uR)
    for k in ("g_hat", "x_hat", "y_hat", "w_hat"):
        np.testing.assert_allclose(db[k], a[k], rtol=0, atol=1e-12 * np.abs(a[k]).max())


def test_double_backward_multilinearity(tiny_double):
    """Each VJP output is linear in G and in each of h, Y, R it depends on
    (dh does not depend on h, dY not on Y, dR not on R), so
    <g_hat, G> = Lam, <x_hat, h> = <uY, dY> + <uR, dR>,
    <y_hat, Y> = <uh, dh> + <uR, dR>, <w_hat, R> = <uh, dh> + <uY, dY>."""
    prob, d, b, (uh, uY, uR), db = tiny_double
    _, _, Y, _, R = prob.edge_terms(np.arange(len(prob.src)))
    t_h = float((uh * b["dh"]).sum())
    t_Y = float((uY * b["dY"]).sum())
    t_R = float((uR * b["dR"]).sum())
    scale = abs(t_h) + abs(t_Y) + abs(t_R)
    G = np.asarray(d["G"], dtype=np.float64)
    h = np.asarray(d["h"], dtype=np.float64)
    assert abs(float((db["g_hat"] * G).sum()) - (t_h + t_Y + t_R)) < 1e-12 * scale
    assert abs(float((db["x_hat"] * h).sum()) - (t_Y + t_R)) < 1e-12 * scale
    assert abs(float((db["y_hat"] * Y).sum()) - (t_h + t_R)) < 1e-12 * scale
    assert abs(float((db["w_hat"] * R).sum()) - (t_h + t_Y)) < 1e-12 * scale


def test_double_backward_rows_match_full(tiny_double):
    prob, d, b, (uh, uY, uR), db = tiny_double
    rows = np.array([0, 5, 17, 31])
    g, x = prob.double_backward_rows(rows, uh, uY, uR)
    np.testing.assert_allclose(g, db["g_hat"][rows], rtol=0, atol=1e-13 * np.abs(db["g_hat"]).max())
    np.testing.assert_allclose(x, db["x_hat"][rows], rtol=0, atol=1e-13 * np.abs(db["x_hat"]).max())
