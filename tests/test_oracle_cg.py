"""Pins of the oracle's coupling coefficients (closed forms, a library routine,
invariances and the FlashCart worked example)."""
import math
import os

import numpy as np
import pytest
from sympy.physics.wigner import real_gaunt

from oracle import cg, paths, sh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL = [(l1, l2, l3) for l1 in range(4) for l2 in range(4) for l3 in range(4)
       if paths.admissible(l1, l2, l3)]


def test_path_lists_of_the_configs():
    import workloads
    for k, c in workloads.CONFIGS.items():
        L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"], c.get("sum_paths", False))
        assert (L.n_paths, L.d_in, L.d_sh, L.d_out) == (c["n_paths"], c["d_in"], c["d_sh"], c["d_out"])
    L = paths.Layout(1, 2, 1, 8)
    assert L.paths == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 2, 1)]


def test_dot_product_closed_form():
    # (1,1) -> 0 is the dot product over sqrt(3)
    np.testing.assert_allclose(cg.coupling(1, 1, 0)[:, :, 0], np.eye(3) / math.sqrt(3), atol=1e-15)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_identity_paths(l):
    d = np.eye(2 * l + 1) / math.sqrt(2 * l + 1)
    np.testing.assert_allclose(cg.coupling(0, l, l)[0], d, atol=1e-14)
    np.testing.assert_allclose(cg.coupling(l, 0, l)[:, 0, :], d, atol=1e-14)
    np.testing.assert_allclose(cg.coupling(l, l, 0)[:, :, 0], d, atol=1e-14)


@pytest.mark.parametrize("p", ALL)
def test_matches_sympy_real_gaunt(p):
    l1, l2, l3 = p
    ref = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for a in range(2 * l1 + 1):
        for b in range(2 * l2 + 1):
            for c in range(2 * l3 + 1):
                ref[a, b, c] = float(real_gaunt(l1, l2, l3, a - l1, b - l2, c - l3))
    ref /= np.linalg.norm(ref)
    np.testing.assert_allclose(cg.coupling(*p), ref, atol=1e-14)


@pytest.mark.parametrize("p", ALL)
def test_norm_exchange_orthogonality(p):
    l1, l2, l3 = p
    C = cg.coupling(*p)
    assert abs(np.linalg.norm(C) - 1.0) < 1e-14
    # exchange symmetry of the inputs (FlashCart §3: exchanged paths share one expression)
    np.testing.assert_allclose(cg.coupling(l2, l1, l3), C.transpose(1, 0, 2), atol=1e-14)
    np.testing.assert_allclose(np.einsum("abk,abl->kl", C, C), np.eye(2 * l3 + 1) / (2 * l3 + 1), atol=1e-14)


def _wigner_D(l, q):
    rng = np.random.default_rng(99)
    v = rng.standard_normal((80, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    s = slice(l * l, (l + 1) ** 2)
    D, *_ = np.linalg.lstsq(sh.sh(v, l)[:, s], sh.sh(v @ q.T, l)[:, s], rcond=None)
    return D.T          # Y_l(Q r) = D Y_l(r)


@pytest.mark.parametrize("p", ALL)
def test_rotation_invariance(p):
    l1, l2, l3 = p
    q, _ = np.linalg.qr(np.random.default_rng(7).standard_normal((3, 3)))
    q *= np.sign(np.linalg.det(q))
    D1, D2, D3 = _wigner_D(l1, q), _wigner_D(l2, q), _wigner_D(l3, q)
    C = cg.coupling(*p)
    np.testing.assert_allclose(np.einsum("ai,bj,ck,ijk->abc", D1, D2, D3, C), C, atol=1e-12)


def _stf_112_from_page():
    terms = {}
    with open(os.path.join(GOLDEN, "stf_112.txt")) as f:
        for line in f:
            if line.startswith("#") or line.startswith("component") or not line.strip():
                continue
            a, b, c = line.split()
            terms[(a, b)] = float(c)
    return terms


def test_112_matches_the_cartesian_worked_example():
    """The spherical (1,1)->2 block equals, up to one overall scale, the
    Cartesian product "contract 0 pairs, symmetrise, remove the trace"; the
    page prints its xx component, which fixes the Cartesian side's scale."""
    terms = _stf_112_from_page()
    ax = {"x": 0, "y": 1, "z": 2}
    rng = np.random.default_rng(3)
    # the Cartesian product, scaled so that its xx component is the printed one
    kappa = None
    stf_to_sph = []
    pts = rng.standard_normal((40, 3))
    pts /= np.linalg.norm(pts, axis=1, keepdims=True)
    Y2 = sh.sh(pts, 2)[:, 4:9]
    quad = np.einsum("qa,qb->qab", pts, pts).reshape(len(pts), 9)
    K, *_ = np.linalg.lstsq(quad, Y2, rcond=None)     # Y_2m(r) = K_m : r r^T on |r| = 1
    K = K.T.reshape(5, 3, 3)
    K = 0.5 * (K + K.transpose(0, 2, 1))
    C = cg.coupling(1, 1, 2)
    for _ in range(20):
        x, y = rng.standard_normal(3), rng.standard_normal(3)
        S = 0.5 * (np.outer(x, y) + np.outer(y, x)) - np.eye(3) * (x @ y) / 3.0
        page_xx = sum(c * x[ax[a]] * y[ax[b]] for (a, b), c in terms.items())
        scale = page_xx / S[0, 0]
        assert abs(scale - 1.5) < 1e-12          # the page's product is 3/2 of the STF part
        cart = np.einsum("mab,ab->m", K, scale * S)
        sph = np.einsum("abk,a,b->k", C, x[[1, 2, 0]], y[[1, 2, 0]])
        r = sph / cart
        if kappa is None:
            kappa = r[0]
        np.testing.assert_allclose(r, kappa, rtol=1e-12)


def test_operation_count_close_to_the_page():
    """Weak pin: 3*nnz - (2 l3 + 1) over the 15 distinct couplings with l <= 3
    (exchanged paths counted once) against the page's 609 for sparse CG."""
    with open(os.path.join(GOLDEN, "opcount.txt")) as f:
        page = dict(line.split() for line in f if line.strip() and not line.startswith("#"))
    distinct = {tuple(sorted(p[:2])) + (p[2],) for p in ALL}
    assert len(distinct) == 15
    nnz = sum(int(np.count_nonzero(cg.coupling(*p))) for p in distinct)
    ops = sum(3 * int(np.count_nonzero(cg.coupling(*p))) - (2 * p[2] + 1) for p in distinct)
    assert nnz == 223
    assert abs(ops - int(page["sparse_clebsch_gordan"])) <= 1
