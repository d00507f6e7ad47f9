"""Pins of the oracle's neighbour list: brute force, closed-form cases,
symmetry, the binned search against brute force, and edge locality."""
import math

import numpy as np
import pytest

import workloads
from oracle import nbr


def test_single_atom_cubic_images():
    # one atom in a cube of side 3: with r_c in (3, 3*sqrt2) its only neighbours
    # are its six face images, each at distance 3
    pos = np.array([[0.5, 1.0, 2.0]])
    cell = np.eye(3) * 3.0
    rp, src, shift = nbr.brute_force(pos, cell, 3.5)
    assert rp.tolist() == [0, 6]
    assert src.tolist() == [0] * 6
    assert sorted(map(tuple, shift.tolist())) == sorted(
        [(-1, 0, 0), (1, 0, 0), (0, -1, 0), (0, 1, 0), (0, 0, -1), (0, 0, 1)])
    # rows are sorted by (src, s1, s2, s3)
    assert [tuple(s) for s in shift.tolist()] == sorted(tuple(s) for s in shift.tolist())


def test_two_atoms_count_closed_form():
    # two atoms 1 A apart in a big cube: exactly one edge each way, no images
    pos = np.array([[5.0, 5.0, 5.0], [6.0, 5.0, 5.0]])
    rp, src, shift = nbr.brute_force(pos, np.eye(3) * 20.0, 1.5)
    assert rp.tolist() == [0, 1, 2] and src.tolist() == [1, 0]
    assert not shift.any()
    # strict cutoff: at exactly r_c the pair is excluded
    rp, _, _ = nbr.brute_force(pos, np.eye(3) * 20.0, 1.0)
    assert rp.tolist() == [0, 0, 0]


def test_triclinic_against_direct_enumeration():
    rng = np.random.default_rng(1)
    cell = np.array([[6.0, 0.0, 0.0], [1.5, 5.5, 0.0], [-1.0, 0.7, 5.0]])
    f = rng.uniform(0, 1, (20, 3))
    pos = f @ cell
    rc = 4.2
    rp, src, shift = nbr.brute_force(pos, cell, rc)
    # independent enumeration over a generous shift box, plain Python
    K = 3
    for i in range(len(pos)):
        want = []
        for j in range(len(pos)):
            for s in np.ndindex(2 * K + 1, 2 * K + 1, 2 * K + 1):
                S = np.array(s) - K
                if i == j and not S.any():
                    continue
                v = pos[j] - pos[i] + S @ cell
                if math.sqrt(v @ v) < rc - 1e-9:
                    want.append((j,) + tuple(S))
        got = [(int(j),) + tuple(int(x) for x in s)
               for j, s in zip(src[rp[i]:rp[i + 1]], shift[rp[i]:rp[i + 1]])]
        assert sorted(want) == got


@pytest.mark.parametrize("k", [0, 1])
def test_binned_equals_brute_force(k):
    pos, cell, _ = workloads.geometry(k)
    r_c = workloads.CONFIGS[k]["r_cut"]
    a = nbr.brute_force(pos, cell, r_c)
    b = nbr.binned(pos, cell, r_c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("k", [2, 4])
def test_binned_equals_brute_force_on_sampled_receivers(k):
    pos, cell, _ = workloads.geometry(k)
    r_c = workloads.CONFIGS[k]["r_cut"]
    rp, src, shift = nbr.binned(pos, cell, r_c) if k == 2 else _large_binned(pos, cell, r_c)
    rows = np.random.default_rng(5).choice(len(pos), 24 if k == 4 else 200, replace=False)
    for i, (s_bf, sh_bf) in zip(rows, nbr.brute_force_rows(pos, cell, r_c, rows)):
        np.testing.assert_array_equal(src[rp[i]:rp[i + 1]], s_bf)
        np.testing.assert_array_equal(shift[rp[i]:rp[i + 1]], sh_bf)


_LARGE = {}


def _large_binned(pos, cell, r_c):
    if "csr" not in _LARGE:
        _LARGE["csr"] = nbr.binned(pos, cell, r_c)
    return _LARGE["csr"]


@pytest.mark.parametrize("k", [0, 1, 2])
def test_symmetry_and_reverse_index(k):
    pos, cell, _ = workloads.geometry(k)
    r_c = workloads.CONFIGS[k]["r_cut"]
    rp, src, shift = nbr.binned(pos, cell, r_c)
    rev = nbr.reverse_index(rp, src, shift)
    assert (rev >= 0).all()
    np.testing.assert_array_equal(rev[rev], np.arange(len(rev)))
    recv = nbr.receivers_of(rp)
    np.testing.assert_array_equal(src[rev], recv)
    np.testing.assert_array_equal(shift[rev], -shift)
    # the reverse edge vector is the exact negation
    v = nbr.edge_vectors(pos, cell, recv, src, shift)
    np.testing.assert_array_equal(v[rev], -v)


@pytest.mark.parametrize("k,expect", [(0, 32 / 512 * 4 / 3 * math.pi * 64),
                                      (1, 0.05 * 4 / 3 * math.pi * 125),
                                      (2, 0.1 * 4 / 3 * math.pi * 216)])
def test_mean_degree_matches_density(k, expect):
    pos, cell, _ = workloads.geometry(k)
    rp, _, _ = nbr.binned(pos, cell, workloads.CONFIGS[k]["r_cut"])
    deg = rp[-1] / len(pos)
    assert abs(deg - expect) / expect < 0.1


def test_edge_locality():
    """Moving one atom changes the vectors of exactly its incident edges
    (Frost model card: a moved atom changes exactly its incident edge rows)."""
    pos, cell, _ = workloads.geometry(1)
    rp, src, shift = nbr.binned(pos, cell, 5.0)
    recv = nbr.receivers_of(rp)
    v0 = nbr.edge_vectors(pos, cell, recv, src, shift)
    k = 1234
    p2 = pos.copy()
    p2[k] += np.array([1e-3, -2e-3, 5e-4])
    v1 = nbr.edge_vectors(p2, cell, recv, src, shift)
    changed = np.nonzero(np.any(v0 != v1, axis=1))[0]
    incident = np.nonzero((recv == k) | (src == k))[0]
    np.testing.assert_array_equal(changed, incident)
