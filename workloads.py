"""Seeded synthetic workloads for the equivariant interaction convolution.

This module only draws inputs: positions, cell, species, node features h,
radial-MLP weights W and an upstream gradient G.  It holds none of the
method's arithmetic (no neighbour search, no harmonics, no couplings), so both
the CPU oracle and the GPU binding can take their inputs from it.

The sizes each configuration needs (number of coupling paths, feature widths)
are stated here as literal data; tests check that the oracle and the library
derive the same numbers from the path-admissibility rule.

Recipes (all synthetic; the pages measure on trained models and datasets that
are not used here):

* tiny   -- 32 atoms uniform in a periodic 8 A cube, sequential rejection at
            0.9 A (minimum image), 4 species, r_c = 4.0, float64.
* small  -- 16^3 simple-cubic lattice at 0.05 atoms/A^3, Gaussian jitter
            sigma = 0.1 A, 10 species, r_c = 5.0, float32.
* medium -- water-like box at 0.1 atoms/A^3: 10,923 O placed by random
            sequential adsorption (O-O >= 2.5 A), two H at 0.96 A and
            104.5 deg with a uniformly random orientation (the last molecule
            is OH so that N = 32,768), every intermolecular pair >= 1.0 A,
            species O=0, H=1, H=2, r_c = 6.0, float32.
* large  -- fcc at 0.085 sites/A^3 (a = 3.6103 A) on a 40x41x41 supercell,
            6,816 random vacancies (N = 262,144), Gaussian jitter
            sigma = 0.15 A, 89 species drawn Zipf(1.1), r_c = 6.0, float32.
* dense  -- 1,024 atoms uniform at 0.286 atoms/A^3 (sequential rejection at
            0.8 A), about 150 neighbours within r_c = 5.0 (rows longer than
            128 edges), parity inputs only.

Atoms of the small, medium and large systems are numbered along a Morton
curve over 3 A bins (molecules kept whole), the order an MD engine keeps for
locality.  Positions are wrapped into the cell.  Every value array is drawn
from ``numpy.random.default_rng(seed)`` in the order: positions, species, h,
W (layer order), G.
"""
from __future__ import annotations

import functools
import math

import numpy as np

__all__ = ["CONFIGS", "config", "generate", "variant", "geometry", "values", "morton_order"]

# Literal per-configuration data.  d_in = sum over node irreps of (2l+1),
# d_sh = (sh_lmax+1)^2, d_out = sum over paths of (2 l3 + 1).
CONFIGS = {
    0: dict(name="tiny", N=32, dtype="float64", C=8, l1max=1, sh_lmax=2,
            out_lmax=1, r_cut=4.0, hidden=[16], n_paths=5, d_in=4, d_sh=9,
            d_out=11, scale="one", seed=0, geometry="uniform"),
    1: dict(name="small", N=4096, dtype="float32", C=128, l1max=1, sh_lmax=3,
            out_lmax=3, r_cut=5.0, hidden=[64, 64, 64], n_paths=10, d_in=4,
            d_sh=16, d_out=40, scale="one", seed=1, geometry="sc"),
    2: dict(name="medium", N=32768, dtype="float32", C=128, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=6.0, hidden=[64, 64, 64], n_paths=17,
            d_in=9, d_sh=16, d_out=71, scale="inv_avg_neighbors", seed=2,
            geometry="water"),
    3: dict(name="medium_bwd", N=32768, dtype="float32", C=128, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=6.0, hidden=[64, 64, 64],
            n_paths=17, d_in=9, d_sh=16, d_out=71, scale="inv_avg_neighbors",
            seed=2, geometry="water"),
    4: dict(name="large", N=262144, dtype="float32", C=64, l1max=3,
            sh_lmax=3, out_lmax=3, r_cut=6.0, hidden=[64, 64], n_paths=23,
            d_in=16, d_sh=16, d_out=99, scale="one", seed=4, geometry="fcc"),
    # Kernel-path cases: the small system with other widths, so that the
    # narrower-channel and narrower-network kernels are checked too.
    5: dict(name="small_c32_h16", N=4096, dtype="float32", C=32, l1max=1,
            sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[16, 16], n_paths=10,
            d_in=4, d_sh=16, d_out=40, scale="one", seed=5, geometry="sc"),
    6: dict(name="small_c64_h32", N=4096, dtype="float32", C=64, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[32], n_paths=17,
            d_in=9, d_sh=16, d_out=71, scale="one", seed=6, geometry="sc"),
    7: dict(name="small_c32_h32", N=4096, dtype="float32", C=32, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[32, 32], n_paths=17,
            d_in=9, d_sh=16, d_out=71, scale="one", seed=7, geometry="sc"),
    # the small system with path-summed outputs (one block per output rank)
    8: dict(name="small_summed", N=4096, dtype="float32", C=128, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[64, 64], n_paths=17,
            d_in=9, d_sh=16, d_out=16, scale="one", seed=8, geometry="sc",
            sum_paths=True),
    # Dense systems whose rows hold more than 128 edges (the long-row loops of
    # the tensor-product kernels): 1,024 atoms at about 150 neighbours each,
    # near the FlashCart microbenchmark shape (1,024 nodes, 128 neighbours,
    # 128 channels, rank <= 3); parity inputs only.
    9: dict(name="dense_c128", N=1024, dtype="float32", C=128, l1max=2,
            sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[64, 64], n_paths=17,
            d_in=9, d_sh=16, d_out=71, scale="one", seed=9, geometry="dense"),
    10: dict(name="dense_c64_l3", N=1024, dtype="float32", C=64, l1max=3,
             sh_lmax=3, out_lmax=3, r_cut=5.0, hidden=[32, 32, 32], n_paths=23,
             d_in=16, d_sh=16, d_out=99, scale="one", seed=10, geometry="dense"),
}

N_BESSEL = 8


def config(k):
    """Return a copy of configuration ``k`` (0-based) with derived layer dims."""
    c = dict(CONFIGS[k])
    c["layer_dims"] = [N_BESSEL] + list(c["hidden"]) + [c["n_paths"] * c["C"]]
    return c


# ----------------------------------------------------------------------------
# geometry

def _wrap(x, lengths):
    x = np.mod(x, lengths)
    x[x >= lengths] = 0.0
    return x


def morton_order(points, box, bin_size=3.0):
    """Stable permutation of ``points`` along a Morton curve over cubic bins."""
    nb = np.maximum(1, np.floor(np.asarray(box) / bin_size).astype(np.int64))
    idx = np.floor(points / (np.asarray(box) / nb)).astype(np.int64)
    idx = np.minimum(np.maximum(idx, 0), nb - 1)
    code = np.zeros(len(points), dtype=np.int64)
    for bit in range(11):
        for ax in range(3):
            code |= ((idx[:, ax] >> bit) & 1) << (3 * bit + ax)
    return np.argsort(code, kind="stable")


def _uniform_tiny(rng, N, L, dmin):
    pts = []
    while len(pts) < N:
        p = rng.uniform(0.0, L, size=3)
        ok = True
        for q in pts:
            d = p - q
            d -= L * np.round(d / L)
            if float(d @ d) < dmin * dmin:
                ok = False
                break
        if ok:
            pts.append(p)
    return np.array(pts)


def _random_rotation(rng):
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
        [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
        [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)],
    ])


def _water(rng, N, L):
    n_mol = (N + 2) // 3          # 10,923 molecules; the last one is OH
    d_oh, ang = 0.96, math.radians(104.5)
    body = np.array([[0.0, 0.0, 0.0],
                     [d_oh, 0.0, 0.0],
                     [d_oh * math.cos(ang), d_oh * math.sin(ang), 0.0]])
    nc = int(L // 2.5)            # bins >= 2.5 A: the 27-bin stencil of an O
    cw = L / nc                   # holds every atom within 2.5 A of it
    cap = 24
    grid = np.zeros((nc, nc, nc, cap, 3))
    is_o = np.zeros((nc, nc, nc, cap), dtype=bool)
    cnt = np.zeros((nc, nc, nc), dtype=np.int64)
    offs = np.stack(np.meshgrid(*[np.arange(-1, 2)] * 3, indexing="ij"), -1).reshape(-1, 3)
    slot = np.arange(cap)
    mols = []
    for m in range(n_mol):
        n_at = 3 if m < n_mol - 1 else 2
        while True:
            o = rng.uniform(0.0, L, size=3)
            rot = _random_rotation(rng)
            atoms = _wrap(o + body[:n_at] @ rot.T, L)
            cells = (np.floor(o / cw).astype(np.int64) + offs) % nc
            cx, cy, cz = cells[:, 0], cells[:, 1], cells[:, 2]
            valid = slot[None, :] < cnt[cx, cy, cz][:, None]
            nb = grid[cx, cy, cz][valid]
            nb_o = is_o[cx, cy, cz][valid]
            if len(nb):
                d = atoms[:, None, :] - nb[None, :, :]
                d -= L * np.round(d / L)
                d2 = np.einsum("abk,abk->ab", d, d)
                lim = np.full(d2.shape, 1.0)
                lim[0, nb_o] = 2.5 * 2.5
                if np.any(d2 < lim):
                    continue
            break
        for a_i, a in enumerate(atoms):
            c = tuple(np.floor(a / cw).astype(np.int64) % nc)
            grid[c][cnt[c]] = a
            is_o[c][cnt[c]] = a_i == 0
            cnt[c] += 1
        mols.append(atoms)
    order = morton_order(np.array([mm[0] for mm in mols]), np.array([L, L, L]))
    pos = np.concatenate([mols[k] for k in order], axis=0)
    species = np.concatenate([np.arange(len(mols[k]), dtype=np.int32) for k in order])
    assert pos.shape[0] == N
    return pos, species


def _fcc(rng, dims, a, n_vac, sigma):
    basis = np.array([[0, 0, 0], [0.5, 0.5, 0], [0.5, 0, 0.5], [0, 0.5, 0.5]])
    g = np.stack(np.meshgrid(*[np.arange(d) for d in dims], indexing="ij"), -1).reshape(-1, 3)
    sites = (g[:, None, :] + basis[None, :, :]).reshape(-1, 3) * a
    keep = np.ones(len(sites), dtype=bool)
    keep[rng.choice(len(sites), size=n_vac, replace=False)] = False
    sites = sites[keep]
    box = np.array(dims, dtype=np.float64) * a
    sites = sites + rng.normal(0.0, sigma, size=sites.shape)
    return _wrap(sites, box), box


@functools.lru_cache(maxsize=8)
def _geometry_cached(k):
    c = config(k)
    rng = np.random.default_rng(c["seed"])
    N = c["N"]
    if c["geometry"] == "uniform":
        L = 8.0
        pos = _uniform_tiny(rng, N, L, 0.9)
        box = np.array([L, L, L])
        species = rng.integers(0, 4, size=N).astype(np.int32)
    elif c["geometry"] == "sc":
        n = 16
        a = 20.0 ** (1.0 / 3.0)
        g = np.stack(np.meshgrid(*[np.arange(n)] * 3, indexing="ij"), -1).reshape(-1, 3)
        box = np.array([n * a] * 3)
        pos = _wrap(g * a + rng.normal(0.0, 0.1, size=(N, 3)), box)
        pos = pos[morton_order(pos, box)]
        species = rng.integers(0, 10, size=N).astype(np.int32)
    elif c["geometry"] == "dense":
        # uniform at 0.286 atoms/A^3 (about 150 neighbours within 5 A), no
        # pair closer than 0.8 A, numbered along the Morton curve
        L = (N / 0.286) ** (1.0 / 3.0)
        pos = _uniform_tiny(rng, N, L, 0.8)
        box = np.array([L, L, L])
        pos = pos[morton_order(pos, box, bin_size=2.0)]
        species = rng.integers(0, 4, size=N).astype(np.int32)
    elif c["geometry"] == "water":
        L = (N / 0.1) ** (1.0 / 3.0)
        box = np.array([L, L, L])
        pos, species = _water(rng, N, L)
    elif c["geometry"] == "fcc":
        a = (4.0 / 0.085) ** (1.0 / 3.0)
        dims = (40, 41, 41)
        n_sites = 4 * dims[0] * dims[1] * dims[2]
        pos, box = _fcc(rng, dims, a, n_sites - N, 0.15)
        pos = pos[morton_order(pos, box)]
        ranks = np.arange(1, 90, dtype=np.float64)
        p = ranks ** -1.1
        p /= p.sum()
        species = rng.choice(89, size=N, p=p).astype(np.int32)
    else:
        raise ValueError(c["geometry"])
    cell = np.diag(box).astype(np.float64)
    return np.ascontiguousarray(pos, dtype=np.float64), cell, species, rng.bit_generator.state


def geometry(k):
    """Positions [N,3] (float64, wrapped), cell [3,3] (rows a1,a2,a3), species [N]."""
    pos, cell, species, _ = _geometry_cached(k)
    return pos.copy(), cell.copy(), species.copy()


def values(k, with_grad=True):
    """Node features h [N,d_in,C], weights W (list of [fan_in,fan_out]), and G.

    Drawn from the generator state left after the geometry draw, in the order
    h, W (layer order), G.  G ~ N(0,1) has the output's shape [N,d_out,C].
    """
    c = config(k)
    _, _, _, state = _geometry_cached(k)
    rng = np.random.default_rng()
    rng.bit_generator.state = state
    dt = np.dtype(c["dtype"])
    N, C = c["N"], c["C"]
    h = rng.standard_normal((N, c["d_in"], C), dtype=dt)
    dims = c["layer_dims"]
    W = []
    for a, b in zip(dims[:-1], dims[1:]):
        W.append((rng.standard_normal((a, b)) / math.sqrt(a)).astype(dt))
    G = rng.standard_normal((N, c["d_out"], C), dtype=dt) if with_grad else None
    return h, W, G


def variant(k, C, l1max, sh_lmax, out_lmax, hidden, dtype, seed, sum_paths=False):
    """Configuration ``k``'s geometry with other feature shapes and widths
    (every kernel instantiation gets a small parity case).  The path count
    and widths are derived by the caller's layout; values are drawn from
    ``default_rng(seed)``: h, W (layer order), G.  Returns the same dict as
    ``generate``."""
    from itertools import product
    pos, cell, species = geometry(k)
    n_paths = sum(1 for l1, l2, l3 in product(range(l1max + 1), range(sh_lmax + 1), range(out_lmax + 1))
                  if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0)
    l3s = sorted({l3 for l1, l2, l3 in product(range(l1max + 1), range(sh_lmax + 1), range(out_lmax + 1))
                  if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0})
    d_out = sum(2 * l3 + 1 for l3 in l3s) if sum_paths else sum(
        2 * l3 + 1 for l1, l2, l3 in product(range(l1max + 1), range(sh_lmax + 1), range(out_lmax + 1))
        if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0)
    base = config(k)
    c = dict(base, name=f"{base['name']}_v{seed}", C=C, l1max=l1max, sh_lmax=sh_lmax, out_lmax=out_lmax,
             hidden=list(hidden), dtype=dtype, seed=seed, n_paths=n_paths, d_in=(l1max + 1) ** 2,
             d_sh=(sh_lmax + 1) ** 2, d_out=d_out, sum_paths=sum_paths, scale="one")
    c["layer_dims"] = [N_BESSEL] + list(hidden) + [n_paths * C]
    rng = np.random.default_rng(seed)
    dt = np.dtype(dtype)
    N = len(pos)
    h = rng.standard_normal((N, c["d_in"], C)).astype(dt)
    W = [(rng.standard_normal((a, b)) / math.sqrt(a)).astype(dt)
         for a, b in zip(c["layer_dims"][:-1], c["layer_dims"][1:])]
    G = rng.standard_normal((N, d_out, C)).astype(dt)
    return dict(cfg=c, pos=pos, cell=cell, species=species, h=h, W=W, G=G, r_cut=c["r_cut"])


def generate(k, with_grad=True):
    """Everything for configuration ``k`` as a dict of NumPy arrays."""
    pos, cell, species = geometry(k)
    h, W, G = values(k, with_grad)
    c = config(k)
    return dict(cfg=c, pos=pos, cell=cell, species=species, h=h, W=W, G=G,
                r_cut=c["r_cut"])
