"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded synthetic inputs, and compare with the oracle."""
import sys

import numpy as np

import tensor_product_conv_amd as tpc
import workloads
from oracle import conv, nbr, paths

# "Rewrites and precision options" (FastMACE docs), "What a rewrite is":
# relative error at most 1e-4 in float32 and 1e-10 in float64.
TOL = {"float32": 1e-4, "float64": 1e-10}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b):
    """max |a - b| / max |b| (the infinity-norm relative error per tensor)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.abs(b).max() if b.size else 0.0
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a - b).max())


def torch():
    import torch as t
    return t


class Case:
    """Inputs of configuration k on the GPU plus an oracle problem."""

    def __init__(self, k, validate=False, with_grad=True, data=None, pair=False):
        t = torch()
        self.k = k
        self.d = data if data is not None else workloads.generate(k, with_grad=with_grad)
        self.cfg = self.d["cfg"]
        self.ctx = tpc.Context(tpc.spec_for(self.cfg, validate, pair_radial=pair))
        self.layout = paths.Layout(self.cfg["l1max"], self.cfg["sh_lmax"], self.cfg["out_lmax"],
                                   self.cfg["C"], self.cfg.get("sum_paths", False))
        dev = "cuda"
        self.pos = t.from_numpy(self.d["pos"]).to(dev)
        self.cell = self.d["cell"]
        self.species = t.from_numpy(self.d["species"]).to(dev)
        self.h = t.from_numpy(self.d["h"]).to(dev)
        self.W = [t.from_numpy(w).to(dev) for w in self.d["W"]]
        self.G = t.from_numpy(self.d["G"]).to(dev) if self.d["G"] is not None else None
        self.N = self.cfg["N"]

    def nbr(self, edge_cap=None):
        say(f"[gpu] nbr_build cfg={self.k} N={self.N}")
        nl = self.ctx.nbr_build(self.pos, self.cell, self.species, edge_cap=edge_cap)
        torch().cuda.synchronize()
        return nl

    def scale(self, nl):
        return conv.scale_for(self.cfg, self.N, nl.n_edges)

    def oracle_csr(self):
        """The oracle's own neighbour list (binned build, itself pinned to
        brute force), computed once per case."""
        if getattr(self, "_csr", None) is None:
            say(f"[cpu] oracle neighbour list cfg={self.k}")
            self._csr = nbr.binned(self.d["pos"], self.cell, self.cfg["r_cut"])
        return self._csr

    def oracle(self, nl_np):
        rp, src, shift = nl_np
        return conv.Problem(self.layout, self.d["pos"], self.cell, rp, src, shift, self.d["h"],
                            self.d["W"], self.cfg["r_cut"], conv.scale_for(self.cfg, self.N, rp[-1]),
                            self.d["G"])


def np_csr(nl):
    return (nl.row_ptr.cpu().numpy(), nl.src.cpu().numpy(), nl.shift.cpu().numpy(),
            nl.rev.cpu().numpy())


def row_bounds(row_ptr, n_chunks):
    """Split receivers into n_chunks ranges with roughly equal edge counts."""
    E = int(row_ptr[-1])
    cuts = [0]
    for c in range(1, n_chunks):
        cuts.append(int(np.searchsorted(row_ptr, E * c // n_chunks)))
    cuts.append(len(row_ptr) - 1)
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def run_chunked(case, nl, chunks=1, keep_edges=None, want_forces=True):
    """Forward and backward over receiver chunks.  Returns out, dh, forces,
    g_edge and the dR rows of ``keep_edges`` (absolute edge indices)."""
    t = torch()
    ctx = case.ctx
    rp = nl.row_ptr.cpu().numpy()
    s = case.scale(nl)
    N = case.N
    out = t.empty((N, ctx.d_out, case.cfg["C"]), dtype=ctx.dtype, device="cuda")
    dh = t.empty_like(case.h)
    g_edge = t.empty((nl.n_edges, 3), dtype=ctx.dtype, device="cuda")
    forces = t.empty((N, 3), dtype=ctx.dtype, device="cuda") if want_forces else None
    bounds = row_bounds(rp, chunks)
    max_e = max(int(rp[b] - rp[a]) for a, b in bounds)
    # chunk-sized: each chunk's call folds its terms into dh before the next
    dh_edge = t.empty((max_e, ctx.d_in, case.cfg["C"]), dtype=ctx.dtype, device="cuda")
    eb = ctx.alloc_edge_buffers(max_e, "cuda")
    dR = t.empty((max_e, ctx.r_width), dtype=ctx.dtype, device="cuda")
    kept = {}
    keep_edges = np.asarray([] if keep_edges is None else keep_edges, dtype=np.int64)
    for n, (a, b) in enumerate(bounds):
        e0, e1 = int(rp[a]), int(rp[b])
        say(f"[gpu] conv_fwd/bwd cfg={case.k} rows=[{a},{b}) edges=[{e0},{e1})")
        ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=out, eb=eb, rows=(a, b),
                     edges=(e0, e1))
        last = n == len(bounds) - 1
        ctx.conv_bwd(nl, case.h, case.W, s, case.G, eb, dh=dh, dR=dR, g_edge=g_edge, dh_edge=dh_edge,
                     want_forces=want_forces and last, forces=forces if last else None)
        sel = keep_edges[(keep_edges >= e0) & (keep_edges < e1)]
        if len(sel):
            idx = t.from_numpy(sel - e0).to("cuda")
            vals = dR.index_select(0, idx).cpu().numpy()
            for e, v in zip(sel, vals):
                kept[int(e)] = v
        t.cuda.synchronize()
    return dict(out=out, dh=dh, forces=forces, g_edge=g_edge, dR=kept, eb=eb)


def cotangents(case, n_edges, seed):
    """Seeded N(0,1) cotangents of the VJP outputs (dh, dY, dR), in the
    context dtype: u_dh [N, d_in, C], u_dY [E, d_sh], u_dR [E, P*C]."""
    rng = np.random.default_rng(seed)
    dt = np.dtype(case.cfg["dtype"])
    ctx = case.ctx
    return (rng.standard_normal((case.N, ctx.d_in, case.cfg["C"])).astype(dt),
            rng.standard_normal((n_edges, ctx.d_sh)).astype(dt),
            rng.standard_normal((n_edges, ctx.r_width)).astype(dt))


def run_double(case, nl, u, chunks=1, keep_edges=None):
    """Forward (for the per-edge buffers) then the double backward over
    receiver chunks.  Returns g_hat, h_hat and the Y_hat / R_hat rows of
    ``keep_edges`` (absolute edge indices)."""
    t = torch()
    ctx = case.ctx
    rp = nl.row_ptr.cpu().numpy()
    s = case.scale(nl)
    uh, uY, uR = [t.from_numpy(a).to("cuda") for a in u]
    out = t.empty((case.N, ctx.d_out, case.cfg["C"]), dtype=ctx.dtype, device="cuda")
    g_hat = t.empty_like(case.G)
    h_hat = t.empty_like(case.h)
    bounds = row_bounds(rp, chunks)
    max_e = max(int(rp[b] - rp[a]) for a, b in bounds)
    eb = ctx.alloc_edge_buffers(max_e, "cuda")
    Yh = t.empty((max_e, ctx.d_sh), dtype=ctx.dtype, device="cuda")
    Rh = t.empty((max_e, ctx.r_width), dtype=ctx.dtype, device="cuda")
    keep = np.asarray([] if keep_edges is None else keep_edges, dtype=np.int64)
    kept_Y, kept_R = {}, {}
    for a, b in bounds:
        e0, e1 = int(rp[a]), int(rp[b])
        say(f"[gpu] conv_fwd/double_bwd cfg={case.k} rows=[{a},{b}) edges=[{e0},{e1})")
        ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=out, eb=eb, rows=(a, b), edges=(e0, e1))
        ctx.conv_double_bwd(nl, case.h, s, case.G, eb, uh, uY, uR, g_hat=g_hat, h_hat=h_hat,
                            Y_hat=Yh, R_hat=Rh)
        sel = keep[(keep >= e0) & (keep < e1)]
        if len(sel):
            idx = t.from_numpy(sel - e0).to("cuda")
            for e, y, r in zip(sel, Yh.index_select(0, idx).cpu().numpy(), Rh.index_select(0, idx).cpu().numpy()):
                kept_Y[int(e)], kept_R[int(e)] = y, r
        t.cuda.synchronize()
    return dict(g_hat=g_hat, h_hat=h_hat, Y_hat=kept_Y, R_hat=kept_R)
