"""MI355X (gfx950) equivariant interaction convolution: Python binding.

A thin ctypes layer over ``libtpconv.so`` (C ABI in ``include/tpconv.h``).
PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

    import tensor_product_conv_amd as tpc
    ctx = tpc.Context(tpc.Spec(dtype="float32", channels=128, node_lmax=2,
                               sh_lmax=3, out_lmax=3, r_cut=6.0,
                               layer_dims=[8, 64, 64, 64, 17 * 128]))
    nl = ctx.nbr_build(pos, cell)                    # receiver-sorted CSR
    out, saved = ctx.conv_fwd(pos, cell, nl, h, W, scale)
    dh, dR, forces, g_edge = ctx.conv_bwd(nl, h, W, scale, G, saved)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

__all__ = ["Spec", "Context", "NeighbourList", "EdgeBuffers", "TpcError", "library",
           "nbr_build", "conv_fwd", "conv_bwd", "conv_double_bwd", "virial", "timing_enable",
           "timing_collect",
           "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpconv.so")

TPC_MAX_LAYERS = 8
TPC_MAX_PATHS = 32
OP_NBR, OP_FWD, OP_BWD, OP_VIRIAL, OP_DOUBLE_BWD, OP_TABLE_FIT = 0, 1, 2, 3, 4, 5
STATUS = {0: "ok", 1: "invalid", 2: "unsupported", 3: "capacity", 4: "precondition",
          5: "workspace", 6: "device"}


class TpcError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"tpconv {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class _Spec(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("channels", ctypes.c_int), ("node_lmax", ctypes.c_int),
                ("sh_lmax", ctypes.c_int), ("out_lmax", ctypes.c_int), ("n_bessel", ctypes.c_int),
                ("poly_p", ctypes.c_int), ("n_species", ctypes.c_int), ("r_cut", ctypes.c_double),
                ("n_layers", ctypes.c_int), ("layer_dims", ctypes.c_int * (TPC_MAX_LAYERS + 1)),
                ("validate", ctypes.c_int), ("sum_paths", ctypes.c_int), ("fp32_mfma_only", ctypes.c_int),
                ("radial_table_pieces", ctypes.c_int), ("radial_table_degree", ctypes.c_int),
                ("fuse_radial", ctypes.c_int), ("pair_radial", ctypes.c_int)]


class _Info(ctypes.Structure):
    _fields_ = [("n_paths", ctypes.c_int), ("d_in", ctypes.c_int), ("d_sh", ctypes.c_int),
                ("d_out", ctypes.c_int), ("r_width", ctypes.c_int), ("nnz_cg", ctypes.c_int),
                ("paths", (ctypes.c_int * 3) * TPC_MAX_PATHS),
                ("edge_buffer_bytes", ctypes.c_size_t), ("dR_bytes", ctypes.c_size_t),
                ("fwd_workspace_bytes", ctypes.c_size_t), ("bwd_workspace_bytes_fixed", ctypes.c_size_t),
                ("bwd_workspace_bytes_per_edge", ctypes.c_size_t), ("dY_parts", ctypes.c_int),
                ("dh_edge_bytes", ctypes.c_size_t), ("table_bytes", ctypes.c_size_t),
                ("fwd_workspace_bytes_per_edge", ctypes.c_size_t),
                ("fused_radial", ctypes.c_int), ("act_bytes", ctypes.c_size_t),
                ("pair_radial", ctypes.c_int)]


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("total_ms", ctypes.c_double), ("launches", ctypes.c_int64)]


class _EdgeBuffers(ctypes.Structure):
    _fields_ = [("Y", ctypes.c_void_p), ("ef", ctypes.c_void_p), ("rv", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("A", ctypes.c_void_p), ("Rrow", ctypes.c_void_p)]


_LIB = None
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64


def library():
    """Load libtpconv.so (built in-tree by ``python -m tensor_product_conv_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tensor_product_conv_amd.build` (needs ROCm hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.tpc_ctx_create.argtypes = [ctypes.POINTER(_Spec), ctypes.POINTER(_VP)]
    lib.tpc_ctx_destroy.argtypes = [_VP]
    lib.tpc_ctx_destroy.restype = None
    lib.tpc_ctx_info.argtypes = [_VP, ctypes.POINTER(_Info)]
    lib.tpc_cg_table.argtypes = [_VP, ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_size_t]
    lib.tpc_workspace_query.argtypes = [_VP, ctypes.c_int, _I64, _I64,
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_size_t)]
    lib.tpc_nbr_build.argtypes = [_VP, _I64, _VP, ctypes.POINTER(ctypes.c_double), _VP, _I64,
                                  _VP, _VP, _VP, _VP, ctypes.POINTER(_I64), _VP, ctypes.c_size_t, _VP]
    lib.tpc_conv_fwd.argtypes = [_VP, _I64, _VP, ctypes.POINTER(ctypes.c_double), _VP, _VP, _VP, _VP,
                                 _I64, _I64, _I64, _I64, _VP, ctypes.POINTER(_VP), ctypes.c_double,
                                 _VP, ctypes.POINTER(_EdgeBuffers), _VP, ctypes.c_size_t, _VP]
    lib.tpc_conv_bwd.argtypes = [_VP, _I64, _I64, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _VP,
                                 ctypes.POINTER(_VP), ctypes.c_double, _VP,
                                 ctypes.POINTER(_EdgeBuffers), _VP, _VP, _VP, _VP, _VP, _VP,
                                 ctypes.c_size_t, _VP]
    lib.tpc_conv_double_bwd.argtypes = [_VP, _I64, _I64, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _VP,
                                        ctypes.c_double, _VP, ctypes.POINTER(_EdgeBuffers), _VP, _VP,
                                        _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.tpc_virial.argtypes = [_VP, _I64, _I64, _VP, ctypes.POINTER(ctypes.c_double), _VP, _VP, _VP,
                               _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.tpc_radial_table_fit.argtypes = [_VP, ctypes.POINTER(_VP), _VP, ctypes.c_size_t,
                                         ctypes.POINTER(ctypes.c_double), _VP, ctypes.c_size_t, _VP]
    lib.tpc_timing_enable.argtypes = [ctypes.c_int]
    lib.tpc_timing_collect.argtypes = [ctypes.POINTER(_KernelTime), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int)]
    lib.tpc_status_string.argtypes = [ctypes.c_int]
    lib.tpc_status_string.restype = ctypes.c_char_p
    lib.tpc_last_error.argtypes = []
    lib.tpc_last_error.restype = ctypes.c_char_p
    for name in ("tpc_ctx_create", "tpc_ctx_info", "tpc_cg_table", "tpc_workspace_query",
                 "tpc_nbr_build", "tpc_conv_fwd", "tpc_conv_bwd", "tpc_conv_double_bwd", "tpc_virial",
                 "tpc_radial_table_fit", "tpc_timing_enable", "tpc_timing_collect"):
        getattr(lib, name).restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(status):
    if status != 0:
        raise TpcError(status, library().tpc_last_error().decode())


def timing_enable(on=True):
    """Record HIP events around every kernel the library launches (this thread)."""
    _check(library().tpc_timing_enable(int(bool(on))))


def timing_collect():
    """{kernel name: (total ms, launches)} since the last collect; waits for the events."""
    buf = (_KernelTime * 64)()
    n = ctypes.c_int()
    _check(library().tpc_timing_collect(buf, 64, ctypes.byref(n)))
    return {buf[k].name.decode(): (buf[k].total_ms, buf[k].launches) for k in range(n.value)}


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _cell_arg(cell):
    import numpy as np
    c = np.ascontiguousarray(np.asarray(cell.cpu() if hasattr(cell, "cpu") else cell,
                                        dtype=np.float64).reshape(9))
    return (ctypes.c_double * 9)(*c.tolist())


@dataclass
class Spec:
    """Python mirror of ``tpc_spec``."""
    channels: int
    node_lmax: int
    sh_lmax: int
    out_lmax: int
    r_cut: float
    layer_dims: list
    dtype: str = "float32"
    n_species: int = 128
    n_bessel: int = 8
    poly_p: int = 5
    validate: bool = False
    sum_paths: bool = False
    fp32_mfma_only: bool = False
    radial_table_pieces: int = 0
    radial_table_degree: int = 0
    fuse_radial: bool = False
    pair_radial: bool = False

    def to_c(self):
        s = _Spec()
        s.dtype = {"float32": 0, "float64": 1}[self.dtype]
        s.channels = self.channels
        s.node_lmax, s.sh_lmax, s.out_lmax = self.node_lmax, self.sh_lmax, self.out_lmax
        s.n_bessel, s.poly_p, s.n_species = self.n_bessel, self.poly_p, self.n_species
        s.r_cut = float(self.r_cut)
        s.n_layers = len(self.layer_dims) - 1
        for k, d in enumerate(self.layer_dims[:TPC_MAX_LAYERS + 1]):
            s.layer_dims[k] = int(d)
        s.validate = int(bool(self.validate))
        s.sum_paths = int(bool(self.sum_paths))
        s.fp32_mfma_only = int(bool(self.fp32_mfma_only))
        s.radial_table_pieces = int(self.radial_table_pieces)
        s.radial_table_degree = int(self.radial_table_degree)
        s.fuse_radial = int(bool(self.fuse_radial))
        s.pair_radial = int(bool(self.pair_radial))
        return s


@dataclass
class NeighbourList:
    row_ptr: object       # int32 [N+1]
    src: object           # int32 [E]
    shift: object         # int32 [E, 3]
    rev: object           # int32 [E]
    n_edges: int


@dataclass
class EdgeBuffers:
    Y: object
    ef: object
    rv: object
    R: object
    A: object = None       # uint8 [E, act_bytes] when the context fuses the radial last layer
    Rrow: object = None    # int32 [E + 1] when an edge and its reverse share a row of R
    edge_begin: int = 0
    edge_end: int = 0
    row_begin: int = 0
    row_end: int = 0

    def to_c(self):
        return _EdgeBuffers(_ptr(self.Y), _ptr(self.ef), _ptr(self.rv), _ptr(self.R), _ptr(self.A),
                            _ptr(self.Rrow))

    def R_per_edge(self):
        """R with one row per edge of the chunk (rows gathered through Rrow
        when an edge and its reverse share one)."""
        if self.Rrow is None or self.R is None:
            return self.R
        ne = self.edge_end - self.edge_begin
        return self.R.index_select(0, self.Rrow[:ne].long())


class Context:
    """A ``tpc_ctx``: immutable spec plus the coupling tables built from it."""

    def __init__(self, spec: Spec):
        self.spec = spec
        lib = library()
        self._h = ctypes.c_void_p()
        self._spec_c = spec.to_c()
        _check(lib.tpc_ctx_create(ctypes.byref(self._spec_c), ctypes.byref(self._h)))
        info = _Info()
        _check(lib.tpc_ctx_info(self._h, ctypes.byref(info)))
        self.n_paths, self.d_in, self.d_sh, self.d_out = info.n_paths, info.d_in, info.d_sh, info.d_out
        self.r_width, self.nnz_cg = info.r_width, info.nnz_cg
        self.paths = [tuple(info.paths[p]) for p in range(info.n_paths)]
        self.sizes = {k: getattr(info, k) for k in (
            "edge_buffer_bytes", "dR_bytes", "fwd_workspace_bytes", "bwd_workspace_bytes_fixed",
            "bwd_workspace_bytes_per_edge", "dY_parts", "dh_edge_bytes", "table_bytes", "act_bytes",
            "fwd_workspace_bytes_per_edge")}
        self.fused_radial = bool(info.fused_radial)
        self.pair_radial = bool(info.pair_radial)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value and _LIB is not None:
            _LIB.tpc_ctx_destroy(h)
            self._h = None

    @property
    def dtype(self):
        t = _torch()
        return t.float64 if self.spec.dtype == "float64" else t.float32

    def cg_table(self, p):
        import numpy as np
        l1, l2, l3 = self.paths[p]
        n = (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1)
        buf = (ctypes.c_double * n)()
        _check(library().tpc_cg_table(self._h, p, buf, n))
        return np.array(buf[:], dtype=np.float64).reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)

    def workspace_bytes(self, op, n_atoms=0, n_edges=0, cell=None):
        out = ctypes.c_size_t()
        c = _cell_arg(cell) if cell is not None else None
        _check(library().tpc_workspace_query(self._h, op, n_atoms, n_edges, c, ctypes.byref(out)))
        return out.value

    def _workspace(self, nbytes, device):
        t = _torch()
        return t.empty(max(int(nbytes), 256), dtype=t.uint8, device=device)

    # ---- neighbour list ---------------------------------------------------
    def nbr_build(self, pos, cell, species=None, edge_cap=None, into=None, workspace=None):
        """Receiver-sorted CSR; grows the edge buffers once if the first guess is short.

        ``into`` (a NeighbourList whose arrays hold ``edge_cap`` edges) reuses
        existing buffers; ``workspace`` reuses a workspace tensor.
        """
        t = _torch()
        N = pos.shape[0]
        dev = pos.device
        ws = workspace if workspace is not None else \
            self._workspace(self.workspace_bytes(OP_NBR, N, 0, cell), dev)
        c = _cell_arg(cell)
        cap = int(edge_cap) if edge_cap is not None else max(64, N * 64)
        row_ptr = into.row_ptr if into is not None else t.empty(N + 1, dtype=t.int32, device=dev)
        for _ in range(2):
            if into is not None:
                src, shift, rev = into.src, into.shift, into.rev
            else:
                src = t.empty(cap, dtype=t.int32, device=dev)
                shift = t.empty((cap, 3), dtype=t.int32, device=dev)
                rev = t.empty(cap, dtype=t.int32, device=dev)
            ne = _I64()
            st = library().tpc_nbr_build(self._h, N, _ptr(pos), c, _ptr(species), cap, _ptr(row_ptr),
                                         _ptr(src), _ptr(shift), _ptr(rev), ctypes.byref(ne), _ptr(ws),
                                         ws.numel(), _stream())
            if st == 3 and edge_cap is None:     # capacity: reallocate and call again
                cap = ne.value
                continue
            _check(st)
            E = ne.value
            return NeighbourList(row_ptr, src[:E], shift[:E], rev[:E], E)
        _check(st)

    # ---- forward ------------------------------------------------------------
    def alloc_edge_buffers(self, n_edges, device, with_R=True):
        """Per-edge buffers of a chunk of ``n_edges``; ``with_R=False`` leaves
        out R when the context fuses the radial last layer (forward only)."""
        t = _torch()
        act = self.sizes["act_bytes"]
        return EdgeBuffers(Y=t.empty((n_edges, self.d_sh), dtype=self.dtype, device=device),
                           ef=t.empty((n_edges, 8), dtype=self.dtype, device=device),
                           rv=t.empty((n_edges, 4), dtype=self.dtype, device=device),
                           R=(t.empty((n_edges, self.r_width), dtype=self.dtype, device=device)
                              if with_R or not self.fused_radial else None),
                           A=t.empty((n_edges, act), dtype=t.uint8, device=device) if act else None,
                           Rrow=(t.empty(n_edges + 1, dtype=t.int32, device=device)
                                 if self.pair_radial else None))

    def conv_fwd(self, pos, cell, nl: NeighbourList, h, W, scale=1.0, out=None, eb=None,
                 rows=None, edges=None, workspace=None):
        """out [N, d_out, C]; returns (out, edge buffers for conv_bwd)."""
        t = _torch()
        N = pos.shape[0]
        rb, re_ = rows if rows is not None else (0, N)
        eb_, ee = edges if edges is not None else (0, nl.n_edges)
        if out is None:
            out = t.empty((N, self.d_out, self.spec.channels), dtype=self.dtype, device=h.device)
        if eb is None:
            eb = self.alloc_edge_buffers(ee - eb_, h.device)
        eb.edge_begin, eb.edge_end, eb.row_begin, eb.row_end = eb_, ee, rb, re_
        wp = (_VP * len(W))(*[w.data_ptr() for w in W])
        ebc = eb.to_c()
        ws = workspace if workspace is not None else \
            self._workspace(self.workspace_bytes(OP_FWD, N, ee - eb_), h.device)
        _check(library().tpc_conv_fwd(self._h, N, _ptr(pos), _cell_arg(cell), _ptr(nl.row_ptr),
                                      _ptr(nl.src), _ptr(nl.shift), _ptr(nl.rev), rb, re_, eb_, ee, _ptr(h), wp,
                                      float(scale), _ptr(out), ctypes.byref(ebc), _ptr(ws), ws.numel(),
                                      _stream()))
        return out, eb

    # ---- backward -------------------------------------------------------------
    def conv_bwd(self, nl: NeighbourList, h, W, scale, G, eb: EdgeBuffers, dh=None, dR=None,
                 g_edge=None, dh_edge=None, want_dR=True, want_dh=True, want_forces=True,
                 forces=None, workspace=None):
        """Backward of L = sum(G * out) for the chunk in ``eb``.

        Returns (dh, dR, forces, g_edge).  A chunked caller passes the same
        dh on every chunk, chunks in ascending row order: each call continues
        every atom's running sum with the chunk's terms (the first chunk
        starts it, the last scales it), and dh_edge is chunk-sized scratch
        that the calls may share.  forces sums g_edge over every edge, so it
        is asked for (want_forces) only on the last chunk, after every chunk's
        g_edge (one shared full-size buffer) is written.
        """
        t = _torch()
        N = h.shape[0]
        ne = eb.edge_end - eb.edge_begin
        if want_dh and dh is None:
            dh = t.empty_like(h)
        if not want_dh:
            dh = None
        if want_dR and dR is None:
            dR = t.empty((ne, self.r_width), dtype=self.dtype, device=h.device)
        if g_edge is None:
            g_edge = t.empty((nl.n_edges, 3), dtype=self.dtype, device=h.device)
        if dh_edge is None:
            dh_edge = t.empty((ne, self.d_in, self.spec.channels), dtype=self.dtype, device=h.device)
        if want_forces and forces is None:
            forces = t.empty((N, 3), dtype=self.dtype, device=h.device)
        if not want_forces:
            forces = None
        wp = (_VP * len(W))(*[w.data_ptr() for w in W])
        ebc = eb.to_c()
        ws = workspace if workspace is not None else \
            self._workspace(self.workspace_bytes(OP_BWD, N, ne), h.device)
        _check(library().tpc_conv_bwd(self._h, N, nl.n_edges, _ptr(nl.row_ptr), _ptr(nl.src),
                                      _ptr(nl.rev), eb.row_begin, eb.row_end, eb.edge_begin,
                                      eb.edge_end, _ptr(h), wp, float(scale), _ptr(G), ctypes.byref(ebc),
                                      _ptr(dR), _ptr(g_edge), _ptr(dh_edge), _ptr(dh), _ptr(forces),
                                      _ptr(ws), ws.numel(), _stream()))
        return dh, dR, forces, g_edge

    # ---- radial tables ------------------------------------------------------------
    def radial_table_fit(self, W, table=None, workspace=None, check=True):
        """Fit and certify the piecewise Chebyshev table of R(r) from the
        radial network's weights W (a context with radial_table_pieces > 0).
        Returns (table, certificate ratios (values, derivatives)); with
        ``check`` an uncertified table raises TpcError (status precondition).
        The convolution calls of this context then take [table] as weights."""
        t = _torch()
        dev = W[0].device
        nbytes = self.sizes["table_bytes"]
        if table is None:
            table = t.empty(nbytes // (8 if self.spec.dtype == "float64" else 4), dtype=self.dtype, device=dev)
        ws = workspace if workspace is not None else self._workspace(self.workspace_bytes(OP_TABLE_FIT), dev)
        wp = (_VP * len(W))(*[w.data_ptr() for w in W])
        cert = (ctypes.c_double * 2)()
        st = library().tpc_radial_table_fit(self._h, wp, _ptr(table), table.numel() * table.element_size(), cert,
                                            _ptr(ws), ws.numel(), _stream())
        if st != 0 and (check or st != 4):
            _check(st)
        return table, (cert[0], cert[1])

    # ---- VJP-of-VJP -------------------------------------------------------------
    def conv_double_bwd(self, nl: NeighbourList, h, scale, G, eb: EdgeBuffers, u_dh, u_dY, u_dR,
                        g_hat=None, h_hat=None, Y_hat=None, R_hat=None, workspace=None):
        """Double backward of the chunk in ``eb`` for cotangents u_dh
        [N, d_in, C], u_dY [n_edges, d_sh] and u_dR [n_edges, P*C] (every edge)
        of the VJP outputs dh, dY, dR.  Returns (g_hat, h_hat, Y_hat, R_hat):
        the gradients of <u_dh, dh> + <u_dY, dY> + <u_dR, dR> with respect to
        G, h, Y and R (rows of the chunk's receivers for g_hat and h_hat; the
        chunk's edges for Y_hat and R_hat)."""
        t = _torch()
        N = h.shape[0]
        ne = eb.edge_end - eb.edge_begin
        if g_hat is None:
            g_hat = t.empty_like(G)
        if h_hat is None:
            h_hat = t.empty_like(h)
        if Y_hat is None:
            Y_hat = t.empty((ne, self.d_sh), dtype=self.dtype, device=h.device)
        if R_hat is None:
            R_hat = t.empty((ne, self.r_width), dtype=self.dtype, device=h.device)
        ebc = eb.to_c()
        ws = workspace if workspace is not None else \
            self._workspace(self.workspace_bytes(OP_DOUBLE_BWD, N, ne), h.device)
        _check(library().tpc_conv_double_bwd(self._h, N, nl.n_edges, _ptr(nl.row_ptr), _ptr(nl.src),
                                             _ptr(nl.rev), eb.row_begin, eb.row_end, eb.edge_begin,
                                             eb.edge_end, _ptr(h), float(scale), _ptr(G), ctypes.byref(ebc),
                                             _ptr(u_dh), _ptr(u_dY), _ptr(u_dR), _ptr(g_hat), _ptr(h_hat),
                                             _ptr(Y_hat), _ptr(R_hat), _ptr(ws), ws.numel(), _stream()))
        return g_hat, h_hat, Y_hat, R_hat

    # ---- virial ----------------------------------------------------------------
    def virial(self, pos, cell, nl: NeighbourList, g_edge, out=None, workspace=None):
        """W [3, 3] = dL/d(strain) = sum_e g_e r_e^T from the edge gradients of
        conv_bwd (every edge written)."""
        t = _torch()
        N = pos.shape[0]
        if out is None:
            out = t.empty((3, 3), dtype=self.dtype, device=pos.device)
        ws = workspace if workspace is not None else \
            self._workspace(self.workspace_bytes(OP_VIRIAL, N), pos.device)
        _check(library().tpc_virial(self._h, N, nl.n_edges, _ptr(pos), _cell_arg(cell),
                                    _ptr(nl.row_ptr), _ptr(nl.src), _ptr(nl.shift), _ptr(g_edge),
                                    _ptr(out), _ptr(ws), ws.numel(), _stream()))
        return out


def conv_double_bwd(ctx: Context, *a, **k):
    return ctx.conv_double_bwd(*a, **k)


def virial(ctx: Context, *a, **k):
    return ctx.virial(*a, **k)


def nbr_build(ctx: Context, *a, **k):
    return ctx.nbr_build(*a, **k)


def conv_fwd(ctx: Context, *a, **k):
    return ctx.conv_fwd(*a, **k)


def conv_bwd(ctx: Context, *a, **k):
    return ctx.conv_bwd(*a, **k)


def spec_for(cfg, validate=False, fp32_mfma_only=False, table=None, fuse_radial=False, pair_radial=False):
    """Spec of a workload configuration dict (see ``workloads.config``);
    ``table`` = (pieces, degree) selects the radial tables."""
    return Spec(channels=cfg["C"], node_lmax=cfg["l1max"], sh_lmax=cfg["sh_lmax"],
                out_lmax=cfg["out_lmax"], r_cut=cfg["r_cut"], layer_dims=list(cfg["layer_dims"]),
                dtype=cfg["dtype"], validate=validate, sum_paths=bool(cfg.get("sum_paths", False)),
                fp32_mfma_only=fp32_mfma_only,
                radial_table_pieces=table[0] if table else 0, radial_table_degree=table[1] if table else 0,
                fuse_radial=fuse_radial, pair_radial=pair_radial)
