"""The forward entry point that allocates nothing (tpc_conv_fwd_noalloc),
called through the C ABI, against tpc_conv_fwd with a caller workspace: two
calls in a row on the same context, the second on a smaller system, each
compared element by element (the same kernels run on the same inputs, so
the outputs are identical)."""
import ctypes

import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import TOL, Case, rel, say, torch

pytestmark = pytest.mark.gpu


def _fwd_both(case, nl, s):
    t = torch()
    ctx, lib = case.ctx, tpc.library()
    lib.tpc_conv_fwd_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.c_double, ctypes.c_void_p, ctypes.POINTER(tpc._EdgeBuffers),
                                         ctypes.c_void_p]
    lib.tpc_conv_fwd_noalloc.restype = ctypes.c_int
    N, E = case.N, nl.n_edges
    ref, eb_ref = ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s)
    out = t.full((N, ctx.d_out, case.cfg["C"]), float("nan"), dtype=ctx.dtype, device="cuda")
    eb = ctx.alloc_edge_buffers(E, "cuda")
    eb.edge_begin, eb.edge_end, eb.row_begin, eb.row_end = 0, E, 0, N
    ebc = eb.to_c()
    wp = (ctypes.c_void_p * len(case.W))(*[w.data_ptr() for w in case.W])
    t.cuda.synchronize()
    say(f"[gpu] tpc_conv_fwd_noalloc N={N} E={E}")
    st = lib.tpc_conv_fwd_noalloc(ctx._h, N, ctypes.c_void_p(case.pos.data_ptr()), tpc._cell_arg(case.cell),
                                  ctypes.c_void_p(nl.row_ptr.data_ptr()), ctypes.c_void_p(nl.src.data_ptr()),
                                  ctypes.c_void_p(nl.shift.data_ptr()), ctypes.c_void_p(nl.rev.data_ptr()),
                                  0, N, 0, E,
                                  ctypes.c_void_p(case.h.data_ptr()), wp, float(s),
                                  ctypes.c_void_p(out.data_ptr()), ctypes.byref(ebc), tpc._stream())
    assert st == 0, lib.tpc_last_error().decode()
    t.cuda.synchronize()
    return ref, eb_ref, out, eb


def test_noalloc_forward_matches_the_workspace_forward_twice():
    # first call: the small system; second: a smaller system (the tiny
    # geometry) with the same spec and other weights
    big = Case(1)
    small_d = workloads.variant(0, 128, 1, 3, 3, [64, 64, 64], "float32", 77)
    small = Case(0, data=small_d)
    assert small.N < big.N
    tol = TOL["float32"]
    for case in (big, small):
        case.ctx = big.ctx                      # one context for both calls
        nl = case.nbr()
        ref, eb_ref, out, eb = _fwd_both(case, nl, 1.0)
        assert torch().equal(out, ref)
        assert rel(out.cpu().numpy(), ref.cpu().numpy()) < tol
        for k in ("Y", "ef", "rv", "R"):
            assert torch().equal(getattr(eb, k), getattr(eb_ref, k)), k


def test_noalloc_scratch_holds_every_built_spec():
    # the largest forward workspaces of the built configurations fit the
    # fixed scratch (16 MiB): 128 channels, three hidden layers of 64, the
    # widest float32 and float64 shapes
    for dt, l1, P in (("float32", 3, 23), ("float64", 1, 10)):
        spec = tpc.Spec(channels=128, node_lmax=l1, sh_lmax=3, out_lmax=3, r_cut=5.0,
                        layer_dims=[8, 64, 64, 64, P * 128], dtype=dt)
        assert tpc.Context(spec).sizes["fwd_workspace_bytes"] <= 16 << 20
