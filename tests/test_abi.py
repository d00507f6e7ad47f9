"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every declared symbol, validates specs and arguments before any device work,
and its compile-time coupling tables match the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from oracle import cg, paths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpconv.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tpc_[a-z_]+)\s*\(", txt)))


def test_header_symbols_are_exported():
    lib = tpc.library()
    names = _declared()
    assert {"tpc_nbr_build", "tpc_conv_fwd", "tpc_conv_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_no_symbol_outside_the_header():
    out = os.popen(f"nm -D --defined-only {tpc.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if l.split()[-2:-1] == ["T"]}
    ours = {n for n in exported if n.startswith("tpc_")}
    assert ours == set(_declared())


@pytest.mark.parametrize("k", [0, 1, 2, 4, 8])
def test_context_sizes_match_configs(k):
    c = workloads.config(k)
    ctx = tpc.Context(tpc.spec_for(c))
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"], c.get("sum_paths", False))
    assert ctx.paths == L.paths
    assert (ctx.n_paths, ctx.d_in, ctx.d_sh, ctx.d_out) == (c["n_paths"], c["d_in"], c["d_sh"], c["d_out"])
    assert ctx.r_width == c["n_paths"] * c["C"]


def test_coupling_tables_match_the_oracle():
    c = workloads.config(4)
    ctx = tpc.Context(tpc.spec_for(c))
    nnz = 0
    for p, (l1, l2, l3) in enumerate(ctx.paths):
        t = ctx.cg_table(p)
        np.testing.assert_allclose(t, cg.coupling(l1, l2, l3), atol=1e-14, rtol=0)
        nnz += int(np.count_nonzero(t))
    assert nnz == ctx.nnz_cg == 353


def _spec(**over):
    c = workloads.config(1)
    s = tpc.spec_for(c)
    for k, v in over.items():
        setattr(s, k, v)
    return s


@pytest.mark.parametrize("over,status,needle", [
    (dict(dtype="float32", channels=0), 1, "channels"),
    (dict(node_lmax=4), 2, "node_lmax"),
    (dict(n_bessel=6), 2, "n_bessel"),
    (dict(poly_p=6), 2, "poly_p"),
    (dict(r_cut=-1.0), 1, "r_cut"),
    (dict(channels=96, layer_dims=[8, 64, 64, 64, 960]), 2, "no fused kernel"),
    (dict(layer_dims=[8, 64, 64, 64, 999]), 1, "paths*channels"),
    (dict(layer_dims=[8, 48, 1280]), 2, "radial MLP"),
    (dict(layer_dims=[7, 64, 1280]), 1, "layer_dims[0]"),
    (dict(radial_table_pieces=-1), 1, "radial_table_pieces"),
    (dict(radial_table_pieces=16, radial_table_degree=0), 1, "radial_table_degree"),
    # float64 is built for node_lmax <= 1 only
    (dict(dtype="float64", node_lmax=2, layer_dims=[8, 64, 64, 64, 17 * 128]), 2, "no fused kernel"),
    (dict(dtype="float64", node_lmax=3, layer_dims=[8, 64, 64, 64, 23 * 128]), 2, "no fused kernel"),
])
def test_spec_validation(over, status, needle):
    with pytest.raises(tpc.TpcError) as ei:
        tpc.Context(_spec(**over))
    assert ei.value.status == status
    assert needle in ei.value.message


def test_every_failed_check_is_listed():
    with pytest.raises(tpc.TpcError) as ei:
        tpc.Context(_spec(n_bessel=6, poly_p=7, r_cut=0.0))
    m = ei.value.message
    assert "n_bessel" in m and "poly_p" in m and "r_cut" in m
    assert ei.value.status == 1        # INVALID outranks UNSUPPORTED


def test_workspace_query():
    c = workloads.config(2)
    ctx = tpc.Context(tpc.spec_for(c))
    cell = np.eye(3) * 68.94
    nb = ctx.workspace_bytes(tpc.OP_NBR, 32768, 0, cell)
    assert nb >= 2 * 4 * 32768
    bw = ctx.workspace_bytes(tpc.OP_BWD, 32768, 1000)
    assert bw >= 1000 * (16 + 8 + 17 * 128) * 4
    with pytest.raises(tpc.TpcError) as ei:
        ctx.workspace_bytes(tpc.OP_NBR, 10, 0, np.zeros((3, 3)))
    assert "singular" in ei.value.message


def _raw(ctx):
    return tpc.library(), ctx._h


def test_nbr_build_argument_checks_run_before_device_work():
    lib, h = _raw(tpc.Context(_spec()))
    ne = ctypes.c_int64()
    cell = (ctypes.c_double * 9)(*([0.0] * 9))
    st = lib.tpc_nbr_build(h, 10, None, cell, None, 5, None, None, None, None, ctypes.byref(ne),
                           None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    for needle in ("row_ptr", "pos", "src, shift and rev", "workspace", "singular"):
        assert needle in m


def test_conv_argument_checks_run_before_device_work():
    lib, h = _raw(tpc.Context(_spec()))
    eb = tpc._EdgeBuffers()
    cell = (ctypes.c_double * 9)(*np.eye(3).reshape(-1).tolist())
    st = lib.tpc_conv_fwd(h, 10, None, cell, None, None, None, None, 0, 11, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    for needle in ("row_begin <= row_end <= n_atoms", "row_ptr", "eb.Y", "weights"):
        assert needle in m
    st = lib.tpc_conv_bwd(h, 10, 3, None, None, None, 0, 5, 0, 5, None, None, float("nan"), None,
                          ctypes.byref(eb), None, None, None, None, None, None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    for needle in ("n_edges must be >= edge_end", "scale", "g_edge", "dh_edge", "rev", "workspace"):
        assert needle in m


def test_virial_argument_checks_run_before_device_work():
    ctx = tpc.Context(_spec())
    lib, h = _raw(ctx)
    cell = (ctypes.c_double * 9)(*([float("inf")] + [0.0] * 8))
    st = lib.tpc_virial(h, 10, 5, None, cell, None, None, None, None, None, None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    for needle in ("cell must be finite", "row_ptr", "pos", "src", "shift", "g_edge", "virial",
                   "workspace"):
        assert needle in m
    assert ctx.workspace_bytes(tpc.OP_VIRIAL, 1000) >= 4 * 9 * 8   # 4 blocks of float64 partials


def test_status_strings():
    lib = tpc.library()
    assert lib.tpc_status_string(3) == b"edge capacity too small"
    assert lib.tpc_status_string(99) == b"unknown status"


def test_table_context_sizes_and_argument_checks():
    """A table context reports its table size (pieces x (2 degree + 1) x P*C
    values), needs no packed-weight workspace, and refuses a fit without a
    table context, weights, certificate or large enough table."""
    c = workloads.config(1)
    ctx = tpc.Context(tpc.spec_for(c, table=(64, 8)))
    assert ctx.sizes["table_bytes"] == 4 * 64 * 17 * ctx.r_width
    # status word and piece counts; the sorted edge order adds 4 bytes per edge
    assert ctx.sizes["fwd_workspace_bytes"] == 256 + 512   # 65 counts round up to 512 bytes
    assert ctx.sizes["fwd_workspace_bytes_per_edge"] == 4
    assert ctx.workspace_bytes(tpc.OP_FWD, 0, 1000) == 256 + 4352
    lib, h = _raw(ctx)
    st = lib.tpc_radial_table_fit(h, None, None, 0, None, None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    for needle in ("weights", "certificate", "table", "workspace"):
        assert needle in m
    plain = tpc.Context(tpc.spec_for(c))
    lib, h = _raw(plain)
    assert plain.sizes["table_bytes"] == 0
    st = lib.tpc_radial_table_fit(h, None, None, 0, None, None, 0, None)
    assert st == 1 and "no radial table" in lib.tpc_last_error().decode()


def test_fused_radial_selection_and_edge_buffer_checks():
    """spec.fuse_radial takes the fused forward where the shapes allow it
    (float32, bf16-split products, hidden width 32 or 64, C a multiple of 16,
    no table) and reports the activation row size (H / 32 x 192 bytes); a
    fused forward needs eb.A and no longer needs eb.R."""
    c = workloads.config(1)
    plain = tpc.Context(tpc.spec_for(c))
    assert not plain.fused_radial and plain.sizes["act_bytes"] == 0
    fused = tpc.Context(tpc.spec_for(c, fuse_radial=True))
    assert fused.fused_radial and fused.sizes["act_bytes"] == 2 * 192
    assert tpc.Context(tpc.spec_for(workloads.config(6), fuse_radial=True)).sizes["act_bytes"] == 192
    # shapes the fused kernel does not take keep the two kernels
    for k, extra in ((5, {}), (0, {}), (1, dict(fp32_mfma_only=True)), (1, dict(table=(64, 8)))):
        assert not tpc.Context(tpc.spec_for(workloads.config(k), fuse_radial=True, **extra)).fused_radial
    lib, h = _raw(fused)
    eb = tpc._EdgeBuffers()
    cell = (ctypes.c_double * 9)(*np.eye(3).reshape(-1).tolist())
    st = lib.tpc_conv_fwd(h, 10, None, cell, None, None, None, None, 0, 10, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    assert "eb.A" in m and "eb.R" not in m
    lib, h = _raw(plain)
    st = lib.tpc_conv_fwd(h, 10, None, cell, None, None, None, None, 0, 10, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, 0, None)
    m = lib.tpc_last_error().decode()
    assert "eb.R" in m and "eb.A" not in m


def test_pair_radial_selection_sizes_and_checks():
    """Shared rows of R (spec.pair_radial): in effect for the unfused network
    only; the forward then needs rev and eb.Rrow, and its workspace grows by
    the rows' basis values."""
    plain, pair = tpc.Context(_spec()), tpc.Context(_spec(pair_radial=1))
    assert pair.pair_radial and not plain.pair_radial
    assert pair.sizes["fwd_workspace_bytes_per_edge"] == 8 * 4
    assert plain.sizes["fwd_workspace_bytes_per_edge"] == 0
    ne = 100_000
    grow = pair.workspace_bytes(tpc.OP_FWD, 0, ne) - plain.workspace_bytes(tpc.OP_FWD, 0, ne)
    assert 32 * ne <= grow <= 32 * ne + 8 * (ne // 4096 + 2) + 512
    # the fused forward and the tables keep one row per edge
    assert not tpc.Context(tpc.spec_for(workloads.config(6), fuse_radial=True, pair_radial=True)).pair_radial
    assert not tpc.Context(tpc.spec_for(workloads.config(1), table=(64, 8), pair_radial=True)).pair_radial
    # nor do the masked kernels of fewer than 64 channels
    assert not tpc.Context(_spec(pair_radial=1, channels=32,
                                 layer_dims=[8, 64, 64, 64, 10 * 32])).pair_radial
    lib, h = _raw(pair)
    eb = tpc._EdgeBuffers()
    cell = (ctypes.c_double * 9)(*np.eye(3).reshape(-1).tolist())
    st = lib.tpc_conv_fwd(h, 10, None, cell, None, None, None, None, 0, 10, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, 0, None)
    assert st == 1
    m = lib.tpc_last_error().decode()
    assert "rev" in m and "eb.Rrow" in m
    st = lib.tpc_conv_bwd(h, 10, 5, None, None, None, 0, 10, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, None, None, None, None, None, 0, None)
    assert st == 1 and "eb.Rrow" in lib.tpc_last_error().decode()
    lib, h = _raw(plain)
    st = lib.tpc_conv_fwd(h, 10, None, cell, None, None, None, None, 0, 10, 0, 5, None, None, 1.0, None,
                          ctypes.byref(eb), None, 0, None)
    assert "eb.Rrow" not in lib.tpc_last_error().decode()
