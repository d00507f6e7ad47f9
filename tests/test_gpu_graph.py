"""The convolution captured in a HIP graph.  Every call of the forward and
backward path enqueues kernels on the caller's stream and nothing else (no
allocation, no host wait when validation is off, no memset nodes: buffers are
cleared by fill kernels), so a caller can capture a whole step and replay it.
Each replay is checked against the eager result bit for bit, with the
program's own eager work and synchronisations between replays."""
import pytest

import tensor_product_conv_amd as tpc
from _gpu import Case, row_bounds, say, torch

pytestmark = pytest.mark.gpu


def _buffers(case, nl, chunks):
    t = torch()
    ctx = case.ctx
    rp = nl.row_ptr.cpu().numpy()
    bounds = [(a, b, int(rp[a]), int(rp[b])) for a, b in row_bounds(rp, chunks)]
    max_e = max(e1 - e0 for _, _, e0, e1 in bounds)
    N, C = case.N, case.cfg["C"]
    return dict(
        bounds=bounds,
        out=t.empty((N, ctx.d_out, C), dtype=ctx.dtype, device="cuda"),
        dh=t.empty_like(case.h),
        forces=t.empty((N, 3), dtype=ctx.dtype, device="cuda"),
        g_edge=t.empty((nl.n_edges, 3), dtype=ctx.dtype, device="cuda"),
        dR=t.empty((max_e, ctx.r_width), dtype=ctx.dtype, device="cuda"),
        dh_edge=t.empty((max_e, ctx.d_in, C), dtype=ctx.dtype, device="cuda"),
        eb=ctx.alloc_edge_buffers(max_e, "cuda"),
        ws_f=ctx._workspace(ctx.workspace_bytes(tpc.OP_FWD, N, max_e), "cuda"),
        ws_b=ctx._workspace(ctx.workspace_bytes(tpc.OP_BWD, N, max_e), "cuda"))


def _step(case, nl, b, s):
    ctx = case.ctx
    for q, (r0, r1, e0, e1) in enumerate(b["bounds"]):
        ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=b["out"], eb=b["eb"], rows=(r0, r1),
                     edges=(e0, e1), workspace=b["ws_f"])
        last = q == len(b["bounds"]) - 1
        ctx.conv_bwd(nl, case.h, case.W, s, case.G, b["eb"], dh=b["dh"], dR=b["dR"], g_edge=b["g_edge"],
                     dh_edge=b["dh_edge"], forces=b["forces"] if last else None, want_forces=last,
                     workspace=b["ws_b"])


KEYS = ("out", "dh", "forces", "g_edge")


@pytest.mark.parametrize("chunks,pair", [(1, False), (3, False), (1, True), (3, True)])
def test_graph_replay_matches_eager(chunks, pair):
    t = torch()
    case = Case(1, pair=pair)
    nl = case.nbr()
    s = case.scale(nl)
    b = _buffers(case, nl, chunks)
    say(f"[gpu] eager step cfg=1 chunks={chunks}")
    _step(case, nl, b, s)
    t.cuda.synchronize()
    ref = {k: b[k].clone() for k in KEYS}
    # capture after a warm-up on a side stream (default priority)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        _step(case, nl, b, s)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    say(f"[gpu] capture cfg=1 chunks={chunks}")
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        _step(case, nl, b, s)
    t.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: poison every output and intermediate
        # (the replay must rewrite them all), run an eager forward of its
        # own, and wait
        for x in [b[k] for k in KEYS] + [b["dR"], b["dh_edge"], b["eb"].Y, b["eb"].ef, b["eb"].rv, b["eb"].R]:
            x.fill_(float("nan"))
        if b["eb"].Rrow is not None:
            b["eb"].Rrow.fill_(0)     # a map the replay must rebuild (row 0: in bounds)
        case.ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, 2.0 * s, out=t.empty_like(b["out"]))
        t.cuda.synchronize()
        say(f"[gpu] replay {rep} cfg=1 chunks={chunks}")
        g.replay()
        t.cuda.synchronize()
        for k in KEYS:
            assert t.equal(b[k], ref[k]), (rep, k)
