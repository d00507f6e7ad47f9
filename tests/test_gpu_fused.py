"""The forward with the radial last layer fused into the tensor-product kernel
(spec.fuse_radial; FastMACE page "Rewrites and precision options", section
"Convolution (OEq streaming)": the fused folded forward), against the
oracle: a forward-only call that stores no R, a forward that also stores R
for the backward (the full backward then runs on it), determinism and
receiver chunks."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import TOL, Case, np_csr, rel, run_chunked, say, torch

pytestmark = pytest.mark.gpu


def _fused_case(k, with_grad=True):
    # "10h64": config 10's dense system (node l <= 3, C = 64) with two hidden
    # layers of 64, the large system's fused instantiation (P = 23 slices of
    # 6 KB in LDS)
    data = workloads.variant(10, 64, 3, 3, 3, [64, 64], "float32", 1064) if k == "10h64" else None
    case = Case(10 if k == "10h64" else k, with_grad=with_grad, data=data)
    case.ctx = tpc.Context(tpc.spec_for(case.cfg, fuse_radial=True))
    assert case.ctx.fused_radial and case.ctx.sizes["act_bytes"] > 0
    return case


def _oracle(case, nl):
    ref = case.oracle_csr()
    for a, b in zip(np_csr(nl)[:3], ref):
        np.testing.assert_array_equal(a, b)
    return case.oracle(ref)


# 1 small; 6, 7 hidden width 32 at 64 and 32 channels (one k-block of the
# split products, 4 and 2 channel slices); 8 path-summed outputs; 9 rows of
# 114-176 edges (up to 11 batches of 16 per row, ragged last batches); 10
# node l <= 3 (P = 23, the largest weight slice in LDS)
@pytest.mark.timeout(300)
@pytest.mark.parametrize("k", [1, 6, 7, 8, 9, 10, "10h64"])
def test_forward_without_R_matches_the_oracle(k):
    case = _fused_case(k, with_grad=False)
    ctx = case.ctx
    nl = case.nbr()
    s = case.scale(nl)
    E = nl.n_edges
    say(f"[gpu] fused conv_fwd with and without R cfg={k}")
    out1, eb1 = ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s,
                             eb=ctx.alloc_edge_buffers(E, "cuda", with_R=True))
    eb2 = ctx.alloc_edge_buffers(E, "cuda", with_R=False)
    assert eb2.R is None and eb2.A is not None
    out2, _ = ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, eb=eb2)
    torch().cuda.synchronize()
    # the same arithmetic in the same order: the R stores change nothing else
    assert torch().equal(out1, out2)
    prob = _oracle(case, nl)
    say(f"[cpu] oracle forward cfg={k}")
    tol = TOL[case.cfg["dtype"]]
    assert rel(out1.cpu().numpy(), prob.forward()) < tol
    _, _, _, _, R = prob.edge_terms(np.arange(E))
    assert rel(eb1.R.cpu().numpy(), R) < tol


@pytest.mark.timeout(300)
@pytest.mark.parametrize("k", [1, 8, 9, 10, "10h64"])
def test_backward_on_the_fused_forward(k):
    case = _fused_case(k)
    nl = case.nbr()
    res = run_chunked(case, nl, chunks=1, keep_edges=np.arange(nl.n_edges))
    prob = _oracle(case, nl)
    say(f"[cpu] oracle cfg={k}")
    tol = TOL[case.cfg["dtype"]]
    assert rel(res["out"].cpu().numpy(), prob.forward()) < tol
    b = prob.backward()
    assert rel(res["dh"].cpu().numpy(), b["dh"]) < tol
    assert rel(np.stack([res["dR"][e] for e in range(nl.n_edges)]), b["dR"]) < tol
    assert rel(res["forces"].cpu().numpy(), b["F"]) < tol


def test_fused_forward_is_deterministic_and_chunk_invariant():
    """Two runs agree bit for bit, and a forward in three receiver chunks
    (whose batches start at other edges) equals the single call."""
    case = _fused_case(1, with_grad=False)
    ctx = case.ctx
    nl = case.nbr()
    s = case.scale(nl)
    E = nl.n_edges
    say("[gpu] fused conv_fwd determinism and chunks cfg=1")
    out_a, _ = ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, eb=ctx.alloc_edge_buffers(E, "cuda"))
    out_b, _ = ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, eb=ctx.alloc_edge_buffers(E, "cuda"))
    torch().cuda.synchronize()
    assert torch().equal(out_a, out_b)
    rp = nl.row_ptr.cpu().numpy()
    out_c = torch().zeros_like(out_a)
    cuts = [0, 1000, 2345, case.N]
    for a, b in zip(cuts[:-1], cuts[1:]):
        e0, e1 = int(rp[a]), int(rp[b])
        ctx.conv_fwd(case.pos, case.cell, nl, case.h, case.W, s, out=out_c, rows=(a, b), edges=(e0, e1),
                     eb=ctx.alloc_edge_buffers(e1 - e0, "cuda", with_R=False))
    torch().cuda.synchronize()
    assert torch().equal(out_a, out_c)


@pytest.mark.timeout(300)
def test_fused_step_medium_sampled():
    """The medium water system through the fused forward (R stored) and the
    backward, in the launch configuration of the fused benchmark line: out,
    dR and g_edge on sampled rows and edges, dh and forces on sampled atoms,
    against the oracle."""
    from test_gpu_conv import _sampled_check, _samples, _spread
    case = _fused_case(3)
    nl = case.nbr()
    rows, edges = _samples(case, 64, 21)
    res = run_chunked(case, nl, chunks=1, keep_edges=edges)
    _sampled_check(case, nl, res, rows, _spread(rows, 24), edges)
