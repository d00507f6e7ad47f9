"""Precision of the float32 radial last layer when its terms cancel.

By default the float32 products R = a W_L (forward) and dA = dR W_L^T
(backward) run as six bf16 matrix products of three-part operand splits, the
split-product option of the FastMACE page "Rewrites and precision options"
(whose tf32 analogue is noted there to differ from IEEE float32 where terms
cancel).  These tests build weights whose last-layer sums cancel: hidden units
come in identical pairs (equal columns of the previous layer, so equal
activations) whose last-layer rows are +M x + y and -M x + y', so each output
is a small difference of terms M times larger.  Every element of R is then
held to the float32 bound of the computation,
    |err| <= 2 K 2^-24 sum_k |a_k| |W_kc| + 8 2^-24 r |dR_c/dr|,
the last layer's dot product plus the rounding of the distance it is given
(the basis is ill-conditioned just inside the cutoff), on the split path and
on the float32-matrix path (spec.fp32_mfma_only), with a_k the oracle's
float64 activations.  The backward through the same weights is compared
between the two paths."""
import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import Case, rel, run_chunked, say, torch
from oracle import radial

pytestmark = pytest.mark.gpu


def _cancelling_case(fp32_only, M=256.0):
    d = workloads.variant(1, 128, 1, 3, 3, [64, 64], "float32", 501)   # the small system
    rng = np.random.default_rng(502)
    W1, W2, WL = [w.astype(np.float64) for w in d["W"]]
    H = W2.shape[1]
    W2[:, 1::2] = W2[:, 0::2]                      # unit pairs with equal activations
    x = rng.standard_normal((H // 2, WL.shape[1])) / np.sqrt(H)
    WL[0::2] = M * x + WL[0::2]
    WL[1::2] = -M * x + WL[1::2]
    d["W"] = [w.astype(np.float32) for w in (W1, W2, WL)]
    case = Case(1, data=d)
    if fp32_only:
        case.ctx = tpc.Context(tpc.spec_for(d["cfg"], fp32_mfma_only=True))
    return case


@pytest.mark.parametrize("fp32_only", [False, True], ids=["bf16-split", "fp32-mfma"])
def test_cancelling_last_layer_within_the_float32_bound(fp32_only):
    case = _cancelling_case(fp32_only)
    nl = case.nbr()
    res = run_chunked(case, nl, chunks=1)
    prob = case.oracle(case.oracle_csr())
    for a, b in zip([nl.row_ptr.cpu().numpy(), nl.src.cpu().numpy(), nl.shift.cpu().numpy()], case.oracle_csr()):
        np.testing.assert_array_equal(a, b)
    e = np.arange(nl.n_edges)
    _, r, _, ef, R = prob.edge_terms(e)
    # the oracle's float64 last hidden activations and the bound
    a = np.asarray(ef, dtype=np.float64)
    W = [np.asarray(w, dtype=np.float64) for w in case.d["W"]]
    for Wk in W[:-1]:
        a = radial.silu(a @ Wk)
    dRdr = radial.radial_weights_dr(r, W, case.cfg["r_cut"])
    bound = 2.0 * a.shape[1] * 2.0 ** -24 * (np.abs(a) @ np.abs(W[-1])) + 8.0 * 2.0 ** -24 * np.abs(r[:, None] * dRdr)
    got = res["eb"].R_per_edge().cpu().numpy().astype(np.float64)
    err = np.abs(got - R)
    ratio = float((err / bound).max())
    cancel = float(np.median((np.abs(a) @ np.abs(W[-1])) / np.maximum(np.abs(R), 1e-30)))
    say(f"[cmp] fp32_only={fp32_only}: max err/bound {ratio:.3f}, median cancellation {cancel:.0f}x")
    assert cancel > 20.0          # the sums do cancel
    assert ratio <= 1.0


def test_cancelling_backward_split_matches_float32_matrix_path():
    """Edge gradients through the cancelling weights: the split path's error
    against the float64 oracle stays within a small factor of the float32
    matrix path's own error."""
    errs = {}
    for fp32_only in (False, True):
        case = _cancelling_case(fp32_only)
        nl = case.nbr()
        res = run_chunked(case, nl, chunks=1)
        prob = case.oracle(case.oracle_csr())
        b = prob.backward()
        errs[fp32_only] = (rel(res["g_edge"].cpu().numpy(), b["g"]), rel(res["forces"].cpu().numpy(), b["F"]),
                           rel(res["dh"].cpu().numpy(), b["dh"]))
    say(f"[cmp] split {errs[False]} fp32 {errs[True]}")
    for k in range(3):
        assert errs[False][k] <= 4.0 * errs[True][k] + 1e-6
