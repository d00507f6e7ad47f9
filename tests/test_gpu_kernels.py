"""Every kernel instantiation the library accepts, element by element against
the oracle on the tiny system's geometry (32 atoms, about 540 edges): each
built tensor-product configuration (node_lmax, sh_lmax, out_lmax in (1,2,1),
(1,3,3), (2,3,3), (3,3,3) in float32; (1,2,1), (1,3,3) in float64; the other
float64 shapes are refused, see test_abi) at each channel class (fewer
than 64 channels with masked lanes, 64, 128), with separate and path-summed
outputs, and the radial MLP at every hidden shape (width 16, 32, 64; one to
three hidden layers) on each of its code paths (float32 products as bf16
splits, float32 and float64 matrix products, vector and scalar weight
loads), and the double backward of every configuration with separate
outputs.  Also checks the sizes the context reports."""
import itertools

import numpy as np
import pytest

import tensor_product_conv_amd as tpc
import workloads
from _gpu import TOL, Case, cotangents, rel, run_chunked, run_double, say
from oracle import conv

TP_CONFIGS = [(1, 2, 1), (1, 3, 3), (2, 3, 3), (3, 3, 3)]
CHANNELS = [8, 64, 128]
SHAPES = [(h, n) for h in (16, 32, 64) for n in (1, 2, 3)]


TP_CONFIGS_F64 = [(1, 2, 1), (1, 3, 3)]


def _cases():
    out = []
    for dt in ("float32", "float64"):
        k = 0
        cfgs = TP_CONFIGS if dt == "float32" else TP_CONFIGS_F64
        for (l1, l2, l3), C, summed in itertools.product(cfgs, CHANNELS, (False, True)):
            H, NH = SHAPES[(k * 4 + (1 if dt == "float64" else 0)) % len(SHAPES)]
            out.append((dt, l1, l2, l3, C, summed, H, NH))
            k += 1
    return out


CASES = _cases()


def test_case_list_covers_every_radial_shape():
    # host-only bookkeeping of the list above: every (dtype, H, NH) occurs,
    # and float32 takes each radial code path at least once
    for dt in ("float32", "float64"):
        assert {(H, NH) for d, *_, H, NH in CASES if d == dt} == set(SHAPES)
    paths32 = set()
    for dt, l1, l2, l3, C, summed, H, NH in CASES:
        if dt != "float32":
            continue
        P = sum(1 for a in range(l1 + 1) for b in range(l2 + 1) for c in range(l3 + 1)
                if abs(a - b) <= c <= a + b and (a + b + c) % 2 == 0)
        pc = P * C
        paths32.add("x6" if H % 32 == 0 and pc % 32 == 0 else
                    "pairs" if pc % 32 == 0 else "vec" if pc % 16 == 0 else "scalar")
    assert paths32 == {"x6", "pairs", "vec", "scalar"}


@pytest.mark.gpu
@pytest.mark.parametrize("dt,l1,l2,l3,C,summed,H,NH", CASES,
                         ids=[f"{c[0][-2:]}-{c[1]}{c[2]}{c[3]}-C{c[4]}-{'sum' if c[5] else 'sep'}-H{c[6]}x{c[7]}"
                              for c in CASES])
def test_instantiation_parity(dt, l1, l2, l3, C, summed, H, NH):
    seed = 1000 + CASES.index((dt, l1, l2, l3, C, summed, H, NH))
    d = workloads.variant(0, C, l1, l2, l3, [H] * NH, dt, seed, summed)
    case = Case(0, data=d)
    info = case.ctx.sizes
    T = 8 if dt == "float64" else 4
    assert info["dR_bytes"] == T * case.ctx.r_width
    assert info["edge_buffer_bytes"] == T * (case.ctx.d_sh + 8 + 4 + case.ctx.r_width)
    nl = case.nbr()
    tol = TOL[dt]
    res = run_chunked(case, nl, chunks=1, keep_edges=np.arange(nl.n_edges))
    ref_csr = case.oracle_csr()
    prob = case.oracle(ref_csr)
    say(f"[cpu] oracle {dt} ({l1},{l2},{l3}) C={C} summed={summed} H={H}x{NH}")
    out_ref = prob.forward()
    b = prob.backward()
    errs = {
        "out": rel(res["out"].cpu().numpy(), out_ref),
        "dh": rel(res["dh"].cpu().numpy(), b["dh"]),
        "dR": rel(np.stack([res["dR"][e] for e in range(nl.n_edges)]), b["dR"]),
        "g_edge": rel(res["g_edge"].cpu().numpy(), b["g"]),
        "forces": rel(res["forces"].cpu().numpy(), b["F"]),
    }
    _, _, Y, ef, R = prob.edge_terms(np.arange(nl.n_edges))
    errs["R"] = rel(res["eb"].R_per_edge().cpu().numpy(), R)
    if not summed:
        u = cotangents(case, nl.n_edges, seed + 500)
        dres = run_double(case, nl, u, keep_edges=np.arange(nl.n_edges))
        dref = prob.double_backward(*u)
        errs["g_hat"] = rel(dres["g_hat"].cpu().numpy(), dref["g_hat"])
        errs["h_hat"] = rel(dres["h_hat"].cpu().numpy(), dref["x_hat"])
        errs["Y_hat"] = rel(np.stack([dres["Y_hat"][e] for e in range(nl.n_edges)]), dref["y_hat"])
        errs["R_hat"] = rel(np.stack([dres["R_hat"][e] for e in range(nl.n_edges)]), dref["w_hat"])
    say(f"[cmp] {errs}")
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, bad
