"""Benchmark of the equivariant interaction convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload medium]

One step is the whole hot path over the synthetic medium water system
(32,768 atoms, C = 128, node irreps 0e+1o+2e, harmonics l <= 3, outputs
l <= 3, radial MLP 8-64-64-64-2176, about 2.97 M directed edges): the
periodic neighbour build, the forward convolution and its backward
(dL/dh, dL/dR, forces).  Inputs are resident in HBM before timing starts.
The metric is directed edges per second through that step.

Per-kernel durations come from HIP events the library records around each
launch on the launch stream during the timed steps; the dominant kernel's
algorithmic bytes (or flops) per launch divided by its average duration gives
the roofline line.  HBM traffic from rocprofv3 counters is read from
profiles/traffic.json when it was measured on the current kernel sources.
The CPU baseline times the float64 oracle on a bounded sample of receivers.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_F32_PEAK = 157.3e12   # flop/s, dense fp32 matrix
VALU_F32_PEAK = 78.6e12    # flop/s, fp32 FMA without packed math: 256 CU x 4 SIMD x 16 lanes x 2 x 2.4 GHz
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 matrix

KERNEL_SOURCES = {
    "tp_fwd": ["tp_impl.hpp", "tp_fwd.hip", "tables.hpp"],
    "tp_bwd_edge": ["tp_impl.hpp", "tp_bwd_edge.hip", "tables.hpp"],
    "dh_gather": ["tp_impl.hpp", "tp_bwd_edge.hip"],
    "radial_fwd": ["radial.hip"],
    "radial_bwd_dA": ["radial.hip"],
    "radial_bwd_mlp": ["radial.hip"],
    "geom_fwd": ["geom.hip"],
    "geom_bwd": ["geom.hip"],
}


# Symbol fragment of each timed kernel, to find its dispatches in rocprofv3 output.
KERNEL_SYMBOLS = {
    "tp_fwd": "k_tp_fwd<",
    "tp_bwd_edge": "k_tp_bwd_edge<",
    "dh_gather": "k_dh_gather<",
    "radial_fwd": "k_radial_fwd<",
    "radial_bwd_dA": "k_radial_bwd_dA",   # also the bf16-split k_radial_bwd_dA_x6
    "radial_bwd_mlp": "k_radial_bwd_mlp<",
    "geom_fwd": "k_geom_fwd<",
    "geom_bwd": "k_geom_bwd<",
}
COPY_PROBE_BYTES = 1 << 30   # one plain device-to-device copy of this size calibrates the counters


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "tensor_product_conv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(kernel, N, E, cfg, ctx):
    """(bytes, flops) one launch of ``kernel`` must move / compute (fp32)."""
    T = 4
    C, P = cfg["C"], ctx.n_paths
    din, dsh, dout, PC = ctx.d_in, ctx.d_sh, ctx.d_out, ctx.r_width
    H = cfg["hidden"][0]
    NH = len(cfg["hidden"])
    tabs = [ctx.cg_table(p) for p in range(ctx.n_paths)]       # the library's own tables
    nnz = sum(int((t != 0).sum()) for t in tabs)
    m13 = sum(int((t != 0).any(axis=1).sum()) for t in tabs)
    csr = 4 * (N + 1) + 4 * E
    if kernel == "tp_fwd":
        return (E * (T * PC + T * dsh) + N * T * C * (din + dout) + csr,
                E * (2 * nnz + C * (2 * m13 + 2 * dout)))
    if kernel == "tp_bwd_edge":
        # reads R, Y, h and G (once per atom); writes dR and dY.  The per-edge
        # dh contributions it also writes are an intermediate of the two-kernel
        # split, not algorithmic traffic.
        return (E * (2 * T * PC + 2 * T * dsh) + N * T * C * (din + dout) + csr,
                E * C * (2 * nnz + 4 * m13 + 2 * din + 2 * dout))
    if kernel == "dh_gather":
        # as a kernel of its own: reads the per-edge contributions, writes dh
        # (the K9 group below counts only dh, the pass's algorithmic output)
        return (E * T * C * din + N * T * C * din + 4 * (N + 1), E * C * din)
    hidden = 2 * (8 * H + (NH - 1) * H * H)
    if kernel == "radial_fwd":
        return E * (8 * T + T * PC), E * (hidden + 2 * H * PC)
    if kernel == "radial_bwd_dA":
        # reads dR, writes dA (H per edge)
        return E * (T * PC + T * H), E * 2 * H * PC
    if kernel == "radial_bwd_mlp":
        # reads ef and dA, writes d(ef); recomputes the hidden layers
        return E * (8 * T + T * H + 8 * T), E * 2 * hidden
    return None, None


def group_rooflines(per_kernel, N, E, cfg, ctx):
    """HBM fraction of the fused tensor-product passes, each taken as the
    kernels that make it up: K8 = tp_fwd; K9 = tp_bwd_edge + dh_gather, whose
    algorithmic bytes are R, Y, h, G and the CSR in, dR, dY and dh out."""
    T = 4
    C, PC, din, dsh, dout = cfg["C"], ctx.r_width, ctx.d_in, ctx.d_sh, ctx.d_out
    csr = 4 * (N + 1) + 4 * E
    groups = {
        "K8_tp_forward": (["tp_fwd"], E * (T * PC + T * dsh) + N * T * C * (din + dout) + csr),
        "K9_tp_backward": (["tp_bwd_edge", "dh_gather"],
                           E * (2 * T * PC + 2 * T * dsh) + N * T * C * (2 * din + dout) + csr),
    }
    out = {}
    for name, (ks, nbytes) in groups.items():
        if not all(k in per_kernel for k in ks):
            continue
        sec = sum(per_kernel[k]["avg_ms"] for k in ks) * 1e-3
        out[name] = dict(kernels=ks, algorithmic_bytes=nbytes, ms=sec * 1e3,
                         achieved_GBps=nbytes / sec / 1e9, frac=nbytes / sec / HBM_PEAK)
    return out


def roofline_for(kernel, per_launch_s, N, E, cfg, ctx):
    nbytes, flops = algorithmic(kernel, N, E, cfg, ctx)
    if nbytes is None:
        return None
    H, PC = cfg["hidden"][0], ctx.r_width
    if kernel in ("radial_fwd", "radial_bwd_dA") and str(ctx.dtype) == "torch.float32" and H % 32 == 0 and PC % 64 == 0:
        # the float32 last-layer products run as six bf16 products (three-part
        # operand split), the hidden layers on fp32 matrix cores; at those
        # rates the matrix work takes well under the time to stream R or dR,
        # so HBM bounds these kernels
        last = E * 2 * H * PC
        ach = nbytes / per_launch_s
        r = dict(bound="hbm", achieved=ach / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s",
                 frac=ach / HBM_PEAK, algorithmic_bytes_per_launch=nbytes,
                 matrix_frac=((flops - last) / MFMA_F32_PEAK + 6 * last / MFMA_BF16_PEAK) / per_launch_s)
    elif kernel.startswith("radial"):
        ach = flops / per_launch_s
        r = dict(bound="mfma", achieved=ach / 1e12, peak=MFMA_F32_PEAK / 1e12, unit="TFLOP/s",
                 frac=ach / MFMA_F32_PEAK, algorithmic_flops_per_launch=flops)
    else:
        ach = nbytes / per_launch_s
        r = dict(bound="hbm", achieved=ach / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s",
                 frac=ach / HBM_PEAK, algorithmic_bytes_per_launch=nbytes,
                 vector_alu_frac=(flops / per_launch_s) / VALU_F32_PEAK)
    r["kernel"] = kernel
    # the committed counters were taken on the default (separate-path) layout
    r["traffic"] = None if cfg.get("sum_paths") else measured_traffic(kernel)
    return r


def measured_traffic(kernel):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    rec = t.get(kernel)
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(directory):
    """(kernel name, dispatch id, counter, value) from every rocprofv3
    counter_collection.csv under ``directory``."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                k = {key.lower(): v for key, v in r.items()}
                rows.append((k.get("kernel_name", ""), k.get("dispatch_id", ""), k.get("counter_name", ""),
                             float(k.get("counter_value", "nan"))))
    return rows


def _per_dispatch(rows, counter):
    acc = {}
    for name, did, cname, v in rows:
        if cname == counter:
            key = (name, did)
            acc[key] = acc.get(key, 0.0) + v
    return acc


def traffic_from(fetch_dir, write_dir, out_path):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, both in KiB
    per dispatch) of ``bench.py --copy-probe`` into HBM bytes per launch of
    each kernel, each counter scaled by what it reads for a plain copy of
    COPY_PROBE_BYTES (read once, written once)."""
    out = {}
    per = {}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        disp = _per_dispatch(_counter_rows(d), counter)
        copies = sorted((v for (name, _), v in disp.items() if "copy" in name.lower()), reverse=True)[:3]
        if not copies:
            raise SystemExit(f"no copy-kernel dispatch with {counter} under {d}")
        copy_kib = sorted(copies)[len(copies) // 2]
        factor = COPY_PROBE_BYTES / (copy_kib * 1024.0)
        out[f"_{label}_calibration"] = {"counter": counter, "copy_bytes": COPY_PROBE_BYTES,
                                        "copy_counter_kib": copy_kib, "factor": factor}
        for kernel, sym in KERNEL_SYMBOLS.items():
            vals = [v for (name, _), v in disp.items() if sym in name]
            if vals:
                per.setdefault(kernel, {})[label] = (sum(vals) / len(vals)) * 1024.0 * factor
                per[kernel][label + "_dispatches"] = len(vals)
    for kernel, v in per.items():
        if "fetch" in v and "write" in v:
            out[kernel] = {"hbm_bytes_per_launch": v["fetch"] + v["write"], "read_bytes": v["fetch"],
                           "write_bytes": v["write"], "dispatches": v["fetch_dispatches"],
                           "source_hash": source_hash(kernel)}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))
    return 0


_CPU_PROB = None   # the oracle problem the CPU-baseline workers inherit by fork


def _cpu_task(rows):
    """One batch of receiver rows through the oracle: forward rows and the
    per-edge backward.  Returns the batch's edge count."""
    from threadpoolctl import threadpool_limits
    from oracle import conv

    prob = _CPU_PROB
    e, _ = conv.edges_of_rows(prob.row_ptr, rows)
    with threadpool_limits(limits=1):
        prob.forward_rows(rows)
        prob.edge_backward(e)
    return len(e)


def cpu_baseline(case_data, budget_s=10.0):
    """The float64 oracle's forward + per-edge backward on random batches of
    receiver rows, one single-threaded worker process per host core of this
    GPU's share (at most 16), for about ``budget_s`` seconds of wall time.
    Runs before the GPU is touched: the workers are forked from this process.
    The oracle works on its own neighbour list (built before the timing)."""
    global _CPU_PROB
    import multiprocessing as mp
    import numpy as np
    from oracle import conv, nbr, paths

    d = case_data
    c = d["cfg"]
    rp, src, shift = nbr.binned(d["pos"], d["cell"], c["r_cut"])
    L = paths.Layout(c["l1max"], c["sh_lmax"], c["out_lmax"], c["C"], c.get("sum_paths", False))
    _CPU_PROB = conv.Problem(L, d["pos"], d["cell"], rp, src, shift, d["h"], d["W"], c["r_cut"],
                             conv.scale_for(c, len(d["pos"]), rp[-1]), d["G"])
    order = np.random.default_rng(0).permutation(len(d["pos"]))
    batches = [np.sort(order[k:k + 64]) for k in range(0, len(order), 64)]
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    done_edges = done_rows = 0
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        for n_e in pool.imap_unordered(_cpu_task, batches, chunksize=1):
            done_edges += n_e
            done_rows += 64
            if time.perf_counter() - t0 > budget_s:
                break
        wall = time.perf_counter() - t0
        pool.terminate()
    _CPU_PROB = None
    return dict(value=done_edges / wall, unit="edges/s", cores=workers, kind="oracle",
                sample=f"{done_rows} random receiver rows ({done_edges} edges) of the same system in "
                       f"batches of 64, completed in {wall:.1f} s of wall time by {workers} single-threaded "
                       f"worker processes: float64 oracle forward + per-edge backward (dR, dY, dh "
                       f"contributions, edge gradients); neighbour build not included")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="medium", choices=["medium", "small"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sum-paths", action="store_true",
                    help="path-summed outputs (one block per output rank) on the same system")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, copy %d bytes device to device three times "
                         "(counter calibration for rocprofv3 --pmc runs)" % COPY_PROBE_BYTES)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output folders and exit")
    a = ap.parse_args(argv)
    if a.traffic_from:
        return traffic_from(a.traffic_from[0], a.traffic_from[1],
                            os.path.join(ROOT, "profiles", "traffic.json"))
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE={world}); "
              "the convolution is benchmarked at N=1 and no multi-GPU path is built", flush=True)
        return 2

    import numpy as np
    import torch

    import tensor_product_conv_amd as tpc
    import workloads

    k = {"small": 1, "medium": 3}[a.workload]
    d = workloads.generate(k)
    cfg = d["cfg"]
    if a.sum_paths:
        cfg = dict(cfg, sum_paths=True, name=cfg["name"] + "_summed")
        cfg["d_out"] = tpc.Context(tpc.spec_for(cfg)).d_out   # host only, no device call
        d = dict(d, cfg=cfg, G=np.random.default_rng(cfg["seed"] + 100).standard_normal(
            (cfg["N"], cfg["d_out"], cfg["C"])).astype(d["G"].dtype))
    # the CPU leg forks its workers, so it runs before anything touches the GPU
    cpu = None if a.no_cpu_baseline else cpu_baseline(d, a.cpu_budget)
    dev = "cuda"
    ctx = tpc.Context(tpc.spec_for(cfg))
    pos = torch.from_numpy(d["pos"]).to(dev)
    species = torch.from_numpy(d["species"]).to(dev)
    h = torch.from_numpy(d["h"]).to(dev)
    W = [torch.from_numpy(w).to(dev) for w in d["W"]]
    G = torch.from_numpy(d["G"]).to(dev)
    cell = d["cell"]
    N = cfg["N"]

    nl = ctx.nbr_build(pos, cell, species)
    E = nl.n_edges
    scale = float(N) / E if cfg["scale"] == "inv_avg_neighbors" else 1.0
    out = torch.empty((N, ctx.d_out, cfg["C"]), dtype=ctx.dtype, device=dev)
    eb = ctx.alloc_edge_buffers(E, dev)
    dh = torch.empty_like(h)
    dR = torch.empty((E, ctx.r_width), dtype=ctx.dtype, device=dev)
    g_edge = torch.empty((E, 3), dtype=ctx.dtype, device=dev)
    dh_edge = torch.empty((E, ctx.d_in, cfg["C"]), dtype=ctx.dtype, device=dev)
    forces = torch.empty((N, 3), dtype=ctx.dtype, device=dev)
    ws_n = ctx._workspace(ctx.workspace_bytes(tpc.OP_NBR, N, 0, cell), dev)
    ws_f = ctx._workspace(ctx.workspace_bytes(tpc.OP_FWD, N, E), dev)
    ws_b = ctx._workspace(ctx.workspace_bytes(tpc.OP_BWD, N, E), dev)

    def step():
        nl2 = ctx.nbr_build(pos, cell, species, edge_cap=E, into=nl, workspace=ws_n)
        ctx.conv_fwd(pos, cell, nl2, h, W, scale, out=out, eb=eb, workspace=ws_f)
        ctx.conv_bwd(nl2, h, W, scale, G, eb, dh=dh, dR=dR, g_edge=g_edge, dh_edge=dh_edge,
                     forces=forces, workspace=ws_b)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    tpc.timing_collect()
    tpc.timing_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(a.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tpc.timing_enable(False)
    kt = tpc.timing_collect()
    ms_per_step = start.elapsed_time(stop) / a.steps
    value = E / (ms_per_step * 1e-3)

    per_kernel = {n: dict(avg_ms=tot / cnt, launches_per_step=cnt / a.steps, ms_per_step=tot / a.steps)
                  for n, (tot, cnt) in kt.items()}

    # the virial (strain derivative) from the step's edge gradients, timed on
    # its own: it is not part of the step
    vir = torch.empty((3, 3), dtype=ctx.dtype, device=dev)
    ws_v = ctx._workspace(ctx.workspace_bytes(tpc.OP_VIRIAL, N), dev)
    for _ in range(2):
        ctx.virial(pos, cell, nl, g_edge, out=vir, workspace=ws_v)
    torch.cuda.synchronize()
    tpc.timing_enable(True)
    for _ in range(a.steps):
        ctx.virial(pos, cell, nl, g_edge, out=vir, workspace=ws_v)
    torch.cuda.synchronize()
    tpc.timing_enable(False)
    vt = tpc.timing_collect()
    virial_ms = vt["virial"][0] / vt["virial"][1] if "virial" in vt else None
    # one launch of each per pass (the weight packing runs once in each pass)
    fwd_ms = sum(per_kernel.get(n, {}).get("avg_ms", 0.0)
                 for n in ("geom_fwd", "radial_pack", "radial_fwd", "tp_fwd"))
    bwd_ms = sum(per_kernel.get(n, {}).get("avg_ms", 0.0)
                 for n in ("tp_bwd_edge", "radial_pack", "radial_bwd_dA", "radial_bwd_mlp", "geom_bwd",
                           "dh_gather", "forces"))
    nbr_ms = sum(v["ms_per_step"] for n, v in per_kernel.items() if n.startswith("nbr"))
    dominant = max((n for n in per_kernel if n in KERNEL_SOURCES), key=lambda n: per_kernel[n]["ms_per_step"])
    roof = roofline_for(dominant, per_kernel[dominant]["avg_ms"] * 1e-3, N, E, cfg, ctx)
    kernels = {}
    for n, v in per_kernel.items():
        r = roofline_for(n, v["avg_ms"] * 1e-3, N, E, cfg, ctx) if n in KERNEL_SOURCES else None
        kernels[n] = dict(avg_ms=round(v["avg_ms"], 4), launches_per_step=v["launches_per_step"],
                          **({"bound": r["bound"], "frac": round(r["frac"], 4)} if r else {}))

    if a.copy_probe:
        src_t = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t


    line = {
        "metric": "edges/s fwd and fwd+bwd, 128ch sh l<=3 TP conv; % of HBM roofline",
        "value": value,
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']} ({'water' if k == 3 else cfg['geometry']}) "
                               f"N={N} E={E} C={cfg['C']} node_lmax={cfg['l1max']} "
                               f"sh_lmax={cfg['sh_lmax']} out_lmax={cfg['out_lmax']} "
                               f"mlp={'-'.join(map(str, cfg['layer_dims']))}: "
                               "nbr_build + conv_fwd + conv_bwd (forces)"
                               + (", path-summed outputs" if cfg.get("sum_paths") else ""),
                   "n_atoms": N, "n_edges": E, "channels": cfg["C"], "paths": ctx.n_paths,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "fwd_edges_per_s": E / (fwd_ms * 1e-3) if fwd_ms else None,
        "fwd_bwd_edges_per_s": E / ((fwd_ms + bwd_ms) * 1e-3) if fwd_ms else None,
        "nbr_build_ms": nbr_ms,
        "virial_ms": virial_ms,
        "kernels": kernels,
        "tp_groups_hbm": group_rooflines(per_kernel, N, E, cfg, ctx),
        "wall_s": wall,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
