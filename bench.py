"""Benchmark of the equivariant interaction convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload medium|small|large]

One step is the whole hot path over one synthetic system: the periodic
neighbour build, the forward convolution and its backward (dL/dh, dL/dR,
forces).  The default workload is the medium water system (32,768 atoms,
C = 128, node irreps 0e+1o+2e, harmonics l <= 3, outputs l <= 3, radial MLP
8-64-64-64-2176, about 2.93 M directed edges).  The small system (4,096
atoms, C = 128) and the large fcc system (262,144 atoms, C = 64, about
19.8 M edges, processed in 2 receiver chunks) are the other lines.  Inputs
are resident in HBM before timing starts.  The metric is directed edges per
second through the step.  An edge and its reverse share one row of radial
weights (spec.pair_radial); --per-edge-radial times one row per edge.

Per-kernel durations come from HIP events the library records around each
launch on the launch stream during the timed steps; the dominant kernel's
algorithmic bytes (or flops) per step divided by its time per step (the
per-launch ratio, chunk by chunk) gives the roofline line.  HBM traffic from
rocprofv3 counters is read from profiles/traffic_<workload>.json when it was
measured on the current kernel sources.  The virial and the VJP-of-VJP are
timed after the steps, outside them.  The CPU baseline times the float64
oracle on a bounded sample of receivers.
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
    "tp_fwd": ["tp_impl.hpp", "tp_fwd.hip", "tables.hpp", "tp_config.hpp"],
    "tp_bwd_edge": ["tp_impl.hpp", "tp_bwd.hip", "tables.hpp", "tp_config.hpp"],
    "dh_gather": ["tp_impl.hpp", "tp_dispatch.hip"],
    "radial_fwd": ["radial.hip"],
    "radial_bwd_dA": ["radial.hip"],
    "radial_bwd_mlp": ["radial.hip"],
    "geom_fwd": ["geom.hip"],
    "geom_bwd": ["geom.hip"],
    "table_fwd": ["radial_table.hip"],
    "table_bwd": ["radial_table.hip"],
    "radial_act": ["radial.hip"],
    "tp_fwd_fused": ["tp_fused.hpp", "tp_fused.hip", "tp_impl.hpp", "tables.hpp", "tp_config.hpp"],
}


# Symbol fragment of each timed kernel, to find its dispatches in rocprofv3 output.
KERNEL_SYMBOLS = {
    "tp_fwd": "k_tp_fwd<",
    "tp_bwd_edge": "k_tp_bwd_edge<",
    "dh_gather": "k_dh_gather_chunk<",
    "radial_fwd": "k_radial_fwd<",
    "radial_bwd_dA": "k_radial_bwd_dA",   # also the bf16-split k_radial_bwd_dA_x6
    "radial_bwd_mlp": "k_radial_bwd_mlp<",
    "geom_fwd": "k_geom_fwd<",
    "geom_bwd": "k_geom_bwd<",
    "table_fwd": "k_table_fwd_sorted<",
    "table_bwd": "k_table_bwd_sorted<",
    "radial_act": "k_radial_act<",
    "tp_fwd_fused": "k_tp_fwd_fused<",
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
    hidden = 2 * (8 * H + (NH - 1) * H * H)
    if kernel == "tp_fwd":
        return (E * (T * PC + T * dsh) + N * T * C * (din + dout) + csr,
                E * (2 * nnz + C * (2 * m13 + 2 * dout)))
    if kernel == "tp_fwd_fused":
        # reads the split activations (an intermediate of the radial split,
        # counted here because this kernel is where they are read), Y, h and
        # the CSR; writes out, and R when the backward needs it
        act = ctx.sizes["act_bytes"]
        r_out = T * PC if cfg.get("_store_R", True) else 0
        tp = E * C * (2 * m13 + 2 * dout)
        return (E * (act + T * dsh + r_out) + N * T * C * (din + dout) + csr,
                tp + E * (2 * nnz * (C // 16)) + E * 2 * H * PC)
    if kernel == "radial_act":
        # reads ef, writes the split activations
        return E * (8 * T + ctx.sizes["act_bytes"]), E * hidden
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
        # one row of R per distinct edge length: with rows shared by edge
        # pairs, half the edges of a symmetric list (plus the pairs cut by a
        # chunk boundary)
        rows = cfg.get("_R_rows", E)
        return rows * (8 * T + T * PC), rows * (hidden + 2 * H * PC)
    if kernel == "radial_bwd_dA":
        # reads dR, writes dA (H per edge)
        return E * (T * PC + T * H), E * 2 * H * PC
    if kernel == "table_fwd":
        # reads the edge length, writes R (the coefficients are cache traffic)
        return E * (T + T * PC), E * PC * 2 * 2 * (cfg.get("_table_degree", 8) + 1)
    if kernel == "table_bwd":
        # reads the edge length and dR, writes dL/dr
        return E * (2 * T + T * PC), E * PC * 2 * 2 * cfg.get("_table_degree", 8)
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
        # the fused forward: ef, Y, h and the CSR in, out (and R for the
        # backward) out; the split activations are an intermediate
        "K7K8_fused_forward": (["radial_act", "tp_fwd_fused"],
                               E * (8 * T + T * dsh + (T * PC if cfg.get("_store_R", True) else 0))
                               + N * T * C * (din + dout) + csr),
        "K9_tp_backward": (["tp_bwd_edge", "dh_gather"],
                           E * (2 * T * PC + 2 * T * dsh) + N * T * C * (2 * din + dout) + csr),
    }
    out = {}
    for name, (ks, nbytes) in groups.items():
        if not all(k in per_kernel for k in ks):
            continue
        # the step's bytes over the group's time in the step (with chunks:
        # every launch of every kernel of the group)
        sec = sum(per_kernel[k]["ms_per_step"] for k in ks) * 1e-3
        out[name] = dict(kernels=ks, algorithmic_bytes_per_step=nbytes, ms_per_step=sec * 1e3,
                         achieved_GBps=nbytes / sec / 1e9, frac=nbytes / sec / HBM_PEAK)
    return out


def roofline_for(kernel, per_launch_s, N, E, cfg, ctx, workload="medium", launches=1, chunks=None):
    """Roofline of one launch: ``per_launch_s`` its mean duration; the step's
    algorithmic bytes and flops (all E edges) are split evenly over the
    ``launches`` launches of a step (equal-edge receiver chunks)."""
    nbytes, flops = algorithmic(kernel, N, E, cfg, ctx)
    if nbytes is None:
        return None
    nbytes, flops = nbytes / launches, flops / launches
    H, PC = cfg["hidden"][0], ctx.r_width
    if kernel in ("radial_fwd", "radial_bwd_dA") and str(ctx.dtype) == "torch.float32" and H % 32 == 0 and PC % 64 == 0:
        # the float32 last-layer products run as six bf16 products (three-part
        # operand split), the hidden layers on fp32 matrix cores; at those
        # rates the matrix work takes well under the time to stream R or dR,
        # so HBM bounds these kernels
        last = E * 2 * H * PC / launches
        ach = nbytes / per_launch_s
        r = dict(bound="hbm", achieved=ach / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s",
                 frac=ach / HBM_PEAK, algorithmic_bytes_per_launch=nbytes,
                 matrix_frac=((flops - last) / MFMA_F32_PEAK + 6 * last / MFMA_BF16_PEAK) / per_launch_s)
    elif kernel == "tp_fwd_fused":
        # three bounds: the bytes it moves, the tensor product on the vector
        # ALUs, and the radial last layer on the matrix cores as six bf16
        # products (executed bf16 flops against the bf16 peak).  The largest
        # ideal time names the bound; at the medium system it is the vector
        # ALUs (the kernel runs well below all three: latency-bound).
        mat = E * 2 * H * PC / launches
        vec = flops - mat
        t_hbm, t_vec, t_mat = nbytes / HBM_PEAK, vec / VALU_F32_PEAK, 6 * mat / MFMA_BF16_PEAK
        fr = dict(hbm_frac=t_hbm / per_launch_s, vector_alu_frac=t_vec / per_launch_s,
                  matrix_frac=t_mat / per_launch_s)
        if t_mat >= max(t_hbm, t_vec):
            r = dict(bound="mfma", achieved=6 * mat / per_launch_s / 1e12, peak=MFMA_BF16_PEAK / 1e12,
                     unit="TFLOP/s", frac=fr["matrix_frac"], executed_bf16_flops_per_launch=6 * mat)
        elif t_vec >= t_hbm:
            r = dict(bound="alu", achieved=vec / per_launch_s / 1e12, peak=VALU_F32_PEAK / 1e12,
                     unit="TFLOP/s", frac=fr["vector_alu_frac"], vector_flops_per_launch=vec)
        else:
            r = dict(bound="hbm", achieved=nbytes / per_launch_s / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s",
                     frac=fr["hbm_frac"])
        r.update(fr, algorithmic_bytes_per_launch=nbytes, algorithmic_matrix_flops_per_launch=mat)
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
    # the committed counters were taken on the default configuration: the
    # separate-path layout and the default radial kernels
    other = cfg.get("sum_paths") or (cfg.get("_radial_variant") and kernel.startswith(("radial", "table")))
    t = None if other else measured_traffic(kernel, workload, chunks)
    r["traffic"] = t
    r["launches_per_step"] = launches
    return r


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(kernel, workload, chunks=None):
    """HBM bytes per launch of ``kernel`` from the committed counters of this
    workload, when they were taken on the current kernel sources and (when
    ``chunks`` is given) with the same number of receiver chunks."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if chunks is not None and t.get("_chunks") != chunks:
        return None
    rec = t.get(kernel)
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(directory):
    """(kernel name, dispatch id, counter, value) from every rocprofv3 counter
    output under ``directory``: counter_collection.csv files, or the SQLite
    databases (*_results.db, view counters_collection) that rocprofv3 writes
    by default."""
    import csv
    import glob
    import sqlite3
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                k = {key.lower(): v for key, v in r.items()}
                rows.append((k.get("kernel_name", ""), k.get("dispatch_id", ""), k.get("counter_name", ""),
                             float(k.get("counter_value", "nan"))))
    for path in glob.glob(os.path.join(directory, "**", "*_results.db"), recursive=True):
        db = sqlite3.connect(path)
        try:
            rows += [(n, str(d), c, float(v)) for n, d, c, v in db.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection")]
        finally:
            db.close()
    return rows


def _kernel_rows(directory):
    """(kernel name, duration ns) of every dispatch in the rocprofv3 kernel
    traces (SQLite databases) under ``directory``."""
    import glob
    import sqlite3
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*_results.db"), recursive=True):
        db = sqlite3.connect(path)
        try:
            rows += [(n, float(d)) for n, d in db.execute("select name, duration from kernels")]
        finally:
            db.close()
    return rows


def _short_name(name):
    import re
    m = re.match(r"(?:void )?(?:tpc::)?(?:\(anonymous namespace\)::)?(\w+)(<[^(]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name


def profile_summary(directory, counter_dirs=()):
    """Markdown tables: per-kernel dispatch count, mean and total duration of
    a rocprofv3 --kernel-trace run, and per-kernel mean counters of --pmc
    runs (one folder each)."""
    stats = {}
    for n, d in _kernel_rows(directory):
        c = stats.setdefault(_short_name(n), [0, 0.0])
        c[0] += 1
        c[1] += d
    lines = ["| kernel | dispatches | mean (ms) | total (ms) |", "|---|---|---|---|"]
    for k, (c, t) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        if t < 1e5:
            continue
        lines.append(f"| `{k}` | {c} | {t / c / 1e6:.3f} | {t / 1e6:.2f} |")
    for d in counter_dirs:
        per = {}
        for n, did, cname, v in _counter_rows(d):
            per.setdefault(_short_name(n), {}).setdefault(cname, {})[did] = v
        names = sorted({c for k in per.values() for c in k})
        lines += ["", "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        rank = lambda kv: -max(sum(x.values()) / len(x) for x in kv[1].values())
        for k, cs in sorted(per.items(), key=rank):
            vals = [sum(cs[c].values()) / len(cs[c]) if c in cs else float("nan") for c in names]
            if max(vals) < 1e6:
                continue
            lines.append(f"| `{k}` | " + " | ".join(f"{v:.4g}" for v in vals) + " |")
    print("\n".join(lines))
    return 0


def _per_dispatch(rows, counter):
    acc = {}
    for name, did, cname, v in rows:
        if cname == counter:
            key = (name, did)
            acc[key] = acc.get(key, 0.0) + v
    return acc


def traffic_from(fetch_dir, write_dir, out_path, chunks=None):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, both in KiB
    per dispatch) of ``bench.py --copy-probe`` into HBM bytes per launch of
    each kernel, each counter scaled by what it reads for a plain copy of
    COPY_PROBE_BYTES (read once, written once).  ``chunks``: the receiver
    chunks the counted runs used (per-launch bytes depend on it)."""
    out = {"_chunks": chunks}
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


def cpu_baseline(case_data, budget_s=10.0, sample_rows=None):
    """The float64 oracle's forward + per-edge backward on random batches of
    receiver rows, one single-threaded worker process per host core of this
    GPU's share (at most 16), for about ``budget_s`` seconds of wall time.
    ``sample_rows`` restricts the batches to a fixed random sample of that
    many receivers (the large system).  Runs before the GPU is touched: the
    workers are forked from this process.  The oracle works on its own
    neighbour list (built before the timing)."""
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
    rng = np.random.default_rng(0)
    pool_rows = rng.permutation(len(d["pos"]))
    if sample_rows:
        pool_rows = np.sort(pool_rows[:sample_rows])
        pool_rows = pool_rows[rng.permutation(len(pool_rows))]
    batches = [np.sort(pool_rows[k:k + 64]) for k in range(0, len(pool_rows), 64)]
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
    where = (f"a fixed random sample of {sample_rows} receivers" if sample_rows else "the same system")
    return dict(value=done_edges / wall, unit="edges/s", cores=workers, kind="oracle",
                sample=f"{done_rows} random receiver rows ({done_edges} edges) of {where} in "
                       f"batches of 64, completed in {wall:.1f} s of wall time by {workers} single-threaded "
                       f"worker processes: float64 oracle forward + per-edge backward (dR, dY, dh "
                       f"contributions, edge gradients); neighbour build not included")


WORKLOADS = {"small": 1, "medium": 3, "large": 4}
# the large system in the fewest receiver chunks whose per-edge buffers (R,
# dR and the dh contributions: 16 KB per edge) fit beside the rest in 288 GB
DEFAULT_CHUNKS = {"small": 1, "medium": 1, "large": 2}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="medium", choices=sorted(WORKLOADS))
    ap.add_argument("--chunks", type=int, default=None,
                    help="receiver chunks per step (default: 1, or 4 for the large system)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the separately timed virial and double backward")
    ap.add_argument("--sum-paths", action="store_true",
                    help="path-summed outputs (one block per output rank) on the same system")
    ap.add_argument("--radial-table", default=None, metavar="PIECES,DEGREE",
                    help="radial weights from certified piecewise Chebyshev tables (fitted before timing)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the neighbour build and conv_fwd only (no backward; with --fuse-radial no R "
                         "buffer is written)")
    ap.add_argument("--fuse-radial", action="store_true",
                    help="the forward forms R inside the tensor-product kernel (spec.fuse_radial)")
    ap.add_argument("--per-edge-radial", action="store_true",
                    help="one row of R per edge (spec.pair_radial off; by default an edge and its "
                         "reverse share one row)")
    ap.add_argument("--fp32-mfma-only", action="store_true",
                    help="float32 radial products on float32 matrix cores only (no bf16 split)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step with its convolution calls replayed from one captured HIP graph "
                         "(the neighbour build, which waits for its edge count, stays eager) even with "
                         "--no-extras; the default run reports it among the extras")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, copy %d bytes device to device three times "
                         "(counter calibration for rocprofv3 --pmc runs)" % COPY_PROBE_BYTES)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc output "
                         "folders and exit")
    ap.add_argument("--profile-summary", nargs="+", metavar="DIR",
                    help="print markdown tables of a rocprofv3 kernel trace (first folder) and the "
                         "mean counters of --pmc runs (further folders), then exit")
    a = ap.parse_args(argv)
    if a.profile_summary:
        return profile_summary(a.profile_summary[0], a.profile_summary[1:])
    if a.traffic_from:
        return traffic_from(a.traffic_from[0], a.traffic_from[1], traffic_path(a.workload),
                            a.chunks or DEFAULT_CHUNKS[a.workload])
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE={world}); "
              "the convolution is benchmarked at N=1 and no multi-GPU path is built", flush=True)
        return 2

    import numpy as np
    import torch

    import tensor_product_conv_amd as tpc
    import workloads

    k = WORKLOADS[a.workload]
    chunks = a.chunks or DEFAULT_CHUNKS[a.workload]
    d = workloads.generate(k)
    cfg = d["cfg"]
    if a.sum_paths:
        cfg = dict(cfg, sum_paths=True, name=cfg["name"] + "_summed")
        cfg["d_out"] = tpc.Context(tpc.spec_for(cfg)).d_out   # host only, no device call
        d = dict(d, cfg=cfg, G=np.random.default_rng(cfg["seed"] + 100).standard_normal(
            (cfg["N"], cfg["d_out"], cfg["C"])).astype(d["G"].dtype))
    # the CPU leg forks its workers, so it runs before anything touches the GPU
    cpu = None if a.no_cpu_baseline else cpu_baseline(
        d, a.cpu_budget, sample_rows=8192 if a.workload == "large" else None)
    dev = "cuda"
    table = tuple(int(v) for v in a.radial_table.split(",")) if a.radial_table else None
    if table:
        cfg = dict(cfg, _table_degree=table[1])
    if table or a.fp32_mfma_only or a.fuse_radial or a.per_edge_radial:
        cfg = dict(cfg, _radial_variant=True)
    if a.forward_only:
        cfg = dict(cfg, _store_R=False)   # the fused forward then writes no R
    ctx = tpc.Context(tpc.spec_for(cfg, fp32_mfma_only=a.fp32_mfma_only, table=table,
                                   fuse_radial=a.fuse_radial, pair_radial=not a.per_edge_radial))
    pos = torch.from_numpy(d["pos"]).to(dev)
    species = torch.from_numpy(d["species"]).to(dev)
    h = torch.from_numpy(d["h"]).to(dev)
    W = [torch.from_numpy(w).to(dev) for w in d["W"]]
    table_info = None
    if table:
        torch.cuda.synchronize()
        t_fit = time.perf_counter()
        tab, cert = ctx.radial_table_fit(W)
        torch.cuda.synchronize()
        table_info = {"pieces": table[0], "degree": table[1], "certificate": list(cert),
                      "fit_s": time.perf_counter() - t_fit, "table_bytes": ctx.sizes["table_bytes"]}
        W = [tab]
    G = torch.from_numpy(d["G"]).to(dev)
    cell = d["cell"]
    N = cfg["N"]

    nl = ctx.nbr_build(pos, cell, species)
    E = nl.n_edges
    scale = float(N) / E if cfg["scale"] == "inv_avg_neighbors" else 1.0
    rp = nl.row_ptr.cpu().numpy()
    # receiver chunks with about equal edge counts
    cuts = [0] + [int(np.searchsorted(rp, E * q // chunks)) for q in range(1, chunks)] + [N]
    bounds = [(r0, r1, int(rp[r0]), int(rp[r1])) for r0, r1 in zip(cuts[:-1], cuts[1:]) if r1 > r0]
    max_e = max(e1 - e0 for _, _, e0, e1 in bounds)
    if ctx.pair_radial:
        # rows of R the network writes: one per pair inside a chunk, one per
        # edge whose reverse lies in another chunk (the library's own count
        # is checked against this after the timed steps)
        rev = nl.rev.cpu().numpy().astype(np.int64)
        owners = 0
        for _, _, e0, e1 in bounds:
            idx = np.arange(e1 - e0)
            r = rev[e0:e1] - e0
            owners += int(((r < 0) | (r >= e1 - e0) | (idx < r)).sum())
        cfg = dict(cfg, _R_rows=owners)
    out = torch.empty((N, ctx.d_out, cfg["C"]), dtype=ctx.dtype, device=dev)
    # a forward-only run of a fused context stores no R
    eb = ctx.alloc_edge_buffers(max_e, dev, with_R=not a.forward_only)
    dh = torch.empty_like(h)
    dh_edge = torch.empty((max_e, ctx.d_in, cfg["C"]), dtype=ctx.dtype, device=dev)
    dR = torch.empty((max_e, ctx.r_width), dtype=ctx.dtype, device=dev)
    g_edge = torch.empty((E, 3), dtype=ctx.dtype, device=dev)
    forces = torch.empty((N, 3), dtype=ctx.dtype, device=dev)
    ws_n = ctx._workspace(ctx.workspace_bytes(tpc.OP_NBR, N, 0, cell), dev)
    ws_f = ctx._workspace(ctx.workspace_bytes(tpc.OP_FWD, N, max_e), dev)
    ws_b = ctx._workspace(ctx.workspace_bytes(tpc.OP_BWD, N, max_e), dev)

    def step_nbr():
        return ctx.nbr_build(pos, cell, species, edge_cap=E, into=nl, workspace=ws_n)

    def step_conv(nl2):
        for q, (r0, r1, e0, e1) in enumerate(bounds):
            ctx.conv_fwd(pos, cell, nl2, h, W, scale, out=out, eb=eb, rows=(r0, r1), edges=(e0, e1),
                         workspace=ws_f)
            if a.forward_only:
                continue
            last = q == len(bounds) - 1
            ctx.conv_bwd(nl2, h, W, scale, G, eb, dh=dh, dR=dR, g_edge=g_edge, dh_edge=dh_edge,
                         forces=forces if last else None, want_forces=last, workspace=ws_b)

    def step():
        step_conv(step_nbr())

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
    if ctx.pair_radial:
        e0, e1 = bounds[-1][2], bounds[-1][3]
        got = int(eb.Rrow[e1 - e0].item())
        idx = np.arange(e1 - e0)
        r = rev[e0:e1] - e0
        assert got == int(((r < 0) | (r >= e1 - e0) | (idx < r)).sum()), "shared R row count"

    extras = {}
    if not a.no_extras and not a.forward_only:
        # the virial (strain derivative) from the step's edge gradients, timed
        # on its own: it is not part of the step
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
        extras["virial_ms"] = vt["virial"][0] / vt["virial"][1] if "virial" in vt else None
        del ws_v
        if chunks == 1 and not cfg.get("sum_paths") and not table:
            extras["double_backward"] = time_double_backward(tpc, ctx, nl, h, G, eb, scale, N, E, cfg, a.steps)

    if a.graph or not a.no_extras:
        try:
            extras["graph_replay"] = time_graph_replay(torch, step_nbr, step_conv, a.steps, E)
        except RuntimeError as exc:   # reported, not fatal: the eager step above is the measurement
            torch.cuda.synchronize()
            extras["graph_replay"] = {"error": str(exc)[:200]}

    # one launch of each per pass (the weight packing runs once in each pass)
    fwd_ms = sum(per_kernel.get(n, {}).get("ms_per_step", 0.0)
                 for n in ("geom_fwd", "pair_rows", "radial_fwd", "radial_act", "table_fwd", "tp_fwd",
                           "tp_fwd_fused")) + \
        per_kernel.get("radial_pack", {}).get("ms_per_step", 0.0) / 2
    bwd_ms = sum(per_kernel.get(n, {}).get("ms_per_step", 0.0)
                 for n in ("tp_bwd_edge", "radial_bwd_dA", "radial_bwd_mlp", "table_bwd", "geom_bwd", "dh_gather",
                           "forces")) + \
        per_kernel.get("radial_pack", {}).get("ms_per_step", 0.0) / 2
    nbr_ms = sum(v["ms_per_step"] for n, v in per_kernel.items() if n.startswith("nbr"))
    dominant = max((n for n in per_kernel if n in KERNEL_SOURCES), key=lambda n: per_kernel[n]["ms_per_step"])
    # algorithmic bytes of a step over the kernel's time in the step: with
    # equal-edge chunks this is the per-launch ratio of every chunk
    roof = roofline_for(dominant, per_kernel[dominant]["avg_ms"] * 1e-3, N, E, cfg, ctx, a.workload,
                        per_kernel[dominant]["launches_per_step"], chunks)
    kernels = {}
    for n, v in per_kernel.items():
        r = (roofline_for(n, v["avg_ms"] * 1e-3, N, E, cfg, ctx, a.workload, v["launches_per_step"], chunks)
             if n in KERNEL_SOURCES else None)
        kernels[n] = dict(avg_ms=round(v["avg_ms"], 4), launches_per_step=v["launches_per_step"],
                          **({"bound": r["bound"], "frac": round(r["frac"], 4)} if r else {}))

    if a.copy_probe:
        src_t = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    geom = {1: "simple cubic", 3: "water", 4: "fcc with vacancies"}[k]
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
        "config": {"workload": f"{cfg['name']} ({geom}) N={N} E={E} C={cfg['C']} node_lmax={cfg['l1max']} "
                               f"sh_lmax={cfg['sh_lmax']} out_lmax={cfg['out_lmax']} "
                               f"mlp={'-'.join(map(str, cfg['layer_dims']))}: "
                               + ("nbr_build + conv_fwd (forward only)" if a.forward_only
                                  else "nbr_build + conv_fwd + conv_bwd (forces)")
                               + (f" in {len(bounds)} receiver chunks" if len(bounds) > 1 else "")
                               + (", path-summed outputs" if cfg.get("sum_paths") else "")
                               + (f", radial tables {table[0]}x{table[1]}" if table else "")
                               + (", float32 radial products on fp32 matrix cores" if a.fp32_mfma_only else "")
                               + (", radial last layer fused into the forward tensor product"
                                  if ctx.fused_radial else "")
                               + (f", R rows shared by edge pairs ({cfg['_R_rows']} rows)"
                                  if ctx.pair_radial else ""),
                   "n_atoms": N, "n_edges": E, "channels": cfg["C"], "paths": ctx.n_paths,
                   "chunks": len(bounds), "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "fwd_edges_per_s": E / (fwd_ms * 1e-3) if fwd_ms else None,
        "fwd_bwd_edges_per_s": E / ((fwd_ms + bwd_ms) * 1e-3) if fwd_ms else None,
        "nbr_build_ms": nbr_ms,
        **extras,
        **({"radial_table": table_info} if table_info else {}),
        "kernels": kernels,
        "tp_groups_hbm": group_rooflines(per_kernel, N, E, cfg, ctx),
        "wall_s": wall,
    }
    print(json.dumps(line), flush=True)
    return 0


def time_graph_replay(torch, step_nbr, step_conv, steps, E):
    """The step with its convolution calls captured once in a HIP graph and
    replayed: the same kernels on the same buffers, launched by one graph
    launch instead of one host call each.  The neighbour build stays eager
    (it waits for its edge count)."""
    nl = step_nbr()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_conv(nl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_conv(nl)
    for _ in range(2):
        step_nbr()
        g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step_nbr()
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    del g
    return {"ms_per_step": ms, "edges_per_s": E / (ms * 1e-3)}


def time_double_backward(tpc, ctx, nl, h, G, eb, scale, N, E, cfg, steps):
    """The VJP-of-VJP on the step's per-edge buffers with seeded N(0,1)
    cotangents, timed on its own (not part of the step): per-launch times of
    its kernels and edges/s."""
    import numpy as np
    import torch
    dev = h.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    u_dh = torch.randn(h.shape, dtype=ctx.dtype, device=dev, generator=gen)
    u_dY = torch.randn((E, ctx.d_sh), dtype=ctx.dtype, device=dev, generator=gen)
    u_dR = torch.randn((E, ctx.r_width), dtype=ctx.dtype, device=dev, generator=gen)
    g_hat, h_hat = torch.empty_like(G), torch.empty_like(h)
    Y_hat = torch.empty((E, ctx.d_sh), dtype=ctx.dtype, device=dev)
    R_hat = torch.empty((E, ctx.r_width), dtype=ctx.dtype, device=dev)
    ws = ctx._workspace(ctx.workspace_bytes(tpc.OP_DOUBLE_BWD, N, E), dev)

    def call():
        ctx.conv_double_bwd(nl, h, scale, G, eb, u_dh, u_dY, u_dR, g_hat=g_hat, h_hat=h_hat, Y_hat=Y_hat,
                            R_hat=R_hat, workspace=ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    tpc.timing_collect()
    tpc.timing_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    tpc.timing_enable(False)
    kt = tpc.timing_collect()
    ms = {n: tot / cnt for n, (tot, cnt) in kt.items()}
    total = sum(ms.values())
    T, C, PC, din, dsh, dout = 4, cfg["C"], ctx.r_width, ctx.d_in, ctx.d_sh, ctx.d_out
    # algorithmic bytes: R, u_dR and their reverse-edge rows are read once
    # (the gather touches each edge's u_dR once more, at its reverse), R_hat
    # written; Y, u_dY (twice), Y_hat; h, u_dh, G read once per atom, g_hat and
    # h_hat written once per atom; CSR and reverse index
    nbytes = (E * T * (3 * PC + PC) + E * T * (3 * dsh + dsh) + N * T * C * (2 * din + dout)
              + N * T * C * (dout + din) + 4 * (N + 1) + 8 * E)
    return dict(ms=total, kernels_ms={n: round(v, 4) for n, v in ms.items()}, edges_per_s=E / (total * 1e-3),
                algorithmic_bytes=nbytes, hbm_frac=nbytes / (total * 1e-3) / HBM_PEAK)


if __name__ == "__main__":
    sys.exit(main())
