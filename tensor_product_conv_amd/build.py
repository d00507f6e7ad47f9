"""Build libtpconv.so (gfx950) in-tree with hipcc.

    python -m tensor_product_conv_amd.build [--incremental] [--jobs N]

Each source compiles to an object under _build/ (in parallel), then the
objects link into tensor_product_conv_amd/libtpconv.so.  The tensor-product
kernel sources compile once per built configuration (-DTPC_CFG=<index>, see
csrc/tp_config.hpp), so the heavy instantiations build side by side.  The
neighbour build is compiled without floating-point contraction so its
float64 edge test is bitwise reproducible; every file is compiled without
packed-FP32 instructions.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtpconv.so")

PLAIN_SOURCES = ["api.cpp", "nbr.hip", "scan.hip", "geom.hip", "radial.hip", "tp_dispatch.hip",
                 "forces.hip", "noalloc.hip", "radial_table.hip", "pair.hip"]
PER_CONFIG_SOURCES = ["tp_fwd.hip", "tp_bwd.hip", "tp_dbl.hip", "tp_fused.hip"]
HEADERS = ["common.hpp", "kernels.hpp", "nbr.hpp", "tables.hpp", "tp_impl.hpp", "tp_config.hpp", "tp_fused.hpp"]


def n_configs():
    with open(os.path.join(CSRC, "tp_config.hpp")) as f:
        for line in f:
            if line.startswith("#define TPC_TP_N_CONFIGS"):
                return int(line.split()[2])
    raise RuntimeError("TPC_TP_N_CONFIGS not found in tp_config.hpp")


def units(only=None):
    """(source, extra flags, object name) for every object of the library;
    ``only`` restricts the per-configuration sources to those indices."""
    out = [(src, [], src + ".o") for src in PLAIN_SOURCES]
    for src in PER_CONFIG_SOURCES:
        for k in range(n_configs()):
            if only is None or k in only:
                out.append((src, [f"-DTPC_CFG={k}"], f"{src}.{k}.o"))
    return out

ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-fconstexpr-steps=200000000",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]
PER_FILE = {"nbr.hip": ["-ffp-contract=off"]}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtpconv.so)")


def _compile(unit, incremental):
    src, extra, name = unit
    obj = os.path.join(BUILD, name)
    path = os.path.join(CSRC, src)
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in [src] + HEADERS)
        newest = max(newest, os.path.getmtime(os.path.join(ROOT, "include", "tpconv.h")))
        if os.path.getmtime(obj) >= newest:
            return obj, None
    cmd = [hipcc()] + COMMON + PER_FILE.get(src, []) + extra + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        return obj, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return obj, None


def build(incremental=False, jobs=None, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    us = units()
    # the slowest objects first, so they do not start last
    us.sort(key=lambda u: (u[0] not in PER_CONFIG_SOURCES, u[2]))
    jobs = jobs or min(len(us), max(1, (os.cpu_count() or 4)))
    objs, errs = [], []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, err in ex.map(lambda u: _compile(u, incremental), us):
            objs.append(obj)
            if err:
                errs.append(err)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    build(incremental=a.incremental, jobs=a.jobs)


if __name__ == "__main__":
    sys.exit(main())
