"""Host logic of bench.py: the roofline accounting (per launch, with receiver
chunks), the HBM-traffic calibration from rocprofv3 counter databases, and
the profile summary.  No GPU: the contexts are host objects and the counter
databases are small synthetic ones in rocprofv3's SQLite layout."""
import json
import os
import sqlite3

import pytest

import bench
import tensor_product_conv_amd as tpc
import workloads


@pytest.fixture(scope="module")
def medium():
    c = workloads.config(3)
    return c, tpc.Context(tpc.spec_for(c))


def test_roofline_splits_a_step_over_its_launches(medium):
    cfg, ctx = medium
    N, E = 32768, 2_934_240
    nbytes, _ = bench.algorithmic("tp_bwd_edge", N, E, cfg, ctx)
    one = bench.roofline_for("tp_bwd_edge", 10e-3, N, E, cfg, ctx, launches=1)
    four = bench.roofline_for("tp_bwd_edge", 2.5e-3, N, E, cfg, ctx, launches=4)
    # a quarter of the bytes in a quarter of the time: the same rate
    assert one["algorithmic_bytes_per_launch"] == nbytes
    assert four["algorithmic_bytes_per_launch"] == pytest.approx(nbytes / 4)
    assert four["frac"] == pytest.approx(one["frac"])
    assert one["frac"] == pytest.approx(nbytes / 10e-3 / bench.HBM_PEAK)
    assert four["launches_per_step"] == 4


def test_group_rooflines_use_the_time_in_the_step(medium):
    cfg, ctx = medium
    N, E = 32768, 2_934_240
    per = {"tp_fwd": dict(avg_ms=1.0, ms_per_step=4.0, launches_per_step=4),
           "tp_bwd_edge": dict(avg_ms=2.0, ms_per_step=8.0, launches_per_step=4),
           "dh_gather": dict(avg_ms=2.0, ms_per_step=2.0, launches_per_step=1)}
    g = bench.group_rooflines(per, N, E, cfg, ctx)
    assert g["K8_tp_forward"]["ms_per_step"] == pytest.approx(4.0)
    assert g["K9_tp_backward"]["ms_per_step"] == pytest.approx(10.0)
    k8 = g["K8_tp_forward"]
    assert k8["frac"] == pytest.approx(k8["algorithmic_bytes_per_step"] / 4e-3 / bench.HBM_PEAK)
    assert "K7K8_fused_forward" not in g


def _counter_db(directory, rows):
    """A rocprofv3-style results database with a counters_collection view's
    columns (as a table): (kernel_name, dispatch_id, counter_name, value)."""
    os.makedirs(directory, exist_ok=True)
    db = sqlite3.connect(os.path.join(directory, "run_results.db"))
    db.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
               "counter_name text, value real)")
    db.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    db.commit()
    db.close()


def test_traffic_calibration_from_counter_databases(tmp_path, monkeypatch):
    gib_kib = (1 << 30) / 1024
    fetch = [("__amd_rocclr_copyBuffer", d, "FETCH_SIZE", gib_kib / 2) for d in (1, 2, 3)] + [
        ("void tpc::k_tp_fwd<float, 2, 3, 3, false, 1, 1, false, 2>(int)", 7, "FETCH_SIZE", 1000.0),
        ("void tpc::k_tp_fwd<float, 2, 3, 3, false, 1, 1, false, 2>(int)", 9, "FETCH_SIZE", 3000.0)]
    write = [("__amd_rocclr_copyBuffer", d, "WRITE_SIZE", gib_kib) for d in (1, 2, 3)] + [
        ("void tpc::k_tp_fwd<float, 2, 3, 3, false, 1, 1, false, 2>(int)", 7, "WRITE_SIZE", 100.0),
        ("void tpc::k_tp_fwd<float, 2, 3, 3, false, 1, 1, false, 2>(int)", 9, "WRITE_SIZE", 300.0)]
    _counter_db(tmp_path / "f", fetch)
    _counter_db(tmp_path / "w", write)
    out = tmp_path / "traffic.json"
    assert bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), str(out)) == 0
    t = json.loads(out.read_text())
    # the copy reads half its bytes in the fetch counter: reads scale by 2
    assert t["_fetch_calibration"]["factor"] == pytest.approx(2.0)
    assert t["_write_calibration"]["factor"] == pytest.approx(1.0)
    rec = t["tp_fwd"]
    assert rec["read_bytes"] == pytest.approx(2000.0 * 1024 * 2)     # mean of 1000 and 3000 KiB, x2
    assert rec["write_bytes"] == pytest.approx(200.0 * 1024)
    assert rec["dispatches"] == 2
    assert rec["source_hash"] == bench.source_hash("tp_fwd")
    # the committed counters apply only while the kernel sources are unchanged
    monkeypatch.setattr(bench, "traffic_path", lambda w: str(out))
    assert bench.measured_traffic("tp_fwd", "medium") == pytest.approx(rec["hbm_bytes_per_launch"])
    # counters taken in other receiver chunks do not apply either
    assert bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), str(out), chunks=2) == 0
    assert bench.measured_traffic("tp_fwd", "medium", chunks=2) == pytest.approx(rec["hbm_bytes_per_launch"])
    assert bench.measured_traffic("tp_fwd", "medium", chunks=4) is None
    monkeypatch.setattr(bench, "source_hash", lambda k: "changed")
    assert bench.measured_traffic("tp_fwd", "medium") is None


def test_profile_summary_reads_kernel_traces(tmp_path, capsys):
    d = tmp_path / "trace"
    d.mkdir()
    db = sqlite3.connect(str(d / "x_results.db"))
    db.execute("create table kernels (name text, duration real)")
    db.executemany("insert into kernels values (?, ?)",
                   [("void tpc::k_tp_fwd<float, 2>(int)", 5.5e6), ("void tpc::k_tp_fwd<float, 2>(int)", 5.7e6),
                    ("k_bin", 1e4)])
    db.commit()
    db.close()
    assert bench.profile_summary(str(d)) == 0
    text = capsys.readouterr().out
    assert "| `k_tp_fwd<float, 2>` | 2 | 5.600 | 11.20 |" in text
    assert "k_bin" not in text          # under 0.1 ms in total


def test_fused_forward_roofline_names_its_largest_bound():
    c = workloads.config(3)
    ctx = tpc.Context(tpc.spec_for(c, fuse_radial=True))
    N, E = 32768, 2_934_240
    H, PC = c["hidden"][0], ctx.r_width
    fwd_only = dict(c, _store_R=False)
    r = bench.roofline_for("tp_fwd_fused", 6e-3, N, E, fwd_only, ctx)
    # without R stores the vector ALUs take longest at their peak: the bound is
    # "alu", measured on the vector flops alone (the matrix flops of the radial
    # last layer are not counted against the vector peak)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    nbytes, flops = bench.algorithmic("tp_fwd_fused", N, E, fwd_only, ctx)
    vec = flops - E * 2 * H * PC
    assert r["frac"] == pytest.approx(vec / 6e-3 / bench.VALU_F32_PEAK)
    assert r["matrix_frac"] == pytest.approx(6 * E * 2 * H * PC / bench.MFMA_BF16_PEAK / 6e-3)
    assert r["hbm_frac"] == pytest.approx(nbytes / bench.HBM_PEAK / 6e-3)
    # storing R for the backward adds 8.7 KB per edge: HBM becomes the bound
    r2 = bench.roofline_for("tp_fwd_fused", 15e-3, N, E, dict(c, _store_R=True), ctx)
    assert r2["bound"] == "hbm" and r2["unit"] == "GB/s"
    assert max(r2["hbm_frac"], r2["vector_alu_frac"], r2["matrix_frac"]) == r2["frac"]


def test_more_than_one_gpu_is_refused_before_any_work(capsys, monkeypatch):
    # one GPU only: --gpus above 1 (or a launcher's WORLD_SIZE) ends at once
    # with a message and a non-zero status, before torch or the library load
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().out
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2
    assert "WORLD_SIZE=4" in capsys.readouterr().out


def test_radial_forward_counts_one_row_per_written_row(medium):
    """With rows shared by edge pairs the radial network writes one row per
    pair: its algorithmic bytes and flops follow the row count, and the
    tensor products' reads of R (one row per edge) do not change."""
    cfg, ctx = medium
    N, E = 32768, 2_934_240
    per_edge = bench.algorithmic("radial_fwd", N, E, cfg, ctx)
    shared = bench.algorithmic("radial_fwd", N, E, dict(cfg, _R_rows=E // 2), ctx)
    assert shared[0] * 2 == per_edge[0] and shared[1] * 2 == per_edge[1]
    assert per_edge[0] == E * 4 * (8 + ctx.r_width)
    for k in ("tp_fwd", "tp_bwd_edge"):
        assert bench.algorithmic(k, N, E, dict(cfg, _R_rows=E // 2), ctx) == bench.algorithmic(k, N, E, cfg, ctx)
