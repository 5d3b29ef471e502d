"""The profile summaries: per-kernel counter averages, outer/inner mean tagging, calibration."""
import csv
import os

from graph_mini_pipeline_amd import rocprof_summary as rs


def _counter_csv(path, counter, rows):
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, grid, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Grid_Size": grid, "Kernel_Name": f"gnnmb::{name}(args)",
                        "Counter_Name": counter, "Counter_Value": val})


def test_counter_summary_tags_outer_mean_and_scales(tmp_path):
    seq = [("k_sample", 100, 10.0), ("k_gather_batch<64, 3, 8>", 200, 1000.0),
           ("k_mean_v5<64, 3, 4>", 300, 500.0), ("k_mean_v5<64, 3, 4>", 400, 50.0),
           ("k_copy_probe", 500, 524288.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", seq)
    _counter_csv(w, "WRITE_SIZE", [(n, g, 2 * v) for n, g, v in seq])
    text = rs.counter_summary("t", str(f), str(w), "cmd")
    out = tmp_path / "c.txt"
    out.write_text(text)
    outer = rs.read_traffic(str(out), "k_mean_v5<64, 3, 4>@outer")
    inner = rs.read_traffic(str(out), "k_mean_v5<64, 3, 4>@inner")
    # calibration: the 1 GiB copy reads as 512 MiB fetched, 1 GiB written -> fetch x2, write x1
    assert outer["fetch_scale"] == 2.0 and outer["write_scale"] == 1.0
    assert outer["fetch_bytes"] == 500.0 * 1024 * 2 and outer["write_bytes"] == 1000.0 * 1024
    assert inner["fetch_bytes"] == 50.0 * 1024 * 2
    g = rs.read_traffic(str(out), "k_gather_batch<64, 3, 8>")
    assert g["bytes"] == 1000.0 * 1024 * 2 + 2000.0 * 1024


def test_read_traffic_stale_source_is_none(tmp_path):
    out = tmp_path / "c.txt"
    out.write_text("counters k_sample dispatches=1 fetch_kib=1.0 write_kib=1.0 source=csrc/sample.hip "
                   "sha256=0000000000000000\ncalibration copy_bytes=1073741824 fetch_kib=1.0 write_kib=1.0\n")
    assert rs.read_traffic(str(out), "k_sample") is None
    assert rs.read_traffic(str(tmp_path / "missing.txt"), "k_sample") is None


def test_copy_after_mean_is_tagged(tmp_path):
    seq = [("k_gather_batch<64, 3, 8>", 200, 1000.0), ("k_mean_v5<64, 3, 4>", 300, 500.0),
           ("k_gather_batch<64, 3, 8>", 100, 30.0), ("k_mean_v5<64, 3, 4>", 400, 50.0),
           ("k_copy_probe", 500, 524288.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", seq)
    _counter_csv(w, "WRITE_SIZE", seq)
    out = tmp_path / "c.txt"
    out.write_text(rs.counter_summary("t", str(f), str(w), "cmd"))
    assert rs.read_traffic(str(out), "k_gather_batch<64, 3, 8>")["fetch_bytes"] == 1000.0 * 1024 * 2
    assert rs.read_traffic(str(out), "k_gather_batch<64, 3, 8>@copy")["fetch_bytes"] == 30.0 * 1024 * 2
    # the mean after the copy is an inner block
    assert rs.read_traffic(str(out), "k_mean_v5<64, 3, 4>@inner")["fetch_bytes"] == 50.0 * 1024 * 2


def test_interleaved_gathers_are_not_copies(tmp_path):
    seq = [("k_gather_rows<32, 1, 4>", 200, 100.0), ("k_mean_v5<32, 1, 4>", 300, 50.0),
           ("k_gather_rows<32, 1, 4>", 200, 100.0), ("k_mean_v5<32, 1, 4>", 300, 50.0),
           ("k_mean_v5<32, 1, 4>", 400, 5.0), ("k_copy_probe", 500, 524288.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", seq)
    _counter_csv(w, "WRITE_SIZE", seq)
    out = tmp_path / "c.txt"
    out.write_text(rs.counter_summary("t", str(f), str(w), "cmd"))
    assert rs.read_traffic(str(out), "k_gather_rows<32, 1, 4>@copy") is None
    assert rs.read_traffic(str(out), "k_mean_v5<32, 1, 4>@outer")["fetch_bytes"] == 50.0 * 1024 * 2
    assert rs.read_traffic(str(out), "k_mean_v5<32, 1, 4>@inner")["fetch_bytes"] == 5.0 * 1024 * 2


def test_short_name_strips_namespaces_and_arguments():
    assert rs.short_name("void gnnmb::(anonymous namespace)::k_sage_update("
                         "gnnmb::(anonymous namespace)::SageArgs)") == "k_sage_update"
    assert rs.short_name("void gnnmb::k_mean_v5<64, 3, 4>(gnnmb::MeanArgs)") == "k_mean_v5<64, 3, 4>"
    assert rs.source_of("k_sage_update") == "csrc/sage.hip"


def test_metrics_summary_averages_per_kernel(tmp_path):
    p = tmp_path / "m.csv"
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (k, c, v) in enumerate([("k_sample", "VALUBusy", 60.0), ("k_sample", "VALUBusy", 70.0),
                                       ("k_sample", "MfmaUtil", 0.0), ("k_sage_update", "MfmaUtil", 40.0)]):
            w.writerow({"Dispatch_Id": i, "Grid_Size": 1, "Kernel_Name": f"void gnnmb::{k}(a)",
                        "Counter_Name": c, "Counter_Value": v})
    text = rs.metrics_summary(str(p), "cmd")
    lines = {l.split()[0]: l.split() for l in text.splitlines() if not l.startswith("#")}
    assert lines["k_sample"][1] == "2" and float(lines["k_sample"][3]) == 65.0   # VALUBusy column
    assert float(lines["k_sage_update"][2]) == 40.0                             # MfmaUtil column
    assert lines["k_sage_update"][3] == "-"


def test_source_of_template_instances():
    """Kernel instances (template arguments, the outer/inner tag) map to the file of their
    kernel, and a name that no library file defines maps to nothing."""
    assert rs.source_of("k_sample<8, false, true>") == "csrc/sample.hip"
    assert rs.source_of("k_sample<4, true, false>") == "csrc/sample.hip"
    assert rs.source_of("k_mean_v5<32, 1, 4>@outer") == "csrc/aggregate.hip"
    assert rs.source_of("k_gather_rows<64, 3, 8, true>") == "csrc/gather.hip"
    assert rs.source_of("Cijk_Ailk_Bljk_SB_MT64x64") is None
