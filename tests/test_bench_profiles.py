"""CPU checks of bench.py's profile summaries: rocprofv3-style CSVs in, the
text tables under profiles/ out, and the rows bench.py reads back from them
(HBM bytes scaled by the plain-copy calibration, SQ-counter derived columns,
source digests that mark a table stale)."""
import csv
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)


def _pmc_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kern, grid, cname, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kern, "Grid_Size": grid, "Counter_Name": cname,
                        "Counter_Value": val})


COMP = "void gear::(anonymous namespace)::compress_kernel<128, 4, 16>(gear::CompressArgs)"
SEL = "void gear::(anonymous namespace)::select_kernel<128, 2, 1024>(gear::CompressArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_hbm_table_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    f, w = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    # the copy reads half its bytes in FETCH_SIZE, all of them in WRITE_SIZE
    _pmc_csv(f, [(COMP, 512, "FETCH_SIZE", 1000.0), (COMP, 512, "FETCH_SIZE", 3000.0),
                 (SEL, 512, "FETCH_SIZE", 500.0), (COPY, bench.COPY_GRID, "FETCH_SIZE", 131072.0),
                 (COPY, "999", "FETCH_SIZE", 7.0)])
    _pmc_csv(w, [(COMP, 512, "WRITE_SIZE", 100.0), (SEL, 512, "WRITE_SIZE", 0.0),
                 (COPY, bench.COPY_GRID, "WRITE_SIZE", 262144.0)])
    text = bench.hbm_table(f, w, "# header\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "gear_kernels_wl_hbm_bytes.txt").write_text(text)
    row = bench.read_profile_row("hbm_bytes", "wl", "compress")
    assert row["read_B"] == pytest.approx(2000.0 * 1024 / 0.5)      # mean 2000 KiB / factor 0.5
    assert row["write_B"] == pytest.approx(100.0 * 1024)
    assert row["total_B"] == pytest.approx(row["read_B"] + row["write_B"])
    assert bench.read_profile_row("hbm_bytes", "wl", "select")["total_B"] == pytest.approx(1024000.0)
    assert bench.read_profile_row("hbm_bytes", "wl", "decompress") is None
    # a table taken from other sources is stale: its rows are not used
    stale = text.replace(bench.source_digest("compress"), "0123456789abcdef")
    (tmp_path / "gear_kernels_wl_hbm_bytes.txt").write_text(stale)
    assert bench.read_profile_row("hbm_bytes", "wl", "compress") is None


def test_sq_table_derived_columns_and_bound(tmp_path, monkeypatch):
    p1, p2 = str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")
    gui = 1.0e6            # summed over the 8 XCDs: 125,000 cycles per SIMD
    valu = 0.5 * 1024 * gui / 8 / 4      # half of the SIMD-cycles issuing VALU
    r1 = [(COMP, 512, c, 0.0) for c in bench.SQ_PASSES[0]
          if c not in ("SQ_INSTS_VALU", "GRBM_GUI_ACTIVE", "SQ_INSTS_LDS")]
    _pmc_csv(p1, r1 + [(COMP, 512, "SQ_INSTS_VALU", valu), (COMP, 512, "GRBM_GUI_ACTIVE", gui),
                       (COMP, 512, "SQ_INSTS_LDS", 100.0)])
    r2 = [(COMP, 512, c, 0.0) for c in bench.SQ_PASSES[1]
          if c not in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_BANK_CONFLICT")]
    _pmc_csv(p2, r2 + [(COMP, 512, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * gui / 8),
                       (COMP, 512, "SQ_VALU_MFMA_COEXEC_CYCLES", 0.1 * 1024 * gui / 8),
                       (COMP, 512, "SQ_LDS_BANK_CONFLICT", 300.0)])
    entries = {"compress": 1_000_000}
    text = bench.sq_table(p1, p2, entries, "# header\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "gear_kernels_wl_sq_counters.txt").write_text(text)
    row = bench.read_profile_row("sq_counters", "wl", "compress")
    assert row["valu%"] == pytest.approx(50.0, abs=0.05)
    assert row["mfma%"] == pytest.approx(25.0, abs=0.05)
    assert row["coexec%"] == pytest.approx(40.0, abs=0.05)
    assert row["lane_ops/entry"] == pytest.approx(valu * 64 / 1e6, rel=1e-3)
    assert row["lds_confl/inst"] == pytest.approx(3.0)
    # no HBM table: the counters alone decide (VALU issue)
    got = bench._bound_from_counters("compress", "wl", 0.1, 1e8)
    assert got["bound"] == "alu" and got["hbm_busy_frac"] is None
    assert got["lane_ops_per_launch"] == pytest.approx(valu * 64, rel=1e-3)


def test_kernel_stats_table_last_launches(tmp_path):
    path = str(tmp_path / "kt.csv")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for dur in [50_000] * 5 + [10_000] * 3:       # warm-up launches, then the last 3
            w.writerow({"Kernel_Name": COMP, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 1000
    text = bench.kernel_stats_table(path, 3, {"kernels_ms": {"compress": 0.0101}, "value": 1.0,
                                              "ms_per_step": 1.0,
                                              "roofline": {"kernel": "compress_kernel", "launch_ms": 0.0101}},
                                    "# header\n")
    line = [l for l in text.splitlines() if l.startswith("compress_kernel<128,4,16>")][0].split()
    assert line[1] == "8" and float(line[5]) == pytest.approx(10.0) and float(line[6]) == pytest.approx(10.1)


def test_kernel_names_match_whole_symbols():
    assert bench._kernel_key("void gear::(anonymous namespace)::decompress_kernel<128, 4>(x)") == "decompress"
    assert bench._kernel_key("void gear::(anonymous namespace)::decompress_mm_kernel<128, 4, 0, 4>(x)") == "decompress"
    assert bench._kernel_key(COMP) == "compress"
    assert bench._kernel_key("void at::native::elementwise_kernel<4>(x)") is None


def test_sweep_table_from_a_sweep_line(tmp_path):
    line = {"metric": "m", "model": "x", "data": "s", "wall_s": 1.0, "configs": {
        "fp16": {"cache_bytes_per_sequence": 2e9, "max_batch": 100, "peak_tok_s": 10.0,
                 "throughput_vs_fp16": 1.0, "max_batch_vs_fp16": 1.0, "peak_memory_vs_fp16_at_batch_64": 1.0,
                 "runs": [{"batch": 64, "tok_s": 10.0, "peak_GB": 128.0}]},
        "gear_4bit": {"cache_bytes_per_sequence": 1e9, "max_batch": 200, "peak_tok_s": 25.0,
                      "throughput_vs_fp16": 2.5, "max_batch_vs_fp16": 2.0, "peak_memory_vs_fp16_at_batch_64": 2.0,
                      "runs": [{"batch": 64, "tok_s": 25.0, "peak_GB": 64.0}, {"batch": 300, "oom": True}]}}}
    import json
    p = tmp_path / "s.json"
    p.write_text("[sweep] progress\n" + json.dumps(line) + "\n")
    t = bench.sweep_table(str(p))
    row = [l for l in t.splitlines() if l.startswith("gear_4bit ")][0].split()
    assert row[1] == "1000.0" and row[2] == "200" and float(row[4]) == 2.5
    assert "(300, oom, -)" in t


@pytest.mark.parametrize("workload", ["7b_layer", "2bit", "long_ctx", "stream_gqa"])
def test_committed_profiles_match_the_current_kernel_sources(workload):
    """The benchmark line's roofline and compress-phase objects take measured
    bytes and counters from the committed profiles only while their source
    digests match the kernels as they are now: after a kernel change the
    profiles must be made again (bench.py --make-profiles)."""
    for kind in ("hbm_bytes", "sq_counters"):
        for kernel in ("select", "compress", "lowrank_a", "decompress"):
            row = bench.read_profile_row(kind, workload, kernel)
            assert row is not None, (f"profiles/gear_kernels_{workload}_{kind}.txt has no {kernel} row "
                                     f"for the current sources ({bench.source_digest(kernel)})")
