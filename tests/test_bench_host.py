"""bench.py's host logic on the CPU: counter ingestion, the source-hash rule for the
traffic figures, and the one-GPU guard. No GPU is touched."""
import csv
import json
import subprocess
import sys

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


COPY = "__amd_rocclr_copyBuffer"
MASS = "void sv::k_sample_mass<sv::bf16_t, true, false>(sv::SampleParams)"
MASS_F = "void sv::k_sample_mass<sv::bf16_t, true, true>(sv::SampleParams)"
DRAW = "void sv::k_sample_draw<sv::bf16_t, false>(sv::SampleParams)"
DRAW_F = "void sv::k_sample_draw<sv::bf16_t, true>(sv::SampleParams)"
FILT = "void sv::k_filter<sv::bf16_t>(sv::SampleParams)"
FROWS = "void sv::k_filter_rows<float>(sv::SampleParams)"


def test_counter_means_split_filtered_variants_and_keep_three_calibration_copies(tmp_path):
    p = tmp_path / "fetch.csv"
    _write_csv(p, "FETCH_SIZE", [(COPY, 131072), (COPY, 131072), (COPY, 131074), (COPY, 5),  # 4th: an input upload
                                 (MASS, 100), (MASS, 300), (DRAW, 7),
                                 # the filtered rounds: top-k 50 / top-p 0.9 first, then top-p 0.9 alone
                                 (FILT, 50), (FROWS, 2), (MASS_F, 1000), (DRAW_F, 9),
                                 (FILT, 70), (FROWS, 4), (MASS_F, 1100), (DRAW_F, 11),
                                 ("void sv::unrelated_kernel()", 1)])
    m = bench._counter_means(str(p), "FETCH_SIZE")
    assert m[COPY] == (131072 + 131072 + 131074) / 3
    assert m["k_sample_mass"] == 200
    assert m["k_sample_draw"] == 7
    # k_filter_rows is not taken for k_filter (a prefix of its name), and each setting keeps its own figures
    assert m["k_filter"] == 50 and m["k_filter_topp"] == 70
    assert m["k_filter_rows"] == 2 and m["k_filter_rows_topp"] == 4
    assert m["k_sample_mass_filtered"] == 1000 and m["k_sample_mass_filtered_topp"] == 1100
    assert m["k_sample_draw_filtered"] == 9 and m["k_sample_draw_filtered_topp"] == 11
    assert len(m) == 11


def test_ingest_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    # the fetch counter reports half the copy's bytes, the write counter all of them
    _write_csv(fp, "FETCH_SIZE", [(COPY, bench.CALIBRATION_KIB / 2)] * 3 + [(MASS, 1000.0)])
    _write_csv(wp, "WRITE_SIZE", [(COPY, bench.CALIBRATION_KIB)] * 3 + [(MASS, 10.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.ingest_counters(str(fp), str(wp)) == 0
    d = json.loads(out.read_text())
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["k_sample_mass"]["bytes_per_launch"] == 1024 * (1000 * 2 + 10)
    assert d["k_sample_mass"]["source_sha"] == bench.kernel_source_sha()
    # the figure is reported while the sources hash as recorded, and null once they do not
    assert bench.measured_traffic("k_sample_mass") == 1024 * 2010
    d["k_sample_mass"]["source_sha"] = "0" * 16
    out.write_text(json.dumps(d))
    assert bench.measured_traffic("k_sample_mass") is None
    assert bench.measured_traffic("k_greedy_argmax") is None


def test_ingest_refuses_files_without_the_calibration_copy(tmp_path, monkeypatch):
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(fp, "FETCH_SIZE", [(MASS, 1.0)])
    _write_csv(wp, "WRITE_SIZE", [(MASS, 1.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    assert bench.ingest_counters(str(fp), str(wp)) == 1
    assert not (tmp_path / "t.json").exists()


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_source_hash_covers_every_kernel_source():
    import glob
    import os
    csrc = os.path.join(os.path.dirname(bench.__file__), "rejection_sampling_verify_sample_amd", "csrc")
    every = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp")))
    assert bench.kernel_sources() == every and len(every) >= 10


def test_counter_means_keep_fp32_variants_apart(tmp_path):
    p = tmp_path / "fetch.csv"
    rows = [(COPY, 131072)] * 3 + [
        ("void sv::k_sample_rowstats<sv::bf16_t>(sv::SampleParams, int)", 100),
        ("void sv::k_sample_rowstats<float>(sv::SampleParams, int)", 500),
        ("void sv::k_sample_mass<float, true, false>(sv::SampleParams)", 70),
        (MASS, 30)]
    _write_csv(p, "FETCH_SIZE", rows)
    m = bench._counter_means(str(p), "FETCH_SIZE")
    assert m["k_sample_rowstats"] == 100 and m["k_sample_rowstats_f32"] == 500
    assert m["k_sample_mass_f32"] == 70 and m["k_sample_mass"] == 30


def test_trace_summary_groups_by_kernel_and_grid(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for g, d in ((1024, 4000), (1024, 6000), (64, 1000)):
            w.writerow({"Kernel_Name": "void sv::k_x<float>(sv::P)", "Grid_Size_X": g, "Start_Timestamp": 10,
                        "End_Timestamp": 10 + d})
    assert bench.trace_summary(str(p)) == 0
    out = capsys.readouterr().out
    assert "| k_x<float> | 1024 | 2 | 5.00 | 4.00 | 6.00 |" in out
    assert "| k_x<float> | 64 | 1 | 1.00 | 1.00 | 1.00 |" in out
