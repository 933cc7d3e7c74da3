"""Host logic of bench.py (no GPU): the one-GPU refusal, the rocprofv3 CSV summary, and the
rule that a committed HBM-traffic figure is used only while its kernel sources are unchanged."""
import hashlib

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def _write_csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_summarize_rocprof_stats_and_counters(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    _write_csv(d / "x_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [["kvb::prefill_kernel<a>", 3, 1500.0, 1000, 2000], ["other_kernel", 1, 5, 5, 5]])
    _write_csv(d / "x_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, "kvb::prefill_kernel<a>", "FETCH_SIZE", 10.0],
                [1, "kvb::prefill_kernel<a>", "FETCH_SIZE", 6.0],     # two rows of one dispatch add up
                [2, "kvb::prefill_kernel<a>", "FETCH_SIZE", 20.0],
                [3, "other_kernel", "FETCH_SIZE", 999.0]])
    out = bench.summarize_rocprof(str(tmp_path), "prefill_kernel").splitlines()
    assert "calls: 3" in out and "avg_ns: 1500.0" in out
    assert "dispatches: 2" in out
    assert "FETCH_SIZE_per_dispatch: 18" in out                  # (16 + 20) / 2


def test_traffic_only_while_sources_match(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    (prof / "kern_work.pmc.txt").write_text(
        "# header: lines starting with # are comments\n"
        f"source_files: k.hip\nsource_sha256_16: {h}\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("kern_work") == 12345.0
    assert bench.read_traffic("missing") is None
    src.write_text("kernel v2\n")                                  # kernel changed since
    assert bench.read_traffic("kern_work") is None


def test_counters_only_while_sources_match(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    (prof / "kern_work.sq.txt").write_text(
        "# command (A): rocprofv3 --pmc MfmaUtil ...\n"
        f"source_files: k.hip\nsource_sha256_16: {h}\nMfmaUtil_per_dispatch: 55.5\n"
        "mfma_util_percent: 55.50\nvalu_per_mfma: 5.852\nl2_hit_rate: 0.8453\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_counters("kern_work") == {"mfma_util_percent": 55.5, "valu_per_mfma": 5.852,
                                                "l2_hit_rate": 0.8453}
    assert bench.read_counters("missing") is None
    src.write_text("kernel v2\n")                                  # kernel changed since
    assert bench.read_counters("kern_work") is None
