"""Host-side checks of the measurement tooling (no GPU): the clock reader's
parsing of the driver's sysfs format and the benchmark's HBM-traffic
bookkeeping."""
import csv
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(name, rel):
    spec = importlib.util.spec_from_file_location(name, os.path.join(ROOT, rel))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


measure = _load("measure_t", "dense_gemm_17_amd/measure.py")


def test_sclk_parsing(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 127Mhz\n0: 500Mhz\n1: 2400Mhz *\n")
    assert measure._current_sclk_mhz(str(f)) == 2400.0
    f.write_text("S: 127Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert measure._current_sclk_mhz(str(f)) == 127.0
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")             # no current level marked
    assert measure._current_sclk_mhz(str(f)) is None
    assert measure._current_sclk_mhz(str(tmp_path / "missing")) is None


def test_power_parsing(tmp_path):
    f = tmp_path / "power1_average"
    f.write_text("1305000000\n")
    assert measure._power_w(str(f)) == pytest.approx(1305.0)
    f.write_text("garbage\n")
    assert measure._power_w(str(f)) is None


def test_sampler_without_sysfs_reports_none():
    s = measure.ClockSampler()
    s.sclk_files, s.power_files = [], []
    with s:
        pass
    assert s.summary() == {"sclk_mhz": None, "power_w": None}


def test_stats():
    assert measure._stats([]) is None
    st = measure._stats([1.0, 2.0, 10.0])
    assert st == {"median": 2.0, "min": 1.0, "max": 10.0, "samples": 3}


# ---------------------------------------------------------------------------
# bench.py's HBM-traffic bookkeeping: counter ingestion, copy calibration and
# the source digest that retires a measurement once the kernel changes.

bench = _load("bench_t", "bench.py")


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": 65536,
                        "Counter_Name": counter, "Counter_Value": kib})


def test_code_text_ignores_comments_and_spacing():
    a = "int x = 1; // one\n/* block\n comment */ int  y =\n 2;\n"
    b = "int x = 1;\nint y = 2; // two\n"
    assert bench.code_text_from(a) == bench.code_text_from(b) == "int x = 1; int y = 2;"


def test_counter_ingestion_and_digest(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for f in {f for _, fs in bench.KERNEL_SOURCES.values() for f in fs} | set(bench.COMMON_SOURCES):
        (csrc / f).write_text(f"// {f}\nint k_{f.replace('.', '_')} = 1;\n")
    traffic = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))

    sym = bench.KERNEL_SOURCES["mfma_f32_direct"][0]
    kname = f"void mi355gemm::(anonymous namespace)::{sym}(long)"
    copy = "__amd_rocclr_copyBuffer"
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    fetch.mkdir()
    write.mkdir()
    # The copy reads back as half its bytes on FETCH_SIZE and as all of them on
    # WRITE_SIZE; a small copy dispatch must not be taken for the calibration.
    _pmc_csv(fetch / "pmc_counter_collection.csv", "FETCH_SIZE",
             [(copy, 4.0), (copy, copy_kib / 2), (kname, 1000.0), (kname, 3000.0)])
    _pmc_csv(write / "pmc_counter_collection.csv", "WRITE_SIZE",
             [(copy, copy_kib), (kname, 500.0), (kname, 500.0)])
    bench.ingest_counters(str(fetch), str(write))

    text = traffic.read_text()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    expected = 2.0 * 2000.0 * 1024 + 1.0 * 500.0 * 1024
    assert bench.traffic_for("mfma_f32_direct") == expected
    assert bench.traffic_for("mfma_bf16_direct") is None          # never measured

    # A comment edit keeps the measurement; a code edit retires it.
    src = csrc / bench.KERNEL_SOURCES["mfma_f32_direct"][1][0]
    src.write_text(src.read_text() + "// note\n")
    assert bench.traffic_for("mfma_f32_direct") == expected
    src.write_text(src.read_text() + "int extra = 2;\n")
    assert bench.traffic_for("mfma_f32_direct") is None


def test_committed_traffic_file_parses():
    rec = bench.json.loads((lambda t: t[t.index("{"):])(open(bench.TRAFFIC_FILE).read()))
    assert rec["copy_bytes"] == bench.COPY_BYTES
    assert 0.5 < rec["fetch_scale"] < 8 and 0.5 < rec["write_scale"] < 8
    for k, v in rec["kernels"].items():
        assert k in bench.KERNEL_SOURCES
        assert v["bytes_per_launch"] == pytest.approx(v["fetch_bytes"] + v["write_bytes"], abs=1)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
