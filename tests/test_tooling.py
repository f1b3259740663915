"""Host-side checks of the measurement tooling (no GPU): the clock reader's
parsing of the driver's sysfs format, and the counter summary's kernel-name
handling and per-dispatch averaging."""
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
counters = _load("counters_t", "dense_gemm_17_amd/counters.py")


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


@pytest.mark.parametrize("name,short", [
    ("void mi355gemm::(anonymous namespace)::mfma_f32_direct_kernel<128, 64, 16>(long, long, "
     "long, float const*, long, float const*, long, float*, long, long, long, int)",
     "mfma_f32_direct_kernel<128, 64, 16>"),
    ("mi355gemm::(anonymous namespace)::mfma_bf16_direct_kernel(long, long, long, unsigned "
     "short const*, long)", "mfma_bf16_direct_kernel"),
    ("void mi355gemm::(anonymous namespace)::skinny_kernel<float, 4, 8, 1024, 4, true, 2>(long)",
     "skinny_kernel<float, 4, 8, 1024, 4, true, 2>"),
])
def test_kernel_name_shortening(name, short):
    assert counters.short(name) == short


def test_counter_averaging(tmp_path):
    d = tmp_path / "gpt_qkv__sq"
    d.mkdir()
    rows = []
    kname = "void mi355gemm::(anonymous namespace)::mfma_f32_direct_kernel<128, 64, 16>(long)"
    # two dispatches, each counter reported per XCD instance (summed per dispatch)
    for disp, (mfma, grbm) in enumerate([(800.0, 80.0), (1200.0, 120.0)]):
        for part in (0.5, 0.5):
            rows.append({"Dispatch_Id": disp, "Kernel_Name": kname,
                         "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": mfma * part})
            rows.append({"Dispatch_Id": disp, "Kernel_Name": kname,
                         "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": grbm * part})
    rows.append({"Dispatch_Id": 9, "Kernel_Name": "at::native::some_torch_kernel",
                 "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1e9})
    with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        w.writerows(rows)
    got = counters.read_dir(str(d))
    assert list(got) == ["mfma_f32_direct_kernel<128, 64, 16>"]
    k = got["mfma_f32_direct_kernel<128, 64, 16>"]
    assert k["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(1000.0)
    assert k["GRBM_GUI_ACTIVE"] == pytest.approx(100.0)
    assert k["_dispatches"] == 2
