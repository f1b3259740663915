"""Context recorded beside every timing: the GPU core clock and board power
while the timed region runs, and the toolchain that built the kernels.

The clock matters on this board: the bf16 matrix-core kernels run at the
board's power limit, where the clock drops with the data being multiplied,
so a throughput figure without the clock it ran at cannot be compared
across runs.  The toolchain matters because a compiler change can move a
kernel across an occupancy cliff without failing any test; "Bare Metal
Bard" (page 1, fourth paragraph) found such a regression only through the
version recorded with its measurements.  Clock and power come from the
amdgpu driver's sysfs files (no GPU call), sampled by a background thread;
the compiler version comes from the library (no process is started).
"""
from __future__ import annotations

import glob
import re
import statistics
import threading
from typing import Dict, List, Optional


def _read(path: str) -> Optional[str]:
    try:
        with open(path) as fh:
            return fh.read()
    except OSError:
        return None


def _current_sclk_mhz(path: str) -> Optional[float]:
    """The level marked '*' in a pp_dpm_sclk file ("1: 2400Mhz *")."""
    text = _read(path)
    if not text:
        return None
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*[Mm]hz", line)
            if m:
                return float(m.group(1))
    return None


def _power_w(path: str) -> Optional[float]:
    text = _read(path)
    try:
        return int(text) / 1e6 if text else None   # microwatts
    except ValueError:
        return None


def _stats(xs: List[float]) -> Optional[Dict[str, float]]:
    if not xs:
        return None
    return {"median": round(statistics.median(xs), 1), "min": round(min(xs), 1),
            "max": round(max(xs), 1), "samples": len(xs)}


class ClockSampler:
    """`with ClockSampler() as cs: <timed work>` then `cs.summary()`."""

    def __init__(self, period_s: float = 0.005):
        self.period = period_s
        self.sclk_files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.power_files = sorted(
            glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average") +
            glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))[:1]
        self.sclk: List[float] = []
        self.power: List[float] = []
        self._stop = threading.Event()
        self._thread: Optional[threading.Thread] = None

    def _run(self):
        while not self._stop.is_set():
            for f in self.sclk_files[:1]:
                v = _current_sclk_mhz(f)
                if v is not None:
                    self.sclk.append(v)
            for f in self.power_files:
                v = _power_w(f)
                if v is not None:
                    self.power.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.sclk_files or self.power_files:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()
        return False

    def summary(self) -> Dict[str, Optional[Dict[str, float]]]:
        return {"sclk_mhz": _stats(self.sclk), "power_w": _stats(self.power)}


def toolchain(build_info: Optional[str] = None) -> Dict[str, Optional[str]]:
    """ROCm release (read from the installation's version file) and the
    toolchain that compiled the kernels, as the library itself reports it
    (gemm_build_info).  Starts no process: the caller may already hold the
    GPU."""
    rocm = _read("/opt/rocm/.info/version")
    return {"rocm": rocm.strip() if rocm else None, "compiler": build_info}
