"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU call): api.hip's validation, extent and overlap arithmetic
(128-bit guards against overflow), the dispatch table and the plan queries
are rebuilt with both sanitizers and the host-side ABI tests run against that
build in a child process; any sanitizer report fails the run."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_mi355gemm_build_san", os.path.join(ROOT, "dense_gemm_17_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    if not all(os.path.exists(os.path.join(b.BUILD, os.path.basename(s)[:-4] + ".o"))
               for s in b.sources()):
        pytest.skip("the library has not been built in this tree")
    lib = b.build_sanitized_host(str(tmp_path / "libmi355gemm_san.so"))
    env = dict(os.environ, MI355GEMM_LIBRARY=lib, LD_PRELOAD=b.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
