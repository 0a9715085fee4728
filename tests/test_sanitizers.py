"""Sanitizer builds of the host-side code, on the CPU.

* The fp64 oracle compiled with AddressSanitizer and UndefinedBehaviorSanitizer
  (every error fatal), with every pin of ``test_oracle_pins.py`` run against it
  in a process of its own.
* The host side of the library (``deltalog.cpp``: validation, aliasing
  rules, log-length bookkeeping, the choice of launch mode) compiled with
  g++ and both sanitizers against launchers that only record what they were
  asked to launch (``tests/sanitize/stub_launch.cpp``), driven by
  ``tests/sanitize/host_check.cpp``.  No device code is built or run.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
ROCM = "/opt/rocm"


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is required")
def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", *SAN_FLAGS, "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "eager_oracle.c")], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = _env()
    env["LD_PRELOAD"] = asan
    r = subprocess.run([sys.executable, os.path.join(SAN, "run_oracle_pins.py"), str(lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "pins under sanitizers" in r.stdout and "FAILED" not in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="g++ and the HIP headers are required")
def test_host_library_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    csrc = os.path.join(ROOT, "recurrent_state_updates_amd", "csrc")
    subprocess.run(["g++", *SAN_FLAGS, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                    os.path.join(csrc, "deltalog.cpp"), os.path.join(SAN, "stub_launch.cpp"),
                    os.path.join(SAN, "host_check.cpp"), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], env=_env(), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is required")
def test_the_sanitizer_is_live_a_planted_overflow_is_caught(tmp_path):
    """A copy of the oracle with its value-factor buffer one element short
    (planted here, on the CPU) must abort the same run with a heap overflow:
    the pin run above really executes under AddressSanitizer."""
    with open(os.path.join(ROOT, "oracle", "eager_oracle.c")) as f:
        src = f.read()
    site = "double *u = (double *)malloc((size_t)dv * sizeof(double));"
    assert src.count(site) == 1
    bad = tmp_path / "oracle_short.c"
    bad.write_text(src.replace(site, "double *u = (double *)malloc((size_t)(dv - 1) * sizeof(double));"))
    lib = tmp_path / "liboracle_short.so"
    subprocess.run(["gcc", *SAN_FLAGS, "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(lib), str(bad)],
                   check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = _env()
    env["LD_PRELOAD"] = asan
    r = subprocess.run([sys.executable, os.path.join(SAN, "run_oracle_pins.py"), str(lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
