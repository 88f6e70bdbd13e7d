"""CPU sanitizer tier: the oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (errors abort, leaks are not tracked).

* The oracle pins (tests/test_oracle_pins.py, tests/test_oracle_fp8_pins.py) run in a child process
  against oracle.c built with both sanitizers (GATTN_ORACLE_LIB).
* The ABI checks (tests/test_abi.py) run in a child process against a host-only build of
  csrc/gattn.cpp with both sanitizers (GATTN_LIBRARY): every argument check, the split plan and the
  workspace sizing execute instrumented; kernel launches are stubs that fail
  (tests/sanitize/host_stubs.cpp), and no check in that file launches one.
The sanitizer runtime is preloaded into the child Python, as an instrumented shared library needs.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

SAN = oracle.SANITIZE_FLAGS


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def _run_child(tests, extra_env, timeout=1200):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra_env)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    _run_child(["tests/test_oracle_pins.py", "tests/test_oracle_fp8_pins.py"], {"GATTN_ORACLE_LIB": lib})


def test_abi_validation_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "global_paged_gqa_amd", "csrc")
    lib = str(tmp_path / "libgattn_hostcheck.so")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I", csrc, "-I", os.path.join(ROOT, "include"), "-o", lib,
                           os.path.join(csrc, "gattn.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp")])
    _run_child(["tests/test_abi.py"], {"GATTN_LIBRARY": lib})


def test_the_harness_reports_a_planted_overflow(tmp_path):
    """Power check of the set-up above (preloaded runtime, instrumented library loaded by ctypes in
    a child Python): a one-past-the-end heap write in a tiny CPU-only library is reported."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint planted(int n) { int *a = malloc(n * sizeof(int));"
                   " a[n] = 1; int r = a[0]; free(a); return r; }\n")
    lib = str(tmp_path / "libplanted.so")
    subprocess.check_call(["gcc", *SAN, "-fPIC", "-shared", "-o", lib, str(src)])
    env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).planted(4)"], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
