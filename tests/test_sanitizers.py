"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The planner (csrc/plan.cpp, plain C++ with no HIP) is built with g++ together
  with tests/c/plan_sanitize.cpp, which plans seeded random batches -- every
  request kind, bf16 and fp32, page sizes 1..64, GQA 1..16, detected and hinted
  shared-prefix trees -- and checks exactly-once coverage of every visible
  (token, head, key), the split and merge numbering, cascade page sharing and
  the metadata capacity, plus the slot_mapping check against brute force.
* The oracle (oracle/rpkv_oracle.c) is built with gcc the same way and the
  oracle pin suite is run against that build, with the sanitizer runtime
  preloaded into the Python process.
Any sanitizer report fails the run (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_paged_kv_store_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
       "-g", "-O1"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _env():
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def test_planner_under_asan_ubsan(tmp_path):
    _need("g++")
    exe = str(tmp_path / "plan_sanitize")
    subprocess.run(["g++", "-std=c++17", "-Wall", *SAN, "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, os.path.join(ROOT, "tests", "c", "plan_sanitize.cpp"),
                    os.path.join(CSRC, "plan.cpp"), "-o", exe], check=True)
    env = _env()
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1"
    r = subprocess.run([exe, "600"], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "600 batches, 0 failures" in r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    _need("gcc")
    lib = str(tmp_path / "librpkv_oracle_asan.so")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-shared", "-fPIC", *SAN,
                    os.path.join(ROOT, "oracle", "rpkv_oracle.c"), "-o", lib, "-lm", "-lpthread"],
                   check=True)
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    if not os.path.isabs(asan_rt) or not os.path.exists(asan_rt):
        pytest.skip("no AddressSanitizer runtime for gcc")
    env = _env()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"   # the interpreter's own leaks
    env["LD_PRELOAD"] = asan_rt
    env["RPKV_ORACLE_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
