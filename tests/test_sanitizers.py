"""The CPU oracle and the library's host-only configuration checks built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++), and driven over
every entry point (tests/sanitize/*): no sanitizer report, every call returns
what it should."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(tmp_path, cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout[-500:], r.stderr[-3000:])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN, "-mpopcnt", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "hkv_oracle.c"),
           "-lm", "-o", exe]
    _run(tmp_path, cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_driver")
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "lsh_eviction_amd", "csrc"),
           os.path.join(HERE, "sanitize", "validate_driver.cpp"),
           os.path.join(ROOT, "lsh_eviction_amd", "csrc", "hkv_validate.cpp"), "-o", exe]
    _run(tmp_path, cmd, exe)
