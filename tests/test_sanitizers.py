"""The CPU oracle and the host layer of the C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, plain gcc / g++, no GPU) and run on
drivers that exercise every entry point: any memory error, leak or undefined
behaviour ends the run with a sanitizer report and a non-zero exit status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", *SAN,
                os.path.join(ROOT, "oracle", "dqk_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                "-o", exe, "-lm"], exe)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    out = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-Wall", *SAN,
                os.path.join(ROOT, "bit_quantized_decode_dqk_amd", "csrc", "dqk_api.cpp"),
                os.path.join(HERE, "host_driver.cpp"), "-o", exe], exe)
    assert "failures 0" in out
