"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the C ABI layer of libsattn
(csrc/api.cpp, built for the host with recording stand-ins for the kernel launchers) and the CPU oracle
(oracle/*.c).  Each driver in tests/native/ exits 0 only if every expectation holds and no sanitizer fires."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_api_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_host_check")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "quantized_attention_05_amd", "csrc", "api.cpp"),
          os.path.join(ROOT, "tests", "native", "api_host_check.cpp"), "-o", exe])
    res = _run([exe], env=ENV)
    assert "api host checks: ok" in res.stdout
    assert "runtime error" not in res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_host_check")
    _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fopenmp",
          os.path.join(ROOT, "oracle", "sattn_oracle.c"), os.path.join(ROOT, "oracle", "linear_oracle.c"),
          os.path.join(ROOT, "tests", "native", "oracle_host_check.c"), "-o", exe, "-lm"])
    res = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"))
    assert "oracle host checks: ok" in res.stdout
    assert "runtime error" not in res.stderr
