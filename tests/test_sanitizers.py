"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code:
libwushkv's C-ABI layer (api.cpp, with stub launchers that check every
launch's arguments against the caller's buffers; no GPU) and the fp64 oracle
(oracle/wko.c).  Each driver exercises every entry point, including the error
paths and the quantizer's edge cases, and must finish clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _have(tool):
    return shutil.which(tool) is not None


@pytest.mark.skipif(not _have("g++"), reason="needs g++")
def test_host_abi_under_sanitizers(tmp_path):
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(ROOT, "decode_attention_wushkv_amd", "csrc", "api.cpp"),
           "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host driver OK" in r.stdout


@pytest.mark.skipif(not _have("gcc"), reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", *SAN, "-ffp-contract=off",
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "wko.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver OK" in r.stdout
