"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host/sanitize_host.cpp calls every host-only path of the C ABI (status
strings, shape checks, workspace layouts over a sweep of shapes, formats and
token counts, argument checks that return before device work, the Mamba verify
shape checks).  The library sources are compiled with the sanitizers on the host
side only (-Xarch_host before each -fsanitize=; device code is built as usual)
and linked into that driver, which runs on the CPU."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_layer_logits_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["latentmoe", "route", "gemm_stream", "gemm_big", "gemm_mid", "misc", "ssm_replay"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"] + SAN

    def compile_one(name):
        out = str(tmp_path / (name + ".o"))
        subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, name + ".hip"), "-o", out], check=True,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        return out

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(tmp_path / "drv.o")
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", *SAN, "-c", os.path.join(ROOT, "tests", "host",
                                                                               "sanitize_host.cpp"), "-o", drv],
                   check=True)
    exe = str(tmp_path / "sanitize_host")
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, drv, *objs], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "host checks ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
