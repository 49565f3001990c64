"""The library's host code under AddressSanitizer and UBSan (CPU only).

api.hip (argument checks, workspace plans, launch descriptors) is compiled
host-only with the sanitizers and linked against tests/host_asan/stubs.hip,
which stands in for the HIP runtime and for every kernel launcher: each
launcher checks that the buffers its kernel would read or write lie inside
the registered caller buffers or the workspace, and that outputs do not
overlap inputs.  tests/host_asan/driver.cpp then calls every entry point with
invalid arguments and with valid ones on all workload shapes and 300 random
mixes of small, thin, tiled, tall and ragged groups.  No GPU is used; device
buffers are address ranges that are never dereferenced."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
# sanitizers on the host side only (nothing here is compiled for the GPU)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_host_code_under_asan_and_ubsan(tmp_path):
    hip = [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer", *HOST_SAN]
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "host_checks")
    run(hip + ["-c", os.path.join(ROOT, "matrix_orthogonalizing_optimizer_muon_amd", "csrc", "api.hip"), "-o", api])
    run(hip + ["-c", os.path.join(ROOT, "tests", "host_asan", "stubs.hip"), "-o", stubs])
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san, "-D__HIP_PLATFORM_AMD__",
         "-I/opt/rocm/include", "-c", os.path.join(ROOT, "tests", "host_asan", "driver.cpp"), "-o", drv])
    run([CLANG, *san, api, stubs, drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
