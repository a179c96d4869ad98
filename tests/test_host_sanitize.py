"""Host code of libmoeep under AddressSanitizer and UBSan (CPU only).

Every HIP source is compiled with the sanitizers on its host pass (device
code is unchanged), linked with tests/host_sanitize_checks.cpp, and run:
the driver exercises every argument check of the C ABI, the workspace
queries, the status strings and the host expert-placement routine, none of
which touches the GPU.  UBSan stops at the first undefined operation
(signed overflow, an out-of-range enum load, a misaligned access), ASan at
the first invalid memory access.
"""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_grouped_gemm_amd", "csrc")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = "address,undefined"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                                reason="needs the ROCm toolchain")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    return r


def test_host_code_under_asan_and_ubsan(tmp_path):
    # the sanitizer options go to the host pass only
    host_only = []
    for flag in (f"-fsanitize={SAN}", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"):
        host_only += ["-Xarch_host", flag]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_hip(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", *common, *host_only,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_hip, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    driver = str(tmp_path / "driver.o")
    _run([CLANGXX, *common, f"-fsanitize={SAN}", "-fno-sanitize-recover=undefined",
          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-c", os.path.join(ROOT, "tests", "host_sanitize_checks.cpp"), "-o", driver])
    exe = str(tmp_path / "host_checks")
    _run([CLANGXX, f"-fsanitize={SAN}", driver, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks ok" in r.stdout, f"{r.stdout}\n{r.stderr}"
