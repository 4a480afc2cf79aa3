"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two small C++ programs drive, over ordinary, degenerate and erroneous inputs:
  * every exported oracle function (tests/sanitize/oracle_driver.cpp), built
    with g++ together with oracle/mfr_oracle.cpp;
  * the library's host side: path query, status text, the launch override
    and every argument check of the three entry points
    (tests/sanitize/abi_driver.cpp), linked against mfr_kernels.hip built by
    hipcc with the sanitizers on its host code only. No call reaches a kernel
    launch, so no GPU is involved.
A sanitizer report, a leak or a wrong status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "top_finalize_residual_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
HOST_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", *HOST_SAN,
          os.path.join(ROOT, "oracle", "mfr_oracle.cpp"), os.path.join(HERE, "oracle_driver.cpp"),
          "-o", exe], timeout=300)
    r = _run([exe], env=ENV, timeout=120)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm")
def test_library_host_code_under_sanitizers(tmp_path):
    obj = str(tmp_path / "mfr_kernels.o")
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "mfr_kernels.hip"), "-o", obj],
         timeout=600)
    _run([CLANG, "-std=c++17", "-O1", "-g", *HOST_SAN, "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
          "-I", CSRC, "-I", "/opt/rocm/include", os.path.join(HERE, "abi_driver.cpp"), obj,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], timeout=300)
    r = _run([exe], env=ENV, timeout=120)
    assert "abi driver: ok" in r.stdout
