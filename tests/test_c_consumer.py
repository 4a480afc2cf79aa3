"""The boundary is a C ABI: a plain C99 program compiles against
include/moe_finalize_rmsnorm.h, links the library and gets the documented
host-side answers (path query, argument errors, status strings). No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "top_finalize_residual_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "moe_finalize_rmsnorm.h"
int main(void) {
    int bad = 0;
    if (moe_finalize_rmsnorm_path(1, 6144, 8) != MFR_PATH_TOKEN) bad |= 1;
    if (moe_finalize_rmsnorm_path(8192, 6144, 8) != MFR_PATH_STREAM) bad |= 2;
    if (moe_finalize_rmsnorm_path(4, 6143, 8) != MFR_PATH_UNSUPPORTED) bad |= 4;
    if (moe_finalize_rmsnorm(NULL, NULL, NULL, NULL, NULL, NULL, 1e-6f, 1.0f, NULL, NULL,
                             4, 2048, 8, NULL) != MFR_ERR_NULL) bad |= 8;
    if (residual_add_rmsnorm(NULL, NULL, NULL, -1.0f, NULL, NULL, 4, 2048, NULL)
        != MFR_ERR_SCALAR) bad |= 16;
    if (moe_finalize_rmsnorm_fp8(NULL, NULL, NULL, NULL, NULL, NULL, 1e-6f, 1.0f, NULL, NULL,
                                 NULL, NULL, 0, 2048, 8, NULL) != MFR_OK) bad |= 32;
    if (strcmp(moe_finalize_rmsnorm_strerror(MFR_ERR_ARG), "unknown status") == 0) bad |= 64;
    if (strlen(moe_finalize_rmsnorm_strerror(MFR_ERR_ALIAS)) == 0) bad |= 128;
    if (moe_finalize_rmsnorm_checked(NULL, -1, NULL, NULL, NULL, NULL, NULL, 1e-6f, 1.0f, NULL,
                                     NULL, NULL, 4, 2048, 8, NULL) != MFR_ERR_SHAPE) bad |= 256;
    printf("%d\n", bad);
    return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs gcc and the ROCm headers")
def test_plain_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libmoe_finalize_rmsnorm.so")):
        pytest.skip("HIP library not built")
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-Wno-unused-function",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-o", str(exe), str(src), "-L", LIBDIR,
                    "-lmoe_finalize_rmsnorm", f"-Wl,-rpath,{LIBDIR}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
