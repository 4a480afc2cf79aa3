"""Build the HIP library (libmoe_finalize_rmsnorm.so) in-tree for gfx950, and
the torch operators on top of it (libmfr_torch_ops.so).

The library is compiled with hipcc straight from csrc/ and placed next to
this file, where the Python binding loads it. Flags:
  --offload-arch=gfx950          CDNA4 (MI355X) code only
  -ffp-contract=off              every FMA in the kernels is written out
  -target-feature -packed-fp32-ops  no packed fp32 VALU ops are emitted
  -amdgpu-kernarg-preload-count=16   (the fused-op library only) the kernel's
                                 leading arguments arrive in SGPRs at wave
                                 launch instead of through a scalar load
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_finalize_rmsnorm.so")
PROBE_LIB = os.path.join(PKG, "libmfr_copy_probe.so")
OPS_LIB = os.path.join(PKG, "libmfr_torch_ops.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CXX = os.environ.get("CXX", "g++")

HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Up to 16 SGPRs of leading kernel arguments (the fused kernel passes 14:
# six pointers and two ints) are loaded by the dispatcher at wave launch.
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]


def _hipcc(sources, out, verbose=False, extra=()):
    cmd = [HIPCC, *HIPFLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", out + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and "(ignoring feature)" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def _torch_ops(verbose=False):
    """The torch operators (host C++ against torch's headers and the
    library above, which it links by its in-tree path)."""
    import torch
    from torch.utils import cpp_extension
    out = OPS_LIB
    torch_lib = cpp_extension.library_paths()[0]
    cmd = [CXX, "-std=c++17", "-O2", "-fPIC", "-shared", "-Wall",
           "-D__HIP_PLATFORM_AMD__", "-DUSE_ROCM",
           f"-D_GLIBCXX_USE_CXX11_ABI={int(torch._C._GLIBCXX_USE_CXX11_ABI)}",
           *[f"-I{p}" for p in cpp_extension.include_paths()],
           "-I", os.path.join(ROCM, "include"), "-I", INCLUDE,
           "-o", out + ".tmp", os.path.join(CSRC, "mfr_torch_ops.cpp"),
           f"-L{torch_lib}", "-lc10", "-lc10_hip", "-ltorch_cpu",
           f"-L{PKG}", "-l:" + os.path.basename(LIB),
           "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{torch_lib}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the torch operators failed:\n" + r.stdout + r.stderr)
    if verbose and (r.stdout + r.stderr).strip():
        print(r.stdout + r.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(verbose=False):
    """Compile the product library, the bench's copy-probe library and the
    torch operators."""
    _hipcc([os.path.join(CSRC, "mfr_kernels.hip")], LIB, verbose, extra=PRELOAD)
    _hipcc([os.path.join(CSRC, "copy_probe.hip")], PROBE_LIB, verbose)
    _torch_ops(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
