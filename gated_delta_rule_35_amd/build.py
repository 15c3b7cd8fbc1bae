"""Builds libkda.so, the HIP library behind the C ABI in include/kda.h, for gfx950.

hipcc compiles the kernels and the C-ABI front end into one shared object next to
this file.  -packed-fp32-ops is turned off for the device code: the compiler then
never forms packed fp32 instructions.  -amdgpu-mfma-vgpr-form keeps MFMA
accumulators in ordinary VGPRs while they fit: the scan kernel's state and
products are scaled and converted by VALU instructions every chunk, which cannot
read accumulation registers, so the other form costs a register move per element.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("kda_fused.hip", "kda_intra.hip", "kda_scan.hip", "kda_compose.hip", "kda_decode.hip", "kda_bwd.hip", "kda_scratch.hip",
              "kda_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"), "-o", LIB + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
