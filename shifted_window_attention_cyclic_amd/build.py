"""Builds the HIP library ``libswa.so`` for gfx950 with hipcc (in-tree).

Packed fp32 VALU instructions are switched off for device code
(``-packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libswa.so")
SOURCES = [os.path.join(CSRC, "swa_kernels.hip"), os.path.join(CSRC, "swa_backward.hip"),
           os.path.join(CSRC, "swa_projection.hip"), os.path.join(CSRC, "swa_layer.hip"),
           os.path.join(CSRC, "swa_api.cpp")]
ARCH = "gfx950"


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA operands and results in VGPRs (no AGPR copies), and let
            # fmaxf skip NaN canonicalisation (inputs are finite; masks use -inf)
            "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compiles every HIP source and links the shared library (always)."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objs, procs = [], []
    # the sources compile independently, side by side
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc] + hipcc_flags() + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", LIBRARY + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    for o in objs:
        os.remove(o)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
