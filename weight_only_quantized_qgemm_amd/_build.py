"""Builds the HIP library (libqgemm.so) in-tree for gfx950 with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemm.so")
SOURCES = ["qgemm_host.cpp", "qgemm_kernels.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose=False):
    """Compile every source into libqgemm.so next to this file; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr)
    # the host pass does not know the gfx-only target feature; that warning is noise
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
