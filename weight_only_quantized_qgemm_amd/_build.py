"""Builds the HIP library (libqgemm.so) in-tree for gfx950 with hipcc.

Each source compiles to its own objects in parallel (the kernel sources once per weight format), then hipcc links the shared library.
The objects stay in _build/obj next to this file (not committed), where the host-sanitizer
build of the host code (_build_asan.py) finds the kernel objects it links against.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemm.so")
OBJ_DIR = os.path.join(PKG, "_build", "obj")
# measurement helpers for the benchmark (streaming-read kernel, host time per call): a library
# of their own, outside the qgemm ABI
PROBE_LIB = os.path.join(PKG, "libqgemm_probe.so")
# Weight formats (the Format enum of csrc/qgemm_internal.h).  Each kernel source is compiled
# once per format (-DQGEMM_FMT_UNIT), so the many kernel instances build in parallel.
N_FORMATS = 6
UNITS = ([("qgemm_host.cpp", []), ("qgemm_run.hip", [])]
         + [(k, [f"-DQGEMM_FMT_UNIT={f}"]) for k in ("qgemm_decode.hip", "qgemm_prefill.hip", "qgemm_prefill_tw.hip")
            for f in range(N_FORMATS)])

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments (up to 16 SGPRs) arrive preloaded in registers
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
]


def unit_object(source, defs):
    """Path of the object file of one compilation unit (a source and its defines)."""
    tag = "".join(d.split("=")[-1] for d in defs)
    return os.path.join(OBJ_DIR, f"{source.replace('.', '_')}{'_' + tag if tag else ''}.o")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx-only target feature; that warning is noise
    lines = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return res.returncode, lines


def build(verbose=False):
    """Compile every source into libqgemm.so next to this file; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include")]
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [unit_object(s, defs) for s, defs in UNITS]
    cmds = [[hipcc, *HIPCC_FLAGS, *defs, *inc, "-c", os.path.join(CSRC, s), "-o", o]
            for (s, defs), o in zip(UNITS, objs)]
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_run, cmds))
    msgs = []
    for (s, defs), (rc, lines) in zip(UNITS, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} {' '.join(defs)}:\n" + "\n".join(lines))
        msgs += lines
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose launch stub the host pass did not emit fails here, not at
    # load time
    rc, lines = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(lines))
    msgs += lines
    os.replace(tmp, LIB)
    pobj = os.path.join(OBJ_DIR, "qgemm_probe_hip.o")
    rc, lines = _run([hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, "qgemm_probe.hip"), "-o", pobj])
    if rc != 0:
        raise RuntimeError("hipcc failed on qgemm_probe.hip:\n" + "\n".join(lines))
    msgs += lines
    ptmp = PROBE_LIB + ".tmp"
    rc, lines = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", pobj, "-L", PKG, "-lqgemm",
                      "-Wl,-rpath,$ORIGIN", "-o", ptmp])
    if rc != 0:
        raise RuntimeError("link failed (probe library):\n" + "\n".join(lines))
    msgs += lines
    os.replace(ptmp, PROBE_LIB)
    if verbose and msgs:
        print("\n".join(msgs))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
