"""Host-sanitizer build of the library, for the CPU tests of the host code (not shipped).

The host code -- validation, launch planning, the quantizer and the packer (qgemm_host.cpp)
and the entry points (qgemm_run.hip) -- is recompiled with AddressSanitizer and
UndefinedBehaviorSanitizer on its host pass only, and linked with the kernel objects of the
regular build (_build/obj) into _build/libqgemm_asan.so.  A process that loads it must
preload the sanitizer runtime (tests/test_host_asan.py runs the packer and ABI tests that way).
"""
import os

import _build as B

ASAN_LIB = os.path.join(B.PKG, "_build", "libqgemm_asan.so")
HOST_UNITS = [("qgemm_host.cpp", []), ("qgemm_run.hip", [])]
# sanitizers on the host compilation only (device code is built exactly as in the library)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build_asan():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(B.ROOT, "include")]
    kernel_objs = [B.unit_object(s, d) for s, d in B.UNITS if (s, d) not in HOST_UNITS]
    missing = [o for o in kernel_objs if not os.path.exists(o)]
    if missing:
        B.build()
    objs = []
    for s, d in HOST_UNITS:
        o = os.path.join(B.OBJ_DIR, s.replace(".", "_") + "_asan.o")
        rc, lines = B._run([hipcc, *B.HIPCC_FLAGS, *HOST_SANITIZE, *d, *inc, "-c", os.path.join(B.CSRC, s), "-o", o])
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s}:\n" + "\n".join(lines))
        objs.append(o)
    tmp = ASAN_LIB + ".tmp"
    rc, lines = B._run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, *kernel_objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(lines))
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
