"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Validation, launch planning, the quantizer and the packer are recompiled with both
sanitizers on their host pass (weight_only_quantized_qgemm_amd/_build_asan.py), and the
packer and C-ABI tests run against that build in a child process that preloads the
sanitizer runtimes; any report ends the child with an error.  FlashInfer PR #7495 analysis,
section 3 (a) and (b), lists the alignment and index-overflow faults this kind of host index
arithmetic is prone to."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_packer_and_abi_tests_pass_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, os.path.join(ROOT, "weight_only_quantized_qgemm_amd"))
    try:
        import _build_asan
    finally:
        sys.path.pop(0)
    lib = _build_asan.build_asan()
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", QGEMM_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_pack.py", "tests/test_abi.py", "-q", "-x", "-s",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
