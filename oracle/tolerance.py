"""Acceptance gates for GEMM outputs (TEST INFRASTRUCTURE ONLY).

Low Bit Triton Kernels (lecture 034): after adding group scales the mean / max relative
error should be around 1e-3 / 5e-3, and the error should be judged as a distribution,
not only by its maximum (validation section and exercise 4).  The reading used here:

* E1: sum|y - r| / sum|r| <= 1e-3   (norm-wise mean relative error; no cut-off needed)
* E2: |y - r| <= max(5e-3 * |r|, 2e-2) per element  (relative where |r| >= 4, absolute
      2e-2 where the reference is near zero; the two clauses meet at |r| = 4)
* E3: a 16-bit output equals the round-to-nearest-even cast of the same kernel's fp32
      output, bit for bit (so E1 of a bf16 result is judged on its fp32 output; a bf16
      number alone carries ~1.4e-3 mean relative rounding error).
"""
import numpy as np

from . import codecs

E1_MAX = 1e-3
E2_REL = 5e-3
E2_ABS = 2e-2


def error_stats(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    d = np.abs(y - r)
    denom = float(np.abs(r).sum())
    e1 = float(d.sum()) / denom if denom > 0 else float(d.sum())
    bound = np.maximum(E2_REL * np.abs(r), E2_ABS)
    ratio = d / bound
    big = np.abs(r) >= 4.0
    return {
        "E1": e1,
        "E2_worst_ratio": float(ratio.max()) if ratio.size else 0.0,
        "E2_fail_count": int((ratio > 1.0).sum()),
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_rel_big": float((d[big] / np.abs(r[big])).max()) if big.any() else 0.0,
        "p99_abs": float(np.percentile(d, 99)) if d.size else 0.0,
        "nonfinite": int((~np.isfinite(y)).sum()),
    }


def check_e1_e2(y, r):
    """Raises AssertionError with the statistics when E1 or E2 fails."""
    st = error_stats(y, r)
    ok = st["nonfinite"] == 0 and st["E1"] <= E1_MAX and st["E2_fail_count"] == 0
    if not ok:
        raise AssertionError(f"tolerance gates failed: {st}")
    return st


def check_e2(y, r):
    st = error_stats(y, r)
    if st["nonfinite"] or st["E2_fail_count"]:
        raise AssertionError(f"E2 gate failed: {st}")
    return st


def check_e3(out16_bits, out32, kind):
    """16-bit output bits == RNE cast of the fp32 output, for kind 'f16' or 'bf16'."""
    o32 = np.asarray(out32, dtype=np.float32).astype(np.float64)
    want = codecs.f16_bits(o32) if kind == "f16" else codecs.bf16_bits(o32)
    got = np.asarray(out16_bits, dtype=np.uint16)
    bad = int((want != got).sum())
    if bad:
        idx = np.argwhere(want != got)[0]
        raise AssertionError(f"E3 failed at {bad} elements, first {tuple(idx)}: "
                             f"got {got[tuple(idx)]:#06x} want {want[tuple(idx)]:#06x}")
    return True
