"""Acceptance gates for GEMM outputs (TEST INFRASTRUCTURE ONLY).

Low Bit Triton Kernels (lecture 034): after adding group scales the mean / max relative
error should be around 1e-3 / 5e-3, and the error should be judged as a distribution,
not only by its maximum (validation section and exercise 4).  The reading used here:

* E1: sum|y - r| / sum|r| <= 1e-3   (norm-wise mean relative error; no cut-off needed)
* E2: |y - r| <= max(5e-3 * |r|, 2e-2) per element  (relative where |r| >= 4, absolute
      2e-2 where the reference is near zero; the two clauses meet at |r| = 4)
* E3: a 16-bit output equals the round-to-nearest-even cast of the same kernel's fp32
      output, bit for bit (so E1 of a bf16 result is judged on its fp32 output; a bf16
      number alone carries ~1.4e-3 mean relative rounding error).  Both outputs must be
      finite everywhere: two NaNs would otherwise compare equal as bit patterns.

Because the validation section asks for the error distribution rather than one number,
error_stats also reports the largest relative error over the elements with |r| >= rms(r)
(where a relative error is meaningful for a zero-mean output) and the sums behind E1, so
that statistics of row chunks can be combined (combine_stats).
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
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    typical = np.abs(r) >= rms if rms > 0 else np.zeros(r.shape, dtype=bool)
    return {
        "E1": e1,
        "abs_err_sum": float(d.sum()),
        "abs_ref_sum": denom,
        "count": int(d.size),
        "max_rel_rms": float((d[typical] / np.abs(r[typical])).max()) if typical.any() else 0.0,
        "E2_worst_ratio": float(ratio.max()) if ratio.size else 0.0,
        "E2_fail_count": int((ratio > 1.0).sum()),
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_rel_big": float((d[big] / np.abs(r[big])).max()) if big.any() else 0.0,
        "p99_abs": float(np.percentile(d, 99)) if d.size else 0.0,
        "nonfinite": int((~np.isfinite(y)).sum()),
    }


def combine_stats(parts):
    """Statistics of a whole output from those of disjoint row chunks (E1 from the summed
    numerators and denominators; worst cases as maxima; p99_abs as the largest chunk p99,
    an upper bound; max_rel_rms per chunk uses that chunk's rms)."""
    num = sum(p["abs_err_sum"] for p in parts)
    den = sum(p["abs_ref_sum"] for p in parts)
    out = {"E1": num / den if den > 0 else num, "abs_err_sum": num, "abs_ref_sum": den,
           "count": sum(p["count"] for p in parts)}
    for k in ("E2_worst_ratio", "max_abs", "max_rel_big", "p99_abs", "max_rel_rms"):
        out[k] = max(p[k] for p in parts)
    for k in ("E2_fail_count", "nonfinite"):
        out[k] = sum(p[k] for p in parts)
    return out


def gates_pass(st):
    """E1 and E2 on (possibly combined) statistics, every value finite."""
    return st["nonfinite"] == 0 and st["E1"] <= E1_MAX and st["E2_fail_count"] == 0


def check_e1_e2(y, r):
    """Raises AssertionError with the statistics when E1 or E2 fails."""
    st = error_stats(y, r)
    if not gates_pass(st):
        raise AssertionError(f"tolerance gates failed: {st}")
    return st


def check_e2(y, r):
    st = error_stats(y, r)
    if st["nonfinite"] or st["E2_fail_count"]:
        raise AssertionError(f"E2 gate failed: {st}")
    return st


def check_e3(out16_bits, out32, kind):
    """16-bit output bits == RNE cast of the fp32 output, for kind 'f16' or 'bf16'; every
    value of both outputs must be finite (a NaN in both would otherwise pass)."""
    o32 = np.asarray(out32, dtype=np.float32).astype(np.float64)
    got = np.asarray(out16_bits, dtype=np.uint16)
    v16 = codecs.f16_from_bits(got) if kind == "f16" else codecs.bf16_from_bits(got)
    n32, n16 = int((~np.isfinite(o32)).sum()), int((~np.isfinite(v16)).sum())
    if n32 or n16:
        raise AssertionError(f"E3 failed: {n32} non-finite fp32 and {n16} non-finite 16-bit outputs")
    want = codecs.f16_bits(o32) if kind == "f16" else codecs.bf16_bits(o32)
    bad = int((want != got).sum())
    if bad:
        idx = np.argwhere(want != got)[0]
        raise AssertionError(f"E3 failed at {bad} elements, first {tuple(idx)}: "
                             f"got {got[tuple(idx)]:#06x} want {want[tuple(idx)]:#06x}")
    return True
