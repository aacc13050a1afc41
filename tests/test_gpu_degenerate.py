"""Degenerate inputs of the method on the GPU: weight groups that quantize to a zero scale
(pruned columns and single all-zero groups, as a pruned layer has them) and non-finite
activations.

* Zero groups: every format's quantizer gives such a group a zero scale (INT4 / INT2 / NF4
  group scale, FP4 block scale) or zero codes (FP8), which dequantize to exact zeros; the
  output is compared with the oracle element by element on every launch path.
* Non-finite activations: out[m, :] depends on A row m only, so a NaN or an infinity in
  row m of A must reach row m of the output and no other.  In such a row each element is
  fixed by IEEE arithmetic whatever the summation order: NaN if any product is NaN
  (a NaN activation, or an infinity times an exact zero weight), else the infinity of the
  products' common sign, else NaN (infinities of both signs).  The expected pattern is formed
  from the oracle's dequantized weights with elementwise fp64 products (no BLAS), and both
  output types must match it exactly; the finite rows pass the usual error gates.  An
  infinity that meets a zero-scale group must give NaN there, which also pins the zero
  groups to exact zeros in the kernel's dequantization."""
import numpy as np
import pytest

import synthetic
from gpu_cases import SIGMA, Prepared, a_values, out16_dtype, out16_kind, out16_values, run_gpu, say
from oracle import reference, tolerance

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_qgemm_amd as lib
    return lib


# (format, M, N, K, G, kernel_hint, split_k_hint, tile_hint)
CASES = [
    ("int4", 1, 512, 1024, 128, 1, 0, 0),      # decode, one row
    ("int4", 16, 512, 2048, 32, 1, 2, 0),      # decode, split K
    ("nf4", 5, 256, 1024, 64, 1, 0, 0),        # decode, NF4 table
    ("fp8", 40, 1024, 1024, 0, 2, 0, 64),      # 64 x 128 tile
    ("fp4", 200, 1024, 2048, 0, 2, 2, 128),    # 128 x 128 tile, split 2
    ("int2", 300, 512, 1024, 128, 2, 0, 256),  # 256 x 256 tile
    ("fp8h", 70, 512, 1024, 0, 3, 0, 64),      # persistent stream-K
    ("nf4", 100, 1024, 2048, 64, 4, 2, 0),     # transform waves, split 2
]


def _zeroed_weights(fmt, N, K, G, key):
    """Seeded weights with zero columns (pruned outputs) and single zero groups."""
    w = synthetic.weights(N, K, SIGMA[fmt], key)
    g = G if G else 16 if fmt == "fp4" else 128
    r = np.random.default_rng(list(key) + [9])
    w[r.choice(N, size=max(1, N // 16), replace=False), :] = 0.0
    for _ in range(max(4, N // 8)):
        n, b = int(r.integers(0, N)), int(r.integers(0, K // g))
        w[n, b * g:(b + 1) * g] = 0.0
    return w


def _ieee_rows(a_rows, wdq, alpha):
    """Elementwise fp64 products summed per output (IEEE special values, no BLAS)."""
    w = np.asarray(wdq, dtype=np.float64)
    out = np.empty((a_rows.shape[0], w.shape[0]))
    with np.errstate(invalid="ignore", over="ignore"):
        for i, a in enumerate(a_rows):
            out[i] = (a[None, :] * w).sum(axis=1) * float(alpha)
    return out


def _same_special_pattern(y, r):
    """Every element of y non-finite exactly where r is, NaN where r is NaN, and the same
    infinity where r is infinite."""
    if not np.array_equal(np.isnan(y), np.isnan(r)):
        return False
    inf = np.isinf(r)
    return bool(np.array_equal(np.isinf(y), inf) and np.array_equal(y[inf], r[inf]))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_zero_groups_and_nonfinite_activations(q, ci):
    fmt, M, N, K, G, hint, split, tile = CASES[ci]
    say(f"case degenerate#{ci} fmt={fmt} M={M} N={N} K={K} G={G} hint={hint} split={split} tile={tile}")
    key = (74, ci)
    prep = Prepared(q, fmt, N, K, G, key, weights=_zeroed_weights(fmt, N, K, G, key))
    kind = out16_kind(fmt)

    # 1. zero groups alone: every element against the oracle
    A = synthetic.activations(M, K, kind, (74, ci, M))
    y32, ws = run_gpu(q, prep, A, q.DT_F32, hint, split, tile_hint=tile)
    y16, _ = run_gpu(q, prep, A, out16_dtype(q, fmt), hint, split, ws, tile)
    r = reference.gemm_fp64(a_values(A), prep.wdq, prep.alpha)
    st = tolerance.error_stats(y32, r)
    assert tolerance.gates_pass(st), st
    st16 = tolerance.error_stats(out16_values(y16, fmt), r)
    assert not st16["nonfinite"] and not st16["E2_fail_count"], st16
    tolerance.check_e3(y16, y32.astype(np.float32), kind)

    # 2. non-finite activations: NaN, +inf, -inf, and +inf with -inf in one row
    Ab = A.clone()
    special = {0: [(3, float("nan"))], M // 2: [(K // 3, float("inf"))], M - 1: [(K - 1, float("-inf"))],
               (M // 2 + 1) % M: [(1, float("inf")), (K // 2, float("-inf"))]}
    for m, entries in special.items():
        for k, v in entries:
            Ab[m, k] = v
    bad = sorted(special)
    good = np.setdiff1d(np.arange(M), bad)
    z32, ws = run_gpu(q, prep, Ab, q.DT_F32, hint, split, tile_hint=tile)
    z16, _ = run_gpu(q, prep, Ab, out16_dtype(q, fmt), hint, split, ws, tile)
    z16v = out16_values(z16, fmt)
    a = a_values(Ab)
    if len(good):
        assert np.isfinite(z32[good]).all() and np.isfinite(z16v[good]).all(), "a non-finite value left its row"
        st = tolerance.error_stats(z32[good], reference.gemm_fp64(a[good], prep.wdq, prep.alpha))
        assert tolerance.gates_pass(st), st
    want = _ieee_rows(a[bad], prep.wdq, prep.alpha)
    assert _same_special_pattern(z32[bad], want), "fp32 output: non-finite pattern differs from the oracle"
    assert _same_special_pattern(z16v[bad], want), "16-bit output: non-finite pattern differs from the oracle"
    # an infinity against an all-zero column is NaN there: the zero groups dequantize to exact zeros
    zero_cols = np.flatnonzero(~np.asarray(prep.wdq, dtype=np.float64).any(axis=1))
    assert len(zero_cols) and np.isnan(z32[M // 2, zero_cols]).all()
