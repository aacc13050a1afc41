"""Dequantization and the fp64 reference GEMM (TEST INFRASTRUCTURE ONLY).

The method's result has a plain definition: out = A . dequant(W) (times alpha for the
formats that carry one), so the reference is that definition written out.  Dequantized
weights are formed in float32 (every product below is exact in float32), the matmul
accumulates in float64 (numpy BLAS dgemm, a library primitive), and alpha multiplies the
float64 result, as the FP8 analysis prescribes applying the per-tensor scale to the
accumulator (FlashInfer PR #7495 analysis, introduction).
"""
import numpy as np

from . import codecs


def dequant_int4(codes, scale_bits, group_size):
    """(nibble - 8) * s  in float32, exact.  codes [N, K], scale_bits uint16 [K/G, N].

    Low Bit Triton Kernels (lecture 034), gemlite snippet: subtract 8, multiply by the
    scale of group k // group_size of the same column.  Returns float32 [N, K].
    """
    q = np.asarray(codes, dtype=np.int64) - 8
    s = codecs.f16_from_bits(scale_bits)               # [K/G, N]
    s_nk = np.repeat(s.T, group_size, axis=1)          # [N, K]
    return (q * s_nk).astype(np.float32)


def dequant_int4_f16(codes, scale_bits, group_size):
    """The 16-bit operand the gemlite snippet forms: RNE_fp16((nibble - 8) * s).

    The snippet converts the signed nibble to fp16 and multiplies by the fp16 scale,
    so the tile it feeds to the matrix unit is the fp16 rounding of the exact product.
    Returns float64 values of fp16 numbers, [N, K].
    """
    return codecs.f16_round(dequant_int4(codes, scale_bits, group_size).astype(np.float64))


def dequant_int2(codes, scale_bits, group_size):
    """(code - 2) * s in float32, exact.  codes [N, K] in 0..3, scale_bits uint16 [K/G, N].

    The INT2 (W2A16) counterpart of dequant_int4: signed value code - 2 times the scale of
    group k // group_size of the same column.  The product has at most 12 significant bits
    and |code - 2| <= 2, so it is also exact in fp16: the 16-bit operand equals it.
    """
    q = np.asarray(codes, dtype=np.int64) - 2
    s = codecs.f16_from_bits(scale_bits)               # [K/G, N]
    s_nk = np.repeat(s.T, group_size, axis=1)          # [N, K]
    return (q * s_nk).astype(np.float32)


def dequant_nf4(codes, scale_bits, group_size, book_bits):
    """T[code] * s in float32, exact (two fp16 values: at most 22 significant bits).

    codes [N, K] in 0..15, scale_bits uint16 [K/G, N], book_bits uint16 [16] (the fp16 code
    book).  The non-uniform 4-bit grid of Low Bit Triton Kernels (lecture 034): the code
    indexes the book, the group scale multiplies the entry.  Returns float32 [N, K].
    """
    t = codecs.f16_from_bits(book_bits)[np.asarray(codes, dtype=np.int64)]
    s = codecs.f16_from_bits(scale_bits)               # [K/G, N]
    s_nk = np.repeat(s.T, group_size, axis=1)          # [N, K]
    return (t * s_nk).astype(np.float32)


def dequant_nf4_f16(codes, scale_bits, group_size, book_bits):
    """The fp16 operand of an NF4 tile: RNE_fp16(T[code] * s), as INT4's RNE_fp16((n - 8) s).
    Returns float64 values of fp16 numbers, [N, K]."""
    return codecs.f16_round(dequant_nf4(codes, scale_bits, group_size, book_bits).astype(np.float64))


def dequant_fp8(codes):
    """e4m3 code -> value (exact); alpha is NOT applied here.  Returns float32 [N, K].

    The same values serve fp16 and bf16 activations (mm_fp16_fp8 and mm_bf16_fp8): every
    e4m3 value is exact in both 16-bit formats."""
    return codecs.e4m3_decode(codes).astype(np.float32)


def dequant_fp4(codes, sf_codes):
    """e2m1 code * e4m3 block scale (exact: 2 x 4 significant bits); alpha not applied."""
    v = codecs.e2m1_decode(codes)                      # [N, K]
    s = codecs.e4m3_decode(sf_codes)                   # [N, K/16]
    return (v * np.repeat(s, 16, axis=1)).astype(np.float32)


def gemm_fp64(a_values, wdq_nk, alpha=1.0, bias=None):
    """R = (A . Wdq^T) * alpha (+ bias[n]) in float64.  a_values [M, K], wdq_nk [N, K].

    The bias is the optional bias argument of mm_bf16_fp8 / mm_fp16_fp8 (FlashInfer PR
    #7495 analysis, section 2), one value per output column, added after alpha.
    """
    a = np.asarray(a_values, dtype=np.float64)
    w = np.asarray(wdq_nk, dtype=np.float64)
    r = (a @ w.T) * float(alpha)
    if bias is not None:
        r = r + np.asarray(bias, dtype=np.float64)[None, :]
    return r


def gemm_fp64_rows(a_values, wdq_nk, rows, alpha=1.0, bias=None):
    """Reference for a subset of output rows (sampled checks at full size)."""
    a = np.asarray(a_values, dtype=np.float64)[np.asarray(rows)]
    return gemm_fp64(a, wdq_nk, alpha, bias)
