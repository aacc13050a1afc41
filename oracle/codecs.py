"""Number-format codecs of the oracle (TEST INFRASTRUCTURE ONLY).

All rounding is written out from the definition of a binary floating-point format with
``m`` explicit mantissa bits and smallest normal exponent ``emin``: a finite x is
rounded to the nearest multiple of its quantum 2**(max(e, emin) - m), where
e = floor(log2|x|), ties to the even multiple (numpy ``rint`` is round-half-even).
All arithmetic is float64, in which every step below is exact for the inputs used.

Formats (the pages name them; their bit layouts are the standard ones):
* fp16  (IEEE binary16): m=10, emin=-14, max 65504, overflow -> inf.
* bf16: m=7, emin=-126, max (2 - 2**-7) * 2**127, overflow -> inf.
* e4m3 (OCP FP8 "e4m3fn", the FP8 weight format of the FlashInfer PR #7495 analysis):
  bias 7, m=3, emin=-6, max 448, no infinities, code S.1111.111 is NaN.
* e2m1 (OCP FP4, the FP4 weight format of the FlashInfer PR #4466 analysis):
  bias 1, m=1, emin=0, values +-{0, .5, 1, 1.5, 2, 3, 4, 6}, no inf / NaN.
"""
import numpy as np

F16_MAX = 65504.0
BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def round_to_format(x, mant_bits, emin):
    """Round float64 values to the nearest value of a binary format, ties to even.

    Returns float64.  No overflow handling here (callers decide: inf or error).
    Zero maps to zero with its sign kept.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    xa = x[nz]
    _, E = np.frexp(xa)             # xa = f * 2**E, 0.5 <= |f| < 1
    e = np.maximum(E - 1, emin)      # exponent of the leading bit, clamped at emin
    quantum = np.ldexp(1.0, e - mant_bits)
    out[nz] = np.rint(xa / quantum) * quantum
    out[~nz] = x[~nz]
    return out


# ----------------------------------------------------------------------------- fp16
def f16_round(x):
    """RNE to IEEE fp16, returned as float64 (inf on overflow)."""
    r = round_to_format(x, 10, -14)
    r = np.where(np.abs(r) > F16_MAX, np.copysign(np.inf, r), r)
    return r


def f16_bits(x):
    """RNE to fp16, returned as uint16 bit patterns."""
    return f16_round(x).astype(np.float16).view(np.uint16)   # exact: already rounded


def f16_from_bits(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------- bf16
def bf16_round(x):
    r = round_to_format(x, 7, -126)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    return r


def bf16_bits(x):
    """RNE to bf16, as uint16 bit patterns (the top half of the fp32 pattern)."""
    r = bf16_round(x).astype(np.float32)        # exact: a bf16 value is an fp32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- e4m3
def e4m3_decode(codes):
    """Closed form of OCP e4m3: (-1)^S * 2^(E-7) * (1 + M/8); E == 0: 2^-6 * M/8."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x):
    """RNE to e4m3 codes; |x| must already be <= 448 (callers clamp first)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values with |x| <= 448")
    r = round_to_format(x, 3, -6)
    sign = (np.signbit(r) & (r != 0)).astype(np.int64)   # -0 is canonicalised to +0
    a = np.abs(r)
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e_unb = E - 1
    normal = a >= 2.0 ** -6
    biased = np.where(normal, e_unb + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, e_unb) - 1.0, a / 2.0 ** -6) * 8.0
    mant = np.rint(mant).astype(np.int64)          # exact integers by construction
    code = (sign << 7) | (biased.astype(np.int64) << 3) | mant
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- e2m1
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Closed form of e2m1: S.EE.M, E == 0: M * 0.5, else 2^(E-1) * (1 + M/2)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(x):
    """RNE to e2m1 codes; |x| must already be <= 6.  -0 becomes code 0."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E2M1_MAX):
        raise ValueError("e2m1_encode expects finite values with |x| <= 6")
    r = round_to_format(x, 1, 0)
    sign = (np.signbit(r) & (r != 0)).astype(np.int64)
    a = np.abs(r)
    # the 8 magnitudes are E2M1_POS in code order, so the code is the index
    idx = np.searchsorted(E2M1_POS, a)
    if np.any(E2M1_POS[np.minimum(idx, 7)] != a):
        raise AssertionError("e2m1 rounding produced a value off the grid")
    return ((sign << 3) | idx).astype(np.uint8)
