"""Quantizers and canonical packing of the oracle (TEST INFRASTRUCTURE ONLY).

Weights are handled in the "nt" orientation of the BitBLAS problem descriptor
(Bitblas lecture 033, API example: ``layout="nt"``) and of the FP4 preparation step
(FlashInfer PR #4466 analysis, section 2: the weight is ``[n, k/2]``): row n of ``wt``
holds column n of the logical W[K, N], i.e. ``wt[n, k] = W[k, n]``.

Readings where the pages are silent (each is listed in the design notes):
* rounding is round-half-even everywhere, divisions are done in float64 and rounded
  once to the target format;
* the quantizer divides by the *stored* (already rounded) scale, so that dequantizing
  the stored codes and scales is self-consistent;
* an all-zero INT4 group gets scale 0 and codes 8 (signed 0), an all-zero INT2 group scale 0
  and codes 2, an all-zero NF4 group scale 0 and the code of the book's 0; an all-zero FP4 block gets scale code 0 and codes 0; an all-zero FP8 tensor
  gets alpha 0 and codes 0.
"""
import numpy as np

from . import codecs


# ----------------------------------------------------------------------------- INT4
def quantize_int4(wt, group_size):
    """Symmetric absmax INT4 per (K-group, column).

    Low Bit Triton Kernels (lecture 034), core pattern: one scale per group of
    ``group_size`` consecutive K, group 128 being the common choice; gemlite snippet:
    the stored nibble is the signed value + 8.  The scale is absmax / 7 rounded to
    fp16, the code is clamp(rint(w / s), -8, 7) + 8.

    wt: float32 [N, K].  Returns (codes uint8 [N, K] in 0..15, scale_bits uint16 [K/G, N]).
    """
    wt = np.asarray(wt, dtype=np.float32)
    N, K = wt.shape
    G = int(group_size)
    if K % G:
        raise ValueError("K must be a multiple of group_size")
    w = wt.astype(np.float64).reshape(N, K // G, G)
    amax = np.abs(w).max(axis=2)                        # [N, K/G]
    s = codecs.f16_round(amax / 7.0)                    # stored scale value
    safe = np.where(s == 0, 1.0, s)
    q = np.clip(np.rint(w / safe[:, :, None]), -8, 7)
    q = np.where(s[:, :, None] == 0, 0.0, q)
    codes = (q + 8).astype(np.uint8).reshape(N, K)
    scale_bits = codecs.f16_bits(s).T.copy()            # [K/G, N]
    return codes, scale_bits


# ----------------------------------------------------------------------------- INT2 (W2A16)
def quantize_int2(wt, group_size):
    """Symmetric absmax INT2 per (K-group, column): the W2A16 combination of the Bitblas
    lecture (033, exercises: "W2A16 (INT2 weight)") with the INT4 recipe carried over to
    2 bits.  Signed range [-2, 1], stored code = signed + 2 (as the nibble is signed + 8);
    the scale is absmax / (2^(2-1) - 1) = absmax rounded to fp16 (INT4's absmax / 7 is
    absmax / (2^(4-1) - 1)); code = clamp(rint(w / s), -2, 1) + 2.  Like -8 for INT4, -2
    is never emitted by the absmax scale.

    wt: float32 [N, K].  Returns (codes uint8 [N, K] in 0..3, scale_bits uint16 [K/G, N]).
    """
    wt = np.asarray(wt, dtype=np.float32)
    N, K = wt.shape
    G = int(group_size)
    if K % G:
        raise ValueError("K must be a multiple of group_size")
    w = wt.astype(np.float64).reshape(N, K // G, G)
    amax = np.abs(w).max(axis=2)                        # [N, K/G]
    s = codecs.f16_round(amax / 1.0)                    # stored scale value
    safe = np.where(s == 0, 1.0, s)
    q = np.clip(np.rint(w / safe[:, :, None]), -2, 1)
    q = np.where(s[:, :, None] == 0, 0.0, q)
    codes = (q + 2).astype(np.uint8).reshape(N, K)
    scale_bits = codecs.f16_bits(s).T.copy()            # [K/G, N]
    return codes, scale_bits


# ----------------------------------------------------------------------------- NF4
NF4_DELTA = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_codebook():
    """The NormalFloat-4 code book as fp16 values (float64 [16], ascending).

    Low Bit Triton Kernels (lecture 034) names NF4 as the non-uniform choice of the 16
    values a 4-bit weight can take, read through a table held in registers; the pages give
    no values.  Reading: QLoRA's construction -- quantiles of the standard normal at evenly
    spaced probabilities, 8 for the positive half (from delta down to, not including, 1/2)
    and 7 for the negative half, plus an exact zero, divided by the largest so the book
    spans [-1, 1]; delta = ((1 - 1/30) + (1 - 1/32)) / 2 lies between the outermost quantile
    estimates of a 15- and a 16-point grid.  Each value is then rounded to fp16, the type
    the book is stored in.
    """
    from scipy.special import ndtri
    pos = ndtri(np.linspace(NF4_DELTA, 0.5, 9)[:-1])      # 8 values, largest first
    neg = -ndtri(np.linspace(NF4_DELTA, 0.5, 8)[:-1])     # 7 values, most negative first
    v = np.sort(np.concatenate([neg, [0.0], pos]))
    return codecs.f16_round(v / v.max())


def quantize_nf4(wt, group_size, book=None):
    """NF4 per (K-group, column): s = RNE_fp16(absmax) (the book spans [-1, 1]), code = index
    of the book entry nearest to w / s, ties to the lower index; all-zero group: s = 0 and
    the code of the entry 0 (7 in the NF4 book).

    wt: float32 [N, K]; book: fp16 values [16] (default: nf4_codebook()).
    Returns (codes uint8 [N, K] in 0..15, scale_bits uint16 [K/G, N], book_bits uint16 [16]).
    """
    wt = np.asarray(wt, dtype=np.float32)
    N, K = wt.shape
    G = int(group_size)
    if K % G:
        raise ValueError("K must be a multiple of group_size")
    book = nf4_codebook() if book is None else np.asarray(book, dtype=np.float64)
    zero_code = int(np.argmin(np.abs(book)))
    w = wt.astype(np.float64).reshape(N, K // G, G)
    s = codecs.f16_round(np.abs(w).max(axis=2))           # [N, K/G]
    safe = np.where(s == 0, 1.0, s)
    x = w / safe[:, :, None]
    codes = np.argmin(np.abs(x[..., None] - book), axis=-1)   # first minimum: lower index
    codes = np.where(s[:, :, None] == 0, zero_code, codes)
    return (codes.astype(np.uint8).reshape(N, K), codecs.f16_bits(s).T.copy(),
            codecs.f16_bits(book).astype(np.uint16))


# ----------------------------------------------------------------------------- FP8
def quantize_fp8(wt):
    """Per-tensor FP8 e4m3 (FlashInfer PR #7495 analysis, introduction).

    alpha = absmax / 448 rounded to fp32; code = e4m3(clamp(w / alpha, +-448)).
    Returns (codes uint8 [N, K], alpha as a Python float that is an fp32 value).
    """
    w = np.asarray(wt, dtype=np.float32).astype(np.float64)
    amax = float(np.abs(w).max()) if w.size else 0.0
    alpha = float(np.float32(amax / 448.0))
    if alpha == 0.0:
        return np.zeros(w.shape, np.uint8), 0.0
    x = np.clip(w / alpha, -codecs.E4M3_MAX, codecs.E4M3_MAX)
    return codecs.e4m3_encode(x), alpha


# ----------------------------------------------------------------------------- FP4
def quantize_fp4(wt):
    """FP4 e2m1 with an e4m3 scale per 16 consecutive K and one fp32 alpha.

    The pages give only the operands (FlashInfer PR #4466 analysis, section 2: weight,
    per-block descale, optional alpha); the recipe is the plainest two-level absmax:
      alpha = absmax(W) / (6 * 448)                  (rounded to fp32)
      s_b   = e4m3(min(absmax_b / (6 * alpha), 448))  per (n, block of 16 k)
      code  = e2m1(clamp(w / (s_b * alpha), +-6)),    code 0 where s_b == 0.
    Returns (codes uint8 [N, K] in 0..15, sf codes uint8 [N, K/16], alpha float).
    """
    w = np.asarray(wt, dtype=np.float32).astype(np.float64)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    amax = float(np.abs(w).max()) if w.size else 0.0
    alpha = float(np.float32(amax / (6.0 * 448.0)))
    wb = w.reshape(N, K // 16, 16)
    if alpha == 0.0:
        return np.zeros((N, K), np.uint8), np.zeros((N, K // 16), np.uint8), 0.0
    bmax = np.abs(wb).max(axis=2)
    sf_codes = codecs.e4m3_encode(np.minimum(bmax / (6.0 * alpha), codecs.E4M3_MAX))
    sb = codecs.e4m3_decode(sf_codes)                  # stored block scale
    denom = sb * alpha                                  # exact in float64
    safe = np.where(denom == 0, 1.0, denom)
    x = np.clip(wb / safe[:, :, None], -codecs.E2M1_MAX, codecs.E2M1_MAX)
    x = np.where(denom[:, :, None] == 0, 0.0, x)
    codes = codecs.e2m1_encode(x).reshape(N, K)
    return codes, sf_codes.astype(np.uint8), alpha


# ----------------------------------------------------------------------------- canonical packing
def pack_nibbles(codes):
    """Two 4-bit codes per byte along K, low nibble = even k (two per byte, low first).

    codes uint8 [N, K] (values 0..15) -> uint8 [N, K/2].
    """
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[1] % 2:
        raise ValueError("K must be even")
    if np.any(c > 15):
        raise ValueError("nibble codes must be < 16")
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles: uint8 [N, K/2] -> codes uint8 [N, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def int4_signed(codes):
    """Signed INT4 value of a stored nibble: nibble - 8 (gemlite snippet, lecture 034)."""
    return np.asarray(codes, dtype=np.int64) - 8


def pack_crumbs(codes):
    """Four 2-bit codes per byte along K, the lowest k in the lowest bits (INT2 canonical).

    codes uint8 [N, K] (values 0..3) -> uint8 [N, K/4].
    """
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[1] % 4:
        raise ValueError("K must be a multiple of 4")
    if np.any(c > 3):
        raise ValueError("2-bit codes must be < 4")
    return (c[:, 0::4] | (c[:, 1::4] << 2) | (c[:, 2::4] << 4) | (c[:, 3::4] << 6)).astype(np.uint8)


def unpack_crumbs(packed):
    """Inverse of pack_crumbs: uint8 [N, K/4] -> codes uint8 [N, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 4), np.uint8)
    for i in range(4):
        out[:, i::4] = (p >> (2 * i)) & 3
    return out


def int2_signed(codes):
    """Signed INT2 value of a stored 2-bit code: code - 2."""
    return np.asarray(codes, dtype=np.int64) - 2
