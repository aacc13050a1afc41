"""Model of the packed device layout (TEST INFRASTRUCTURE ONLY).

An independent numpy statement of the index map that the library's packer must
produce; written from the layout specification, sharing no code with the packer.

The specification targets the operand fragment of the gfx950 16x16x32 MFMA: in a
64-lane wavefront, lane l supplies column (or row) ``l & 15`` and the 8 consecutive
K values ``8 * (l >> 4) + j``, j = 0..7, of each 32-wide K step.  Each weight block is
exactly what one wavefront loads with one 16-byte load per lane, so a lane's 16 bytes
are its operand registers with no LDS re-layout in between (the Bitblas lecture 033,
layout section, attributes more than half the runtime to such a re-layout when the
fragment order is wrong).

INT4 (w_dtype INT4) and FP4 (w_dtype FP4_E2M1) weights
    block (nb, kb) = columns 16*nb .. 16*nb+15, k = 128*kb .. 128*kb+127, 1024 bytes,
    blocks ordered nb-major: block index = nb * (K/128) + kb.
    Inside a block, lane l owns bytes [16*l, 16*l + 16): dword t (t = 0..3) holds the
    8 nibbles of column n = 16*nb + (l & 15) at k = 128*kb + 32*t + 8*(l >> 4) + J[s]
    for nibble slot s = 0..7 (slot s = bits 4s .. 4s+3 of the little-endian dword).
      INT4: J = (0, 2, 4, 6, 1, 3, 5, 7)
      FP4 : J = (0, 1, 2, 3, 4, 5, 6, 7)
      NF4 : J = (0, 4, 1, 5, 2, 6, 3, 7)  (byte b: k offsets b and b + 4, the order in which
            a byte-wise table lookup yields fp16 pairs (k, k+1) with one byte shuffle)
INT2 (w_dtype INT2) weights
    block (nb, kb) = columns 16*nb .. 16*nb+15, k = 128*kb .. 128*kb+127, 512 bytes, block
    index nb * (K/128) + kb.  Lane l owns bytes [8*l, 8*l + 8): dword d (d = 0..1) holds 16
    2-bit codes; the code at bits 16*h + 8*b + 2*f (h, b = 0..1, f = 0..3) is column
    16*nb + (l & 15) at k = 128*kb + 32*(2*d + b) + 8*(l >> 4) + 2*f + h.  So byte b of
    either 16-bit half carries K step 2d + b, field f of it the k pair (2f, 2f + 1) with
    the even k in the low half: a mask of the field and an OR of an fp16 exponent give an
    fp16 pair 2^(10 - 2f) + code with no shift but the one for b = 1.
FP8 weights
    block (nb, kb) = 16 columns x 64 k, 1024 bytes, block index nb * (K/64) + kb;
    lane l owns 16 bytes: byte 8*t + j (t = 0..1, j = 0..7) is column 16*nb + (l & 15),
    k = 64*kb + 32*t + 8*(l >> 4) + j.
NF4 scales
    a 256-byte header, then the INT4 scale layout.  Header byte c (0..15) = low byte of the
    fp16 code-book entry T[c], byte 16 + c = its high byte, bytes 32..255 = 0.
INT4 and INT2 scales (fp16)
    span = max(G, 128); T = max(1, 128 / G) scales per (column, span).
    Element index ((nb * (K/span) + kb) * 16 + c) * T + t holds the scale of column
    16*nb + c for group  kb * (span / G) + t.
FP4 block scales (e4m3 bytes)
    Byte index ((nb * (K/128) + kb) * 16 + c) * 8 + 4*h + t holds the scale of column
    16*nb + c for 16-k block  8*kb + 2*t + h  (h = 0..1, t = 0..3), so that lane l
    reads one dword at ((l & 15) * 2 + (l >> 5)) * 4 with the scale of K step t in byte t.
"""
import numpy as np

J_INT4 = (0, 2, 4, 6, 1, 3, 5, 7)
J_FP4 = (0, 1, 2, 3, 4, 5, 6, 7)
J_NF4 = (0, 4, 1, 5, 2, 6, 3, 7)
LUT_HEADER_BYTES = 256


def _nibble_positions(N, K, J):
    """For every packed nibble position, the (n, k) it holds.

    Returns (n, k) int64 arrays of shape [N/16, K/128, 64 lanes, 4 dwords, 8 slots];
    the packed byte of a position is  block*1024 + 16*lane + 4*t + slot//2.
    """
    assert N % 16 == 0 and K % 128 == 0
    nb = np.arange(N // 16)[:, None, None, None, None]
    kb = np.arange(K // 128)[None, :, None, None, None]
    l = np.arange(64)[None, None, :, None, None]
    t = np.arange(4)[None, None, None, :, None]
    s = np.arange(8)[None, None, None, None, :]
    n = 16 * nb + (l & 15) + 0 * (kb + t + s)
    k = 128 * kb + 32 * t + 8 * (l >> 4) + np.asarray(J)[s] + 0 * nb
    return n, k


def _nibble_layout(codes, J):
    """codes uint8 [N, K] (0..15) -> packed bytes per the 4-bit block spec."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    n, k = _nibble_positions(N, K, J)
    nib = codes[n, k]                                  # [NB, KB, 64, 4, 8]
    lo, hi = nib[..., 0::2], nib[..., 1::2]            # slot 2i -> low, 2i+1 -> high
    return (lo | (hi << 4)).astype(np.uint8).reshape(-1)


def _nibble_unlayout(packed, N, K, J):
    packed = np.asarray(packed, dtype=np.uint8).reshape(N // 16, K // 128, 64, 4, 4)
    nib = np.empty(packed.shape[:-1] + (8,), np.uint8)
    nib[..., 0::2] = packed & 0xF
    nib[..., 1::2] = packed >> 4
    n, k = _nibble_positions(N, K, J)
    codes = np.zeros((N, K), np.uint8)
    codes[n, k] = nib
    return codes


def device_int4_weights(codes):
    return _nibble_layout(codes, J_INT4)


def device_int4_weights_inverse(packed, N, K):
    return _nibble_unlayout(packed, N, K, J_INT4)


def device_fp4_weights(codes):
    return _nibble_layout(codes, J_FP4)


def device_fp4_weights_inverse(packed, N, K):
    return _nibble_unlayout(packed, N, K, J_FP4)


def _int2_positions(N, K):
    """(n, k) of every packed 2-bit code, shape [N/16, K/128, 64 lanes, 2 dwords, 2 halves,
    2 bytes, 4 fields]; its bit position is 16*h + 8*b + 2*f of dword d."""
    assert N % 16 == 0 and K % 128 == 0
    sh = (N // 16, K // 128, 64, 2, 2, 2, 4)
    nb = np.arange(N // 16).reshape(-1, 1, 1, 1, 1, 1, 1)
    kb = np.arange(K // 128).reshape(1, -1, 1, 1, 1, 1, 1)
    l = np.arange(64).reshape(1, 1, -1, 1, 1, 1, 1)
    d = np.arange(2).reshape(1, 1, 1, -1, 1, 1, 1)
    h = np.arange(2).reshape(1, 1, 1, 1, -1, 1, 1)
    b = np.arange(2).reshape(1, 1, 1, 1, 1, -1, 1)
    f = np.arange(4).reshape(1, 1, 1, 1, 1, 1, -1)
    n = np.broadcast_to(16 * nb + (l & 15), sh)
    k = np.broadcast_to(128 * kb + 32 * (2 * d + b) + 8 * (l >> 4) + 2 * f + h, sh)
    return n, k


def device_int2_weights(codes):
    """codes uint8 [N, K] (0..3) -> packed bytes per the INT2 block spec."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    n, k = _int2_positions(N, K)
    c = codes[n, k].astype(np.uint32)                  # [NB, KB, 64, 2, 2(h), 2(b), 4(f)]
    h = np.arange(2).reshape(1, 1, 1, 1, -1, 1, 1)
    b = np.arange(2).reshape(1, 1, 1, 1, 1, -1, 1)
    f = np.arange(4).reshape(1, 1, 1, 1, 1, 1, -1)
    dword = (c << (16 * h + 8 * b + 2 * f).astype(np.uint32)).sum(axis=(4, 5, 6)).astype(np.uint32)
    return dword.astype("<u4").view(np.uint8).reshape(-1)


def device_int2_weights_inverse(packed, N, K):
    dw = np.asarray(packed, dtype=np.uint8).view("<u4").reshape(N // 16, K // 128, 64, 2)
    h = np.arange(2).reshape(1, 1, 1, 1, -1, 1, 1)
    b = np.arange(2).reshape(1, 1, 1, 1, 1, -1, 1)
    f = np.arange(4).reshape(1, 1, 1, 1, 1, 1, -1)
    c = (dw[..., None, None, None] >> (16 * h + 8 * b + 2 * f).astype(np.uint32)) & 3
    n, k = _int2_positions(N, K)
    codes = np.zeros((N, K), np.uint8)
    codes[n, k] = c.astype(np.uint8)
    return codes


def _fp8_positions(N, K):
    """(n, k) of every packed FP8 byte, shape [N/16, K/64, 64 lanes, 2, 8]."""
    assert N % 16 == 0 and K % 64 == 0
    nb = np.arange(N // 16)[:, None, None, None, None]
    kb = np.arange(K // 64)[None, :, None, None, None]
    l = np.arange(64)[None, None, :, None, None]
    t = np.arange(2)[None, None, None, :, None]
    j = np.arange(8)[None, None, None, None, :]
    n = 16 * nb + (l & 15) + 0 * (kb + t + j)
    k = 64 * kb + 32 * t + 8 * (l >> 4) + j + 0 * nb
    return n, k


def device_fp8_weights(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = _fp8_positions(*codes.shape)
    return codes[n, k].reshape(-1)


def device_fp8_weights_inverse(packed, N, K):
    n, k = _fp8_positions(N, K)
    codes = np.zeros((N, K), np.uint8)
    codes[n, k] = np.asarray(packed, dtype=np.uint8).reshape(n.shape)
    return codes


def device_int4_scales(scale_bits, N, K, G):
    """scale_bits uint16 [K/G, N] -> packed uint16 per the INT4 scale spec."""
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    span = max(G, 128)
    T = max(1, 128 // G)
    nb = np.arange(N // 16)[:, None, None, None]
    kb = np.arange(K // span)[None, :, None, None]
    c = np.arange(16)[None, None, :, None]
    t = np.arange(T)[None, None, None, :]
    g = kb * (span // G) + t + 0 * (nb + c)
    n = 16 * nb + c + 0 * (kb + t)
    return scale_bits[g, n].reshape(-1)


def device_fp4_scales(sf_codes, N, K):
    """sf_codes uint8 [N, K/16] -> packed bytes per the FP4 scale spec."""
    sf_codes = np.asarray(sf_codes, dtype=np.uint8)
    nb = np.arange(N // 16)[:, None, None, None, None]
    kb = np.arange(K // 128)[None, :, None, None, None]
    c = np.arange(16)[None, None, :, None, None]
    h = np.arange(2)[None, None, None, :, None]
    t = np.arange(4)[None, None, None, None, :]
    n = 16 * nb + c + 0 * (kb + h + t)
    blk = 8 * kb + 2 * t + h + 0 * (nb + c)
    return sf_codes[n, blk].reshape(-1)


def device_nf4_weights(codes):
    return _nibble_layout(codes, J_NF4)


def device_nf4_weights_inverse(packed, N, K):
    return _nibble_unlayout(packed, N, K, J_NF4)


def device_nf4_scales(book_bits, scale_bits, N, K, G):
    """book_bits uint16 [16], scale_bits uint16 [K/G, N] -> packed bytes per the NF4 scale spec."""
    book = np.asarray(book_bits, dtype=np.uint16)
    head = np.zeros(LUT_HEADER_BYTES, np.uint8)
    head[:16] = book & 0xFF
    head[16:32] = book >> 8
    body = device_int4_scales(scale_bits, N, K, G).astype("<u2").view(np.uint8)
    return np.concatenate([head, body])
