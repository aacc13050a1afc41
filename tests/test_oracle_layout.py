"""Pins of the device-layout model: hand-computed single-hot placements and round trips."""
import numpy as np
import pytest

from oracle import layout


@pytest.mark.parametrize("n,k,byte,shift", [
    # INT4, N=32, K=256 (K/128 = 2 blocks per column block)
    # (n=0,k=0): nb0 kb0 lane0 t0 J-slot0 -> byte 0, low nibble
    (0, 0, 0, 0),
    # (n=0,k=1): slot 4 (J[4]=1) -> byte 2, low nibble
    (0, 1, 2, 0),
    # (n=0,k=2): slot 1 -> byte 0, high nibble
    (0, 2, 0, 4),
    # (n=5,k=8): lane = 5 + 16*1 = 21, t0, slot0 -> byte 16*21 = 336
    (5, 8, 336, 0),
    # (n=17,k=130): nb1 kb1 -> block 3, base 3072; lane 1, t0, J=2 -> slot 1 -> byte 3072+16
    (17, 130, 3072 + 16, 4),
    # (n=31,k=255): nb1 kb1 block 3; k-128=127 = 32*3 + 8*3 + 7 -> t3, lane 15+48=63, J=7 -> slot 7
    (31, 255, 3072 + 16 * 63 + 12 + 3, 4),
])
def test_int4_single_hot(n, k, byte, shift):
    codes = np.zeros((32, 256), np.uint8)
    codes[n, k] = 0xB
    p = layout.device_int4_weights(codes)
    nz = np.flatnonzero(p)
    assert list(nz) == [byte]
    assert p[byte] == 0xB << shift


@pytest.mark.parametrize("n,k,byte,shift", [
    (0, 1, 0, 4),                  # FP4 keeps k order: k=1 -> slot 1 -> byte 0 high
    (3, 9, 16 * (3 + 16), 4),      # lane 19, t0, j=1
    # n=16 -> nb1, c=0; k=200 -> kb1, 72 = 32*2 + 8*1 + 0 -> t2, lane 0+16, j0
    (16, 200, 3072 + 16 * 16 + 4 * 2, 0),
])
def test_fp4_single_hot(n, k, byte, shift):
    codes = np.zeros((32, 256), np.uint8)
    codes[n, k] = 0x9
    p = layout.device_fp4_weights(codes)
    assert list(np.flatnonzero(p)) == [byte]
    assert p[byte] == 0x9 << shift


def test_fp8_single_hot():
    codes = np.zeros((32, 128), np.uint8)
    # n=18 -> nb1, c=2; k=100 -> kb1 (64-wide), r=36 = 32*1 + 8*0 + 4 -> t1, lane 2, j4
    codes[18, 100] = 0x5A
    p = layout.device_fp8_weights(codes)
    base = (1 * 2 + 1) * 1024
    assert list(np.flatnonzero(p)) == [base + 16 * 2 + 8 + 4]


def test_int4_scales_layout():
    N, K = 32, 512
    for G in (32, 64, 128, 256):
        s = np.arange((K // G) * N, dtype=np.uint16).reshape(K // G, N)
        p = layout.device_int4_scales(s, N, K, G)
        assert p.size == s.size
        assert sorted(p.tolist()) == sorted(s.ravel().tolist())
    # G=32: T=4; element ((nb*KS + kb)*16 + c)*4 + t = scale[g = 4kb + t][16nb + c]
    s = np.arange(16 * 32, dtype=np.uint16).reshape(16, 32)
    p = layout.device_int4_scales(s, 32, 512, 32)
    assert p[((1 * 4 + 2) * 16 + 5) * 4 + 3] == s[4 * 2 + 3, 16 + 5]
    # G=256: span 256, T=1
    s = np.arange(2 * 32, dtype=np.uint16).reshape(2, 32)
    p = layout.device_int4_scales(s, 32, 512, 256)
    assert p[(1 * 2 + 1) * 16 + 7] == s[1, 16 + 7]


def test_fp4_scales_layout():
    N, K = 32, 256
    sf = np.arange(N * K // 16, dtype=np.uint8).reshape(N, K // 16)
    p = layout.device_fp4_scales(sf, N, K)
    # lane l of column block 1, k-block 1 reads dword ((l&15)*2 + (l>>5)); byte t is
    # the scale of K step t: 16-k block 8*kb + 2t + (l>>5)
    for l in (0, 5, 37, 63):
        dword = ((1 * 2 + 1) * 16 + (l & 15)) * 8 + 4 * (l >> 5)
        for t in range(4):
            k = 128 + 32 * t + 8 * (l >> 4)
            assert p[dword + t] == sf[16 + (l & 15), k // 16]


def test_round_trips():
    g = np.random.default_rng(9)
    c4 = g.integers(0, 16, (48, 384)).astype(np.uint8)
    assert np.array_equal(layout.device_int4_weights_inverse(layout.device_int4_weights(c4), 48, 384), c4)
    assert np.array_equal(layout.device_fp4_weights_inverse(layout.device_fp4_weights(c4), 48, 384), c4)
    c8 = g.integers(0, 256, (48, 192)).astype(np.uint8)
    assert np.array_equal(layout.device_fp8_weights_inverse(layout.device_fp8_weights(c8), 48, 192), c8)


@pytest.mark.parametrize("n,k,byte,shift", [
    # INT2, N=32, K=256: 512-byte blocks, lane l owns bytes 8l..8l+7 (dwords d = 0, 1);
    # a code sits at bit 16h + 8b + 2f of dword d for k = 32(2d+b) + 8(l>>4) + 2f + h
    (0, 0, 0, 0),                      # d0 b0 f0 h0 -> bit 0
    (0, 1, 2, 0),                      # h1 -> bit 16 -> byte 2
    (0, 2, 0, 2),                      # f1 -> bit 2
    (0, 7, 2, 6),                      # f3 h1 -> bit 22 -> byte 2, shift 6
    (0, 32, 1, 0),                     # step 1 -> b1 -> bit 8 -> byte 1
    (0, 64, 4, 0),                     # step 2 -> d1 -> byte 4
    (5, 8, 8 * 21, 0),                 # lane 5 + 16 = 21
    (17, 130, 3 * 512 + 8, 2),         # nb1 kb1 (block 3), lane 1, k' = 2 -> f1
    # n=31 k=255: block 3; k' = 127 = 32*3 + 8*3 + 7 -> d1 b1, lane 63, f3 h1 -> bit 30 of dword 1
    (31, 255, 3 * 512 + 8 * 63 + 4 + 3, 6),
])
def test_int2_single_hot(n, k, byte, shift):
    codes = np.zeros((32, 256), np.uint8)
    codes[n, k] = 3
    p = layout.device_int2_weights(codes)
    assert p.size == 32 * 256 // 4
    assert list(np.flatnonzero(p)) == [byte]
    assert p[byte] == 3 << shift


def test_int2_round_trip():
    c = np.random.default_rng(4).integers(0, 4, (48, 384)).astype(np.uint8)
    assert np.array_equal(layout.device_int2_weights_inverse(layout.device_int2_weights(c), 48, 384), c)


@pytest.mark.parametrize("n,k,byte,shift", [
    # NF4, N=32, K=256: J = (0,4,1,5,2,6,3,7), so byte b of a dword holds k offsets b (low
    # nibble) and b + 4 (high nibble)
    (0, 0, 0, 0),
    (0, 1, 1, 0),                      # offset 1 -> slot 2 -> byte 1 low
    (0, 4, 0, 4),                      # offset 4 -> slot 1 -> byte 0 high
    (0, 7, 3, 4),                      # offset 7 -> slot 7 -> byte 3 high
    (5, 14, 16 * 21 + 2, 4),           # lane 21, t0, offset 6 -> slot 5 -> byte 2 high
    (17, 131, 3072 + 16 + 3, 0),       # block 3, lane 1, offset 3 -> slot 6 -> byte 3 low
    # n=31 k=255: block 3; k' = 127 = 32*3 + 8*3 + 7 -> t3, lane 63, offset 7 -> byte 3 high
    (31, 255, 3072 + 16 * 63 + 12 + 3, 4),
])
def test_nf4_single_hot(n, k, byte, shift):
    codes = np.zeros((32, 256), np.uint8)
    codes[n, k] = 0xD
    p = layout.device_nf4_weights(codes)
    assert list(np.flatnonzero(p)) == [byte]
    assert p[byte] == 0xD << shift


def test_nf4_round_trip_and_scale_header():
    c = np.random.default_rng(5).integers(0, 16, (48, 384)).astype(np.uint8)
    assert np.array_equal(layout.device_nf4_weights_inverse(layout.device_nf4_weights(c), 48, 384), c)
    N, K, G = 32, 256, 64
    book = (0x1234 + 0x0101 * np.arange(16)).astype(np.uint16)
    s = np.arange((K // G) * N, dtype=np.uint16).reshape(K // G, N)
    p = layout.device_nf4_scales(book, s, N, K, G)
    assert p.size == 256 + 2 * s.size
    assert list(p[:16]) == [0x34 + i for i in range(16)]    # low bytes of the book
    assert list(p[16:32]) == [0x12 + i for i in range(16)]  # high bytes
    assert not p[32:256].any()
    assert np.array_equal(p[256:].view("<u2"), layout.device_int4_scales(s, N, K, G))
