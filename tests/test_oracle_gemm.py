"""Pins of the oracle's dequant + fp64 GEMM: brute force, closed forms, identity A."""
import math

import numpy as np

from oracle import codecs, quant, reference


def test_gemm_fp64_vs_brute_force():
    g = np.random.default_rng(11)
    for M, N, K in [(1, 3, 8), (3, 5, 16), (4, 32, 256)]:
        a = g.standard_normal((M, K))
        w = g.standard_normal((N, K))
        r = reference.gemm_fp64(a, w, 0.75)
        for m in range(M):
            for n in range(N):
                exact = math.fsum(a[m, k] * w[n, k] for k in range(K)) * 0.75
                tol = K * 2.0 ** -52 * math.fsum(abs(a[m, k] * w[n, k]) for k in range(K))
                assert abs(r[m, n] - exact) <= tol + 1e-300


def test_int4_closed_form_all_equal_nibbles():
    M, N, K, G = 3, 32, 256, 128
    a = np.random.default_rng(12).standard_normal((M, K)).astype(np.float16).astype(np.float64)
    one = codecs.f16_bits(np.ones((K // G, N)))
    for c in (0, 3, 8, 15):
        codes = np.full((N, K), c, np.uint8)
        r = reference.gemm_fp64(a, reference.dequant_int4(codes, one, G))
        want = (c - 8) * a.sum(axis=1)
        assert np.allclose(r, want[:, None], rtol=0, atol=1e-12)


def test_int4_closed_form_one_nonzero_group():
    M, N, K, G = 2, 16, 512, 64
    g = np.random.default_rng(13)
    a = g.standard_normal((M, K))
    codes = np.full((N, K), 8, np.uint8)
    q = g.integers(0, 16, (N, G)).astype(np.uint8)
    codes[:, 3 * G:4 * G] = q
    s = np.zeros((K // G, N))
    s[3] = 0.5 + np.arange(N) / 64.0
    r = reference.gemm_fp64(a, reference.dequant_int4(codes, codecs.f16_bits(s), G))
    want = (a[:, 3 * G:4 * G] @ (q.astype(np.float64) - 8).T) * s[3][None, :]
    assert np.allclose(r, want, rtol=1e-14, atol=1e-14)


def test_identity_a_returns_dequantized_weights():
    N, K, G = 16, 128, 32
    wt = (np.random.default_rng(14).standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, sb = quant.quantize_int4(wt, G)
    eye = np.eye(K)
    assert np.array_equal(reference.gemm_fp64(eye, reference.dequant_int4(codes, sb, G)),
                          reference.dequant_int4(codes, sb, G).T.astype(np.float64))
    c8, alpha = quant.quantize_fp8(wt)
    assert np.array_equal(reference.gemm_fp64(eye, reference.dequant_fp8(c8), 1.0),
                          codecs.e4m3_decode(c8).T)
    c4, sf, a4 = quant.quantize_fp4(wt)
    want = codecs.e2m1_decode(c4) * np.repeat(codecs.e4m3_decode(sf), 16, axis=1)
    assert np.array_equal(reference.gemm_fp64(eye, reference.dequant_fp4(c4, sf)), want.T)


def test_fp8_closed_form_all_equal_codes():
    M, N, K = 2, 16, 128
    a = np.random.default_rng(15).standard_normal((M, K))
    for code, v in ((0x38, 1.0), (0x42, 2.5), (0xF0, -128.0)):
        r = reference.gemm_fp64(a, reference.dequant_fp8(np.full((N, K), code, np.uint8)), 0.125)
        assert np.allclose(r, (0.125 * v * a.sum(axis=1))[:, None], rtol=1e-14, atol=1e-14)


def test_int4_f16_operand_is_rounded_product():
    codes = np.array([[1, 15, 8, 3]], np.uint8)
    s = codecs.f16_bits(np.array([[0.1]]))                  # 0.1 is not an fp16 value
    v = reference.dequant_int4_f16(codes, s, 4)
    sval = codecs.f16_from_bits(s)[0, 0]
    for i, q in enumerate([-7, 7, 0, -5]):
        assert v[0, i] == np.float64(np.float16(q * sval))


def test_gemm_fp64_bias_vs_brute_force():
    # the bias lands on its own column, after alpha: a triple loop with the bias written out
    g = np.random.default_rng(15)
    M, N, K = 3, 7, 64
    a = g.standard_normal((M, K))
    w = g.standard_normal((N, K))
    b = g.standard_normal(N)
    r = reference.gemm_fp64(a, w, 0.5, b)
    for m in range(M):
        for n in range(N):
            exact = math.fsum(a[m, k] * w[n, k] for k in range(K)) * 0.5 + b[n]
            tol = K * 2.0 ** -52 * (math.fsum(abs(a[m, k] * w[n, k]) for k in range(K)) + abs(b[n]))
            assert abs(r[m, n] - exact) <= tol + 1e-300
    # zero activations leave exactly the bias in every row; rows keep their own columns
    z = reference.gemm_fp64(np.zeros((M, K)), w, 3.0, b)
    assert np.array_equal(z, np.tile(b, (M, 1)))
    rows = reference.gemm_fp64_rows(a, w, [2, 0], 0.5, b)
    assert np.array_equal(rows, r[[2, 0]])


def test_fp8_values_are_exact_in_fp16_and_bf16():
    # mm_fp16_fp8 feeds the same dequantized weights to an fp16 matrix unit: every finite
    # e4m3 value must survive both 16-bit casts unchanged
    v = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = v[np.isfinite(v)]
    assert np.array_equal(codecs.f16_round(fin), fin)
    assert np.array_equal(codecs.bf16_round(fin), fin)


def test_int2_closed_forms_and_identity():
    M, N, K, G = 3, 32, 256, 128
    a = np.random.default_rng(16).standard_normal((M, K)).astype(np.float16).astype(np.float64)
    one = codecs.f16_bits(np.ones((K // G, N)))
    for c in (0, 1, 2, 3):
        codes = np.full((N, K), c, np.uint8)
        r = reference.gemm_fp64(a, reference.dequant_int2(codes, one, G))
        assert np.allclose(r, ((c - 2) * a.sum(axis=1))[:, None], rtol=0, atol=1e-12)
    wt = (np.random.default_rng(17).standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, sb = quant.quantize_int2(wt, 32)
    dq = reference.dequant_int2(codes, sb, 32)
    assert np.array_equal(reference.gemm_fp64(np.eye(K), dq), dq.T.astype(np.float64))
    # the products are exact in fp16 too: the 16-bit operand equals the exact value
    assert np.array_equal(codecs.f16_round(dq.astype(np.float64)), dq.astype(np.float64))


def test_nf4_closed_forms_and_identity():
    M, N, K, G = 3, 32, 256, 128
    a = np.random.default_rng(19).standard_normal((M, K)).astype(np.float16).astype(np.float64)
    one = codecs.f16_bits(np.ones((K // G, N)))
    book_bits = codecs.f16_bits(quant.nf4_codebook())
    book = codecs.f16_from_bits(book_bits)
    for c in range(16):
        codes = np.full((N, K), c, np.uint8)
        r = reference.gemm_fp64(a, reference.dequant_nf4(codes, one, G, book_bits))
        assert np.allclose(r, (book[c] * a.sum(axis=1))[:, None], rtol=0, atol=1e-12)
    # one nonzero group: s * (A_group . book[q_group])
    codes = np.full((N, K), 7, np.uint8)
    q = np.random.default_rng(20).integers(0, 16, G)
    codes[4, G:2 * G] = q
    sb = np.zeros((K // G, N), np.uint16)
    sb[1, 4] = 0x3555                                       # an fp16 scale with a full mantissa
    r = reference.gemm_fp64(a, reference.dequant_nf4(codes, sb, G, book_bits))
    s = float(codecs.f16_from_bits(np.array([0x3555], np.uint16))[0])
    want = s * (a[:, G:2 * G] @ book[q])
    assert np.allclose(r[:, 4], want, rtol=1e-14, atol=0) and not np.any(np.delete(r, 4, axis=1))
    # identity A returns the dequantized weights; the fp16 operand is their RNE_fp16
    wt = (np.random.default_rng(21).standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, sb, bb = quant.quantize_nf4(wt, 32)
    dq = reference.dequant_nf4(codes, sb, 32, bb)
    assert np.array_equal(reference.gemm_fp64(np.eye(K), dq), dq.T.astype(np.float64))
    f16 = reference.dequant_nf4_f16(codes, sb, 32, bb)
    assert np.array_equal(f16, codecs.f16_round(dq.astype(np.float64)))
    assert np.max(np.abs(f16 - dq)) <= np.max(np.abs(dq)) * 2.0 ** -11
