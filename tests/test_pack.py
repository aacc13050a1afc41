"""Library quantizer and packer vs the oracle, byte for byte (CPU, through the C ABI)."""
import numpy as np
import pytest

import synthetic
import weight_only_quantized_qgemm_amd as q
from oracle import layout, quant


def _w(N, K, sigma, seed):
    return synthetic.weights(N, K, sigma, (90, seed))


@pytest.mark.parametrize("N,K,G", [(16, 128, 32), (16, 128, 64), (16, 128, 128), (16, 256, 256),
                                   (48, 384, 128), (256, 512, 128), (64, 1024, 32), (64, 1024, 256)])
def test_int4_quantize_and_pack_match_oracle(N, K, G):
    w = _w(N, K, 0.02, N + K + G)
    w[0, :G] = 0.0                                      # an all-zero group
    p = q.problem(1, N, K, "int4", group_size=G)
    codes_b, scales_b, alpha = q.quantize(p, w)
    codes_o, sbits_o = quant.quantize_int4(w, G)
    assert alpha == 1.0
    assert np.array_equal(codes_b, quant.pack_nibbles(codes_o))
    assert np.array_equal(scales_b, sbits_o)
    wpk, spk = q.pack(p, codes_b, scales_b)
    assert np.array_equal(wpk, layout.device_int4_weights(codes_o))
    assert np.array_equal(spk.view(np.uint16), layout.device_int4_scales(sbits_o, N, K, G))


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 512), (32, 1024)])
def test_fp8_quantize_and_pack_match_oracle(N, K):
    w = _w(N, K, 0.05, N * 3 + K)
    p = q.problem(1, N, K, "fp8")
    codes_b, _, alpha_b = q.quantize(p, w)
    codes_o, alpha_o = quant.quantize_fp8(w)
    assert alpha_b == alpha_o
    assert np.array_equal(codes_b, codes_o)
    wpk, spk = q.pack(p, codes_b, None)
    assert spk is None
    assert np.array_equal(wpk, layout.device_fp8_weights(codes_o))


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 512), (32, 1024)])
def test_fp4_quantize_and_pack_match_oracle(N, K):
    w = _w(N, K, 0.02, N * 5 + K)
    w[1, 16:32] = 0.0                                   # an all-zero block
    p = q.problem(1, N, K, "fp4")
    codes_b, sf_b, alpha_b = q.quantize(p, w)
    codes_o, sf_o, alpha_o = quant.quantize_fp4(w)
    assert alpha_b == alpha_o
    assert np.array_equal(codes_b, quant.pack_nibbles(codes_o))
    assert np.array_equal(sf_b, sf_o)
    wpk, spk = q.pack(p, codes_b, sf_b)
    assert np.array_equal(wpk, layout.device_fp4_weights(codes_o))
    assert np.array_equal(spk, layout.device_fp4_scales(sf_o, N, K))


def test_pack_at_workload_size_int4():
    N, K = 4096, 4096
    g = np.random.default_rng(5)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    sb = g.integers(0, 0x7C00, (K // 128, N)).astype(np.uint16)
    p = q.problem(1, N, K, "int4")
    wpk, spk = q.pack(p, quant.pack_nibbles(codes), sb)
    assert np.array_equal(wpk, layout.device_int4_weights(codes))
    assert np.array_equal(spk.view(np.uint16), layout.device_int4_scales(sb, N, K, 128))


def test_quantizer_edge_cases():
    # worked example values (hand-derived fixture) through the library quantizer
    from golden_io import tagged
    g = tagged("worked_fp8.txt")
    w = np.zeros((16, 128), np.float32)
    w[0, :4] = g["w"][0]
    w[1, :4] = g["w"][1]
    codes, _, alpha = q.quantize(q.problem(1, 16, 128, "fp8"), w)
    assert alpha == g["alpha"]
    assert list(codes[0, :4]) == g["codes"][0] and list(codes[1, :4]) == g["codes"][1]
    # non-finite weights are rejected
    w[3, 3] = np.inf
    with pytest.raises(q.QgemmError):
        q.quantize(q.problem(1, 16, 128, "fp8"), w)
    # an all-zero tensor quantizes to zero codes and alpha 0
    codes, sf, alpha = q.quantize(q.problem(1, 16, 128, "fp4"), np.zeros((16, 128), np.float32))
    assert alpha == 0.0 and not codes.any() and not sf.any()


@pytest.mark.parametrize("N,K,G", [(16, 128, 32), (16, 128, 128), (16, 256, 256), (48, 384, 64),
                                   (256, 512, 128), (64, 1024, 32)])
def test_int2_quantize_and_pack_match_oracle(N, K, G):
    w = _w(N, K, 0.02, 7 * N + K + G)
    w[2, G:2 * G] = 0.0                                 # an all-zero group
    p = q.problem(1, N, K, "int2", group_size=G)
    codes_b, scales_b, alpha = q.quantize(p, w)
    codes_o, sbits_o = quant.quantize_int2(w, G)
    assert alpha == 1.0
    assert np.array_equal(codes_b, quant.pack_crumbs(codes_o))
    assert np.array_equal(scales_b, sbits_o)
    wpk, spk = q.pack(p, codes_b, scales_b)
    assert wpk.size == N * K // 4
    assert np.array_equal(wpk, layout.device_int2_weights(codes_o))
    assert np.array_equal(spk.view(np.uint16), layout.device_int4_scales(sbits_o, N, K, G))


def test_int2_pack_every_code_position():
    # random codes (the quantizer never emits code 0, the layout must still carry it)
    N, K = 64, 512
    codes = np.random.default_rng(9).integers(0, 4, (N, K)).astype(np.uint8)
    sb = np.full((K // 128, N), 0x3C00, np.uint16)
    wpk, _ = q.pack(q.problem(1, N, K, "int2"), quant.pack_crumbs(codes), sb)
    assert np.array_equal(wpk, layout.device_int2_weights(codes))
    assert np.array_equal(layout.device_int2_weights_inverse(wpk, N, K), codes)


@pytest.mark.parametrize("N,K,G", [(16, 128, 32), (16, 128, 128), (16, 256, 256), (48, 384, 64),
                                   (256, 512, 128), (64, 1024, 32)])
def test_nf4_quantize_and_pack_match_oracle(N, K, G):
    w = _w(N, K, 0.02, 11 * N + K + G)
    w[2, G:2 * G] = 0.0                                 # an all-zero group
    p = q.problem(1, N, K, "nf4", group_size=G)
    codes_b, scales_b, alpha = q.quantize(p, w)
    codes_o, sbits_o, book_o = quant.quantize_nf4(w, G)
    assert alpha == 1.0
    # the library derives the code book on its own (bisection on erfc); the oracle uses scipy
    assert np.array_equal(scales_b[:16], book_o)
    assert np.array_equal(scales_b[16:].reshape(K // G, N), sbits_o)
    assert np.array_equal(codes_b, quant.pack_nibbles(codes_o))
    wpk, spk = q.pack(p, codes_b, scales_b)
    assert wpk.size == N * K // 2 and spk.size == 256 + 2 * (K // G) * N
    assert np.array_equal(wpk, layout.device_nf4_weights(codes_o))
    assert np.array_equal(spk, layout.device_nf4_scales(book_o, sbits_o, N, K, G))


def test_nf4_pack_every_code_and_any_book():
    # every code at every position, and a code book that is not NF4's: the packer copies the
    # caller's book into the header unchanged
    N, K, G = 64, 512, 128
    codes = np.random.default_rng(10).integers(0, 16, (N, K)).astype(np.uint8)
    book = np.random.default_rng(12).integers(0, 0x7C00, 16).astype(np.uint16)
    sb = np.full((K // G, N), 0x3C00, np.uint16)
    scales = np.concatenate([book, sb.reshape(-1)])
    wpk, spk = q.pack(q.problem(1, N, K, "nf4"), quant.pack_nibbles(codes), scales)
    assert np.array_equal(wpk, layout.device_nf4_weights(codes))
    assert np.array_equal(layout.device_nf4_weights_inverse(wpk, N, K), codes)
    assert np.array_equal(spk, layout.device_nf4_scales(book, sb, N, K, G))
