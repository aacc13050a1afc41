"""Pins of the oracle's quantizers and canonical packing: hand-worked fixtures,
brute-force nearest-grid searches and invariants."""
import numpy as np

from oracle import codecs, quant, reference
from golden_io import table, tagged


def test_unpack_fixture_and_all_bytes():
    for byte, lo, hi in table("int4_nibbles.txt"):
        codes = quant.unpack_nibbles(np.array([[byte]], np.uint8))
        assert list(quant.int4_signed(codes)[0]) == [lo, hi]
    allb = np.arange(256, dtype=np.uint8)[None, :]
    codes = quant.unpack_nibbles(allb)
    assert np.array_equal(codes[0, 0::2], allb[0] & 0xF)
    assert np.array_equal(codes[0, 1::2], allb[0] >> 4)
    assert np.array_equal(quant.pack_nibbles(codes), allb)


def test_pack_round_trip_random():
    c = np.random.default_rng(1).integers(0, 16, (48, 384)).astype(np.uint8)
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(c)), c)


def _w(d):
    return np.array([d[i] for i in sorted(d)], dtype=np.float32)


def test_int4_worked_example():
    g = tagged("worked_int4.txt")
    wt = _w(g["w"])
    codes, sbits = quant.quantize_int4(wt, 4)
    want_s = np.array([g["scale"][i] for i in sorted(g["scale"])], np.uint16)
    assert np.array_equal(sbits, want_s)
    want_b = np.array([g["bytes"][i] for i in sorted(g["bytes"])], np.uint8)
    assert np.array_equal(quant.pack_nibbles(codes), want_b)
    a = np.array([g["a"][i] for i in sorted(g["a"])])
    out = reference.gemm_fp64(a, reference.dequant_int4(codes, sbits, 4))
    want = np.array([g["out"][i] for i in sorted(g["out"])])
    assert np.array_equal(out, want)


def test_fp8_worked_example():
    g = tagged("worked_fp8.txt")
    codes, alpha = quant.quantize_fp8(_w(g["w"]))
    assert alpha == g["alpha"]
    assert np.array_equal(codes, np.array([g["codes"][i] for i in sorted(g["codes"])], np.uint8))
    a = np.array([g["a"][0]])
    out = reference.gemm_fp64(a, reference.dequant_fp8(codes), alpha)
    assert np.array_equal(out[0], np.array(g["out"][0]))


def test_fp4_worked_example():
    g = tagged("worked_fp4.txt")
    codes, sf, alpha = quant.quantize_fp4(_w(g["w"]))
    assert alpha == g["alpha"]
    assert np.array_equal(sf[0], np.array(g["sf"][0], np.uint8))
    assert np.array_equal(quant.pack_nibbles(codes)[0], np.array(g["bytes"][0], np.uint8))
    a = np.array([g["a"][0]])
    out = reference.gemm_fp64(a, reference.dequant_fp4(codes, sf), alpha)
    assert out[0, 0] == g["out"][0][0]


def test_int4_brute_force_nearest_and_invariants():
    G = 32
    wt = (np.random.default_rng(2).standard_normal((32, 256)) * 0.02).astype(np.float32)
    wt[3, 64:96] = 0.0                                      # an all-zero group
    codes, sbits = quant.quantize_int4(wt, G)
    s = codecs.f16_from_bits(sbits)                         # [K/G, N]
    s_nk = np.repeat(s.T, G, axis=1)
    q = codes.astype(np.int64) - 8
    # brute force: for every element try all 16 signed values, nearest to w/s, ties even
    cand = np.arange(-8, 8)
    x = np.where(s_nk == 0, 0.0, wt.astype(np.float64) / np.where(s_nk == 0, 1, s_nk))
    d = np.abs(x[..., None] - cand)
    dmin = d.min(axis=-1, keepdims=True)
    tie_even = np.where(d == dmin, (cand % 2 != 0) * 1.0 + d, np.inf)
    best = cand[np.argmin(tie_even, axis=-1)]
    assert np.array_equal(q, best)
    assert q.min() >= -7 and q.max() <= 7                   # absmax/7 never emits -8
    # the absmax element of each non-zero group lands on +-7
    grp = np.abs(wt).reshape(32, -1, G)
    arg = grp.argmax(axis=2)
    qg = q.reshape(32, -1, G)
    hit = np.take_along_axis(np.abs(qg), arg[..., None], axis=2)[..., 0]
    nz = s.T > 0
    assert np.all(hit[nz] == 7)
    assert np.all(codes[3, 64:96] == 8) and s[2, 3] == 0
    err = np.abs(wt - reference.dequant_int4(codes, sbits, G))
    assert np.all(err <= s_nk / 2 * (1 + 1e-6) + 1e-12)


def test_fp8_brute_force_nearest():
    wt = (np.random.default_rng(3).standard_normal((16, 256)) * 0.05).astype(np.float32)
    codes, alpha = quant.quantize_fp8(wt)
    assert alpha == float(np.float32(np.abs(wt).max() / 448.0))
    allc = np.arange(256)
    vals = codecs.e4m3_decode(allc)
    fin = ~np.isnan(vals)
    vals, allc = vals[fin], allc[fin]
    x = np.clip(wt.astype(np.float64) / alpha, -448, 448).ravel()
    d = np.abs(x[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    # among the nearest, prefer an even mantissa (code bit 0 clear) and +0 over -0
    score = np.where(d == dmin, (allc % 2) * 1.0 + (allc == 0x80) * 2.0, np.inf)
    best = allc[np.argmin(score, axis=1)]
    assert np.array_equal(codes.ravel(), best)
    # the absmax element maps to +-448
    i = np.unravel_index(np.abs(wt).argmax(), wt.shape)
    assert codecs.e4m3_decode(codes[i]) in (448.0, -448.0)


def test_fp4_brute_force_nearest_and_block_scales():
    wt = (np.random.default_rng(4).standard_normal((16, 256)) * 0.02).astype(np.float32)
    wt[5, 32:48] = 0.0
    codes, sf, alpha = quant.quantize_fp4(wt)
    assert alpha == float(np.float32(np.abs(wt).max() / (6 * 448.0)))
    sb = codecs.e4m3_decode(sf)
    assert sf[5, 2] == 0 and np.all(codes[5, 32:48] == 0)
    # brute-force the block scale: nearest e4m3 to absmax_b / (6 alpha)
    bmax = np.abs(wt.astype(np.float64)).reshape(16, -1, 16).max(axis=2)
    target = np.minimum(bmax / (6 * alpha), 448)
    allv = codecs.e4m3_decode(np.arange(0x7F))
    nearest = allv[np.argmin(np.abs(target[..., None] - allv), axis=-1)]
    assert np.array_equal(sb, nearest)
    grid = codecs.e2m1_decode(np.arange(16))
    den = np.repeat(sb * alpha, 16, axis=1)
    x = np.where(den == 0, 0, np.clip(wt / np.where(den == 0, 1, den), -6, 6))
    d = np.abs(x[..., None] - grid)
    best = np.argmin(np.where(d == d.min(-1, keepdims=True), (np.arange(16) % 2) + (np.arange(16) == 8) * 2.0, np.inf), -1)
    assert np.array_equal(codes, best.astype(np.uint8))


def test_crumbs_every_byte_and_round_trip():
    # INT2 canonical packing: byte j holds k = 4j .. 4j+3, lowest k in the lowest two bits
    allb = np.arange(256, dtype=np.uint8)[None, :]
    codes = quant.unpack_crumbs(allb)
    for i in range(4):
        assert np.array_equal(codes[0, i::4], (allb[0] >> (2 * i)) & 3)
    assert np.array_equal(quant.pack_crumbs(codes), allb)
    assert list(quant.int2_signed(codes[0, :8])) == [-2, -2, -2, -2, -1, -2, -2, -2]   # bytes 0, 1
    c = np.random.default_rng(7).integers(0, 4, (48, 384)).astype(np.uint8)
    assert np.array_equal(quant.unpack_crumbs(quant.pack_crumbs(c)), c)


def test_int2_worked_example():
    g = tagged("worked_int2.txt")
    wt = _w(g["w"])
    codes, sbits = quant.quantize_int2(wt, 4)
    want_s = np.array([g["scale"][i] for i in sorted(g["scale"])], np.uint16)
    assert np.array_equal(sbits, want_s)
    want_b = np.array([g["bytes"][i] for i in sorted(g["bytes"])], np.uint8)
    assert np.array_equal(quant.pack_crumbs(codes), want_b)
    a = np.array([g["a"][i] for i in sorted(g["a"])])
    out = reference.gemm_fp64(a, reference.dequant_int2(codes, sbits, 4))
    want = np.array([g["out"][i] for i in sorted(g["out"])])
    assert np.array_equal(out, want)


def test_int2_brute_force_nearest_and_invariants():
    G = 64
    wt = (np.random.default_rng(8).standard_normal((32, 256)) * 0.02).astype(np.float32)
    wt[5, 128:192] = 0.0                                    # an all-zero group
    codes, sbits = quant.quantize_int2(wt, G)
    s = codecs.f16_from_bits(sbits)                         # [K/G, N]
    s_nk = np.repeat(s.T, G, axis=1)
    q = codes.astype(np.int64) - 2
    # brute force over the four signed values, nearest to w/s, ties to the even one
    cand = np.arange(-2, 2)
    x = np.where(s_nk == 0, 0.0, wt.astype(np.float64) / np.where(s_nk == 0, 1, s_nk))
    d = np.abs(x[..., None] - cand)
    dmin = d.min(axis=-1, keepdims=True)
    tie_even = np.where(d == dmin, (cand % 2 != 0) * 1.0 + d, np.inf)
    assert np.array_equal(q, cand[np.argmin(tie_even, axis=-1)])
    assert q.min() >= -1 and q.max() <= 1                   # absmax / 1 never emits -2
    grp = np.abs(wt).reshape(32, -1, G)
    hit = np.take_along_axis(np.abs(q.reshape(32, -1, G)), grp.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.all(hit[s.T > 0] == 1)                        # each group's absmax lands on +-1
    assert np.all(codes[5, 128:192] == 2) and s[2, 5] == 0
    err = np.abs(wt - reference.dequant_int2(codes, sbits, G))
    assert np.all(err <= s_nk / 2 * (1 + 1e-6) + 1e-12)


def _phi_inverse_by_bisection(p):
    """Standard normal quantile from math.erf alone (independent of scipy's ndtri)."""
    import math
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_nf4_codebook_definition():
    book = quant.nf4_codebook()
    assert book.shape == (16,)
    assert np.all(np.diff(book) > 0)                        # strictly ascending
    assert book[0] == -1.0 and book[7] == 0.0 and book[15] == 1.0
    assert np.sum(book < 0) == 7 and np.sum(book > 0) == 8  # asymmetric: exact zero, 8 positive
    assert np.array_equal(codecs.f16_round(book), book)     # stored in fp16
    # the quantile construction, recomputed with a different routine, gives the same fp16 book
    d = ((1 - 1 / 30) + (1 - 1 / 32)) / 2
    top = _phi_inverse_by_bisection(d)
    pos = [_phi_inverse_by_bisection(d + (0.5 - d) * i / 8) / top for i in range(8)]
    neg = [-_phi_inverse_by_bisection(d + (0.5 - d) * i / 7) / top for i in range(7)]
    want = codecs.f16_round(np.sort(np.array(pos + neg + [0.0])))
    assert np.array_equal(book, want)
    # equal-probability spacing: Phi of consecutive positive quantiles differs by (d - 1/2) / 8
    import math
    phi = [0.5 * (1 + math.erf(p * top / math.sqrt(2))) for p in pos]
    assert np.allclose(np.diff(phi), -(d - 0.5) / 8, rtol=0, atol=1e-12)


def test_nf4_worked_example():
    g = tagged("worked_nf4.txt")
    wt = _w(g["w"])
    codes, sbits, book_bits = quant.quantize_nf4(wt, 4)
    for i, v in g["book"].items():
        assert book_bits[i] == v[0]
    want_s = np.array([g["scale"][i] for i in sorted(g["scale"])], np.uint16)
    assert np.array_equal(sbits, want_s)
    want_b = np.array([g["bytes"][i] for i in sorted(g["bytes"])], np.uint8)
    assert np.array_equal(quant.pack_nibbles(codes), want_b)
    a = np.array([g["a"][i] for i in sorted(g["a"])])
    out = reference.gemm_fp64(a, reference.dequant_nf4(codes, sbits, 4, book_bits))
    want = np.array([g["out"][i] for i in sorted(g["out"])])
    assert np.array_equal(out, want)


def test_nf4_brute_force_nearest_and_invariants():
    G = 64
    wt = (np.random.default_rng(18).standard_normal((16, 256)) * 0.02).astype(np.float32)
    wt[3, 64:128] = 0.0                                     # an all-zero group
    codes, sbits, book_bits = quant.quantize_nf4(wt, G)
    book = codecs.f16_from_bits(book_bits)
    s = codecs.f16_from_bits(sbits)                         # [K/G, N]
    for n in range(16):
        for k in range(256):
            sk = s[k // G, n]
            if sk == 0:
                assert codes[n, k] == 7
                continue
            x = float(wt[n, k]) / float(sk)
            best, bd = 0, abs(x - book[0])
            for c in range(1, 16):                          # first strict minimum: lower index on ties
                if abs(x - book[c]) < bd:
                    best, bd = c, abs(x - book[c])
            assert codes[n, k] == best
    grp = np.abs(wt).reshape(16, -1, G)
    hit = np.take_along_axis(codes.reshape(16, -1, G), grp.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.all(np.isin(hit[s.T > 0], (0, 15)))           # each group's absmax lands on -1 or +1
    gap = np.max(np.diff(book))
    err = np.abs(wt - reference.dequant_nf4(codes, sbits, G, book_bits))
    assert np.all(err <= np.repeat(s.T, G, axis=1) * gap / 2 * (1 + 1e-6) + 1e-12)
    # ties go to the lower index: a value exactly between two entries
    w2 = np.zeros((1, 64), np.float32)
    w2[0, 0] = 1.0
    w2[0, 1] = np.float32((book[7] + book[8]) / 2)
    c2, _, _ = quant.quantize_nf4(w2, 64)
    if float(w2[0, 1]) == (book[7] + book[8]) / 2:
        assert c2[0, 1] == 7
