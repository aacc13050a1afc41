"""Pins of the oracle's number codecs against library casts, closed forms and brute force."""
import numpy as np
import pytest
import torch

from oracle import codecs
from golden_io import table


# ----------------------------------------------------------------------------- fp16
def test_f16_every_code_round_trips():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    got = codecs.f16_bits(vals[fin])
    want = bits[fin].copy()
    want[want == 0x8000] = 0x8000        # -0 keeps its sign
    assert np.array_equal(got, want)


def test_f16_midpoints_tie_to_even_and_match_numpy():
    # every midpoint between consecutive positive finite fp16 values
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                                   # exact in float64
    got = codecs.f16_bits(mid)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    # numpy's own float64 -> float16 cast is an independent implementation
    assert np.array_equal(got, mid.astype(np.float16).view(np.uint16))
    r = np.random.default_rng(3).standard_normal(200000) * 10.0 ** np.random.default_rng(4).uniform(-9, 4.5, 200000)
    assert np.array_equal(codecs.f16_bits(r), r.astype(np.float16).view(np.uint16))


def test_f16_overflow_and_specials():
    assert codecs.f16_round(65504.0) == 65504.0
    assert codecs.f16_round(65519.99) == 65504.0
    assert np.isinf(codecs.f16_round(65520.0))           # tie above max goes to inf
    assert codecs.f16_round(2.0 ** -24) == 2.0 ** -24     # smallest subnormal
    assert codecs.f16_round(2.0 ** -25) == 0.0            # tie to even (zero)
    assert codecs.f16_round(1.0 + 2.0 ** -11) == 1.0
    assert codecs.f16_round(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9


# ----------------------------------------------------------------------------- bf16
def test_bf16_matches_torch_cast():
    g = np.random.default_rng(5)
    x = (g.standard_normal(300000) * 10.0 ** g.uniform(-30, 30, 300000)).astype(np.float32)
    # plus every exact midpoint pattern: low 16 bits = 0x8000
    hi = g.integers(0, 0x7F00, 50000, dtype=np.uint32)
    mids = ((hi << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_every_code_round_trips():
    bits = np.arange(65536, dtype=np.uint16)
    vals = codecs.bf16_from_bits(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(codecs.bf16_bits(vals[fin]), bits[fin])


# ----------------------------------------------------------------------------- e4m3
def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.nanmax(ours) == 448.0


def test_e4m3_points_from_fixture():
    for code, val in table("e4m3_points.txt"):
        got = codecs.e4m3_decode(np.array([code]))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val, hex(code)
            if code != 0x80:
                assert codecs.e4m3_encode(np.array([val]))[0] == code


def test_e4m3_encode_midpoints_and_random_vs_torch():
    codes = np.arange(0, 0x7E, dtype=np.uint8)           # positive finite, below max
    lo = codecs.e4m3_decode(codes)
    hi = codecs.e4m3_decode(codes + 1)
    mid = (lo + hi) / 2
    got = codecs.e4m3_encode(mid)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, even)
    g = np.random.default_rng(6)
    x = np.clip(g.standard_normal(200000) * 10.0 ** g.uniform(-4, 2.7, 200000), -448, 448)
    x = np.concatenate([x, mid, -mid])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch casts from fp32; x drawn here is fp32-exact only after the cast, so compare
    # against our encoder on the same fp32 values
    got = codecs.e4m3_encode(x.astype(np.float32).astype(np.float64))
    want = want.copy()
    want[want == 0x80] = 0x00                            # we canonicalise -0 to +0
    assert np.array_equal(got, want)


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([449.0]))


# ----------------------------------------------------------------------------- e2m1
def test_e2m1_table_from_fixture():
    for code, val in table("e2m1_grid.txt"):
        assert codecs.e2m1_decode(np.array([code]))[0] == val
        if code != 0x8:
            assert codecs.e2m1_encode(np.array([val]))[0] == code
    assert codecs.e2m1_encode(np.array([-0.0]))[0] == 0


def test_e2m1_midpoints_ties_to_even():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    got = codecs.e2m1_decode(codecs.e2m1_encode(mids))
    assert np.array_equal(got, want)
    assert np.array_equal(codecs.e2m1_decode(codecs.e2m1_encode(-mids)), -want)


def test_e2m1_brute_force_nearest():
    grid = codecs.e2m1_decode(np.arange(8))
    x = np.random.default_rng(7).uniform(-6, 6, 50000)
    got = codecs.e2m1_decode(codecs.e2m1_encode(x))
    d = np.abs(np.abs(x)[:, None] - grid[None, :])
    best = grid[np.argmin(d, axis=1)]                    # no exact ties in random draws
    assert np.array_equal(np.abs(got), best)
