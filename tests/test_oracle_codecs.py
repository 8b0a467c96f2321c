"""Pins of the oracle's number formats against their definitions, brute force and torch's CPU casts."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as C


def _all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32)
    return v[np.isfinite(v)]


# --- E4M3 -------------------------------------------------------------------------------------

def _e4m3_value_exact(code: int) -> Fraction:
    """Independent statement of OFP8 E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def test_e4m3_decode_all_codes():
    dec = C.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if c & 0x7F == 0x7F:
            assert np.isnan(dec[c])
        else:
            assert Fraction(float(dec[c])) == _e4m3_value_exact(c), hex(c)
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6


def _brute_e4m3(vals: np.ndarray) -> np.ndarray:
    """Nearest of the 127 non-negative finite magnitudes, ties to the even code; saturate."""
    mags = np.array([float(_e4m3_value_exact(c)) for c in range(0x7F)])
    a = np.minimum(np.abs(vals.astype(np.float64)), 448.0)
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & ((np.arange(0x7F) % 2) == 0)[None, :]
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (code | np.where(np.signbit(vals), 0x80, 0)).astype(np.uint8)


def test_e4m3_encode_exhaustive_bf16():
    v = _all_bf16_finite()
    got = C.e4m3_encode(v)
    for chunk in np.array_split(np.arange(v.size), 16):
        np.testing.assert_array_equal(got[chunk], _brute_e4m3(v[chunk]))


def test_e4m3_encode_midpoints_fp32():
    # every rounding boundary between adjacent magnitudes, and one fp32 ulp either side
    mags = np.array([float(_e4m3_value_exact(c)) for c in range(0x7F)])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (mags[:-1] + mags[1:]) / 2)   # exact in fp32
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                          mags.astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    np.testing.assert_array_equal(C.e4m3_encode(pts), _brute_e4m3(pts))


def test_e4m3_special_values():
    f = np.float32
    cases = [(448.0, 0x7E), (464.0, 0x7E), (464.0001, 0x7E), (1e30, 0x7E), (2.0 ** -10, 0x00),
             (1.5 * 2.0 ** -10, 0x01), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (1.0, 0x38),
             (-1.0, 0xB8), (-448.0, 0xFE), (-1e9, 0xFE), (0.0, 0x00), (-0.0, 0x80), (240.0, 0x77),
             (17.0, 0x58), (18.0, 0x59), (19.0, 0x5A)]   # 17 is a tie 16|18 -> even (16)
    for v, c in cases:
        assert C.e4m3_encode(np.array([v], f))[0] == c, (v, hex(c))
    assert C.e4m3_encode(np.array([np.nan], f))[0] == 0x7F
    assert C.e4m3_encode(np.array([np.inf], f))[0] == 0x7E


def test_e4m3_encode_matches_torch_after_clamp():
    # torch's CPU cast is RNE but does not saturate (464.0001 -> NaN), hence the clamp
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 50,
                        rng.standard_normal(200000).astype(np.float32) * 0.01])
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(C.e4m3_encode(v), ref)


def test_e4m3_roundtrip_of_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(C.e4m3_encode(C.e4m3_decode(codes).astype(np.float32)), codes)


# --- bf16 / INT8 ------------------------------------------------------------------------------

def test_f64_to_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(C.f64_to_bf16(v.astype(np.float64)), ref)


def test_f64_to_bf16_single_rounding():
    # 1 + 2^-8 + 2^-40 is above the bf16 midpoint 1 + 2^-8: a single rounding goes up; rounding
    # through fp32 first would land on the midpoint and go to the even neighbour 1.0
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert C.bf16_to_f64(C.f64_to_bf16(np.array([x])))[0] == 1.0 + 2.0 ** -7
    assert C.bf16_to_f64(C.f64_to_bf16(np.array([1.0 + 2.0 ** -8])))[0] == 1.0


def test_bf16_decode_exhaustive_vs_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = C.bf16_to_f64(b)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_int8_round_half_even_and_clip():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.4, 200.0, -300.0], np.float32)
    q = C.int8_encode(x, np.float32(1.0))
    np.testing.assert_array_equal(q, [0, 2, 2, 0, -2, -2, 126, 127, 127, -127])


def test_int8_uses_fp32_product():
    # the product is rounded to fp32 before rint: 0.49999997 * (1 + 2^-23) = 0.5 in fp32 -> 0
    x = np.array([np.nextafter(np.float32(0.5), np.float32(0))], np.float32)
    inv = np.nextafter(np.float32(1.0), np.float32(2))
    assert np.float32(x[0] * inv) == np.float32(0.5)
    assert C.int8_encode(x, inv)[0] == 0


# --- E2M1 / E8M0 ------------------------------------------------------------------------------

def test_e2m1_decode_table():
    vals = C.e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(vals[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(vals[8:], -np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6]))


def test_e2m1_encode_brute_force():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    grid = np.concatenate([np.linspace(-8, 8, 64001), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0]])
    a = np.minimum(np.abs(grid), 6.0)
    dist = np.abs(a[:, None] - mags[None, :])
    cand = dist == dist.min(axis=1, keepdims=True)
    even = cand & ((np.arange(8) % 2) == 0)[None, :]
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = code | np.where(np.signbit(grid), 8, 0)
    np.testing.assert_array_equal(C.e2m1_encode(grid), code.astype(np.uint8))
    assert C.e2m1_encode(np.array([5.0]))[0] == 6          # tie 4|6 -> even code (4)
    assert C.e2m1_encode(np.array([7.9]))[0] == 7          # saturates at 6


def test_e8m0_floor_rule():
    amax = np.array([6.0, 4.0, 3.99, 8.0, 1.0, 0.75, 3.0, 2.0 ** -20, 0.0])
    X = C.e8m0_decode(C.e8m0_shared_exponent(amax))
    np.testing.assert_array_equal(X, [1.0, 1.0, 0.5, 2.0, 0.25, 0.125, 0.5, 2.0 ** -22, 1.0])
    # X is a power of two and amax / X lands in [4, 8) (the top E2M1 binade) for non-zero blocks
    r = np.abs(np.random.default_rng(0).standard_normal(1000)) * 10.0 ** np.random.default_rng(1).integers(-6, 6, 1000)
    Xr = C.e8m0_decode(C.e8m0_shared_exponent(r))
    q = r / Xr
    assert np.all((q >= 4) & (q < 8))
    assert np.all(np.frexp(Xr)[0] == 0.5)
