"""Number formats of the method, written from their definitions (test infrastructure only).

* bf16 / fp16 / fp32 value <-> bit-pattern conversions (IEEE-754 round to nearest, ties to even).
* E4M3 ("FN" variant of the OCP OFP8 spec): the FP8 format of the per-tensor-scaled linear layers
  ([TRIM] "运行速度如何", note under the table: the RTX 4090 path runs the transformer's matmuls in
  FP8 with one scale per tensor).  Bias 7, 3 mantissa bits, largest finite 448, smallest subnormal
  2^-9, no infinities, S.1111.111 is NaN.  Encoding rounds to nearest with ties to even and
  saturates: every finite magnitude above 448 becomes 448.
* symmetric INT8 codes, used for the query/key score computation (same note).
* E2M1 elements and E8M0 shared scales of the OCP MX spec (the 4-bit weight format standing in
  for the pages' NVFP4 layers, [FARWALK] post 6/8 and [TRIM] "ComfyUI 重打包包含什么").

Every encoder here takes the exact value as float64 (fp32 inputs convert exactly), finds the
quantum of its binade with frexp, and rounds the count of quanta half-to-even with np.rint, which
is exact because that count is an integer-or-half below 2^53.
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------------------------------------
# IEEE binary formats


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def f64_to_f32(x) -> np.ndarray:
    """One round-to-nearest-even from float64 to fp32 (numpy's cast is correctly rounded)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _round_binary(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 x to a binary format with ``mant_bits`` fraction bits whose smallest normal
    binade is [2^min_exp, 2^(min_exp+1)) (subnormal quantum 2^(min_exp - mant_bits)); RNE; no
    overflow handling (the caller saturates or maps to infinity)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                    # a = m * 2^e, 0.5 <= m < 1  ->  binade exponent e-1
    q = np.maximum(e - 1, min_exp) - mant_bits
    n = np.rint(np.ldexp(a, -q))          # exact: ldexp by a power of two, rint half-to-even
    return np.copysign(np.ldexp(n, q), x)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, one round-to-nearest-even (bf16: 7 fraction bits, binades
    down to 2^-126, overflow to infinity)."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_binary(x, 7, -126)
    big = np.abs(r) >= 2.0 ** 128
    r = np.where(big, np.copysign(np.inf, x), r)
    r = np.where(np.isnan(x), np.nan, r)
    bits = r.astype(np.float32).view(np.uint32)    # r is a bf16 value: the cast is exact
    out = (bits >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), out)


def f64_to_bf16_value(x) -> np.ndarray:
    return bf16_to_f64(f64_to_bf16(x))


# ------------------------------------------------------------------------------------------------
# E4M3 (OFP8 "FN")

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte -> float64.  exp field 0: m * 2^-9; else (1 + m/8) * 2^(e-7); S.1111.111 -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(x) -> np.ndarray:
    """fp32 -> E4M3 byte: round to nearest, ties to even, saturating at 448; NaN -> 0x7F.

    The sign bit is carried over unchanged (so a negative value that rounds to zero gives 0x80).
    Reading of "saturating round-to-nearest-even": magnitudes above 448 -- including the interval
    (448, 464] that RNE would send to 448 anyway and everything beyond -- encode as 448 (0x7E).
    """
    x = f32_to_f64(x)
    nan = np.isnan(x)
    a = np.abs(np.where(nan, 0.0, x))
    r = _round_binary(a, 3, -6)                      # 3 fraction bits, min normal 2^-6
    r = np.minimum(r, E4M3_MAX)
    _, e = np.frexp(r)
    be = np.maximum(e - 1, -6)                       # binade exponent (subnormals share -6)
    normal = r >= 2.0 ** -6
    mant = np.where(normal, np.ldexp(r, -be) - 1.0, np.ldexp(r, 9))   # fraction*8 or m
    mant = np.where(normal, mant * 8.0, mant)
    field_e = np.where(normal, be + 7, 0)
    code = (field_e.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


# ------------------------------------------------------------------------------------------------
# INT8


def int8_encode(x_f32, inv_f32) -> np.ndarray:
    """Symmetric INT8 code: round-half-even of the fp32 product x*inv, clipped to [-127, 127]."""
    prod = np.asarray(x_f32, dtype=np.float32) * np.float32(inv_f32)   # fp32 multiply
    return np.clip(np.rint(prod.astype(np.float64)), -127, 127).astype(np.int8)


# ------------------------------------------------------------------------------------------------
# E2M1 and E8M0 (OCP MX v1.0)

E2M1_MAX = 6.0
E2M1_EMAX = 2            # exponent of the largest E2M1 binade (4 = 2^2)


def e2m1_decode(codes) -> np.ndarray:
    """4-bit code S.EE.M -> float64: exp 0 -> M*0.5; else (1 + M/2) * 2^(E-1)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, e - 1))
    return s * mag


def e2m1_encode(x) -> np.ndarray:
    """float64 -> E2M1 4-bit code (in the low nibble of a uint8): RNE, saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = np.minimum(_round_binary(a, 1, 0), E2M1_MAX)  # 1 fraction bit, min normal 2^0
    _, e = np.frexp(r)
    be = np.maximum(e - 1, 0)
    normal = r >= 1.0
    mant = np.where(normal, (np.ldexp(r, -be) - 1.0) * 2.0, r * 2.0)
    field_e = np.where(normal, be + 1, 0)
    code = (field_e.astype(np.int64) << 1) | np.rint(mant).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x8, 0)
    return code.astype(np.uint8)


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 0xFF, np.nan, np.ldexp(1.0, c - 127))


def e8m0_shared_exponent(amax) -> np.ndarray:
    """Shared scale of one 32-element block (OCP MX v1.0): X = 2^(floor(log2 amax) - emax_elem),
    emax_elem = 2 for E2M1, returned as the biased E8M0 code (127 + exponent), clamped to the
    representable [-127, 127].  An all-zero block takes X = 1 (code 127)."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    k = np.where(a > 0, (e - 1) - E2M1_EMAX, 0)
    return (np.clip(k, -127, 127) + 127).astype(np.uint8)
