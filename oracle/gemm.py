"""Scaled low-precision linear layers (test infrastructure only).

[TRIM] "运行速度如何", note under the table: on the RTX 4090 the transformer's linear layers run as
FP8 matmuls with one scale per tensor, the scales applied to the output of a fused kernel.  Here:
y = (sum_k dec(a_mk) dec(w_nk)) * fp32(s_a * s_w) + b.

The float64 sum is exact: every E4M3 x E4M3 product is a multiple of 2^-18 below 2^18, so a sum of
up to 2^17 of them needs fewer than 53 bits; any summation order gives the same float64 (the
library matmul is used only as a sum).  For the 4-bit weights (E2M1 x 2^k) the products are
multiples of 2^(-10 + k_min) and the same argument holds for the block scales drawn here.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _sp_erf

from .codecs import e4m3_decode, e2m1_decode, e8m0_decode
from .quant import unpack_e2m1


def gemm_acc_fp8(a_codes, w_codes) -> np.ndarray:
    """Exact accumulator acc[m][n] = sum_k dec(a[m][k]) * dec(w[n][k]) (float64)."""
    A = e4m3_decode(a_codes)
    W = e4m3_decode(w_codes)
    return A @ W.T


def output_scale(s_a, s_w) -> np.float32:
    """The single fp32 factor applied to the accumulator: fp32(s_a * s_w)."""
    return np.float32(s_a) * np.float32(s_w)


def gemm_fp8(a_codes, s_a, w_codes, s_w, bias=None) -> np.ndarray:
    """y = acc * fp32(s_a*s_w) + bias, float64 [M][N]."""
    y = gemm_acc_fp8(a_codes, w_codes) * float(output_scale(s_a, s_w))
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def dequant_mxfp4(packed, e8) -> np.ndarray:
    """Packed E2M1 [N][K/2] + E8M0 [N][K/32] -> float64 [N][K]."""
    codes = unpack_e2m1(packed)
    N, K = codes.shape
    X = e8m0_decode(e8)
    return (e2m1_decode(codes).reshape(N, K // 32, 32) * X[..., None]).reshape(N, K)


def gemm_mxfp4(a_codes, s_a, w_packed, w_e8, bias=None) -> np.ndarray:
    """E4M3 activations (per-tensor scale s_a) times MXFP4 weights: y = s_a * sum dec(a) dec(w) + b."""
    y = (e4m3_decode(a_codes) @ dequant_mxfp4(w_packed, w_e8).T) * float(np.float32(s_a))
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def gemm_mxfp4_w4a4(a_packed, a_e8, w_packed, w_e8, bias=None) -> np.ndarray:
    """Both operands MXFP4 (E2M1 elements, an E8M0 scale per 32 consecutive K; the activations
    quantized per token row exactly as the weights are per output row): y = sum_k dec(a) dec(w) + b,
    float64 [M][N].  [farwalk] post 6/8 runs the transformer's linear layers in 4 bits on both
    operands (NVFP4 on Blackwell); OCP MX v1.0 fixes the block format used here instead.  No
    per-tensor factor: the block scales carry the magnitudes.  Each product is a multiple of
    2^(e_a + e_w - 256) below 36 * 2^(e_a + e_w - 254), so the float64 sum is exact while the block
    exponents of a row pair span fewer than about 45 binades, as they do for every input drawn here."""
    y = dequant_mxfp4(a_packed, a_e8) @ dequant_mxfp4(w_packed, w_e8).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def gelu(u) -> np.ndarray:
    """Exact (erf) GELU: u * (1 + erf(u / sqrt 2)) / 2 in float64 (scipy's erf as the library
    primitive).  Reading: the workloads name a GELU MLP; the erf form is taken, not tanh."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + _sp_erf(u / math.sqrt(2.0)))
