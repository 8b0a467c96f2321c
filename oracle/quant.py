"""Quantizers of the hot path (test infrastructure only).

* Per-tensor FP8: [TRIM] "运行速度如何", note under the table -- the FP8 path uses one scale per
  tensor and applies it to the matmul output instead of per-token / per-channel FP8 scaling.
  Reading (the pages give no rule): s = amax/448, the codes are E4M3(x * 448/amax) computed in
  fp32; a dynamic scale takes amax over the tensor itself, a static (calibrated) one is passed in
  and the codes are E4M3(x * (1/s)).  An all-zero tensor takes s = 1.
* INT8 query/key: same note -- Q and K are quantized to INT8 for the score computation.  Reading:
  one symmetric scale per (head, 128-token tile), s = amax/127 over the tile's valid rows, codes
  rint(x * 127/amax) clipped to +-127; an all-zero tile takes s = 1.
* MXFP4 weights (E2M1 + one E8M0 scale per 32 consecutive inputs): the 4-bit transformer format of
  [FARWALK] post 6/8 and [TRIM] "ComfyUI 重打包包含什么", in the OCP MX form.
* Static activation-scale calibration and clipping: [FARWALK] post 6/8 -- under scales that were
  not calibrated the activations clip (40 of 42 blocks; one block at 137x the limit), so every
  4-bit layer was calibrated on 1,000 prompts.  Reading: s = amax over the calibration set / 448,
  raised by one fp32 ulp when s*448 would fall below that amax; an element clips when |x| > s*448.
"""
from __future__ import annotations

import numpy as np

from .codecs import (bf16_to_f64, e4m3_encode, int8_encode, e2m1_encode, e8m0_shared_exponent,
                     E4M3_MAX)

TILE = 128


def fp8_scale_dynamic(amax_f32: float) -> tuple[np.float32, np.float32]:
    """(s, inv) for a dynamic per-tensor scale: s = fp32(amax/448), inv = fp32(448/amax)."""
    a = np.float32(amax_f32)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a) / np.float32(E4M3_MAX), np.float32(E4M3_MAX) / np.float32(a)


def quant_fp8_per_tensor(x_f32, scale_in=None):
    """fp32 values -> (E4M3 codes, s).  Dynamic when scale_in is None, else static."""
    x = np.asarray(x_f32, dtype=np.float32)
    if scale_in is None:
        amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
        s, inv = fp8_scale_dynamic(amax)
    else:
        s = np.float32(scale_in)
        inv = np.float32(1.0) / s
    return e4m3_encode(x * inv), s


def quant_fp8_with_amax(x_f32, amax_f32):
    """The dynamic per-tensor rule applied to part of a tensor whose amax (over the whole tensor) is
    given: codes E4M3(x * fp32(448/amax)), s = fp32(amax/448).  Lets rows of a large tensor be
    checked one by one once its amax is known."""
    x = np.asarray(x_f32, dtype=np.float32)
    s, inv = fp8_scale_dynamic(amax_f32)
    return e4m3_encode(x * inv), s


def quant_fp8_bf16(x_bits, scale_in=None):
    """Per-tensor FP8 of a bf16 tensor (given as bit patterns)."""
    return quant_fp8_per_tensor(bf16_to_f64(x_bits).astype(np.float32), scale_in)


def quant_int8_qk(x_bits, L: int, H: int, head_dim: int = 128, tile: int = TILE):
    """bf16 [L][H][head_dim] -> (int8 codes [L][H][head_dim], scales fp32 [H][ceil(L/tile)])."""
    x = bf16_to_f64(np.asarray(x_bits).reshape(L, H, head_dim)).astype(np.float32)
    T = (L + tile - 1) // tile
    q = np.zeros((L, H, head_dim), dtype=np.int8)
    s = np.ones((H, T), dtype=np.float32)
    for h in range(H):
        for i in range(T):
            rows = slice(i * tile, min(L, (i + 1) * tile))
            blk = x[rows, h, :]
            a = np.float32(np.abs(blk).max())
            if a == 0:
                inv = np.float32(1.0)
                s[h, i] = np.float32(1.0)
            else:
                inv = np.float32(127.0) / a
                s[h, i] = a / np.float32(127.0)
            q[rows, h, :] = int8_encode(blk, inv)
    return q, s


def quant_mxfp4_weight(w_bits):
    """bf16 master weight [N][K] -> (packed E2M1 [N][K/2] uint8, E8M0 scales [N][K/32] uint8):
    quant_mxfp4 of the bf16 values."""
    return quant_mxfp4(bf16_to_f64(w_bits))


def quant_mxfp4(x):
    """Real values [N][K] (the exact values given: fp32 or float64, not rounded further) ->
    (packed E2M1 [N][K/2] uint8, E8M0 scales [N][K/32] uint8).

    Per row and per 32 consecutive K: X = 2^(floor(log2 amax) - 2), element = E2M1(x / X) (RNE,
    saturating at 6).  Element 2j sits in the low nibble of byte j, element 2j+1 in the high one.
    The same rule quantizes activations per token row (W4A4: both GEMM operands MXFP4).
    """
    w = np.asarray(x, dtype=np.float64)
    N, K = w.shape
    assert K % 32 == 0
    blocks = w.reshape(N, K // 32, 32)
    e8 = e8m0_shared_exponent(np.abs(blocks).max(axis=-1))
    X = np.ldexp(1.0, e8.astype(np.int64) - 127)[..., None]
    codes = e2m1_encode(blocks / X).reshape(N, K)
    packed = (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)
    return packed.astype(np.uint8), e8


def unpack_e2m1(packed):
    p = np.asarray(packed, dtype=np.uint8)
    N, Kh = p.shape
    out = np.empty((N, 2 * Kh), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def calibrated_scale(amax: float) -> np.float32:
    """Static per-tensor scale from a calibration amax: s = fp32(amax/448), raised by one fp32
    ulp if s*448 (exact, float64) would be below amax, so that the calibration set never clips."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    s = a / np.float32(E4M3_MAX)
    if float(s) * E4M3_MAX < float(a):
        s = np.nextafter(s, np.float32(np.inf))
    return np.float32(s)


def clip_count(x, s) -> int:
    """Elements with |x| > s*448 (float64 comparison): the ones a static scale s saturates."""
    return int(np.count_nonzero(np.abs(np.asarray(x, dtype=np.float64)) > float(s) * E4M3_MAX))
