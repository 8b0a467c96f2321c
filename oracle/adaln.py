"""AdaLN timestep conditioning and the modulated LayerNorm (test infrastructure only).

[TRIM] "Trim 改变了什么", timestep-conditioning bullet: each block is conditioned on the diffusion
timestep through an AdaLN projection that turns the 2,688-dim time embedding into six modulation
vectors; Trim replaces the per-block projection by a 2,688->16 basis shared by all blocks and a
small per-block projection, both kept in fp16.

Readings of what the pages leave open:
* embedding: e(t) = [cos(t*f_i), sin(t*f_i)], f_i = 10000^(-i/(dim/2)), i < dim/2, dim = d; no MLP
  or SiLU in front of the basis; c = B e and mod = P_k c (+ b_k) are formed in float64 and the six
  vectors are handed on as fp32;
* the six vectors, in order: shift1, scale1, gate1 (attention branch), shift2, scale2, gate2 (MLP);
* modulate: LayerNorm over d without affine parameters, biased variance, eps passed as an fp32;
  y = ((x - mean) * (1/sqrt(var + eps))) * (1 + scale) + shift in float64, rounded once to fp32
  and quantized per tensor to E4M3.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64, fp16_to_f64, f64_to_f32, f32_to_f64
from .quant import quant_fp8_per_tensor, quant_mxfp4

N_MOD = 6


def timestep_embedding(t: float, dim: int) -> np.ndarray:
    half = dim // 2
    freqs = np.exp(-np.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    arg = float(t) * freqs
    return np.concatenate([np.cos(arg), np.sin(arg)])


def adaln_basis_coords(t: float, basis_bits) -> np.ndarray:
    """c = B e(t): the 16 coordinates of the timestep in the shared basis (float64)."""
    B = fp16_to_f64(basis_bits)
    return B @ timestep_embedding(t, B.shape[1])


def adaln_project(t: float, basis_bits, proj_bits, bias_bits=None) -> np.ndarray:
    """Modulation table [6][d] fp32 of one block at timestep t: P_k (B e(t)) (+ b_k)."""
    c = adaln_basis_coords(t, basis_bits)
    P = fp16_to_f64(proj_bits)
    m = P @ c
    if bias_bits is not None:
        m = m + fp16_to_f64(bias_bits)
    return f64_to_f32(m).reshape(N_MOD, -1)


def layernorm_modulate(x_bits, mod_f32, half: int, eps: float) -> np.ndarray:
    """fp32 y = LN(x) * (1 + scale) + shift for x bf16 [L][d]; half 0 uses (shift1, scale1),
    half 1 uses (shift2, scale2)."""
    x = bf16_to_f64(x_bits)
    mod = f32_to_f64(mod_f32)
    shift, scale = mod[3 * half], mod[3 * half + 1]
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    eps64 = float(np.float32(eps))
    rstd = 1.0 / np.sqrt(var + eps64)
    y = ((x - mu) * rstd) * (1.0 + scale) + shift
    return f64_to_f32(y)


def adaln_modulate(x_bits, mod_f32, half: int, eps: float = 1e-6, act_scale=None):
    """-> (E4M3 codes [L][d], per-tensor scale s)."""
    return quant_fp8_per_tensor(layernorm_modulate(x_bits, mod_f32, half, eps), act_scale)


def adaln_modulate_mxfp4(x_bits, mod_f32, half: int, eps: float = 1e-6):
    """-> (packed E2M1 [L][d/2], E8M0 [L][d/32]): the fp32 modulated LayerNorm output quantized per
    token row and 32 consecutive channels (MXFP4 activations; no per-tensor scale)."""
    return quant_mxfp4(layernorm_modulate(x_bits, mod_f32, half, eps))
