"""One quantized DiT block, and the 42-block stack over the sampler timesteps (test infra only).

The pages describe the model as a diffusion transformer that denoises the video and audio latents
together ([TRIM] "Trim 改变了什么", first paragraph), conditioned per block by six AdaLN modulation
vectors (timestep-conditioning bullet), with FP8 per-tensor linear layers and INT8 query/key
scores ([TRIM] "运行速度如何", note under the table) and 80% attention sparsity (training bullet).

Reading of the block (the pages give no topology): the adaLN-Zero pre-norm DiT block
  h1 = E4M3(LN(x)(1 + scale1) + shift1)                     per-tensor scale s1
  qkv = bf16(h1 W_qkv^T * s1 s_qkv + b_qkv)                 columns: Q | K | V, heads of 128
  Q8, K8 = INT8 per (head, 128-token tile) of the bf16 Q, K
  O = bf16(block-sparse softmax(Q8 K8^T sQ sK / sqrt 128) V)
  x1 = bf16(x + gate1 * (E4M3(O) W_o^T s_O s_o + b_o))
  h2 = E4M3(LN(x1)(1 + scale2) + shift2)
  g = bf16(GELU(h2 W_up^T s2 s_up + b_up))
  x2 = bf16(x1 + gate2 * (E4M3(g) W_down^T s_g s_down + b_down))
with no text cross-attention, rotary embedding or QK normalisation (none is on the pages).  Every
per-tensor activation scale is dynamic (amax of the tensor) unless static scales are given.
Residual sums are formed in float64 and rounded once to bf16.

fmt "w4a4" (both GEMM operands 4-bit, the pages' NVFP4 transformer in OCP MX form): the four GEMM
inputs are MXFP4 instead of E4M3 -- h1 and h2 quantize the fp32 modulated LayerNorm output, O and g
their bf16 tensors, each per token row and 32 channels -- and the weights are MXFP4; there are no
per-tensor activation scales.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64, f64_to_bf16, f32_to_f64
from .quant import quant_fp8_bf16, quant_int8_qk, quant_mxfp4_weight
from .adaln import adaln_modulate, adaln_modulate_mxfp4
from .gemm import gemm_fp8, gemm_mxfp4, gemm_mxfp4_w4a4, gelu
from .attention import sparse_attn

SITES = ("qkv", "o", "up", "down")   # the four quantized GEMM inputs of a block


def quantize_block_weights(wbits: dict) -> dict:
    """bf16 master weights -> E4M3 codes and per-tensor scales (dynamic amax/448 per tensor)."""
    out = {}
    for site in SITES:
        codes, s = quant_fp8_bf16(wbits["w_" + site])
        out["w_" + site] = codes
        out["s_" + site] = s
    return out


def _linear(a_codes, s_a, qw: dict, site: str, fmt: str):
    b = qw.get("b_" + site)
    if fmt == "w4a4":                       # a_codes = (packed E2M1, E8M0) of the activations
        return gemm_mxfp4_w4a4(a_codes[0], a_codes[1], qw["w_" + site], qw["e8_" + site], b)
    if fmt == "mxfp4":
        return gemm_mxfp4(a_codes, s_a, qw["w_" + site], qw["e8_" + site], b)
    return gemm_fp8(a_codes, s_a, qw["w_" + site], qw["s_" + site], b)


def dit_block(x_bits, mod_f32, qw: dict, kv_idx, kv_cnt, n_heads: int, eps: float = 1e-6,
              act_scales=None, fmt: str = "fp8", keep: bool = False):
    """x bf16 [L][d] -> bf16 [L][d].  ``qw`` holds the quantized weights (and optional fp32
    biases ``b_<site>``); ``act_scales`` = None (dynamic) or four static scales for the inputs of
    the QKV, out, up and down GEMMs (unused by fmt "w4a4").  With keep=True, returns (x2, dict of
    intermediates)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    L, d = x_bits.shape
    H, D = n_heads, d // n_heads
    st = (lambda k: None) if act_scales is None else (lambda k: act_scales[k])
    mod = f32_to_f64(mod_f32)
    gate1, gate2 = mod[2], mod[5]
    x = bf16_to_f64(x_bits)

    a4 = fmt == "w4a4"
    if a4:
        h1, s1 = adaln_modulate_mxfp4(x_bits, mod_f32, 0, eps), None
    else:
        h1, s1 = adaln_modulate(x_bits, mod_f32, 0, eps, st(0))
    qkv = f64_to_bf16(_linear(h1, s1, qw, "qkv", fmt))                 # [L][3d] bf16
    q8, sq = quant_int8_qk(qkv[:, :d], L, H, D)
    k8, sk = quant_int8_qk(qkv[:, d:2 * d], L, H, D)
    v = qkv[:, 2 * d:].reshape(L, H, D)
    o = f64_to_bf16(sparse_attn(q8, sq, k8, sk, v, kv_idx, kv_cnt)).reshape(L, d)
    o8, so = (quant_mxfp4_weight(o), None) if a4 else quant_fp8_bf16(o, st(1))
    y1 = _linear(o8, so, qw, "o", fmt)
    x1_bits = f64_to_bf16(x + gate1[None, :] * y1)

    if a4:
        h2, s2 = adaln_modulate_mxfp4(x1_bits, mod_f32, 1, eps), None
    else:
        h2, s2 = adaln_modulate(x1_bits, mod_f32, 1, eps, st(2))
    g = f64_to_bf16(gelu(_linear(h2, s2, qw, "up", fmt)))
    g8, sg = (quant_mxfp4_weight(g), None) if a4 else quant_fp8_bf16(g, st(3))
    y2 = _linear(g8, sg, qw, "down", fmt)
    x2_bits = f64_to_bf16(bf16_to_f64(x1_bits) + gate2[None, :] * y2)
    if not keep:
        return x2_bits
    inter = dict(h1=h1, s1=s1, qkv=qkv, q8=q8, sq=sq, k8=k8, sk=sk, o=o, o8=o8, so=so,
                 y1=y1, x1=x1_bits, h2=h2, s2=s2, g=g, g8=g8, sg=sg, y2=y2)
    return x2_bits, inter


def dit_stack_step(x_bits, mods: list, qws: list, masks: list, n_heads: int, eps: float = 1e-6):
    """One denoising step through the stack: x <- block_k(x) for k = 0 .. len(qws)-1."""
    for mod, qw, (idx, cnt) in zip(mods, qws, masks):
        x_bits = dit_block(x_bits, mod, qw, idx, cnt, n_heads, eps)
    return x_bits
