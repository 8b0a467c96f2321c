"""MI355X (gfx950) quantized DiT-block forward: the FastH3 / FastH3 Trim hot path.

The computation lives in ``libqvd.so`` (HIP kernels behind the C ABI of ``include/qvd.h``); this
package only marshals torch device tensors into those calls.  Importing it does not load the
library; the first call does, and fails loudly if the library has not been built.
"""
from . import _lib  # noqa: F401
from .ops import (  # noqa: F401
    quant_fp8_per_tensor, quant_int8_qk, adaln_project, adaln_modulate, adaln_modulate_mxfp4, sparse_attn,
    adaln_modulate_noalloc,
    sparse_attn_vt, sparse_attn_vt_e4m3, sparse_attn_vt_mxfp4, qk_int32_tile, select_tiles, VT, VTiles,
    vt_from_bf16, vt_unify,
    gemm_fp8, gemm_mxfp4, gemm_mxfp4_w4a4, gemm_tiles, quant_mxfp4, amax_update, clip_count, BlockWeights,
    quantize_block_weights, block_ws_bytes, dit_block_forward, block_forward_until, block_intermediates, from_bits, to_bits, timing_enable, timing_report,
    calibrated_scale, Sampler, mfma_probe, layernorm_modulate_f32, inject_launch_failure, capture_graph,
)
