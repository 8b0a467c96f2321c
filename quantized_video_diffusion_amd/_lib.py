"""ctypes view of the C ABI in include/qvd.h (argument marshalling only).

The shared library is the in-tree ``libqvd.so`` built by ``build.py``.  Loading fails loudly when it
is missing: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqvd.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qvd.h")

QVD_OK, QVD_EINVAL, QVD_ESHAPE, QVD_EALIGN, QVD_EWORKSPACE, QVD_EUNSUPPORTED, QVD_EHIP = (
    0, -1, -2, -3, -4, -5, -6)
(QVD_EPI_F32, QVD_EPI_BF16, QVD_EPI_RESID_GATE, QVD_EPI_GELU, QVD_EPI_QKV, QVD_EPI_GELU_E4M3,
 QVD_EPI_GELU_MXFP4) = range(7)
QVD_W_FP8, QVD_W_MXFP4, QVD_W_MXFP4_A4 = 0, 1, 2
QVD_PROBE_FP8, QVD_PROBE_FP4, QVD_PROBE_INT8, QVD_PROBE_F16 = 0, 1, 2, 3
QVD_PROBE_INT8_32, QVD_PROBE_F16_32, QVD_PROBE_FP8_16 = 4, 5, 6
(QVD_STAGE_MODULATE1, QVD_STAGE_QKV, QVD_STAGE_VT, QVD_STAGE_ATTN, QVD_STAGE_OQUANT, QVD_STAGE_OPROJ,
 QVD_STAGE_MODULATE2, QVD_STAGE_UP, QVD_STAGE_GQUANT, QVD_STAGE_ALL) = range(1, 11)
WS_SLOTS = ("h", "q8", "k8", "vt", "vt_tile_exp", "vt_head_exp", "o", "g", "g8", "h_e8m0", "g_e8m0",
            "q_scale", "k_scale", "scales", "sel_idx", "sel_cnt")
ABI_VERSION = 2

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_f32 = C.c_float
_sz = C.c_size_t


class Epilogue(C.Structure):
    _fields_ = [
        ("mode", _i32), ("n_heads", _i32),
        ("out_f32", _p), ("out_bf16", _p), ("resid", _p), ("gate", _p), ("amax_partials", _p),
        ("q8", _p), ("k8", _p), ("v", _p), ("q_scale", _p), ("k_scale", _p), ("v_exp", _p),
        ("out_e4m3", _p), ("out_scale", _p), ("out_e2m1", _p), ("out_e8m0", _p),
    ]


class SamplerConfig(C.Structure):
    _fields_ = [("n_steps", _i32), ("timesteps", _p), ("shift_video", _f32), ("shift_audio", _f32),
                ("L_video", _i32)]


class BlockParams(C.Structure):
    _fields_ = [
        ("version", _i32), ("d", _i32), ("n_heads", _i32), ("head_dim", _i32), ("mlp", _i32),
        ("weight_format", _i32),
        ("w_qkv", _p), ("w_o", _p), ("w_up", _p), ("w_down", _p),
        ("e8m0_qkv", _p), ("e8m0_o", _p), ("e8m0_up", _p), ("e8m0_down", _p),
        ("s_qkv", _p), ("s_o", _p), ("s_up", _p), ("s_down", _p),
        ("b_qkv", _p), ("b_o", _p), ("b_up", _p), ("b_down", _p),
        ("act_scale", _p),
        ("ln_eps", _f32),
    ]


SIGNATURES = {
    "qvd_abi_version": (C.c_int, []),
    "qvd_last_error": (C.c_char_p, []),
    "qvd_init": (C.c_int, []),
    "qvd_inject_launch_failure": (C.c_int, [C.c_int32]),
    "qvd_quant_ws_bytes": (_sz, [_i64]),
    "quant_fp8_per_tensor": (C.c_int, [_p, _i64, _p, _p, _p, _p, _sz, _p]),
    "quant_int8_qk": (C.c_int, [_p, _i32, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "qvd_adaln_project": (C.c_int, [_f32, _p, _i32, _p, _p, _i32, _p, _p]),
    "qvd_adaln_project_stack": (C.c_int, [_f32, _p, _i32, _p, _p, _i32, _i32, _p, _p]),
    "qvd_adaln_modulate_ws_bytes": (_sz, [_i32, _i32]),
    "adaln_modulate": (C.c_int, [_p, _i32, _i32, _p, _i32, _f32, _p, _p, _p, _p, _sz, _p]),
    "adaln_modulate_mxfp4": (C.c_int, [_p, _i32, _i32, _p, _i32, _f32, _p, _p, _p]),
    "adaln_modulate_noalloc": (C.c_int, [_p, _i32, _i32, _p, _i32, _f32, _p, _p, _p, _p]),
    "qvd_sparse_attn_ws_bytes": (_sz, [_i32, _i32]),
    "sparse_attn": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _p, _p, _i32, _f32, _p, _p, _p, _sz,
                              _p]),
    "qvd_vt_from_bf16": (C.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "qvd_vt_unify": (C.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "qvd_sparse_attn_vt": (C.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _f32, _p, _p,
                                     _p]),
    "qvd_sparse_attn_vt_e4m3": (C.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _f32, _p,
                                          _p, _p]),
    "qvd_sparse_attn_vt_mxfp4": (C.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _f32,
                                           _p, _p, _p]),
    "qvd_select_tiles_ws_bytes": (_sz, [_i32, _i32]),
    "qvd_select_tiles": (C.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p, _sz, _p]),
    "qvd_qk_int32_tile": (C.c_int, [_p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "qvd_gemm_tiles": (_i64, [_i32, _i32]),
    "qvd_gemm_fp8": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, C.POINTER(Epilogue), _p]),
    "qvd_gemm_mxfp4": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, C.POINTER(Epilogue), _p]),
    "qvd_gemm_mxfp4_w4a4": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, C.POINTER(Epilogue), _p]),
    "qvd_block_ws_bytes": (_sz, [C.POINTER(BlockParams), _i32]),
    "dit_block_forward": (C.c_int, [C.POINTER(BlockParams), _p, _p, _i32, _p, _p, _i32, _p, _sz, _p]),
    "qvd_block_forward_until": (C.c_int, [C.POINTER(BlockParams), _p, _p, _i32, _p, _p, _i32, _i32, _p,
                                          _sz, _p]),
    "qvd_block_ws_layout": (C.c_int, [C.POINTER(BlockParams), _i32, C.POINTER(_i64)]),
    "qvd_quant_mxfp4": (C.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "qvd_amax_update": (C.c_int, [_p, _i64, _p, _p]),
    "qvd_clip_count": (C.c_int, [_p, _i64, _p, _p, _p]),
    "qvd_amax_update_bf16": (C.c_int, [_p, _i64, _p, _p]),
    "qvd_clip_count_bf16": (C.c_int, [_p, _i64, _p, _p, _p]),
    "adaln_layernorm_modulate_f32": (C.c_int, [_p, _i32, _i32, _p, _i32, _f32, _p, _p]),
    "qvd_calibrated_scale": (C.c_int, [_p, _p, _i32, _p]),
    "qvd_sampler_sigmas": (C.c_int, [C.POINTER(SamplerConfig), _i32, C.POINTER(C.c_double)]),
    "qvd_mfma_probe": (C.c_int, [_i32, _i32, _i32, _p, _p, _p]),
    "qvd_mfma_probe_flops": (C.c_double, [_i32, _i32, _i32]),
    "qvd_wall_clock_khz": (_i32, []),
    "qvd_sampler_start": (C.c_int, [C.POINTER(SamplerConfig), _p, _i32, _i32, _p, _p, _p]),
    "qvd_sampler_step": (C.c_int, [C.POINTER(SamplerConfig), _i32, _p, _p, _p, _p, _i32, _i32, _p]),
    "qvd_timing_enable": (C.c_int, [C.c_int]),
    "qvd_timing_report": (C.c_int, [C.c_char_p, _sz]),
}


class QvdError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status}: {msg}")
        self.status = status


_LIB = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                "g.build()' or python quantized_video_diffusion_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.qvd_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libqvd ABI {L.qvd_abi_version()} != binding {ABI_VERSION}")
        _LIB = L
    return _LIB


def call(name: str, *args) -> int:
    st = getattr(lib(), name)(*args)
    if st != QVD_OK:
        raise QvdError(name, st, lib().qvd_last_error().decode(errors="replace"))
    return st


def header_functions() -> list[str]:
    """Names of the functions include/qvd.h declares (for the export check)."""
    import re
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))
