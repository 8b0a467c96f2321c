"""Torch-facing wrappers of the C ABI, one per entry point and with the same names.

PyTorch supplies device memory and the current stream; every step of the computation runs in the
HIP kernels of libqvd.so.  Inputs are validated for dtype/shape/device here, allocation of outputs
and workspaces happens here, and the call goes straight to the library.
"""
from __future__ import annotations

import ctypes as C
import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib
from ._lib import call, Epilogue, BlockParams

SM_SCALE = 1.0 / math.sqrt(128.0)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, dtype, name, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


# When set (the GPU tests set it), every output and workspace this module allocates is first filled
# with 0xFF bytes -- NaN for bf16/fp32, -1 for int8/int32, 255 for codes -- so an element a kernel
# fails to write shows up in the comparison instead of passing on stale zeros.
POISON = False


def _out(shape, dtype, device):
    t = torch.empty(shape, dtype=dtype, device=device)
    if POISON and t.numel():
        t.view(torch.uint8).fill_(0xFF)
    return t


def _empty(shape, dtype, like):
    return _out(shape, dtype, like.device)


def from_bits(bits, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """Host 16-bit patterns (numpy uint16) -> device tensor of that 16-bit dtype."""
    import numpy as np
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to(device).view(dtype)


def to_bits(t: torch.Tensor):
    """Device 16-bit tensor -> host numpy uint16 patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view("uint16")


# ----------------------------------------------------------------------------------------------

def quant_fp8_per_tensor(x: torch.Tensor, scale_in: torch.Tensor | None = None):
    """bf16 tensor -> (E4M3 codes uint8 of the same shape, fp32 scale [1])."""
    _check(x, torch.bfloat16, "x")
    q = _empty(x.shape, torch.uint8, x)
    s = _empty((1,), torch.float32, x)
    n = x.numel()
    ws = _empty((_lib.lib().qvd_quant_ws_bytes(n),), torch.uint8, x)
    if scale_in is not None:
        _check(scale_in, torch.float32, "scale_in")
    call("quant_fp8_per_tensor", _ptr(x), n, _ptr(scale_in), _ptr(q), _ptr(s), _ptr(ws), ws.numel(),
         _stream())
    return q, s


def quant_int8_qk(x: torch.Tensor, n_heads: int, row_stride: int | None = None):
    """bf16 [L][H*128] (or [L][H][128]) -> (int8 [L][H][128], fp32 scales [H][ceil(L/128)])."""
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("x: expected a bf16 device tensor")
    if row_stride is None and not x.is_contiguous():
        raise ValueError("x: must be contiguous (or pass row_stride for a strided row view)")
    L = x.shape[0]
    rs = n_heads * 128 if row_stride is None else row_stride
    q = _out((L, n_heads, 128), torch.int8, x.device)
    s = _out((n_heads, (L + 127) // 128), torch.float32, x.device)
    call("quant_int8_qk", _ptr(x), L, n_heads, 128, 128, rs, _ptr(q), _ptr(s), _stream())
    return q, s


def adaln_project(t: float, basis: torch.Tensor, proj: torch.Tensor, bias=None) -> torch.Tensor:
    """fp16 basis [16][dt], proj [6d][16] (or [n][6d][16]) -> fp32 mod [6][d] (or [n][6][d])."""
    _check(basis, torch.float16, "basis")
    _check(proj, torch.float16, "proj")
    dt = basis.shape[1]
    stacked = proj.dim() == 3
    nb = proj.shape[0] if stacked else 1
    six_d = proj.shape[-2]
    d = six_d // 6
    mod = _out((nb, 6, d) if stacked else (6, d), torch.float32, basis.device)
    call("qvd_adaln_project_stack", float(t), _ptr(basis), dt, _ptr(proj), _ptr(bias), d, nb,
         _ptr(mod), _stream())
    return mod


def adaln_modulate(x: torch.Tensor, mod: torch.Tensor, half: int, eps: float = 1e-6,
                   act_scale: torch.Tensor | None = None):
    """bf16 [L][d] -> (E4M3 [L][d], fp32 scale [1])."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    L, d = x.shape
    q = _empty((L, d), torch.uint8, x)
    s = _empty((1,), torch.float32, x)
    ws = _empty((_lib.lib().qvd_adaln_modulate_ws_bytes(L, d),), torch.uint8, x)
    call("adaln_modulate", _ptr(x), L, d, _ptr(mod), half, float(eps), _ptr(act_scale), _ptr(q),
         _ptr(s), _ptr(ws), ws.numel(), _stream())
    return q, s


def adaln_modulate_noalloc(x: torch.Tensor, mod: torch.Tensor, half: int, q: torch.Tensor,
                           scale_out: torch.Tensor, eps: float = 1e-6,
                           act_scale: torch.Tensor | None = None):
    """adaln_modulate into caller-owned q (uint8 [L][d]) and scale_out (fp32 [1]); the library
    allocates nothing (its per-GPU scratch holds the workspace)."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    _check(q, torch.uint8, "q")
    _check(scale_out, torch.float32, "scale_out")
    L, d = x.shape
    call("adaln_modulate_noalloc", _ptr(x), L, d, _ptr(mod), half, float(eps), _ptr(act_scale), _ptr(q),
         _ptr(scale_out), _stream())
    return q, scale_out


def adaln_modulate_mxfp4(x: torch.Tensor, mod: torch.Tensor, half: int, eps: float = 1e-6):
    """bf16 [L][d] -> (packed E2M1 uint8 [L][d/2], E8M0 uint8 [L][d/32])."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    L, d = x.shape
    packed = _empty((L, d // 2), torch.uint8, x)
    e8 = _empty((L, d // 32), torch.uint8, x)
    call("adaln_modulate_mxfp4", _ptr(x), L, d, _ptr(mod), half, float(eps), _ptr(packed), _ptr(e8),
         _stream())
    return packed, e8


def sparse_attn(q8, q_scale, k8, k_scale, v, kv_idx, kv_cnt, sm_scale: float = SM_SCALE,
                want_amax: bool = False):
    """int8 Q/K [L][H][128], fp32 scales [H][T], bf16 V [L][H][128], int32 masks -> bf16 out."""
    L, H, D = q8.shape
    _check(q8, torch.int8, "q8")
    _check(k8, torch.int8, "k8")
    _check(v, torch.bfloat16, "v")
    _check(kv_idx, torch.int32, "kv_idx")
    _check(kv_cnt, torch.int32, "kv_cnt")
    out = _out((L, H, D), torch.bfloat16, q8.device)
    part = _out(q_scale.shape, torch.float32, q8.device) if want_amax else None
    ws = _out((_lib.lib().qvd_sparse_attn_ws_bytes(L, H),), torch.uint8, q8.device)
    call("sparse_attn", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), L, H, D,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out), _ptr(part),
         _ptr(ws), ws.numel(), _stream())
    return (out, part) if want_amax else out


@dataclass
class VTiles:
    """V^T as the QKV GEMM epilogue writes it: fp16 [H][128][T*128] with one power-of-two exponent
    per (head, 128-token tile), int32 [H][T]."""
    t: torch.Tensor
    tile_exp: torch.Tensor


@dataclass
class VT:
    """V^T as the attention reads it: fp16 [H][128][T*128] holding V 2^-exp[h], int32 exp [H]."""
    t: torch.Tensor
    exp: torch.Tensor


def vt_from_bf16(v: torch.Tensor) -> VTiles:
    """bf16 V [L][H][128] -> VTiles (the transpose sparse_attn applies to its V)."""
    _check(v, torch.bfloat16, "v")
    L, H, D = v.shape
    T = (L + 127) // 128
    vt = _out((H, 128, T * 128), torch.float16, v.device)
    te = _out((H, T), torch.int32, v.device)
    call("qvd_vt_from_bf16", _ptr(v), L, H, _ptr(vt), _ptr(te), _stream())
    return VTiles(vt, te)


def vt_unify(vt: VTiles) -> VT:
    """One exponent per head (qvd_vt_unify, in place on vt.t)."""
    H, _, Lp = vt.t.shape
    he = _out((H,), torch.int32, vt.t.device)
    call("qvd_vt_unify", _ptr(vt.t), Lp, H, _ptr(vt.tile_exp), _ptr(he), _stream())
    return VT(vt.t, he)


def _vt_args(vt: VT):
    _check(vt.t, torch.float16, "vt")
    _check(vt.exp, torch.int32, "vt.exp")
    return _ptr(vt.t), _ptr(vt.exp)


def sparse_attn_vt_e4m3(q8, q_scale, k8, k_scale, vt: VT, kv_idx, kv_cnt, out_scale,
                        sm_scale: float = SM_SCALE):
    """As sparse_attn_vt, returning the E4M3 codes of bf16 O under the static scale out_scale
    (a device fp32 [1] tensor) instead of O: uint8 [L][H][128]."""
    L, H, D = q8.shape
    _check(out_scale, torch.float32, "out_scale")
    out = _out((L, H, D), torch.uint8, q8.device)
    call("qvd_sparse_attn_vt_e4m3", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), *_vt_args(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out_scale), _ptr(out),
         _stream())
    return out


def sparse_attn_vt_mxfp4(q8, q_scale, k8, k_scale, vt: VT, kv_idx, kv_cnt, sm_scale: float = SM_SCALE):
    """As sparse_attn_vt, returning the MXFP4 codes of bf16 O per (token, head, 32 dims) instead of
    O: (packed E2M1 uint8 [L][H*64], E8M0 uint8 [L][H*4])."""
    L, H, D = q8.shape
    packed = _out((L, H * D // 2), torch.uint8, q8.device)
    e8 = _out((L, H * D // 32), torch.uint8, q8.device)
    call("qvd_sparse_attn_vt_mxfp4", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), *_vt_args(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(packed), _ptr(e8), _stream())
    return packed, e8


def sparse_attn_vt(q8, q_scale, k8, k_scale, vt: VT, kv_idx, kv_cnt, sm_scale: float = SM_SCALE,
                   want_amax: bool = False):
    """As sparse_attn, with V given transposed (VT: fp16 V^T [H][128][ceil(L/128)*128] and the head
    exponents)."""
    L, H, D = q8.shape
    out = _out((L, H, D), torch.bfloat16, q8.device)
    part = _out(q_scale.shape, torch.float32, q8.device) if want_amax else None
    call("qvd_sparse_attn_vt", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), *_vt_args(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out), _ptr(part),
         _stream())
    return (out, part) if want_amax else out


def qk_int32_tile(q8, k8, h: int, i: int, j: int) -> torch.Tensor:
    L, H, _ = q8.shape
    out = _out((128, 128), torch.int32, q8.device)
    call("qvd_qk_int32_tile", _ptr(q8), _ptr(k8), L, H, h, i, j, _ptr(out), _stream())
    return out


def gemm_tiles(M: int, N: int) -> int:
    return int(_lib.lib().qvd_gemm_tiles(M, N))


def gemm_fp8(a, s_a, w, s_w, bias=None, mode: int = _lib.QVD_EPI_F32, out=None, resid=None,
             gate=None, amax_partials=None, n_heads: int = 0, out_scale=None):
    """E4M3 a [M][K] x E4M3 w [N][K] with the per-tensor scales fused in the epilogue.

    mode F32/BF16/GELU: returns the output tensor; RESID_GATE: writes ``out`` (may be ``resid``);
    QKV: returns (q8, k8, v, q_scale, k_scale)."""
    _check(w, torch.uint8, "w")
    return _gemm("qvd_gemm_fp8", a, s_a, w, s_w, w.shape[0], bias, mode, out, resid, gate,
                 amax_partials, n_heads, out_scale)


def gemm_mxfp4(a, s_a, w_packed, e8m0, bias=None, mode: int = _lib.QVD_EPI_F32, out=None,
               resid=None, gate=None, amax_partials=None, n_heads: int = 0, out_scale=None):
    """E4M3 a [M][K] (scale s_a) x MXFP4 weights (packed E2M1 [N][K/2] + E8M0 [N][K/32])."""
    _check(w_packed, torch.uint8, "w_packed")
    _check(e8m0, torch.uint8, "e8m0")
    return _gemm("qvd_gemm_mxfp4", a, s_a, w_packed, e8m0, w_packed.shape[0], bias, mode, out, resid,
                 gate, amax_partials, n_heads, out_scale)


def gemm_mxfp4_w4a4(a_packed, a_e8m0, w_packed, w_e8m0, bias=None, mode: int = _lib.QVD_EPI_F32,
                    out=None, resid=None, gate=None, amax_partials=None, n_heads: int = 0,
                    out_scale=None):
    """MXFP4 activations (packed E2M1 [M][K/2] + E8M0 [M][K/32], as quant_mxfp4 makes them) x
    MXFP4 weights (packed E2M1 [N][K/2] + E8M0 [N][K/32]); no per-tensor factor."""
    for t, name in ((a_e8m0, "a_e8m0"), (w_packed, "w_packed"), (w_e8m0, "w_e8m0")):
        _check(t, torch.uint8, name)
    return _gemm("qvd_gemm_mxfp4_w4a4", a_packed, a_e8m0, w_packed, w_e8m0, w_packed.shape[0], bias,
                 mode, out, resid, gate, amax_partials, n_heads, out_scale, packed_a=True)


def _gemm(fn, a, s_a, w, extra, N, bias, mode, out, resid, gate, amax_partials, n_heads, out_scale=None,
          packed_a=False):
    M, K = a.shape
    if packed_a:
        K *= 2
    _check(a, torch.uint8, "a")
    e = Epilogue()
    e.mode = mode
    ret = None
    if mode == _lib.QVD_EPI_F32:
        out = _out((M, N), torch.float32, a.device) if out is None else out
        e.out_f32 = out.data_ptr()
        ret = out
    elif mode in (_lib.QVD_EPI_BF16, _lib.QVD_EPI_GELU):
        out = _out((M, N), torch.bfloat16, a.device) if out is None else out
        e.out_bf16 = out.data_ptr()
        if amax_partials is not None:
            e.amax_partials = amax_partials.data_ptr()
        ret = out
    elif mode == _lib.QVD_EPI_GELU_E4M3:
        out = _out((M, N), torch.uint8, a.device) if out is None else out
        _check(out, torch.uint8, "out")
        _check(out_scale, torch.float32, "out_scale")
        e.out_e4m3 = out.data_ptr()
        e.out_scale = out_scale.data_ptr()
        ret = out
    elif mode == _lib.QVD_EPI_GELU_MXFP4:
        packed = _out((M, N // 2), torch.uint8, a.device)
        e8 = _out((M, N // 32), torch.uint8, a.device)
        e.out_e2m1 = packed.data_ptr()
        e.out_e8m0 = e8.data_ptr()
        ret = (packed, e8)
    elif mode == _lib.QVD_EPI_RESID_GATE:
        e.out_bf16 = out.data_ptr()
        e.resid = resid.data_ptr()
        e.gate = gate.data_ptr()
        ret = out
    elif mode == _lib.QVD_EPI_QKV:
        H = n_heads
        T = (M + 127) // 128
        q8 = _out((M, H, 128), torch.int8, a.device)
        k8 = _out(q8.shape, q8.dtype, q8.device)
        v = VTiles(_out((H, 128, T * 128), torch.float16, a.device), _out((H, T), torch.int32, a.device))
        qs = _out((H, T), torch.float32, a.device)
        ks = _out(qs.shape, qs.dtype, qs.device)
        e.n_heads = H
        e.q8, e.k8, e.v, e.q_scale, e.k_scale, e.v_exp = (q8.data_ptr(), k8.data_ptr(), v.t.data_ptr(),
                                                          qs.data_ptr(), ks.data_ptr(),
                                                          v.tile_exp.data_ptr())
        ret = (q8, k8, v, qs, ks)
    call(fn, _ptr(a), _ptr(s_a), _ptr(w), _ptr(extra), _ptr(bias), M, N, K, C.byref(e), _stream())
    return ret


def quant_mxfp4(w: torch.Tensor):
    """bf16 [N][K] -> (packed E2M1 uint8 [N][K/2], E8M0 uint8 [N][K/32])."""
    _check(w, torch.bfloat16, "w")
    N, K = w.shape
    packed = _out((N, K // 2), torch.uint8, w.device)
    e8 = _out((N, K // 32), torch.uint8, w.device)
    call("qvd_quant_mxfp4", _ptr(w), N, K, _ptr(packed), _ptr(e8), _stream())
    return packed, e8


def amax_update(x: torch.Tensor, amax: torch.Tensor):
    """amax (device fp32 [1]) <- max(amax, max|x|) for fp32 or bf16 x."""
    if x.dtype == torch.bfloat16:
        _check(x, torch.bfloat16, "x")
        call("qvd_amax_update_bf16", _ptr(x), x.numel(), _ptr(amax), _stream())
        return
    _check(x, torch.float32, "x")
    call("qvd_amax_update", _ptr(x), x.numel(), _ptr(amax), _stream())


def clip_count(x: torch.Tensor, scale: torch.Tensor, count: torch.Tensor):
    """count (device int64 [1]) += #{|x| > 448 scale} for fp32 or bf16 x."""
    if x.dtype == torch.bfloat16:
        _check(x, torch.bfloat16, "x")
        call("qvd_clip_count_bf16", _ptr(x), x.numel(), _ptr(scale), _ptr(count), _stream())
        return
    _check(x, torch.float32, "x")
    call("qvd_clip_count", _ptr(x), x.numel(), _ptr(scale), _ptr(count), _stream())


def layernorm_modulate_f32(x: torch.Tensor, mod: torch.Tensor, half: int, eps: float = 1e-6) -> torch.Tensor:
    """bf16 [L][d] -> fp32 [L][d]: the modulated LayerNorm values the modulate quantizers encode."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    L, d = x.shape
    y = _out((L, d), torch.float32, x.device)
    call("adaln_layernorm_modulate_f32", _ptr(x), L, d, _ptr(mod), half, float(eps), _ptr(y), _stream())
    return y


# ----------------------------------------------------------------------------------------------
# block

def calibrated_scale(amax: torch.Tensor) -> torch.Tensor:
    """Device fp32 calibration maxima [n] -> their static per-tensor scales [n] (qvd_calibrated_scale)."""
    _check(amax, torch.float32, "amax")
    s = _out(amax.shape, torch.float32, amax.device)
    call("qvd_calibrated_scale", _ptr(amax), _ptr(s), amax.numel(), _stream())
    return s


@dataclass
class BlockWeights:
    """Device weights of one block.  FP8: E4M3 codes [N][K] + fp32 scale [1] per site.
    MXFP4 and MXFP4_A4 (W4A4): packed E2M1 [N][K/2] + E8M0 [N][K/32] per site (scales unused)."""
    d: int
    n_heads: int
    mlp: int
    fmt: int
    w: dict                      # site -> codes
    s: dict = field(default_factory=dict)     # site -> fp32 [1]
    e8: dict = field(default_factory=dict)    # site -> E8M0
    b: dict = field(default_factory=dict)     # site -> fp32 [N] or absent
    act_scale: torch.Tensor | None = None     # fp32 [4] static activation scales
    eps: float = 1e-6

    def params(self) -> BlockParams:
        p = BlockParams()
        p.version = _lib.ABI_VERSION
        p.d, p.n_heads, p.head_dim, p.mlp, p.weight_format = self.d, self.n_heads, 128, self.mlp, self.fmt
        for site in ("qkv", "o", "up", "down"):
            setattr(p, "w_" + site, self.w[site].data_ptr())
            if site in self.s:
                setattr(p, "s_" + site, self.s[site].data_ptr())
            if site in self.e8:
                setattr(p, "e8m0_" + site, self.e8[site].data_ptr())
            if site in self.b:
                setattr(p, "b_" + site, self.b[site].data_ptr())
        if self.act_scale is not None:
            p.act_scale = self.act_scale.data_ptr()
        p.ln_eps = self.eps
        return p


def quantize_block_weights(wbits: dict, d: int, n_heads: int, mlp: int, fmt: int = _lib.QVD_W_FP8,
                           device="cuda") -> BlockWeights:
    """bf16 master weights (device tensors keyed 'w_qkv', ...) -> BlockWeights, quantized on the GPU."""
    bw = BlockWeights(d=d, n_heads=n_heads, mlp=mlp, fmt=fmt, w={})
    for site in ("qkv", "o", "up", "down"):
        w = wbits["w_" + site]
        if fmt == _lib.QVD_W_FP8:
            bw.w[site], bw.s[site] = quant_fp8_per_tensor(w)
        else:
            bw.w[site], bw.e8[site] = quant_mxfp4(w)
    return bw


def block_ws_bytes(bw: BlockWeights, L: int) -> int:
    p = bw.params()
    return int(_lib.lib().qvd_block_ws_bytes(C.byref(p), L))


def dit_block_forward(bw: BlockWeights, mod: torch.Tensor, x: torch.Tensor, kv_idx: torch.Tensor | None,
                      kv_cnt: torch.Tensor | None, ws: torch.Tensor | None = None,
                      kmax: int | None = None) -> torch.Tensor:
    """x bf16 [L][d] is updated in place with the block output (and returned).  With kv_idx and kv_cnt
    None the block selects kmax key tiles per query tile itself (select_tiles' rule)."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    if kv_idx is None:
        assert kv_cnt is None and kmax is not None, "pass both masks, or neither and kmax"
    else:
        _check(kv_idx, torch.int32, "kv_idx")
        _check(kv_cnt, torch.int32, "kv_cnt")
        kmax = kv_idx.shape[-1]
    L = x.shape[0]
    p = bw.params()
    need = int(_lib.lib().qvd_block_ws_bytes(C.byref(p), L))
    if ws is None:
        ws = _out((need,), torch.uint8, x.device)
    call("dit_block_forward", C.byref(p), _ptr(mod), _ptr(x), L, _ptr(kv_idx), _ptr(kv_cnt),
         int(kmax), _ptr(ws), ws.numel(), _stream())
    return x


def block_forward_until(bw: BlockWeights, mod, x, kv_idx, kv_cnt, stage: int, ws=None,
                        kmax: int | None = None) -> torch.Tensor:
    """dit_block_forward stopped after ``stage`` (_lib.QVD_STAGE_*); returns the workspace, whose
    intermediates block_intermediates() exposes.  x is updated as far as the stage goes."""
    _check(x, torch.bfloat16, "x")
    _check(mod, torch.float32, "mod")
    if kv_idx is not None:
        kmax = kv_idx.shape[-1]
    L = x.shape[0]
    p = bw.params()
    need = int(_lib.lib().qvd_block_ws_bytes(C.byref(p), L))
    if ws is None:
        ws = _out((need,), torch.uint8, x.device)
    call("qvd_block_forward_until", C.byref(p), _ptr(mod), _ptr(x), L, _ptr(kv_idx), _ptr(kv_cnt),
         int(kmax), int(stage), _ptr(ws), ws.numel(), _stream())
    return ws


def block_intermediates(bw: BlockWeights, ws: torch.Tensor, L: int) -> dict:
    """Views (no copies) of the block's intermediates in its workspace, by qvd_block_ws_layout."""
    p = bw.params()
    offs = (C.c_int64 * len(_lib.WS_SLOTS))()
    call("qvd_block_ws_layout", C.byref(p), L, offs)
    d, H, F = bw.d, bw.n_heads, bw.mlp
    T = (L + 127) // 128
    a4 = bw.fmt == _lib.QVD_W_MXFP4_A4
    shapes = {
        "h": ((L, d // 2) if a4 else (L, d), torch.uint8), "q8": ((L, H, 128), torch.int8),
        "k8": ((L, H, 128), torch.int8), "vt": ((H, 128, T * 128), torch.float16),
        "vt_tile_exp": ((H, T), torch.int32), "vt_head_exp": ((H,), torch.int32),
        "o": ((L, d), torch.bfloat16), "g": ((L, F), torch.bfloat16),
        "g8": ((L, F // 2) if a4 else (L, F), torch.uint8), "h_e8m0": ((L, d // 32), torch.uint8),
        "g_e8m0": ((L, F // 32), torch.uint8), "q_scale": ((H, T), torch.float32),
        "k_scale": ((H, T), torch.float32), "scales": ((4,), torch.float32),
    }
    unused = set()
    if a4 or bw.act_scale is not None:
        unused |= {"o", "g"}                       # O and g exist only as codes
    if not a4:
        unused |= {"h_e8m0", "g_e8m0"}
    out = {}
    for i, name in enumerate(_lib.WS_SLOTS):
        if name not in shapes or name in unused:
            continue
        shape, dt = shapes[name]
        n = int(np.prod(shape)) * torch.tensor([], dtype=dt).element_size()
        o = int(offs[i])
        if o + n > ws.numel():
            continue
        out[name] = ws[o:o + n].view(dt).view(shape)
    return out


def select_tiles(q8: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor, kept: int):
    """int8 Q/K [L][H][128] and K scales [H][T] -> (kv_idx int32 [H][T][kept], kv_cnt int32 [H][T]):
    the diagonal and the kept - 1 key tiles of highest mean-pooled score, in tile order."""
    _check(q8, torch.int8, "q8")
    _check(k8, torch.int8, "k8")
    _check(k_scale, torch.float32, "k_scale")
    L, H, _ = q8.shape
    T = (L + 127) // 128
    idx = _out((H, T, kept), torch.int32, q8.device)
    cnt = _out((H, T), torch.int32, q8.device)
    ws = _out((int(_lib.lib().qvd_select_tiles_ws_bytes(L, H)),), torch.uint8, q8.device)
    call("qvd_select_tiles", _ptr(q8), _ptr(k8), _ptr(k_scale), L, H, kept, _ptr(idx), _ptr(cnt), _ptr(ws),
         ws.numel(), _stream())
    return idx, cnt


# ----------------------------------------------------------------------------------------------
# per-kernel event timing

_TIMING_ON = False


def timing_enable(on: bool = True):
    global _TIMING_ON
    call("qvd_timing_enable", 1 if on else 0)
    _TIMING_ON = bool(on)


def timing_report() -> dict:
    """{kernel key: {"count": n, "total_ms": t}} for the launches since the last report."""
    import json
    buf = C.create_string_buffer(1 << 20)
    call("qvd_timing_report", buf, len(buf))
    return json.loads(buf.value.decode())


# ----------------------------------------------------------------------------------------------
# sampler

@dataclass
class Sampler:
    """The eight-step sampler's configuration (qvd_sampler_config) and its device state."""
    L_video: int
    shift_video: float = 10.0
    shift_audio: float = 3.0
    timesteps: tuple | None = None            # None: the eight of the pages
    x_state: torch.Tensor | None = None       # fp32 [L][d]
    x0_hat: torch.Tensor | None = None        # fp32 [L][d]

    def config(self):
        c = _lib.SamplerConfig()
        n = 8 if self.timesteps is None else len(self.timesteps)
        c.n_steps, c.shift_video, c.shift_audio, c.L_video = n, self.shift_video, self.shift_audio, self.L_video
        if self.timesteps is not None:
            self._ts = (C.c_float * n)(*self.timesteps)
            c.timesteps = C.cast(self._ts, C.c_void_p)
        return c

    def sigmas(self, modality: int) -> np.ndarray:
        c = self.config()
        out = (C.c_double * (c.n_steps + 1))()
        call("qvd_sampler_sigmas", C.byref(c), modality, out)
        return np.array(out[:])

    def start(self, eps: torch.Tensor, x_in: torch.Tensor | None = None) -> torch.Tensor:
        """eps bf16 [L][d] -> the first stack input (bf16); allocates the fp32 state."""
        _check(eps, torch.bfloat16, "eps")
        L, d = eps.shape
        self.x_state = _out((L, d), torch.float32, eps.device)
        self.x0_hat = _out((L, d), torch.float32, eps.device)
        x_in = _out((L, d), torch.bfloat16, eps.device) if x_in is None else x_in
        c = self.config()
        call("qvd_sampler_start", C.byref(c), _ptr(eps), L, d, _ptr(self.x_state), _ptr(x_in), _stream())
        return x_in

    def step(self, i: int, v: torch.Tensor, x_in: torch.Tensor | None = None) -> torch.Tensor:
        """After the stack ran at step i with output v (bf16 [L][d]): advance the state; returns the
        next stack input (written into x_in, which may be v)."""
        _check(v, torch.bfloat16, "v")
        L, d = v.shape
        x_in = v if x_in is None else x_in
        c = self.config()
        call("qvd_sampler_step", C.byref(c), int(i), _ptr(v), _ptr(self.x_state), _ptr(self.x0_hat), _ptr(x_in),
             L, d, _stream())
        return x_in


def mfma_probe(kind: int, iters: int = 4000, workgroups: int = 1024, reps: int = 3) -> dict:
    """Measured matrix-core rate of one MFMA kind (_lib.QVD_PROBE_*): TFLOP/s (TOP/s for INT8), the
    median over `reps` timed launches of qvd_mfma_probe after one warm-up, and the shader clock the
    loop ran at (MHz, median over workgroups of the last launch)."""
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * workgroups, dtype=torch.int64, device="cuda")
    flops = _lib.lib().qvd_mfma_probe_flops(kind, iters, workgroups)
    call("qvd_mfma_probe", kind, iters, workgroups, _ptr(out), None, _stream())
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call("qvd_mfma_probe", kind, iters, workgroups, _ptr(out), _ptr(clocks), _stream())
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ck = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
    wall_khz = int(_lib.lib().qvd_wall_clock_khz())
    mhz = None
    if wall_khz > 0:
        mhz = float(np.median(ck[:, 0] / np.maximum(ck[:, 1], 1.0)) * wall_khz / 1e3)
    return {"tflops": flops / (sorted(ms)[len(ms) // 2] * 1e-3) / 1e12, "clock_mhz": mhz}


def inject_launch_failure(after: int):
    """The launch `after` launches from now on this thread reports QVD_EHIP (qvd_inject_launch_failure);
    -1 cancels.  For tests of error handling."""
    call("qvd_inject_launch_failure", int(after))


def capture_graph(fn, warmup: int = 1) -> torch.cuda.CUDAGraph:
    """Record the launches fn() makes on the current stream into a HIP graph (torch's CUDAGraph over
    stream capture); graph.replay() runs them again on the same buffers.  The library allocates and
    synchronises nothing inside its calls, so a block forward or a whole stack step captures as it is;
    tensors fn allocates come from the graph's private pool.  fn should be repeatable (it runs warmup
    times on a side stream first, so that every kernel has been loaded before capture).  Per-kernel
    timing must be off (it records events), and the output poisoning of the tests is suspended while
    capturing (its byte fill could be recorded as a memset node)."""
    global POISON
    if _TIMING_ON:
        raise RuntimeError("capture_graph: per-kernel timing is on; call timing_enable(False) first")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    saved, POISON = POISON, False
    try:
        with torch.cuda.graph(g):
            fn()
    finally:
        POISON = saved
    return g
