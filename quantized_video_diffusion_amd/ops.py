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


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


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
    q = torch.empty((L, n_heads, 128), dtype=torch.int8, device=x.device)
    s = torch.empty((n_heads, (L + 127) // 128), dtype=torch.float32, device=x.device)
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
    mod = torch.empty((nb, 6, d) if stacked else (6, d), dtype=torch.float32, device=basis.device)
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
    out = torch.empty((L, H, D), dtype=torch.bfloat16, device=q8.device)
    part = torch.empty(q_scale.shape, dtype=torch.float32, device=q8.device) if want_amax else None
    ws = torch.empty((_lib.lib().qvd_sparse_attn_ws_bytes(L, H),), dtype=torch.uint8, device=q8.device)
    call("sparse_attn", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), L, H, D,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out), _ptr(part),
         _ptr(ws), ws.numel(), _stream())
    return (out, part) if want_amax else out


def sparse_attn_vt_e4m3(q8, q_scale, k8, k_scale, vt, kv_idx, kv_cnt, out_scale,
                        sm_scale: float = SM_SCALE):
    """As sparse_attn_vt, returning the E4M3 codes of bf16 O under the static scale out_scale
    (a device fp32 [1] tensor) instead of O: uint8 [L][H][128]."""
    L, H, D = q8.shape
    _check(vt, torch.float16, "vt")
    _check(out_scale, torch.float32, "out_scale")
    out = torch.empty((L, H, D), dtype=torch.uint8, device=q8.device)
    call("qvd_sparse_attn_vt_e4m3", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out_scale), _ptr(out),
         _stream())
    return out


def sparse_attn_vt_mxfp4(q8, q_scale, k8, k_scale, vt, kv_idx, kv_cnt, sm_scale: float = SM_SCALE):
    """As sparse_attn_vt, returning the MXFP4 codes of bf16 O per (token, head, 32 dims) instead of
    O: (packed E2M1 uint8 [L][H*64], E8M0 uint8 [L][H*4])."""
    L, H, D = q8.shape
    _check(vt, torch.float16, "vt")
    packed = torch.empty((L, H * D // 2), dtype=torch.uint8, device=q8.device)
    e8 = torch.empty((L, H * D // 32), dtype=torch.uint8, device=q8.device)
    call("qvd_sparse_attn_vt_mxfp4", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(packed), _ptr(e8), _stream())
    return packed, e8


def sparse_attn_vt(q8, q_scale, k8, k_scale, vt, kv_idx, kv_cnt, sm_scale: float = SM_SCALE,
                   want_amax: bool = False):
    """As sparse_attn, with V given as fp16 V^T [H][128][ceil(L/128)*128]."""
    L, H, D = q8.shape
    _check(vt, torch.float16, "vt")
    out = torch.empty((L, H, D), dtype=torch.bfloat16, device=q8.device)
    part = torch.empty(q_scale.shape, dtype=torch.float32, device=q8.device) if want_amax else None
    call("qvd_sparse_attn_vt", _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt), L, H,
         _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], float(sm_scale), _ptr(out), _ptr(part),
         _stream())
    return (out, part) if want_amax else out


def qk_int32_tile(q8, k8, h: int, i: int, j: int) -> torch.Tensor:
    L, H, _ = q8.shape
    out = torch.empty((128, 128), dtype=torch.int32, device=q8.device)
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
        out = torch.empty((M, N), dtype=torch.float32, device=a.device) if out is None else out
        e.out_f32 = out.data_ptr()
        ret = out
    elif mode in (_lib.QVD_EPI_BF16, _lib.QVD_EPI_GELU):
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if out is None else out
        e.out_bf16 = out.data_ptr()
        if amax_partials is not None:
            e.amax_partials = amax_partials.data_ptr()
        ret = out
    elif mode == _lib.QVD_EPI_GELU_E4M3:
        out = torch.empty((M, N), dtype=torch.uint8, device=a.device) if out is None else out
        _check(out, torch.uint8, "out")
        _check(out_scale, torch.float32, "out_scale")
        e.out_e4m3 = out.data_ptr()
        e.out_scale = out_scale.data_ptr()
        ret = out
    elif mode == _lib.QVD_EPI_GELU_MXFP4:
        packed = torch.empty((M, N // 2), dtype=torch.uint8, device=a.device)
        e8 = torch.empty((M, N // 32), dtype=torch.uint8, device=a.device)
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
        q8 = torch.empty((M, H, 128), dtype=torch.int8, device=a.device)
        k8 = torch.empty_like(q8)
        v = torch.empty((H, 128, T * 128), dtype=torch.float16, device=a.device)   # V^T, fp16
        qs = torch.empty((H, T), dtype=torch.float32, device=a.device)
        ks = torch.empty_like(qs)
        e.n_heads = H
        e.q8, e.k8, e.v, e.q_scale, e.k_scale = (q8.data_ptr(), k8.data_ptr(), v.data_ptr(),
                                                 qs.data_ptr(), ks.data_ptr())
        ret = (q8, k8, v, qs, ks)
    call(fn, _ptr(a), _ptr(s_a), _ptr(w), _ptr(extra), _ptr(bias), M, N, K, C.byref(e), _stream())
    return ret


def quant_mxfp4(w: torch.Tensor):
    """bf16 [N][K] -> (packed E2M1 uint8 [N][K/2], E8M0 uint8 [N][K/32])."""
    _check(w, torch.bfloat16, "w")
    N, K = w.shape
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    e8 = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    call("qvd_quant_mxfp4", _ptr(w), N, K, _ptr(packed), _ptr(e8), _stream())
    return packed, e8


def amax_update(x: torch.Tensor, amax: torch.Tensor):
    _check(x, torch.float32, "x")
    call("qvd_amax_update", _ptr(x), x.numel(), _ptr(amax), _stream())


def clip_count(x: torch.Tensor, scale: torch.Tensor, count: torch.Tensor):
    _check(x, torch.float32, "x")
    call("qvd_clip_count", _ptr(x), x.numel(), _ptr(scale), _ptr(count), _stream())


# ----------------------------------------------------------------------------------------------
# block

def calibrated_scale(amax: float) -> np.float32:
    """Static per-tensor FP8 scale from a calibration amax: fp32(amax / 448), moved up by one fp32 ulp
    when 448 s (exact) would fall below amax, so that no calibration value exceeds the E4M3 range.
    amax = 0 gives 1."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    s = np.float32(a / np.float32(448.0))
    while float(s) * 448.0 < float(a):
        s = np.nextafter(s, np.float32(np.inf))
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
        ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
    call("dit_block_forward", C.byref(p), _ptr(mod), _ptr(x), L, _ptr(kv_idx), _ptr(kv_cnt),
         int(kmax), _ptr(ws), ws.numel(), _stream())
    return x


def select_tiles(q8: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor, kept: int):
    """int8 Q/K [L][H][128] and K scales [H][T] -> (kv_idx int32 [H][T][kept], kv_cnt int32 [H][T]):
    the diagonal and the kept - 1 key tiles of highest mean-pooled score, in tile order."""
    _check(q8, torch.int8, "q8")
    _check(k8, torch.int8, "k8")
    _check(k_scale, torch.float32, "k_scale")
    L, H, _ = q8.shape
    T = (L + 127) // 128
    idx = torch.empty((H, T, kept), dtype=torch.int32, device=q8.device)
    cnt = torch.empty((H, T), dtype=torch.int32, device=q8.device)
    ws = torch.empty((int(_lib.lib().qvd_select_tiles_ws_bytes(L, H)),), dtype=torch.uint8, device=q8.device)
    call("qvd_select_tiles", _ptr(q8), _ptr(k8), _ptr(k_scale), L, H, kept, _ptr(idx), _ptr(cnt), _ptr(ws),
         ws.numel(), _stream())
    return idx, cnt


# ----------------------------------------------------------------------------------------------
# per-kernel event timing

def timing_enable(on: bool = True):
    call("qvd_timing_enable", 1 if on else 0)


def timing_report() -> dict:
    """{kernel key: {"count": n, "total_ms": t}} for the launches since the last report."""
    import json
    buf = C.create_string_buffer(1 << 20)
    call("qvd_timing_report", buf, len(buf))
    return json.loads(buf.value.decode())
