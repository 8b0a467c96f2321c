"""Teacher-forced, stage-by-stage parity of dit_block_forward against the oracle (FP8 block, dynamic
per-tensor scales).

The block chains four per-tensor requantizations, so a comparison of its output alone mixes each
stage's own error with codes moved upstream.  Here every stage is checked on its own: the GPU block is
stopped after each stage (qvd_block_forward_until runs the block's own launches), its intermediates
are read from the workspace, and the oracle computes the next stage from the GPU's own inputs and
scales.  With the scales forced, every stage is row-local (modulate, the GEMMs, the quantizers with
the tensor's amax given) or tile-local (INT8 Q/K, attention), so large blocks are checked on sampled
token tiles; the per-tensor amax values are taken over the whole tensors.

Bars (stated per stage below):
  codes of the fused modulate quantizer (h1, h2): equal, except within 2^-12 of a rounding midpoint of
      the oracle's pre-rounding value (counted; the near-tie rule);
  the QKV and down-projection GEMMs: their fp32 accumulator output (the same GEMM run with the fp32
      epilogue) within 1e-3 RMS of the oracle's exact one; the QKV epilogue from those fp32 values --
      bf16 V, INT8 Q/K codes and scales -- bit-exact;
  standalone quantizers (O and g) and the per-tensor scales s1, s_O, s2, s_g: bit-exact;
  bf16 GEMM outputs x1 and GELU(g): one bf16 ulp + 1e-3 RMS;
  attention output: one bf16 ulp + 1e-2 RMS;
  block output x2: max |err| <= 1e-2 RMS(x2); beyond it only a one-ulp rounding flip of an element whose
      oracle value lies within |gate2 (y_gpu - y)| (+ two fp32 roundings) of a bf16 midpoint (counted,
      at most 1e-3 of the elements).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from oracle import codecs as OC, quant as OQ, adaln as OA, gemm as OG, attention as OAT
from _gpu_util import (say, bf16_dev, host, host_bits, assert_codes_equal_except_ties, assert_bf16_close,
                       assert_close_rms)

SM_SCALE = 1.0 / math.sqrt(128.0)


def _ln_amax(x_bits, mod, half, eps, chunk=4096):
    """max |LN(x)(1 + scale) + shift| over the whole tensor (the oracle's fp32 values), by row chunks."""
    a = np.float32(0.0)
    for r in range(0, x_bits.shape[0], chunk):
        y = OA.layernorm_modulate(x_bits[r:r + chunk], mod, half, eps)
        a = max(a, np.float32(np.abs(y).max()))
    return np.float32(a)


def _bf16_amax(bits) -> np.float32:
    """max |v| of a bf16 tensor from its bit patterns (finite magnitudes order as their patterns)."""
    m = int((np.asarray(bits).reshape(-1) & 0x7FFF).max())
    return np.float32(OC.bf16_to_f64(np.array([m], np.uint16))[0])


def _near_bf16_mid(v, win):
    """|v - nearest bf16 rounding midpoint| <= win, elementwise (v float64, win >= 0)."""
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    q = np.ldexp(1.0, e - 1 - 7)                      # bf16 spacing in a's binade
    t = a / q
    return np.abs(t - (np.floor(t) + 0.5)) * q <= win


def run_stages(bw, mod_d, x_bits, idx_d, cnt_d, rows=None):
    """Run the GPU block whole and stopped after the stages whose outputs later stages overwrite;
    return host copies of every intermediate.  Also the GPU's own fp32 accumulator outputs of the QKV
    and down-projection GEMMs on `rows` (the same GEMM run with the fp32-output epilogue: the main
    loop and its accumulation order are the same, only the epilogue differs), which the fused
    epilogues then round (y_qkv, y_down)."""
    L = x_bits.shape[0]
    rows_d = None if rows is None else torch.from_numpy(np.asarray(rows)).cuda()
    pick = (lambda t: host(t)) if rows is None else (lambda t: host(t[rows_d]))
    xd = bf16_dev(x_bits)
    ws = Q.block_forward_until(bw, mod_d, xd, idx_d, cnt_d, _lib.QVD_STAGE_ALL)
    it = Q.block_intermediates(bw, ws, L)
    g = {"x2": host_bits(xd), "q8": host(it["q8"]), "k8": host(it["k8"]), "qs": host(it["q_scale"]),
         "ks": host(it["k_scale"]), "vt": host(it["vt"]), "v_exp": host(it["vt_head_exp"]),
         "o": host_bits(it["o"]), "h2": host(it["h"]), "g": host_bits(it["g"]), "g8": host(it["g8"]),
         "scales": host(it["scales"])}
    y = Q.gemm_fp8(it["g8"], it["scales"][3:4].clone(), bw.w["down"], bw.s["down"], bias=bw.b.get("down"))
    g["y_down"] = pick(y)
    del it, ws, y
    for stage, keys in ((_lib.QVD_STAGE_MODULATE1, ("h1",)), (_lib.QVD_STAGE_OQUANT, ("o8",)),
                        (_lib.QVD_STAGE_OPROJ, ("x1",))):
        xd = bf16_dev(x_bits)
        ws = Q.block_forward_until(bw, mod_d, xd, idx_d, cnt_d, stage)
        it = Q.block_intermediates(bw, ws, L)
        if stage == _lib.QVD_STAGE_OPROJ:
            g["x1"] = host_bits(xd)
        else:
            g[keys[0]] = host(it["h"])
            g["scales_" + keys[0]] = host(it["scales"])
        if stage == _lib.QVD_STAGE_MODULATE1:
            y = Q.gemm_fp8(it["h"], it["scales"][0:1].clone(), bw.w["qkv"], bw.s["qkv"], bias=bw.b.get("qkv"))
            g["y_qkv"] = pick(y)
            del y
        del it, ws
    torch.cuda.synchronize()
    return g


def v_bits_from_vt(vt, v_exp, L):
    """The bf16 V the attention consumed: fp16 V^T [H][128][Lp] times 2^E[h], as bf16 bit patterns
    [L][H][128] (exact: each value is a bf16 value scaled by a power of two)."""
    v = vt[:, :, :L].astype(np.float32) * np.ldexp(np.float32(1.0), v_exp.astype(np.int32))[:, None, None]
    return OC.f64_to_bf16(v.transpose(2, 0, 1).astype(np.float64))


def check_block_stages(name, qw, mod, x_bits, idx, cnt, g, n_heads, rows=None, eps=1e-6):
    """Every stage of the FP8 block against the oracle, fed the GPU's own inputs.  qw: the oracle's
    quantized weights (codes and scales, as the GPU block holds them); mod: fp32 [6][d] (the GPU's);
    rows: the token rows checked (whole 128-row tiles, or None for all).  Returns per-stage stats."""
    L, d = x_bits.shape
    H = n_heads
    T = (L + 127) // 128
    if rows is None:
        rows = np.arange(L)
    tiles = np.unique(rows // 128)
    assert np.array_equal(np.concatenate([np.arange(i * 128, min(L, (i + 1) * 128)) for i in tiles]),
                          rows), "rows must be whole tiles"
    mod64 = mod.astype(np.float64)
    st = {}

    # S1: modulate (attention branch) -> E4M3 with the dynamic scale s1
    a1 = _ln_amax(x_bits, mod, 0, eps)
    s1 = g["scales_h1"][0]
    assert s1 == OQ.fp8_scale_dynamic(a1)[0], f"{name}: s1 {s1} != oracle {OQ.fp8_scale_dynamic(a1)[0]}"
    y = OA.layernorm_modulate(x_bits[rows], mod, 0, eps)
    want, _ = OQ.quant_fp8_with_amax(y, a1)
    inv = OQ.fp8_scale_dynamic(a1)[1]
    st["h1_flips"] = assert_codes_equal_except_ties(g["h1"][rows], want, y * inv, "e4m3", name=name + " h1")

    # S2: QKV GEMM from the GPU's h1 and s1 (fp32 accumulator output within 1e-3 RMS of the oracle's
    # exact one); its epilogue from the GPU's own fp32 values: bf16 V, and INT8 Q/K per (head, tile)
    # with their scales, bit for bit as the oracle's quantizer gives them from bf16(y_gpu)
    yq = OG.gemm_fp8(g["h1"][rows], s1, qw["w_qkv"], qw["s_qkv"], qw.get("b_qkv"))
    yg = g["y_qkv"].astype(np.float64)
    st["qkv_gemm_err_rel"] = assert_close_rms(yg, yq, 1e-3, name + " QKV GEMM (fp32)")
    yb = OC.f64_to_bf16(yg)                          # fp32 -> bf16 in one rounding, as the epilogue
    for part, (c8, sc) in enumerate(((g["q8"], g["qs"]), (g["k8"], g["ks"]))):
        blk = np.ascontiguousarray(yb[:, part * d:(part + 1) * d]).reshape(len(rows), H, 128)
        for k, i in enumerate(tiles):
            r = slice(k * 128, k * 128 + min(128, L - i * 128))
            cw, sw = OQ.quant_int8_qk(blk[r], r.stop - r.start, H)
            np.testing.assert_array_equal(sc[:, i], sw[:, 0], err_msg=f"{name} part {part} tile {i} scales")
            np.testing.assert_array_equal(c8[rows[r]], cw, err_msg=f"{name} part {part} tile {i} codes")
    v_bits = v_bits_from_vt(g["vt"], g["v_exp"], L)
    vr = v_bits[rows].reshape(len(rows), d)
    vn = np.abs(OC.bf16_to_f64(vr)) >= 2.0 ** -14 * np.ldexp(1.0, np.repeat(g["v_exp"], 128))[None, :]
    np.testing.assert_array_equal(vr[vn], yb[:, 2 * d:][vn], err_msg=name + " V = bf16 of the GEMM output")

    # S3: attention from the GPU's Q8, K8, scales and V
    o_gpu = g["o"].reshape(L, H, 128)
    for h in range(H):
        for i in tiles:
            r = slice(i * 128, min(L, (i + 1) * 128))
            want = OAT.sparse_attn_tile(g["q8"], g["qs"], g["k8"], g["ks"], v_bits, idx, cnt, h, i, SM_SCALE)
            assert_bf16_close(np.ascontiguousarray(o_gpu[r, h]), want, 1e-2, f"{name} attention ({h}, {i})")

    # S4: per-tensor FP8 of O (standalone quantizer: bit-exact), amax over the whole O
    ao = _bf16_amax(g["o"])
    so = g["scales_o8"][1]
    assert so == OQ.fp8_scale_dynamic(ao)[0], f"{name}: s_O"
    want, _ = OQ.quant_fp8_with_amax(OC.bf16_to_f64(g["o"][rows]).astype(np.float32), ao)
    np.testing.assert_array_equal(g["o8"][rows], want)

    # S5: out-projection + gated residual from the GPU's O8 and s_O
    y1 = OG.gemm_fp8(g["o8"][rows], so, qw["w_o"], qw["s_o"], qw.get("b_o"))
    x1_want = OC.bf16_to_f64(x_bits[rows]) + mod64[2][None, :] * y1
    assert_bf16_close(g["x1"][rows], x1_want, 1e-3, name + " x1")

    # S6: modulate (MLP branch) of the GPU's x1
    a2 = _ln_amax(g["x1"], mod, 1, eps)
    s2 = g["scales"][2]
    assert s2 == OQ.fp8_scale_dynamic(a2)[0], f"{name}: s2"
    y = OA.layernorm_modulate(g["x1"][rows], mod, 1, eps)
    want, _ = OQ.quant_fp8_with_amax(y, a2)
    st["h2_flips"] = assert_codes_equal_except_ties(g["h2"][rows], want, y * OQ.fp8_scale_dynamic(a2)[1],
                                                    "e4m3", name=name + " h2")

    # S7: up-projection + GELU from the GPU's h2 and s2
    gw = OG.gelu(OG.gemm_fp8(g["h2"][rows], s2, qw["w_up"], qw["s_up"], qw.get("b_up")))
    assert_bf16_close(g["g"][rows], gw, 1e-3, name + " GELU")

    # S8: per-tensor FP8 of g (standalone: bit-exact), amax over the whole g
    ag = _bf16_amax(g["g"])
    sg = g["scales"][3]
    assert sg == OQ.fp8_scale_dynamic(ag)[0], f"{name}: s_g"
    want, _ = OQ.quant_fp8_with_amax(OC.bf16_to_f64(g["g"][rows]).astype(np.float32), ag)
    np.testing.assert_array_equal(g["g8"][rows], want)

    # S9: down-projection + gated residual from the GPU's g8, s_g and x1: the block output.  The GEMM's
    # fp32 output is within 1e-3 RMS of the exact one; the block output is then compared with the
    # oracle's, x2 = bf16(x1 + gate2 y) from the exact y.  Where the two differ, the oracle's value must
    # lie within |gate2 (y_gpu - y)| + two fp32 roundings of a bf16 midpoint (a rounding flip).
    y2 = OG.gemm_fp8(g["g8"][rows], sg, qw["w_down"], qw["s_down"], qw.get("b_down"))
    y2g = g["y_down"].astype(np.float64)
    st["down_gemm_err_rel"] = assert_close_rms(y2g, y2, 1e-3, name + " down GEMM (fp32)")
    gy = mod64[5][None, :] * y2
    x2_f64 = OC.bf16_to_f64(g["x1"][rows]) + gy
    x2_want = OC.bf16_to_f64(OC.f64_to_bf16(x2_f64))
    got = OC.bf16_to_f64(g["x2"][rows])
    err = np.abs(got - x2_want)
    rms = float(np.sqrt(np.mean(x2_want ** 2)))
    win = np.abs(mod64[5][None, :] * (y2g - y2)) + 2.0 ** -23 * np.abs(x2_f64)
    tie = _near_bf16_mid(x2_f64, win)
    ulp = np.abs(x2_want) * 2.0 ** -7
    far = ~tie
    st["x2_max_err_rel"] = float(err.max() / rms)
    st["x2_max_err_rel_off_ties"] = float(err[far].max() / rms) if far.any() else 0.0
    big = err > 1e-2 * rms
    st["x2_tie_flips"] = int(np.count_nonzero(big))
    say(f"{name}: stages ok; h1 {st['h1_flips']} / h2 {st['h2_flips']} near-tie code flips; GEMM fp32 max|err| "
        f"QKV {st['qkv_gemm_err_rel']:.1e} / down {st['down_gemm_err_rel']:.1e} RMS; "
        f"block output max|err| {st['x2_max_err_rel']:.2e} RMS "
        f"({st['x2_max_err_rel_off_ties']:.2e} away from bf16 near-ties; {st['x2_tie_flips']} one-ulp flips of "
        f"large outputs at near-ties)")
    # every output within 1e-2 RMS; beyond it only a one-ulp rounding flip of a large output whose
    # oracle value sits within the GEMM's accumulation error of a bf16 midpoint
    assert (~big | (tie & (err <= ulp))).all(), f"{name}: block output beyond 1e-2 RMS away from a near-tie"
    assert st["x2_tie_flips"] <= max(8, 1e-3 * err.size), f"{name}: {st['x2_tie_flips']} near-tie flips"
    return st


# ---- blocks whose producers write the next GEMM's codes ------------------------------------------------
# Static E4M3 activation scales act_scale = (s1, s_O, s2, s_g) with FP8 weights (W8A8) or MXFP4 weights
# (W4A8): modulate -> E4M3 under s1; QKV GEMM and its INT8 Q/K / V^T epilogue; the attention writing
# E4M3(bf16(O)) under s_O (no bf16 O); out-projection + gated residual; modulate -> E4M3 under s2;
# up-projection with the GELU -> E4M3 epilogue under s_g (no bf16 g); down-projection + gated residual.
# W4A4 (QVD_W_MXFP4_A4): the same chain with every GEMM input in MXFP4 per token row and 32 channels
# (E2M1 codes + an E8M0 scale per block) and no per-tensor scale.
# Bars as for the FP8 block.  The two fused producers are checked in two parts: the bf16 tensor they
# encode (the attention's bf16 output from the same inputs, the GELU epilogue's bf16 output from the same
# accumulators) against the oracle at the bf16 bar, and their codes against the oracle's quantizer
# applied to that bf16 tensor, bit for bit.  The MXFP4 modulate codes are bit-exact (the kernel rounds
# the float64 modulation once to fp32, as the oracle does); the E4M3 ones follow the near-tie rule.

def run_stages_fused(bw, mod_d, x_bits, idx_d, cnt_d, rows):
    """GPU side of the stage check of a block with fused producers: the block whole and stopped after the stages later ones
    overwrite, plus, on `rows`, the fp32 accumulator outputs of the QKV, up and down GEMMs and the
    bf16 GELU of the up-projection's accumulators; the bf16 attention output from the block's own
    Q8/K8/V^T.  Host copies."""
    L = x_bits.shape[0]
    a4 = bw.fmt == _lib.QVD_W_MXFP4_A4
    fp8 = bw.fmt == _lib.QVD_W_FP8
    rows_d = torch.from_numpy(np.asarray(rows)).cuda()
    a = bw.act_scale
    wq = {s: (bw.w[s], bw.s[s] if fp8 else bw.e8[s]) for s in ("qkv", "o", "up", "down")}

    def gemm(it, codes, e8_slot, k, site, mode=_lib.QVD_EPI_F32):
        c = it[codes][rows_d].contiguous()
        if a4:
            return Q.gemm_mxfp4_w4a4(c, it[e8_slot][rows_d].contiguous(), *wq[site], mode=mode)
        if fp8:
            return Q.gemm_fp8(c, a[k:k + 1], *wq[site], mode=mode)
        return Q.gemm_mxfp4(c, a[k:k + 1], *wq[site], mode=mode)

    def acts(it, codes, e8_slot):
        return (host(it[codes]), host(it[e8_slot])) if a4 else (host(it[codes]), None)

    xd = bf16_dev(x_bits)
    ws = Q.block_forward_until(bw, mod_d, xd, idx_d, cnt_d, _lib.QVD_STAGE_ALL)
    it = Q.block_intermediates(bw, ws, L)
    g = {"x2": host_bits(xd), "q8": host(it["q8"]), "k8": host(it["k8"]), "qs": host(it["q_scale"]),
         "ks": host(it["k_scale"]), "vt": host(it["vt"]), "v_exp": host(it["vt_head_exp"]),
         "h2": acts(it, "h", "h_e8m0"), "g8": acts(it, "g8", "g_e8m0")}
    o = Q.sparse_attn_vt(it["q8"], it["q_scale"], it["k8"], it["k_scale"],
                         Q.VT(it["vt"], it["vt_head_exp"]), idx_d, cnt_d)
    g["o_bf16"] = host_bits(o)
    del o
    g["y_up"] = host(gemm(it, "h", "h_e8m0", 2, "up"))
    g["g_bf16"] = host_bits(gemm(it, "h", "h_e8m0", 2, "up", mode=_lib.QVD_EPI_GELU))
    g["y_down"] = host(gemm(it, "g8", "g_e8m0", 3, "down"))
    del it, ws
    for stage in (_lib.QVD_STAGE_MODULATE1, _lib.QVD_STAGE_OQUANT, _lib.QVD_STAGE_OPROJ):
        xd = bf16_dev(x_bits)
        ws = Q.block_forward_until(bw, mod_d, xd, idx_d, cnt_d, stage)
        it = Q.block_intermediates(bw, ws, L)
        if stage == _lib.QVD_STAGE_MODULATE1:
            g["h1"] = acts(it, "h", "h_e8m0")
            g["y_qkv"] = host(gemm(it, "h", "h_e8m0", 0, "qkv"))
        elif stage == _lib.QVD_STAGE_OQUANT:
            g["o8"] = acts(it, "h", "h_e8m0")
        else:
            g["x1"] = host_bits(xd)
        del it, ws
    torch.cuda.synchronize()
    return g


def check_block_stages_fused(name, wm, act, mod, x_bits, idx, cnt, g, n_heads, rows, eps=1e-6):
    """Every stage of a block with fused producers against the oracle, fed the GPU's own inputs.  wm:
    the GPU's weights on the host, MXFP4 ('w_<site>' packed E2M1, 'e8_<site>' E8M0) or FP8 ('w_<site>'
    E4M3 codes, 's_<site>' the per-tensor scale); act: the four static E4M3 scales (W8A8, W4A8), or
    None for MXFP4 activations (W4A4)."""
    L, d = x_bits.shape
    H = n_heads
    a4 = act is None
    tiles = np.unique(rows // 128)
    assert np.array_equal(np.concatenate([np.arange(i * 128, min(L, (i + 1) * 128)) for i in tiles]),
                          rows), "rows must be whole tiles"
    mod64 = mod.astype(np.float64)
    s1, so, s2, sg = (None,) * 4 if a4 else (np.float32(v) for v in act)
    st = {}
    fp8 = "s_qkv" in wm
    w = {s: (wm["w_" + s], wm["s_" + s] if fp8 else wm["e8_" + s]) for s in ("qkv", "o", "up", "down")}
    kind = "W4A4" if a4 else ("W8A8" if fp8 else "W4A8")

    def sub(c):
        """The checked rows of a GPU activation (codes, E8M0 or None)."""
        return (c[0][rows], None if c[1] is None else c[1][rows])

    def gemm(c, s, site):
        """The oracle's GEMM of the GPU's activation codes (rows already taken) with the site's weights."""
        if a4:
            return OG.gemm_mxfp4_w4a4(c[0], c[1], *w[site])
        if fp8:
            return OG.gemm_fp8(c[0], s, *w[site])
        return OG.gemm_mxfp4(c[0], s, *w[site])

    def check_modulate(c, half, s, what):
        y = OA.layernorm_modulate(x_bits[rows] if half == 0 else g["x1"][rows], mod, half, eps)
        if a4:
            p, e = OQ.quant_mxfp4(y)
            np.testing.assert_array_equal(c[1], e, err_msg=f"{name} {what} E8M0")
            np.testing.assert_array_equal(c[0], p, err_msg=f"{name} {what} E2M1")
            return 0
        codes, _ = OQ.quant_fp8_per_tensor(y, scale_in=s)
        pre = np.asarray(y, np.float32) * (np.float32(1.0) / s)
        return assert_codes_equal_except_ties(c[0], codes, pre, "e4m3", name=f"{name} {what}")

    def check_codes_of_bf16(c, bits, s, what):
        """The GPU's codes of a fused producer equal the oracle's quantizer of its bf16 output."""
        v = OC.bf16_to_f64(bits)
        if a4:
            p, e = OQ.quant_mxfp4(v)
            np.testing.assert_array_equal(c[1], e, err_msg=f"{name} {what} E8M0")
            np.testing.assert_array_equal(c[0], p, err_msg=f"{name} {what} E2M1")
        else:
            np.testing.assert_array_equal(c[0], OQ.quant_fp8_per_tensor(v.astype(np.float32), scale_in=s)[0],
                                          err_msg=f"{name} {what}")

    # S1: modulate (attention branch) of the input
    st["h1_flips"] = check_modulate(sub(g["h1"]), 0, s1, "h1")

    # S2: QKV GEMM from the GPU's h1; its epilogue from the GPU's fp32 values
    yq = gemm(sub(g["h1"]), s1, "qkv")
    yg = g["y_qkv"].astype(np.float64)
    st["qkv_gemm_err_rel"] = assert_close_rms(yg, yq, 1e-3, name + " QKV GEMM (fp32)")
    yb = OC.f64_to_bf16(yg)
    for part, (c8, sc) in enumerate(((g["q8"], g["qs"]), (g["k8"], g["ks"]))):
        blk = np.ascontiguousarray(yb[:, part * d:(part + 1) * d]).reshape(len(rows), H, 128)
        for k, i in enumerate(tiles):
            r = slice(k * 128, k * 128 + min(128, L - i * 128))
            cw, sw = OQ.quant_int8_qk(blk[r], r.stop - r.start, H)
            np.testing.assert_array_equal(sc[:, i], sw[:, 0], err_msg=f"{name} part {part} tile {i} scales")
            np.testing.assert_array_equal(c8[rows[r]], cw, err_msg=f"{name} part {part} tile {i} codes")
    v_bits = v_bits_from_vt(g["vt"], g["v_exp"], L)
    vr = v_bits[rows].reshape(len(rows), d)
    vn = np.abs(OC.bf16_to_f64(vr)) >= 2.0 ** -14 * np.ldexp(1.0, np.repeat(g["v_exp"], 128))[None, :]
    np.testing.assert_array_equal(vr[vn], yb[:, 2 * d:][vn], err_msg=name + " V = bf16 of the GEMM output")

    # S3: attention from the GPU's Q8, K8, scales and V^T: the bf16 output at the attention bar, and the
    # block's codes of O equal to the oracle's quantizer on that bf16 output
    o_gpu = g["o_bf16"].reshape(L, H, 128)
    for h in range(H):
        for i in tiles:
            r = slice(i * 128, min(L, (i + 1) * 128))
            want = OAT.sparse_attn_tile(g["q8"], g["qs"], g["k8"], g["ks"], v_bits, idx, cnt, h, i, SM_SCALE)
            assert_bf16_close(np.ascontiguousarray(o_gpu[r, h]), want, 1e-2, f"{name} attention ({h}, {i})")
    o8 = sub(g["o8"])
    check_codes_of_bf16((o8[0].reshape(len(rows), -1), o8[1]), g["o_bf16"].reshape(L, d)[rows], so,
                        "O codes = quantizer of the bf16 O")

    # S5: out-projection + gated residual from the GPU's O codes
    y1 = gemm((o8[0].reshape(len(rows), -1), o8[1]), so, "o")
    assert_bf16_close(g["x1"][rows], OC.bf16_to_f64(x_bits[rows]) + mod64[2][None, :] * y1, 1e-3, name + " x1")

    # S6: modulate (MLP branch) of the GPU's x1
    st["h2_flips"] = check_modulate(sub(g["h2"]), 1, s2, "h2")

    # S7: up-projection from the GPU's h2: fp32 accumulators at the GEMM bar, bf16 GELU of them at the
    # bf16 bar, and the block's codes of g equal to the oracle's quantizer on that bf16 GELU
    yu = gemm(sub(g["h2"]), s2, "up")
    st["up_gemm_err_rel"] = assert_close_rms(g["y_up"].astype(np.float64), yu, 1e-3, name + " up GEMM (fp32)")
    assert_bf16_close(g["g_bf16"], OG.gelu(g["y_up"].astype(np.float64)), 1e-3, name + " GELU")
    check_codes_of_bf16(sub(g["g8"]), g["g_bf16"], sg, "g codes = quantizer of the bf16 GELU")

    # S9: down-projection + gated residual from the GPU's g codes: the block output (the FP8 block's rule)
    y2 = gemm(sub(g["g8"]), sg, "down")
    y2g = g["y_down"].astype(np.float64)
    st["down_gemm_err_rel"] = assert_close_rms(y2g, y2, 1e-3, name + " down GEMM (fp32)")
    x2_f64 = OC.bf16_to_f64(g["x1"][rows]) + mod64[5][None, :] * y2
    x2_want = OC.bf16_to_f64(OC.f64_to_bf16(x2_f64))
    got = OC.bf16_to_f64(g["x2"][rows])
    err = np.abs(got - x2_want)
    rms = float(np.sqrt(np.mean(x2_want ** 2)))
    win = np.abs(mod64[5][None, :] * (y2g - y2)) + 2.0 ** -23 * np.abs(x2_f64)
    tie = _near_bf16_mid(x2_f64, win)
    big = err > 1e-2 * rms
    st["x2_max_err_rel"] = float(err.max() / rms)
    st["x2_tie_flips"] = int(np.count_nonzero(big))
    say(f"{name}: {kind} stages ok; h1 {st['h1_flips']} / h2 {st['h2_flips']} near-tie "
        f"code flips; GEMM fp32 max|err| QKV {st['qkv_gemm_err_rel']:.1e} / up {st['up_gemm_err_rel']:.1e} / "
        f"down {st['down_gemm_err_rel']:.1e} RMS; block output max|err| {st['x2_max_err_rel']:.2e} RMS")
    assert (~big | (tie & (err <= np.abs(x2_want) * 2.0 ** -7))).all(), \
        f"{name}: block output beyond 1e-2 RMS away from a near-tie"
    assert st["x2_tie_flips"] <= max(8, 1e-3 * err.size), f"{name}: {st['x2_tie_flips']} near-tie flips"
    return st
