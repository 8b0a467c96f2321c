"""GPU parity of the FP8 / MXFP4 GEMM epilogues and of the block-sparse INT8-QK attention."""
import math

import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from oracle import codecs as OC, quant as OQ, gemm as OG, attention as OAT
from _gpu_util import (say, bf16_dev, u8_dev, i32_dev, f32_dev, host, host_bits, bf16_f64,
                       assert_codes_equal_except_ties, assert_close_rms, assert_bf16_close)

pytestmark = pytest.mark.gpu


def _codes(M, K, seed, tensor="codes_a"):
    return W.random_e4m3_codes((M, K), seed=seed, tensor=tensor)


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (391, 384, 256), (33, 2688, 2688), (700, 768, 1024),
                                   (1, 256, 128)])
def test_gemm_fp8_f32_epilogue(M, N, K):
    say("gemm f32", M, N, K)
    a, w = _codes(M, K, M), _codes(N, K, N, "codes_b")
    sa, sw = np.float32(0.0123), np.float32(0.37)
    bias = (np.arange(N) % 7).astype(np.float32) - 3
    y = host(Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]), bias=f32_dev(bias)))
    want = OG.gemm_fp8(a, sa, w, sw, bias)
    assert_close_rms(y, want, 1e-3, "gemm f32")


def test_gemm_fp8_480p_qkv_shape_sampled():
    """M = 33,784 (ragged last tile), N = 8,064, K = 2,688; 64 sampled rows checked exactly."""
    M, N, K = W.TOKENS_480P, 3 * 2688, 2688
    a, w = _codes(M, K, 1), _codes(N, K, 2, "codes_b")
    sa, sw = np.float32(1e-2), np.float32(2e-3)
    y = Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]))
    rows = np.r_[np.random.default_rng(0).choice(M, 60, replace=False), [0, M - 1, M - 120, M - 248]]
    got = host(y[torch.from_numpy(rows).cuda()])
    want = OG.gemm_fp8(a[rows], sa, w, sw)
    assert_close_rms(got, want, 1e-3, "gemm 480p rows")


def test_gemm_fp8_480p_down_shape_sampled():
    """The 480p down-projection shape: M = 33,784 (ragged last tile), N = 2,688 (10.5 tiles wide),
    K = 10,752; realistic codes (per-tensor quantized N(0,1) activations and Glorot weights); 64
    sampled rows in fp32 at 1e-3 RMS, and the gated-residual epilogue the block uses at that shape on
    the same rows at 1 bf16 ulp + 1e-3 RMS."""
    M, N, K = W.TOKENS_480P, 2688, 10752
    say("gemm 480p down", M, N, K)
    # 2,048 distinct activation rows, quantized by the oracle, repeated down the 33,784 rows (the
    # oracle quantizer would take about a minute over the whole tensor)
    a0, sa = OQ.quant_fp8_bf16(W.normal_bf16((2048, K), seed=41))
    a = np.ascontiguousarray(np.resize(a0, (M, K)))
    wt, sw = OQ.quant_fp8_bf16(W.f32_to_bf16_bits(W.glorot_uniform(N, K, W.rng_for(41, 81, 0, "w_down"))))
    rows = np.r_[np.random.default_rng(2).choice(M, 60, replace=False), [0, M - 1, M - 120, M - 248]]
    rows_d = torch.from_numpy(rows).cuda()
    ad, wd = u8_dev(a), u8_dev(wt)
    y = Q.gemm_fp8(ad, f32_dev([sa]), wd, f32_dev([sw]))
    got = host(y[rows_d])
    del y
    want = OG.gemm_fp8(a[rows], sa, wt, sw)
    assert_close_rms(got, want, 1e-3, "gemm 480p down rows")
    x = W.normal_bf16((M, N), seed=42)
    gate = np.linspace(-0.2, 0.2, N).astype(np.float32)
    xd = bf16_dev(x)
    Q.gemm_fp8(ad, f32_dev([sa]), wd, f32_dev([sw]), mode=_lib.QVD_EPI_RESID_GATE, out=xd, resid=xd,
               gate=f32_dev(gate))
    want_r = OC.bf16_to_f64(x[rows]) + gate[None, :].astype(np.float64) * want
    assert_bf16_close(host_bits(xd[rows_d]), want_r, 1e-3, "gemm 480p down resid-gate rows")


def test_gemm_bf16_and_resid_gate_epilogues():
    M, N, K = 300, 512, 384
    a, w = _codes(M, K, 3), _codes(N, K, 4, "codes_b")
    sa, sw = np.float32(0.01), np.float32(0.02)
    yb = Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]), mode=_lib.QVD_EPI_BF16)
    want = OG.gemm_fp8(a, sa, w, sw)
    assert_bf16_close(host_bits(yb), want, 1e-3, "bf16 epilogue")
    x = W.normal_bf16((M, N), seed=5)
    gate = np.linspace(-1, 1, N).astype(np.float32)
    xd = bf16_dev(x)
    Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]), mode=_lib.QVD_EPI_RESID_GATE,
               out=xd, resid=xd, gate=f32_dev(gate))
    want_r = OC.bf16_to_f64(x) + gate[None, :].astype(np.float64) * want
    assert_bf16_close(host_bits(xd), want_r, 1e-3, "resid-gate epilogue (in place)")


def test_gemm_gelu_epilogue_and_amax_partials():
    M, N, K = 333, 1024, 256
    a, w = _codes(M, K, 6), _codes(N, K, 7, "codes_b")
    sa, sw = np.float32(0.002), np.float32(0.003)
    parts = torch.zeros(Q.gemm_tiles(M, N), dtype=torch.float32, device="cuda")
    g = Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]), mode=_lib.QVD_EPI_GELU,
                   amax_partials=parts)
    want = OG.gelu(OG.gemm_fp8(a, sa, w, sw))
    assert_bf16_close(host_bits(g), want, 1e-3, "gelu epilogue")
    assert float(host(parts).max()) == float(np.abs(bf16_f64(g)).max())


@pytest.mark.parametrize("fmt,M,N,K", [("fp8", 333, 1024, 256), ("mxfp4", 391, 768, 512)])
def test_gemm_gelu_e4m3_epilogue_static_scale(fmt, M, N, K):
    """GELU -> bf16 -> E4M3 under a static scale, in the epilogue: within the admissible range of the
    oracle's static quantization of bf16(GELU(y)) (below), mostly equal to it, and bit for bit the
    standalone static quantizer applied to the same kernel's bf16 GELU output.  Two scales: one that
    covers the tensor and one that saturates about half of it at 448."""
    say("gemm gelu e4m3", fmt, M, N, K)
    a = _codes(M, K, 8)
    if fmt == "fp8":
        w = _codes(N, K, 9, "codes_b")
        sa, sw = np.float32(0.002), np.float32(0.003)
        y = OG.gemm_fp8(a, sa, w, sw)
        run = lambda **kw: Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]), **kw)
    else:
        wb = W.normal_bf16((N, K), seed=N + K, scale=0.03)
        pw, ew = OQ.quant_mxfp4_weight(wb)
        sa = np.float32(0.05)
        y = OG.gemm_mxfp4(a, sa, pw, ew)
        run = lambda **kw: Q.gemm_mxfp4(u8_dev(a), f32_dev([sa]), u8_dev(pw), u8_dev(ew), **kw)
    g = OG.gelu(y)
    gb = OC.f64_to_bf16_value(g).astype(np.float32)
    gbits = run(mode=_lib.QVD_EPI_GELU)
    for f in (1.25, 0.02):
        s = np.float32(float(np.abs(gb).max()) / 448.0 * f)
        want, _ = OQ.quant_fp8_per_tensor(gb, scale_in=s)
        got = host(run(mode=_lib.QVD_EPI_GELU_E4M3, out_scale=f32_dev([s])))
        inv = np.float32(1.0) / s
        # The codes are those of bf16(GELU(y')) for the GPU's fp32 y', which differs from the exact
        # y by the GEMM's accumulation error.  Bound it by 2.5e-4 RMS(y) (4x inside the 1e-3 RMS GEMM
        # bar); GELU's slope is below 1.13.  bf16 rounding and the encoder are monotone, so every
        # admissible code lies between the codes of bf16(g - e) and bf16(g + e).  Most codes are
        # the oracle's own (at most 1% differ: under a static scale many outputs fall on the fine
        # small codes, where that error spans a code or more; 0.27% measured at the FP8 shape).
        e = 2.5e-4 * 1.13 * float(np.sqrt(np.mean(y ** 2)))
        lo, _ = OQ.quant_fp8_per_tensor(OC.f64_to_bf16_value(g - e).astype(np.float32), scale_in=s)
        hi, _ = OQ.quant_fp8_per_tensor(OC.f64_to_bf16_value(g + e).astype(np.float32), scale_in=s)
        vg, vlo, vhi = (OC.e4m3_decode(c.reshape(-1)) for c in (got, lo, hi))
        out = np.nonzero((vg < vlo) | (vg > vhi))[0]
        assert out.size == 0, (f"gelu e4m3 {fmt} x{f}: {out.size} codes outside the admissible range, "
                               f"e.g. {out[:4].tolist()} got {vg[out[:4]].tolist()} range "
                               f"{vlo[out[:4]].tolist()}..{vhi[out[:4]].tolist()}")
        assert np.mean(got.reshape(-1) != want.reshape(-1)) <= 1e-2
        two_pass, _ = Q.quant_fp8_per_tensor(gbits, scale_in=f32_dev([s]))
        np.testing.assert_array_equal(got, host(two_pass))


def _vt_tile_exponent(amax: float) -> int:
    """The V^T tile exponent rule as the header states it: 0 while max|v| is in [2^-6, 2^15) (or the
    tile is zero), else floor(log2 max|v|) - 14."""
    if amax == 0 or 2.0 ** -6 <= amax < 2.0 ** 15:
        return 0
    return int(np.floor(np.log2(amax))) - 14


def _realistic_codes(M, N, K, seed):
    """Activation codes of N(0,1) data and weight codes of Glorot-uniform weights, both through the
    oracle's per-tensor quantizer (so the accumulators have a realistic dynamic range)."""
    a, sa = OQ.quant_fp8_bf16(W.normal_bf16((M, K), seed=seed))
    wt = W.Workload("t", 80, d=K, n_heads=K // 128, mlp=4 * K, L=M, sparse=False, outliers=False)
    w, sw = OQ.quant_fp8_bf16(W.f32_to_bf16_bits(W.glorot_uniform(N, K, W.rng_for(seed, 80, 0, "w_qkv"))))
    return a, sa, w, sw


@pytest.mark.parametrize("M,H", [(256, 2), (391, 2), (130, 21)])
def test_gemm_qkv_epilogue(M, H):
    d = 128 * H
    N, K = 3 * d, d
    a, sa, w, sw = _realistic_codes(M, N, K, 8 + H)
    q8, k8, v, qs, ks = Q.gemm_fp8(u8_dev(a), f32_dev([sa]), u8_dev(w), f32_dev([sw]),
                                   mode=_lib.QVD_EPI_QKV, n_heads=H)
    y = OG.gemm_fp8(a, sa, w, sw)
    ybits = OC.f64_to_bf16(y)
    # V part: fp16 V^T [H][128][Lp] holding the bf16-rounded values times 2^-e per (head, tile),
    # zeros past M; the exponents follow the tile rule, and fp16 * 2^e is a bf16 value exactly
    T = (M + 127) // 128
    vt = host(v.t).astype(np.float64)
    te = host(v.tile_exp)
    assert vt.shape == (H, 128, T * 128) and te.shape == (H, T)
    assert not vt[:, :, M:].any()
    vv = vt[:, :, :M] * np.ldexp(1.0, np.repeat(te, 128, axis=1)[:, None, :M])
    v_got = vv.transpose(2, 0, 1).reshape(M, d)
    v_bits = OC.f64_to_bf16(v_got)
    normal = np.abs(vt[:, :, :M].transpose(2, 0, 1).reshape(M, d)) >= 2.0 ** -14
    np.testing.assert_array_equal(OC.bf16_to_f64(v_bits)[normal], v_got[normal])
    assert_bf16_close(v_bits, y[:, 2 * d:], 1e-3, "V part")
    for h in range(H):
        for i in range(T):
            a_ = np.abs(v_got[i * 128: min(M, (i + 1) * 128), h * 128: (h + 1) * 128]).max()
            assert te[h, i] == _vt_tile_exponent(a_), (h, i, a_, te[h, i])
    for part, (g8, gs) in enumerate(((q8, qs), (k8, ks))):
        cw, sw_ = OQ.quant_int8_qk(np.ascontiguousarray(ybits[:, part * d:(part + 1) * d]), M, H)
        # scales: bf16 rounding of the fp32 accumulators can differ at near-ties only
        np.testing.assert_allclose(host(gs), sw_, rtol=2 ** -7)
        xv = OC.bf16_to_f64(ybits[:, part * d:(part + 1) * d]).reshape(M, H, 128).astype(np.float32)
        T = (M + 127) // 128
        pre = np.empty_like(xv)
        for h in range(H):
            for i in range(T):
                r = slice(i * 128, min(M, (i + 1) * 128))
                a_ = np.float32(np.abs(xv[r, h]).max())
                pre[r, h] = xv[r, h] * (np.float32(127) / a_)
        n = assert_codes_equal_except_ties(host(g8), cw, pre, "int8", max_frac=1e-3,
                                           name=f"qkv part {part}",
                                           upstream=y[:, part * d:(part + 1) * d].reshape(M, H, 128))
        say(f"qkv part {part}: {n} tie flips")


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (391, 384, 256), (300, 2688, 2688), (130, 256, 10752),
                                   (257, 128, 1152), (1, 256, 128)])
def test_gemm_mxfp4_f32_and_bf16(M, N, K):
    say("gemm mxfp4", M, N, K)
    a = _codes(M, K, M + 1)
    wb = W.normal_bf16((N, K), seed=N + K, scale=0.03)
    pw, ew = OQ.quant_mxfp4_weight(wb)
    sa = np.float32(0.05)
    bias = np.linspace(-1, 1, N).astype(np.float32)
    want = OG.gemm_mxfp4(a, sa, pw, ew, bias)
    y = host(Q.gemm_mxfp4(u8_dev(a), f32_dev([sa]), u8_dev(pw), u8_dev(ew), bias=f32_dev(bias)))
    assert_close_rms(y, want, 1e-3, "mxfp4 f32")
    yb = Q.gemm_mxfp4(u8_dev(a), f32_dev([sa]), u8_dev(pw), u8_dev(ew), bias=f32_dev(bias),
                      mode=_lib.QVD_EPI_BF16)
    assert_bf16_close(host_bits(yb), want, 1e-3, "mxfp4 bf16")


def test_gemm_mxfp4_768p_qkv_shape_sampled():
    """The 768p QKV shape with MXFP4 weights: M = 85,696 (ragged last tile), N = 8,064, K = 2,688;
    64 sampled rows against the oracle."""
    M, N, K = W.TOKENS_768P, 3 * 2688, 2688
    say("gemm mxfp4 768p", M, N, K)
    a = _codes(M, K, 11)
    wb = W.normal_bf16((N, K), seed=12, scale=0.03)
    pw, ew = OQ.quant_mxfp4_weight(wb)
    sa = np.float32(0.02)
    y = Q.gemm_mxfp4(u8_dev(a), f32_dev([sa]), u8_dev(pw), u8_dev(ew))
    rows = np.r_[np.random.default_rng(1).choice(M, 60, replace=False), [0, M - 1, M - 64, M - 200]]
    got = host(y[torch.from_numpy(rows).cuda()])
    del y
    want = OG.gemm_mxfp4(a[rows], sa, pw, ew)
    assert_close_rms(got, want, 1e-3, "mxfp4 768p rows")


# --- attention ---------------------------------------------------------------------------------

def _attn_inputs(L, H, seed, sparse, w=None):
    qb, kb, vb = W.qkv_heads(L, H, seed=seed)
    wl = W.Workload("t", 90 + H, d=128 * H, n_heads=H, mlp=512 * H, L=L, sparse=sparse,
                    outliers=False) if w is None else w
    idx, cnt = W.block_mask(wl, seed=seed, L=L)
    return qb, kb, vb, idx, cnt


def _quantize_both(qb, kb, L, H):
    q8, qs = Q.quant_int8_qk(bf16_dev(qb.reshape(L, H * 128)), H)
    k8, ks = Q.quant_int8_qk(bf16_dev(kb.reshape(L, H * 128)), H)
    oq, oqs = OQ.quant_int8_qk(qb, L, H)
    ok, oks = OQ.quant_int8_qk(kb, L, H)
    np.testing.assert_array_equal(host(q8), oq)       # identical inputs to both attentions
    np.testing.assert_array_equal(host(k8), ok)
    return (q8, qs, k8, ks), (oq, oqs, ok, oks)


@pytest.mark.parametrize("L,i,j", [(256, 0, 1), (391, 3, 3), (391, 1, 3), (1000, 7, 2)])
def test_qk_int32_accumulators_bit_exact(L, i, j):
    H = 2
    qb, kb, _, _, _ = _attn_inputs(L, H, 3, False)
    (q8, _, k8, _), (oq, _, ok, _) = _quantize_both(qb, kb, L, H)
    for h in range(H):
        got = host(Q.qk_int32_tile(q8, k8, h, i, j))
        want = np.zeros((128, 128), np.int64)
        r = np.arange(i * 128, min(L, (i + 1) * 128))
        c = np.arange(j * 128, min(L, (j + 1) * 128))
        want[: len(r), : len(c)] = oq[r, h].astype(np.int64) @ ok[c, h].astype(np.int64).T
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("L,H,sparse", [(256, 2, False), (391, 2, False), (1290, 2, True),
                                        (2000, 3, True), (128, 1, False), (1, 2, False), (37, 3, False)])
def test_sparse_attn_vs_oracle(L, H, sparse):
    say("attn", L, H, sparse)
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, L, sparse)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb, kb, L, H)
    out, part = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt), want_amax=True)
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt)
    got = bf16_f64(out)
    assert_bf16_close(host_bits(out), want, 1e-2, f"attn L={L}")
    T = (L + 127) // 128
    gp = host(part)
    for h in range(H):
        for i in range(T):
            rr = slice(i * 128, min(L, (i + 1) * 128))
            assert gp[h, i] == np.abs(got[rr, h]).max()


def test_sparse_attn_peaked_rows_large_logit_gap():
    """Every query row has one dominant key (the same unit direction in Q and K, |.| = 20 against
    0.05-scaled noise), about 50 log2 units above the other scores.  For three rows in four that key
    lies outside the first 8 keys of its 32-key block, so a row maximum taken over part of a tile
    would leave numerators far above one (beyond fp16 range): the result must stay finite and equal
    the oracle's, which is the mean of the V rows of the dominant keys."""
    L, H = 256, 2
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, 5, False)
    hot = np.zeros((L, H, 128), np.float32)
    rows = np.arange(L)
    hot[rows, :, rows % 128] = 20.0
    qb2 = W.f32_to_bf16_bits(0.05 * W.bf16_bits_to_f32(qb) + hot)
    kb2 = W.f32_to_bf16_bits(0.05 * W.bf16_bits_to_f32(kb) + hot)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb2, kb2, L, H)
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt)
    assert np.isfinite(bf16_f64(out)).all()
    assert_bf16_close(host_bits(out), want, 1e-2, "peaked rows")


def test_sparse_attn_e4m3_output_static_scale():
    """The E4M3 entry equals, bit for bit, the standalone static quantizer applied to the bf16
    entry's output, and its dequantized codes stay within E4M3 rounding (2^-4 relative) plus 1e-2 RMS
    of the oracle attention; a second, small scale saturates part of the output."""
    L, H = 1290, 2
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, 13, True)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb, kb, L, H)
    vt_d = Q.vt_unify(Q.vt_from_bf16(bf16_dev(vb)))
    out = Q.sparse_attn_vt(q8, qs, k8, ks, vt_d, i32_dev(idx), i32_dev(cnt))
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt)
    rms = float(np.sqrt(np.mean(want ** 2)))
    for f in (1.1, 0.1):
        s = np.float32(float(np.abs(want).max()) / 448.0 * f)
        got = Q.sparse_attn_vt_e4m3(q8, qs, k8, ks, vt_d, i32_dev(idx), i32_dev(cnt), f32_dev([s]))
        two_pass, _ = Q.quant_fp8_per_tensor(out, scale_in=f32_dev([s]))
        np.testing.assert_array_equal(host(got), host(two_pass))
        deq = OC.e4m3_decode(host(got).reshape(-1)) * float(s)
        ref = np.clip(want.reshape(-1), -448.0 * float(s), 448.0 * float(s))
        err = np.abs(deq - ref)
        assert (err <= 2.0 ** -4 * np.abs(ref) + 1e-2 * rms + 2.0 ** -9 * float(s)).all(), \
            f"attn e4m3 x{f}: worst {float(err.max()):.3e} (RMS {rms:.3e})"


def test_sparse_attn_vt_entry_matches_bf16_entry():
    """The V^T entry point, on V transposed by qvd_vt_from_bf16 and unified per head, gives the same
    bits as the bf16 entry."""
    L, H = 1290, 2
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, 12, True)
    (q8, qs, k8, ks), _ = _quantize_both(qb, kb, L, H)
    a = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    b = Q.sparse_attn_vt(q8, qs, k8, ks, Q.vt_unify(Q.vt_from_bf16(bf16_dev(vb))), i32_dev(idx),
                         i32_dev(cnt))
    np.testing.assert_array_equal(host_bits(a), host_bits(b))


def test_vt_transpose_and_unify():
    """qvd_vt_from_bf16 then qvd_vt_unify on a V whose tiles need different exponents: one tile of
    head 0 is scaled up to 1e6 (exponent 5), one of head 1 down to 1e-4 (exponent -28), the rest are
    in the usual range (exponent 0).  Every tile's exponent follows the rule; each head then holds
    fp16(v 2^-E) with E the head's largest exponent, equal to the bf16 value times 2^-E wherever that
    is an fp16 normal, and within the fp16 subnormal spacing (2^-25) below it."""
    L, H = 700, 2
    _, _, vb = W.qkv_heads(L, H, seed=17)
    v = OC.bf16_to_f64(vb)
    v[256:384, 0, :] *= 1e6 / np.abs(v[256:384, 0, :]).max()
    v[128:256, 1, :] *= 1e-4 / np.abs(v[128:256, 1, :]).max()
    vb2 = OC.f64_to_bf16(v)
    v = OC.bf16_to_f64(vb2)
    T = (L + 127) // 128
    tiles = Q.vt_from_bf16(bf16_dev(vb2))
    te = host(tiles.tile_exp)
    for h in range(H):
        for j in range(T):
            assert te[h, j] == _vt_tile_exponent(np.abs(v[j * 128: (j + 1) * 128, h]).max()), (h, j)
    assert te[0, 2] == 5 and te[1, 1] == -28 and te[0, 0] == 0
    vt = Q.vt_unify(tiles)
    he = host(vt.exp)
    np.testing.assert_array_equal(he, te.max(axis=1))
    got = host(vt.t).astype(np.float64)
    assert not got[:, :, L:].any()
    want = np.ldexp(v.transpose(1, 2, 0), -he[:, None, None])
    err = np.abs(got[:, :, :L] - want)
    normal = np.abs(want) >= 2.0 ** -14
    assert not err[normal].any()
    assert (err[~normal] <= 2.0 ** -25).all()


def test_sparse_attn_v_outside_fp16_range():
    """V as bf16 at magnitudes fp16 cannot hold: head 0 has every third key row scaled by 1e6 in
    dims 0..31 (above 65,504; those outputs are dominated by them), head 1 is scaled by 1e-9
    throughout (below fp16's smallest normal, 2^-14).  Each head must match the oracle within one
    bf16 ulp + 1e-2 of its own output RMS."""
    L, H = 1290, 2
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, 21, True)
    v = OC.bf16_to_f64(vb)
    v[::3, 0, :32] *= 1e6
    v[:, 1, :] *= 1e-9
    vb2 = OC.f64_to_bf16(v)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb, kb, L, H)
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb2), i32_dev(idx), i32_dev(cnt))
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb2, idx, cnt)
    ob = host_bits(out)
    assert np.abs(want[:, 0, :32]).max() > 65504 * 4
    for h in range(H):
        assert_bf16_close(np.ascontiguousarray(ob[:, h]), want[:, h], 1e-2, f"V outside fp16, head {h}")
    # the same through the V^T entry (the layout the QKV epilogue writes)
    out_t = Q.sparse_attn_vt(q8, qs, k8, ks, Q.vt_unify(Q.vt_from_bf16(bf16_dev(vb2))), i32_dev(idx),
                             i32_dev(cnt))
    np.testing.assert_array_equal(host_bits(out_t), ob)


def test_sparse_attn_large_qk_scales_tile_varying_k():
    """Q and K scaled so that tile maxima reach about 100, and each key tile's K rows further scaled by
    its own factor in [1/4, 4]: the per-tile score factors sQ sK / sqrt(128) log2(e) then differ by up
    to 16x within one row and reach ~0.5 log2 units per integer score step.  The numerator arguments
    must stay exact up to fp32 rounding across tiles (a constant rounded per tile would skew the
    tiles' relative weights by up to ~0.4 log2 units here)."""
    L, H = 1290, 2
    qb, kb, vb, idx, cnt = _attn_inputs(L, H, 23, True)
    T = (L + 127) // 128
    f = np.exp(np.random.default_rng(5).uniform(np.log(0.25), np.log(4.0), size=(H, T)))
    qv = OC.bf16_to_f64(qb) * 25.0
    kv = OC.bf16_to_f64(kb) * 25.0
    for h in range(H):
        kv[:, h, :] *= f[h][np.arange(L) // 128][:, None]
    qb2, kb2 = OC.f64_to_bf16(qv), OC.f64_to_bf16(kv)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb2, kb2, L, H)
    say("large scales: max q scale", float(host(qs).max()), "k scale range",
        float(host(ks).min()), float(host(ks).max()))
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt)
    assert_bf16_close(host_bits(out), want, 1e-2, "large Q/K scales")


def test_sparse_attn_row_varying_kept_counts():
    """Each (head, query tile) keeps its own number of tiles, 0 .. kmax, drawn so that the two work
    items of one workgroup (neighbouring query tiles of a head) mostly differ; the lists are random
    ascending tile sets with or without the diagonal.  Rows with no kept tile give zeros."""
    L, H = 2000, 3
    T = (L + 127) // 128
    kmax = 12
    rng = np.random.default_rng(31)
    qb, kb, vb = W.qkv_heads(L, H, seed=31)
    idx = np.full((H, T, kmax), -1, np.int32)
    cnt = np.zeros((H, T), np.int32)
    for h in range(H):
        for i in range(T):
            c = int(rng.integers(0, kmax + 1)) if (h * T + i) % 5 else 0
            tiles = np.sort(rng.choice(T, size=c, replace=False)).astype(np.int32)
            idx[h, i, :c] = tiles
            cnt[h, i] = c
    pairs = cnt.reshape(-1)[: (H * T) // 2 * 2].reshape(-1, 2)
    assert (pairs[:, 0] != pairs[:, 1]).mean() > 0.5
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb, kb, L, H)
    out, part = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt), want_amax=True)
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt)
    got = bf16_f64(out)
    assert_bf16_close(host_bits(out), want, 1e-2, "row-varying counts")
    for h in range(H):
        for i in range(T):
            if cnt[h, i] == 0:
                assert not got[i * 128: min(L, (i + 1) * 128), h].any()


def test_sparse_attn_diag_only_and_out_of_range_entries():
    L, H = 391, 2
    qb, kb, vb, _, _ = _attn_inputs(L, H, 9, False)
    (q8, qs, k8, ks), (oq, oqs, ok, oks) = _quantize_both(qb, kb, L, H)
    T = 4
    idx = np.full((H, T, 3), -1, np.int32)
    idx[:, :, 0] = np.arange(T)
    idx[:, :, 1] = 99                   # out of range: ignored by the kernel
    cnt = np.full((H, T), 2, np.int32)
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx[:, :, :1].copy(), np.ones((H, T), np.int32))
    assert_bf16_close(host_bits(out), want, 1e-2, "diag only")
    # a row with no kept key outputs zeros
    cnt0 = np.zeros((H, T), np.int32)
    out0 = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt0))
    assert not host_bits(out0).any()


def test_sparse_attn_768p_sampled_tiles():
    """The 768p token count (85,696 tokens: 670 tiles, last one of 64 rows; 135 kept per row), three
    heads of the 768p mask; sampled query tiles against the oracle."""
    w = W.WORKLOADS["block_768p_mxfp4"]
    L, H = w.L, 3
    T = w.n_tiles
    say("attn 768p", L, T)
    qb, kb, vb = W.qkv_heads(L, H, seed=3, tag=w.tag)
    idx, cnt = W.block_mask(w, seed=0)
    idx, cnt = np.ascontiguousarray(idx[:H]), np.ascontiguousarray(cnt[:H])
    q8, qs = Q.quant_int8_qk(bf16_dev(qb.reshape(L, -1)), H)
    k8, ks = Q.quant_int8_qk(bf16_dev(kb.reshape(L, -1)), H)
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    tiles = [(0, 0), (1, T - 1), (2, 335), (0, 669), (1, 2)]
    qq, kq = np.zeros((L, H, 128), np.int8), np.zeros((L, H, 128), np.int8)
    qsc, ksc = np.ones((H, T), np.float32), np.ones((H, T), np.float32)
    for h, i in tiles:
        rows = slice(i * 128, min(L, (i + 1) * 128))
        cw, sw = OQ.quant_int8_qk(np.ascontiguousarray(qb[rows, h:h + 1]), rows.stop - rows.start, 1)
        qq[rows, h], qsc[h, i] = cw[:, 0], sw[0, 0]
        for j in idx[h, i, : cnt[h, i]]:
            rk = slice(j * 128, min(L, (j + 1) * 128))
            cw, sw = OQ.quant_int8_qk(np.ascontiguousarray(kb[rk, h:h + 1]), rk.stop - rk.start, 1)
            kq[rk, h], ksc[h, j] = cw[:, 0], sw[0, 0]
    ob = host_bits(out)
    for h, i in tiles:
        rows = slice(i * 128, min(L, (i + 1) * 128))
        want = OAT.sparse_attn_tile(qq, qsc, kq, ksc, vb, idx, cnt, h, i, 1 / math.sqrt(128))
        assert_bf16_close(ob[rows, h], want, 1e-2, f"768p tile {(h, i)}")


def test_sparse_attn_480p_sampled_tiles():
    """The attention-only 480p workload: 21 heads, 264 tiles, 53 kept per row; sampled tiles."""
    w = W.WORKLOADS["attn_480p"]
    L, H = w.L, w.n_heads
    qb, kb, vb = W.qkv_heads(L, H, seed=0, tag=w.tag)
    idx, cnt = W.block_mask(w, seed=0)
    q8, qs = Q.quant_int8_qk(bf16_dev(qb.reshape(L, -1)), H)
    k8, ks = Q.quant_int8_qk(bf16_dev(kb.reshape(L, -1)), H)
    out = Q.sparse_attn(q8, qs, k8, ks, bf16_dev(vb), i32_dev(idx), i32_dev(cnt))
    T = w.n_tiles
    tiles = [(0, 0), (20, T - 1), (5, 131), (17, 263), (11, 7)]
    # oracle inputs come from the oracle's own quantizer, for the query tiles sampled and every key
    # tile they read; the GPU's codes for the same tiles are compared to them separately
    gq, gk = host(q8), host(k8)
    qq = np.zeros((L, H, 128), np.int8)
    kq = np.zeros((L, H, 128), np.int8)
    qsc = np.ones((H, T), np.float32)
    ksc = np.ones((H, T), np.float32)
    for h, i in tiles:
        rows = slice(i * 128, min(L, (i + 1) * 128))
        cw, sw = OQ.quant_int8_qk(np.ascontiguousarray(qb[rows, h:h + 1]), rows.stop - rows.start, 1)
        qq[rows, h], qsc[h, i] = cw[:, 0], sw[0, 0]
        np.testing.assert_array_equal(gq[rows, h], cw[:, 0])
        for j in idx[h, i, : cnt[h, i]]:
            rk = slice(j * 128, min(L, (j + 1) * 128))
            cw, sw = OQ.quant_int8_qk(np.ascontiguousarray(kb[rk, h:h + 1]), rk.stop - rk.start, 1)
            kq[rk, h], ksc[h, j] = cw[:, 0], sw[0, 0]
            np.testing.assert_array_equal(gk[rk, h], cw[:, 0])
    got = bf16_f64(out)
    for h, i in tiles:
        rows = slice(i * 128, min(L, (i + 1) * 128))
        want = OAT.sparse_attn_tile(qq, qsc, kq, ksc, vb, idx, cnt, h, i, 1 / math.sqrt(128))
        assert_bf16_close(host_bits(out)[rows, h], want, 1e-2, f"480p tile {(h, i)}")
