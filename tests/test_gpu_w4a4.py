"""GPU parity of the MXFP4 x MXFP4 (W4A4) GEMM against the oracle: activations quantized per token row
and 32-element block exactly as weights are (E2M1 elements, E8M0 block scales), both operands on the
block-scaled matrix cores, fp32 accumulation."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from oracle import codecs as OC, quant as OQ, gemm as OG, adaln as OA, attention as OAT
from _gpu_util import (say, bf16_dev, u8_dev, i32_dev, f32_dev, host, host_bits, assert_close_rms,
                       assert_bf16_close)

pytestmark = pytest.mark.gpu


def _acts(M, K, seed):
    """bf16 [M][K] activations: N(0,1), three outlier channels x30, token rows scaled over 2^-12..2^6
    (so row block scales differ), and every 7th 32-element block of every 5th row zeroed (all-zero
    blocks take E8M0 127 with zero elements)."""
    rng = W.rng_for(seed, 17, 0, "x")
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, size=min(3, K), replace=False)] *= np.float32(30.0)
    x *= np.exp2(rng.integers(-12, 7, size=(M, 1))).astype(np.float32)
    z = x.reshape(M, K // 32, 32)
    z[::5, ::7, :] = 0.0
    return W.f32_to_bf16_bits(z.reshape(M, K))


def _weights(N, K, seed):
    return OQ.quant_mxfp4_weight(W.normal_bf16((N, K), seed=seed, scale=0.03))


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (391, 384, 256), (33, 2688, 2688), (700, 768, 1024),
                                   (1, 128, 384), (130, 256, 10752), (300, 128, 1152)])
def test_w4a4_f32_and_bf16_vs_oracle(M, N, K):
    say("w4a4", M, N, K)
    ap, ae = OQ.quant_mxfp4_weight(_acts(M, K, M + K))
    wp, we = _weights(N, K, N + 3 * K)
    bias = np.linspace(-2, 2, N).astype(np.float32)
    want = OG.gemm_mxfp4_w4a4(ap, ae, wp, we, bias)
    y = host(Q.gemm_mxfp4_w4a4(u8_dev(ap), u8_dev(ae), u8_dev(wp), u8_dev(we), bias=f32_dev(bias)))
    assert_close_rms(y, want, 1e-3, "w4a4 f32")
    yb = Q.gemm_mxfp4_w4a4(u8_dev(ap), u8_dev(ae), u8_dev(wp), u8_dev(we), bias=f32_dev(bias),
                           mode=_lib.QVD_EPI_BF16)
    assert_bf16_close(host_bits(yb), want, 1e-3, "w4a4 bf16")


def test_w4a4_device_activation_quant_chain():
    """bf16 activations -> quant_mxfp4 on the device (bit-exact against the oracle's codes and scales)
    -> W4A4 GEMM with the GELU epilogue, against the oracle's chain from the same bf16 input."""
    M, N, K = 515, 512, 2688
    xb = _acts(M, K, 5)
    ap_d, ae_d = Q.quant_mxfp4(bf16_dev(xb))
    ap, ae = OQ.quant_mxfp4_weight(xb)
    np.testing.assert_array_equal(host(ae_d), ae)
    np.testing.assert_array_equal(host(ap_d), ap)
    wp, we = _weights(N, K, 9)
    lin = OG.gemm_mxfp4_w4a4(ap, ae, wp, we)
    y = host(Q.gemm_mxfp4_w4a4(ap_d, ae_d, u8_dev(wp), u8_dev(we)))
    assert_close_rms(y, lin, 1e-3, "w4a4 chain f32")
    g = Q.gemm_mxfp4_w4a4(ap_d, ae_d, u8_dev(wp), u8_dev(we), mode=_lib.QVD_EPI_GELU)
    assert_bf16_close(host_bits(g), OG.gelu(lin), 1e-3, "w4a4 gelu")


def test_w4a4_exact_small_integers():
    """Operands whose partial sums all fit fp32's 24-bit significand, so any accumulation order is exact
    and the result equals the oracle bit for bit.  Block scales 2^(r + e): a row (column) offset r in
    -20 .. 20 and a per-block e in -2 .. 2, so one output's terms span at most 21 binades."""
    M, N, K = 130, 256, 512
    rng = np.random.default_rng(3)
    # E2M1 codes of 0, +-0.5, +-1, +-2 (0, 1, 9, 2, 10, 4, 12) keep every partial sum representable
    pick = np.array([0, 1, 9, 2, 10, 4, 12], dtype=np.uint8)
    ca = pick[rng.integers(0, 7, size=(M, K))]
    cw = pick[rng.integers(0, 7, size=(N, K))]
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    ae = (127 + rng.integers(-20, 21, size=(M, 1)) + rng.integers(-2, 3, size=(M, K // 32))).astype(np.uint8)
    we = (127 + rng.integers(-20, 21, size=(N, 1)) + rng.integers(-2, 3, size=(N, K // 32))).astype(np.uint8)
    ap, wp = pack(ca), pack(cw)
    want = OG.gemm_mxfp4_w4a4(ap, ae, wp, we)
    assert np.all(want == want.astype(np.float32))
    y = host(Q.gemm_mxfp4_w4a4(u8_dev(ap), u8_dev(ae), u8_dev(wp), u8_dev(we)))
    np.testing.assert_array_equal(y, want.astype(np.float32))


def test_w4a4_empty_and_shape_errors():
    wp, we = _weights(128, 128, 1)
    ap = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    ae = torch.zeros((0, 4), dtype=torch.uint8, device="cuda")
    y = Q.gemm_mxfp4_w4a4(ap, ae, u8_dev(wp), u8_dev(we))
    assert tuple(y.shape) == (0, 128)
    with pytest.raises(Exception):
        Q.gemm_mxfp4_w4a4(torch.zeros((4, 48), dtype=torch.uint8, device="cuda"),
                          torch.zeros((4, 3), dtype=torch.uint8, device="cuda"), u8_dev(wp), u8_dev(we))


def test_w4a4_768p_mlp_up_shape_sampled():
    """The 768p MLP-up shape: M = 85,696 (ragged last tile), N = 10,752, K = 2,688; 64 sampled rows."""
    M, N, K = W.TOKENS_768P, 4 * 2688, 2688
    say("w4a4 768p", M, N, K)
    xb = _acts(M, K, 21)
    ap, ae = Q.quant_mxfp4(bf16_dev(xb))
    wp, we = _weights(N, K, 22)
    y = Q.gemm_mxfp4_w4a4(ap, ae, u8_dev(wp), u8_dev(we))
    rows = np.r_[np.random.default_rng(2).choice(M, 60, replace=False), [0, M - 1, M - 64, M - 200]]
    got = host(y[torch.from_numpy(rows).cuda()])
    del y
    oap, oae = OQ.quant_mxfp4_weight(xb[rows])
    want = OG.gemm_mxfp4_w4a4(oap, oae, wp, we)
    assert_close_rms(got, want, 1e-3, "w4a4 768p rows")


# --- MXFP4 producers of the W4A4 block -------------------------------------------------------------

@pytest.mark.parametrize("d,L,half", [(256, 300, 0), (2688, 133, 1), (1024, 64, 0)])
def test_adaln_modulate_mxfp4_bit_exact(d, L, half):
    """Modulated LayerNorm -> MXFP4: the kernel forms y as the float64 modulation rounded once to fp32,
    as the oracle does, so codes and block scales agree bit for bit."""
    say("modulate mxfp4", d, L, half)
    w = W.Workload("m", 60 + d // 128, d=d, n_heads=d // 128, mlp=4 * d, L=L, sparse=False,
                   outliers=d >= 1000)
    x = W.activations(w, 3, L=L)
    mod = W.random_mod(d, seed=4, tag=w.tag)
    p, e = Q.adaln_modulate_mxfp4(bf16_dev(x), f32_dev(mod), half)
    op, oe = OA.adaln_modulate_mxfp4(x, mod, half)
    np.testing.assert_array_equal(host(e), oe)
    np.testing.assert_array_equal(host(p), op)


def _vt_dev(vb, L, H):
    return Q.vt_unify(Q.vt_from_bf16(bf16_dev(np.ascontiguousarray(vb).reshape(L, H, 128))))


@pytest.mark.parametrize("L,H,sparse", [(1290, 2, True), (391, 3, False)])
def test_sparse_attn_mxfp4_output(L, H, sparse):
    """The MXFP4 entry equals, bit for bit, quant_mxfp4 of the bf16 entry's output viewed as
    [L][H*128]; dequantized, it lies within half an E2M1 step (or the saturation at 6 X) of the
    oracle attention, up to the attention's own tolerance (one bf16 ulp + 1e-2 RMS)."""
    say("attn mxfp4", L, H, sparse)
    qb, kb, vb = W.qkv_heads(L, H, seed=L)
    wl = W.Workload("t", 90 + H, d=128 * H, n_heads=H, mlp=512 * H, L=L, sparse=sparse, outliers=False)
    idx, cnt = W.block_mask(wl, seed=L, L=L)
    q8, qs = Q.quant_int8_qk(bf16_dev(qb.reshape(L, H * 128)), H)
    k8, ks = Q.quant_int8_qk(bf16_dev(kb.reshape(L, H * 128)), H)
    vt = _vt_dev(vb, L, H)
    out = Q.sparse_attn_vt(q8, qs, k8, ks, vt, i32_dev(idx), i32_dev(cnt))
    p, e = Q.sparse_attn_vt_mxfp4(q8, qs, k8, ks, vt, i32_dev(idx), i32_dev(cnt))
    p2, e2 = Q.quant_mxfp4(out.reshape(L, H * 128))
    np.testing.assert_array_equal(host(e), host(e2))
    np.testing.assert_array_equal(host(p), host(p2))
    oq, oqs = OQ.quant_int8_qk(qb, L, H)
    ok, oks = OQ.quant_int8_qk(kb, L, H)
    want = OAT.sparse_attn(oq, oqs, ok, oks, vb, idx, cnt).reshape(L, H * 128)
    deq = OG.dequant_mxfp4(host(p), host(e))
    X = np.repeat(OC.e8m0_decode(host(e)), 32, axis=1)
    r = np.abs(want) / X
    half_step = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0)) * X
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = np.abs(deq - np.clip(want, -6 * X, 6 * X))
    # the codes are those of bf16 O, which lies within the attention's own bar of the exact value:
    # one bf16 ulp (2^-7 |O| covers it) + 1e-2 RMS
    slack = np.abs(want) * 2.0 ** -7 + 1e-2 * rms
    assert (err <= half_step + slack).all(), f"worst {float((err - half_step - slack).max()):.3e}, RMS {rms:.3e}"


@pytest.mark.parametrize("fmt,M,N,K", [("w4a4", 391, 768, 512), ("w4a4", 256, 256, 2688), ("fp8", 333, 1024, 256)])
def test_gemm_gelu_mxfp4_epilogue(fmt, M, N, K):
    """GELU -> bf16 -> MXFP4 in the epilogue equals, bit for bit, the GELU epilogue followed by
    quant_mxfp4; and the W4A4 chain agrees with the oracle's within half an E2M1 step (1% of the
    elements may sit one step off where GELU lands within the accumulation error of a midpoint)."""
    say("gelu mxfp4", fmt, M, N, K)
    wp, we = _weights(N, K, N + K)
    bias = np.linspace(-1, 1, N).astype(np.float32)
    if fmt == "w4a4":
        ap, ae = OQ.quant_mxfp4_weight(_acts(M, K, 31))
        args = (u8_dev(ap), u8_dev(ae), u8_dev(wp), u8_dev(we))
        gm = Q.gemm_mxfp4_w4a4
        lin = OG.gemm_mxfp4_w4a4(ap, ae, wp, we, bias)
    else:
        a, w8 = W.random_e4m3_codes((M, K), seed=6), W.random_e4m3_codes((N, K), seed=7, tensor="codes_b")
        args = (u8_dev(a), f32_dev([np.float32(0.002)]), u8_dev(w8), f32_dev([np.float32(0.003)]))
        gm = Q.gemm_fp8
        lin = OG.gemm_fp8(a, np.float32(0.002), w8, np.float32(0.003), bias)
    g = gm(*args, bias=f32_dev(bias), mode=_lib.QVD_EPI_GELU)
    p, e = gm(*args, bias=f32_dev(bias), mode=_lib.QVD_EPI_GELU_MXFP4)
    p2, e2 = Q.quant_mxfp4(g)
    np.testing.assert_array_equal(host(e), host(e2))
    np.testing.assert_array_equal(host(p), host(p2))
    op, oe = OQ.quant_mxfp4_weight(OC.f64_to_bf16(OG.gelu(lin)))
    same = (OQ.unpack_e2m1(host(p)) == OQ.unpack_e2m1(op)) & np.repeat(host(e) == oe, 32, axis=1)
    assert same.mean() >= 0.99, f"{1 - same.mean():.4f} of the codes differ from the oracle's"
