"""GPU parity of the quantizers and the AdaLN kernels against the oracle (bit-exact codes)."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from oracle import codecs as OC, quant as OQ, adaln as OA
from _gpu_util import (say, bf16_dev, fp16_dev, f32_dev, host, host_bits,
                       assert_codes_equal_except_ties)

pytestmark = pytest.mark.gpu


def test_fp8_encoder_all_bf16_patterns_static_scale_one():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = OC.bf16_to_f64(b)
    b = b[np.isfinite(v)]
    say("fp8 static s=1 over", b.size, "bf16 patterns")
    q, s = Q.quant_fp8_per_tensor(bf16_dev(b), scale_in=f32_dev([1.0]))
    want, _ = OQ.quant_fp8_bf16(b, scale_in=np.float32(1.0))
    np.testing.assert_array_equal(host(q), want)
    assert host(s)[0] == 1.0


@pytest.mark.parametrize("n,scale", [(1, 1.0), (7, 3.0), (4096 * 3 + 5, 0.01), (1 << 20, 50.0)])
def test_fp8_dynamic_bit_exact(n, scale):
    say("fp8 dynamic n =", n)
    x = W.normal_bf16((n,), seed=n, scale=scale)
    q, s = Q.quant_fp8_per_tensor(bf16_dev(x))
    want, ws = OQ.quant_fp8_bf16(x)
    assert host(s)[0] == ws
    np.testing.assert_array_equal(host(q), want)


def test_fp8_zero_and_empty():
    q, s = Q.quant_fp8_per_tensor(bf16_dev(np.zeros(1000, np.uint16)))
    assert host(s)[0] == 1.0 and not host(q).any()
    q, s = Q.quant_fp8_per_tensor(torch.empty((0,), dtype=torch.bfloat16, device="cuda"))
    assert host(s)[0] == 1.0


def test_fp8_static_scale_saturates():
    x = W.normal_bf16((5000,), seed=2, scale=10.0)
    sc = np.float32(0.02)                    # 448 * 0.02 = 8.96: most |x| > 9 saturate
    q, s = Q.quant_fp8_per_tensor(bf16_dev(x), scale_in=f32_dev([sc]))
    want, _ = OQ.quant_fp8_bf16(x, scale_in=sc)
    np.testing.assert_array_equal(host(q), want)
    assert (np.abs(OC.e4m3_decode(want)) == 448).sum() > 100


def test_fp8_full_480p_activation_size_sampled():
    """[33,784 x 2,688] bf16 (the 480p block input): exact scale, then 2M sampled codes."""
    w = W.WORKLOADS["trim_stack42_480p"]
    x = W.activations(w, 0)
    say("fp8 480p", x.shape)
    q, s = Q.quant_fp8_per_tensor(bf16_dev(x))
    xf = OC.bf16_to_f64(x).astype(np.float32)
    amax = np.float32(np.abs(xf).max())
    s_want, inv = OQ.fp8_scale_dynamic(amax)
    assert host(s)[0] == s_want
    idx = np.random.default_rng(0).choice(x.size, size=2_000_000, replace=False)
    want = OC.e4m3_encode(xf.reshape(-1)[idx] * inv)
    np.testing.assert_array_equal(host(q).reshape(-1)[idx], want)


@pytest.mark.parametrize("L,H,stride_mult", [(391, 3, 1), (256, 2, 3), (1, 1, 1), (128 * 5, 21, 3)])
def test_int8_qk_bit_exact(L, H, stride_mult):
    say("int8 qk", L, H, stride_mult)
    x = W.normal_bf16((L, stride_mult * H * 128), seed=L + H)
    xd = bf16_dev(x)
    view = xd[:, : H * 128]               # the first H heads of each (possibly wider) row
    q, s = Q.quant_int8_qk(view, H, row_stride=stride_mult * H * 128)
    qw, sw = OQ.quant_int8_qk(np.ascontiguousarray(x[:, : H * 128]), L, H)
    np.testing.assert_array_equal(host(s), sw)
    np.testing.assert_array_equal(host(q), qw)


def test_int8_qk_480p_sampled_tiles():
    L, H = W.TOKENS_480P, 21
    qb, _, _ = W.qkv_heads(L, H, seed=11)
    q, s = Q.quant_int8_qk(bf16_dev(qb.reshape(L, H * 128)), H)
    qh, sh = host(q), host(s)
    T = (L + 127) // 128
    for (h, i) in [(0, 0), (20, T - 1), (7, 100), (13, T - 2)]:
        rows = slice(i * 128, min(L, (i + 1) * 128))
        qw, sw = OQ.quant_int8_qk(np.ascontiguousarray(qb[rows, h:h + 1, :]), rows.stop - rows.start, 1)
        assert sh[h, i] == sw[0, 0]
        np.testing.assert_array_equal(qh[rows, h], qw[:, 0])


# --- AdaLN ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,t", [("toy_d256_L256", 999.0), ("trim_block_L4096", 999.0),
                                    ("trim_block_L4096", 125.0), ("trim_block_L4096", 0.0)])
def test_adaln_project_vs_oracle(name, t):
    w = W.WORKLOADS[name]
    Bb, Pb = W.adaln_basis(w), W.adaln_proj(w)
    got = host(Q.adaln_project(t, fp16_dev(Bb), fp16_dev(Pb)))
    want = OA.adaln_project(t, Bb, Pb)
    diff = got != want
    # both sides form the float64 result and round once; a flip needs a value within ~1e-16 of an
    # fp32 rounding boundary
    assert diff.sum() <= 2, int(diff.sum())
    np.testing.assert_allclose(got, want, rtol=2 ** -23, atol=0)


def test_adaln_project_stack_matches_single():
    w = W.WORKLOADS["toy_d256_L256"]
    Bb = W.adaln_basis(w)
    Ps = np.stack([W.adaln_proj(w, 0, b) for b in range(3)])
    bias = W.normal_bf16((3, 6 * 256), seed=4, scale=0.1)     # any 16-bit payload; read as fp16
    bias = np.asarray(W.f32_to_fp16_bits(OC.bf16_to_f64(bias).astype(np.float32)))
    got = host(Q.adaln_project(874.0, fp16_dev(Bb), fp16_dev(Ps), bias=fp16_dev(bias)))
    for b in range(3):
        want = OA.adaln_project(874.0, Bb, Ps[b], bias[b])
        np.testing.assert_allclose(got[b], want, rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("name,L,half,static", [("toy_d256_L256", 256, 0, False),
                                                ("toy_d256_L256", 77, 1, False),
                                                ("trim_block_L4096", 4096, 0, False),
                                                ("trim_block_L4096", 1000, 1, True)])
def test_adaln_modulate_codes(name, L, half, static):
    w = W.WORKLOADS[name]
    say("modulate", name, L, half, static)
    x = W.activations(w, 1, L=L)
    mod = W.random_mod(w.d, seed=5, tag=w.tag)
    y = OA.layernorm_modulate(x, mod, half, 1e-6)
    if static:
        sc = np.float32(np.abs(y).max() * 0.5 / 448)      # half the range: also exercises saturation
        want, ws = OQ.quant_fp8_per_tensor(y, sc)
        inv = np.float32(1) / sc
        q, s = Q.adaln_modulate(bf16_dev(x), f32_dev(mod), half, 1e-6, act_scale=f32_dev([sc]))
    else:
        want, ws = OQ.quant_fp8_per_tensor(y)
        inv = np.float32(448) / np.float32(np.abs(y).max())
        q, s = Q.adaln_modulate(bf16_dev(x), f32_dev(mod), half, 1e-6)
    assert host(s)[0] == ws
    n = assert_codes_equal_except_ties(host(q), want, y * inv, "e4m3", name=f"modulate {name}")
    say("near-tie flips:", n)


def test_adaln_modulate_zero_modulation_is_plain_ln():
    w = W.WORKLOADS["toy_d256_L256"]
    x = W.activations(w, 2)
    mod = np.zeros((6, 256), np.float32)
    q, s = Q.adaln_modulate(bf16_dev(x), f32_dev(mod), 0)
    xv = OC.bf16_to_f64(x)
    ln = (xv - xv.mean(1, keepdims=True)) / np.sqrt(xv.var(1, keepdims=True) + float(np.float32(1e-6)))
    deq = OC.e4m3_decode(host(q)) * float(host(s)[0])
    assert np.max(np.abs(deq - ln)) <= np.abs(ln).max() * 2 ** -4


# --- MXFP4 weights and calibration ----------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(6, 96), (256, 2688), (384, 1024)])
def test_mxfp4_weight_quant_bit_exact(N, K):
    wb = W.normal_bf16((N, K), seed=N + K, scale=0.03)
    p, e = Q.quant_mxfp4(bf16_dev(wb))
    pw, ew = OQ.quant_mxfp4_weight(wb)
    np.testing.assert_array_equal(host(e), ew)
    np.testing.assert_array_equal(host(p), pw)


def test_calibration_amax_and_clip_counts():
    d_in, nb, tok = 1024, 6, 128
    ch, fac, a0 = W.outlier_spec(d_in, 137.0, site=3, n_batches=nb, tokens=tok)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    batches = [W.apply_outliers(W.calibration_batch(d_in, b, site=3, tokens=tok), ch, fac)
               for b in range(nb)]
    for b in batches:
        Q.amax_update(f32_dev(b), amax)
    want = max(float(np.abs(b).max()) for b in batches)
    assert float(host(amax)[0]) == np.float32(want)
    s_cal = OQ.calibrated_scale(want)
    s_unc = OQ.calibrated_scale(a0)
    for s_val, expect_zero in ((s_cal, True), (s_unc, False)):
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        for b in batches:
            Q.clip_count(f32_dev(b), f32_dev([s_val]), cnt)
        want_cnt = sum(OQ.clip_count(b, s_val) for b in batches)
        assert int(host(cnt)[0]) == want_cnt
        assert (want_cnt == 0) == expect_zero


def test_calibrated_scale_vs_oracle():
    """qvd_calibrated_scale equals the oracle's rule bit for bit: values whose fp32(a/448) needs the
    one-ulp raise (448 s < a) and values that do not, powers of two, 0, the extremes of fp32."""
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.uniform(0, 1000, 3000), np.exp(rng.uniform(-80, 80, 3000)),
                        2.0 ** np.arange(-120, 120, 7), [0.0, 448.0, 1.0, 3.4e38, 1.2e-38]]).astype(np.float32)
    got = host(Q.calibrated_scale(f32_dev(a)))
    want = np.array([OQ.calibrated_scale(v) for v in a], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    raised = np.array([float(np.float32(v / np.float32(448.0))) * 448.0 < float(v) for v in a])
    assert raised.sum() > 100 and (~raised).sum() > 100
    assert ((got.astype(np.float64) * 448.0) >= a.astype(np.float64)).all()


@pytest.mark.parametrize("wname,L,half", [("toy_d256_L256", 300, 0), ("trim_block_L4096", 257, 1)])
def test_layernorm_modulate_f32_bit_exact(wname, L, half):
    """The fp32 modulated LayerNorm values equal the oracle's (float64 statistics and affine map,
    rounded once) bit for bit."""
    w = W.WORKLOADS[wname]
    x = W.activations(w, 5, L=L)
    mod = W.random_mod(w.d, seed=6, tag=w.tag)
    got = host(Q.layernorm_modulate_f32(bf16_dev(x), f32_dev(mod), half))
    want = OA.layernorm_modulate(x, mod, half, 1e-6)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_amax_and_clip_counts():
    """qvd_amax_update_bf16 / qvd_clip_count_bf16 against the same reductions on the host."""
    x = W.normal_bf16((1237, 96), seed=8, scale=3.0)
    xv = OC.bf16_to_f64(x)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    Q.amax_update(bf16_dev(x), amax)
    assert float(host(amax)[0]) == float(np.abs(xv).max())
    for s in (np.float32(0.01), np.float32(0.02), np.float32(1.0)):
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        Q.clip_count(bf16_dev(x), f32_dev([s]), cnt)
        assert int(host(cnt)[0]) == int(np.count_nonzero(np.abs(xv) > float(s) * 448.0))


def test_mfma_probe_rates_are_sane():
    """The register-only MFMA probe (measurement support): every kind runs, reports a positive rate
    below its nominal peak at 2.4 GHz, and a shader clock between 0.5 and 2.6 GHz."""
    from quantized_video_diffusion_amd import _lib
    nominal = {_lib.QVD_PROBE_FP8: 5000.0, _lib.QVD_PROBE_FP4: 10100.0, _lib.QVD_PROBE_INT8: 5000.0,
               _lib.QVD_PROBE_F16: 2500.0, _lib.QVD_PROBE_INT8_32: 5000.0, _lib.QVD_PROBE_F16_32: 2500.0,
               _lib.QVD_PROBE_FP8_16: 5000.0}
    for kind, peak in nominal.items():
        r = Q.mfma_probe(kind, iters=200, workgroups=512, reps=1)
        assert 0.0 < r["tflops"] < 1.02 * peak, (kind, r)
        assert r["clock_mhz"] is None or 500.0 < r["clock_mhz"] < 2600.0, (kind, r)
