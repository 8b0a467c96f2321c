"""GPU parity of the whole DiT block forward (dit_block_forward) against the oracle's block."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from oracle import codecs as OC, quant as OQ, adaln as OA, block as OB
from _gpu_util import (say, bf16_dev, fp16_dev, i32_dev, f32_dev, host, host_bits, assert_close_rms,
                       assert_bf16_close)

pytestmark = pytest.mark.gpu


def _gpu_weights(wbits, w, fmt=_lib.QVD_W_FP8, act_scale=None):
    dev = {k: bf16_dev(v) for k, v in wbits.items()}
    bw = Q.quantize_block_weights(dev, w.d, w.n_heads, w.mlp, fmt=fmt)
    if act_scale is not None:
        bw.act_scale = f32_dev(act_scale)
    return bw


def _oracle_weights(wbits, fmt="fp8"):
    if fmt == "fp8":
        return OB.quantize_block_weights(wbits)
    qm = {}
    for site in OB.SITES:
        qm["w_" + site], qm["e8_" + site] = OQ.quant_mxfp4_weight(wbits["w_" + site])
    return qm


def _run_both(w, L, seed=0, mod=None, t=999.0, sparse=None, act_scale=None, fmt="fp8"):
    x = W.activations(w, seed, L=L)
    wbits = W.block_weights(w, seed)
    idx, cnt = W.block_mask(w, seed, L=L, sparse=sparse)
    if mod is None:
        Bb, Pb = W.adaln_basis(w, seed), W.adaln_proj(w, seed)
        mod_gpu = Q.adaln_project(t, fp16_dev(Bb), fp16_dev(Pb))
        mod_orc = OA.adaln_project(t, Bb, Pb)
    else:
        mod_gpu, mod_orc = f32_dev(mod), mod
    gfmt = {"fp8": _lib.QVD_W_FP8, "mxfp4": _lib.QVD_W_MXFP4, "w4a4": _lib.QVD_W_MXFP4_A4}[fmt]
    bw = _gpu_weights(wbits, w, gfmt, act_scale)
    xd = bf16_dev(x)
    Q.dit_block_forward(bw, mod_gpu, xd, i32_dev(idx), i32_dev(cnt))
    got = host_bits(xd)
    want = OB.dit_block(x, mod_orc, _oracle_weights(wbits, fmt), idx, cnt, w.n_heads,
                        act_scales=None if act_scale is None else [np.float32(a) for a in act_scale],
                        fmt=fmt)
    return x, got, want


# Block-level parity.  The block chains four per-tensor E4M3 requantizations; any sub-ulp difference
# upstream (the FP8 MFMA's accumulation error of ~2^-14.6, fp16 vs float64 exp) moves a small
# fraction of codes to the neighbouring value (one E4M3 step = 2^-4 relative), and each moved code
# perturbs the next GEMM.  Measured here: 0.5-1% of the attention-output codes and ~10% of the GELU
# codes move, giving a branch RMS error of 1-2%.  The criteria:
#   RMS(out - ref) <= 1e-2 RMS(ref)                (the block-output tolerance, on RMS)
#   RMS(branch error) <= 2.5e-2 RMS(branch)         (branch = out - x, gates included)
#   max |out - ref| <= 2 bf16 ulp + 0.1 RMS(ref)    (two residual roundings; gross-error guard)
# W4A4 moves codes on the same near-midpoint inputs, but one E2M1 step is up to 1/3 of the value
# (2^-4 for E4M3), so a single moved code of g shifts one output row by a step times a column of
# W_down.  There the guard reads: at most 0.1% of the outputs beyond 2 ulp + 0.1 RMS(ref), none
# beyond 2 ulp + 0.5 RMS(ref).  And the RMS bars are three times the FP8 ones (3e-2 output, 7.5e-2
# branch): the oracle's own W4A4 block at Trim width moves by 6.4e-3 / 1.4e-2 (output / branch) when
# its attention output is perturbed by 1e-5 relative, 2.5e-2 / 5.5e-2 at 2e-4, about three times what
# its FP8 block does under the same perturbations, and the kernel's attention differs from the
# oracle's at that level (fp16 numerators).
def _check(x, got, want, name, branch_rel=2.5e-2, a4=False):
    g, o, xi = OC.bf16_to_f64(got), OC.bf16_to_f64(want), OC.bf16_to_f64(x)
    err = np.abs(g - o)
    rms = float(np.sqrt(np.mean(o ** 2)))
    k = int(np.argmax(err))
    bo, bg = o - xi, g - xi
    rel = float(np.sqrt(np.mean((bg - bo) ** 2) / np.mean(bo ** 2)))
    say(f"{name}: out RMS rel err {np.sqrt(np.mean(err ** 2)) / rms:.2e}; max {err.max():.3e} at "
        f"{np.unravel_index(k, g.shape)} (want {o.flat[k]:.4f}, got {g.flat[k]:.4f}, x {xi.flat[k]:.4f}); "
        f"branch RMS rel err {rel:.2e}")
    out_rel = 3e-2 if a4 else 1e-2
    branch_rel = 3 * branch_rel if a4 else branch_rel
    assert np.sqrt(np.mean(err ** 2)) <= out_rel * rms, f"{name}: block output RMS error"
    if a4:
        ulp2 = 2 * np.abs(o) * 2.0 ** -7
        frac = float(np.mean(err > ulp2 + 0.1 * rms))
        assert frac <= 1e-3, f"{name}: {frac:.2e} of the outputs beyond 2 ulp + 0.1 RMS"
        assert_bf16_close(got, o, 0.5, name + " block output", ulps=2)
    else:
        assert_bf16_close(got, o, 0.1, name + " block output", ulps=2)
    assert rel <= branch_rel, f"{name}: branch (out - x) relative RMS error {rel:.3e}"


def test_block_toy_full_path():
    w = W.WORKLOADS["toy_d256_L256"]
    x, got, want = _run_both(w, w.L)
    _check(x, got, want, "toy t=999")


def test_block_toy_gates_one_ragged_sparse():
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=3, tag=w.tag, gate=1.0)
    x, got, want = _run_both(w, 391, seed=1, mod=mod, sparse=True)
    _check(x, got, want, "toy gate=1 L=391 sparse")


def test_block_zero_gates_identity():
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=4, tag=w.tag, gate=0.0)
    x, got, want = _run_both(w, 300, seed=2, mod=mod)
    np.testing.assert_array_equal(got, x)
    np.testing.assert_array_equal(want, x)


def test_block_static_scales():
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=5, tag=w.tag, gate=1.0)
    act = np.array([0.01, 0.004, 0.01, 0.002], np.float32)
    x, got, want = _run_both(w, 256, seed=3, mod=mod, act_scale=act)
    _check(x, got, want, "toy static scales")


def test_block_mxfp4_weights_static_scales():
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=6, tag=w.tag, gate=1.0)
    act = np.array([0.01, 0.004, 0.01, 0.002], np.float32)
    x, got, want = _run_both(w, 391, seed=4, mod=mod, act_scale=act, fmt="mxfp4", sparse=True)
    _check(x, got, want, "toy mxfp4")


def test_block_mxfp4_weights_dynamic_scales():
    """MXFP4 weights with dynamic per-tensor E4M3 activations (act_scale NULL: the configuration the
    static scales are calibrated from)."""
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=16, tag=w.tag, gate=1.0)
    x, got, want = _run_both(w, 391, seed=14, mod=mod, fmt="mxfp4", sparse=True)
    _check(x, got, want, "toy mxfp4 dynamic")


def test_block_w4a4_dynamic_block_scales():
    """W4A4: every GEMM input MXFP4 (h1, O, h2, g), MXFP4 weights, no per-tensor activation scale."""
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=8, tag=w.tag, gate=1.0)
    x, got, want = _run_both(w, 391, seed=5, mod=mod, fmt="w4a4", sparse=True)
    _check(x, got, want, "toy w4a4", a4=True)


def test_block_w4a4_zero_gates_identity_and_timestep_mod():
    w = W.WORKLOADS["toy_d256_L256"]
    mod = W.random_mod(w.d, seed=9, tag=w.tag, gate=0.0)
    x, got, want = _run_both(w, 130, seed=6, mod=mod, fmt="w4a4")
    np.testing.assert_array_equal(got, x)
    np.testing.assert_array_equal(want, x)
    x, got, want = _run_both(w, 256, seed=7, t=500.0, fmt="w4a4")
    _check(x, got, want, "toy w4a4 t=500", a4=True)


def test_block_two_block_stack():
    w = W.WORKLOADS["toy_d256_L256"]
    x = W.activations(w, 7)
    Bb = W.adaln_basis(w, 7)
    xd = bf16_dev(x)
    mods, qws, masks = [], [], []
    for blk in range(2):
        wbits = W.block_weights(w, 7, blk)
        Pb = W.adaln_proj(w, 7, blk)
        idx, cnt = W.block_mask(w, 7, blk)
        Q.dit_block_forward(_gpu_weights(wbits, w), Q.adaln_project(874.0, fp16_dev(Bb), fp16_dev(Pb)),
                            xd, i32_dev(idx), i32_dev(cnt))
        mods.append(OA.adaln_project(874.0, Bb, Pb))
        qws.append(_oracle_weights(wbits))
        masks.append((idx, cnt))
    want = OB.dit_stack_step(x, mods, qws, masks, w.n_heads)
    _check(x, host_bits(xd), want, "2-block stack")


def test_block_trim_width_L4096():
    """Full Trim width (d = 2,688, 21 heads, MLP 10,752), 4,096 tokens, dense attention."""
    w = W.WORKLOADS["trim_block_L4096"]
    say("trim block L=4096: oracle takes ~30 s")
    mod = W.random_mod(w.d, seed=8, tag=w.tag, gate=1.0)
    x, got, want = _run_both(w, w.L, seed=0, mod=mod)
    _check(x, got, want, "trim L=4096 gate=1")


@pytest.mark.parametrize("fmt", ["mxfp4", "w4a4"])
def test_block_trim_width_4bit(fmt):
    """Full Trim width with 4-bit weights, 1,100 tokens (9 tiles, ragged), 80%-sparse masks: W4A8 with
    static activation scales, and W4A4 with dynamic MXFP4 activation blocks."""
    w = W.WORKLOADS["trim_block_L4096"]
    say("trim block 4-bit", fmt)
    mod = W.random_mod(w.d, seed=9, tag=w.tag, gate=1.0)
    act = np.array([0.02, 0.01, 0.02, 0.004], np.float32) if fmt == "mxfp4" else None
    x, got, want = _run_both(w, 1100, seed=3, mod=mod, act_scale=act, fmt=fmt, sparse=True)
    _check(x, got, want, f"trim {fmt} L=1100", a4=fmt == "w4a4")


def test_block_deterministic():
    w = W.WORKLOADS["toy_d256_L256"]
    x = W.activations(w, 9)
    bw = _gpu_weights(W.block_weights(w, 9), w)
    mod = f32_dev(W.random_mod(w.d, seed=9, tag=w.tag, gate=1.0))
    idx, cnt = W.block_mask(w, 9)
    outs = []
    for _ in range(2):
        xd = bf16_dev(x)
        Q.dit_block_forward(bw, mod, xd, i32_dev(idx), i32_dev(cnt))
        outs.append(host_bits(xd))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_block_480p_full_size_equals_its_steps():
    """The 480p block at full size, in the configuration the stack step times (33,784 tokens, Trim
    width, block 0's weights and 80%-sparse mask, the timestep-999 modulation): dit_block_forward must
    equal, bit for bit, the same block computed step by step through the separately exported entry
    points -- modulate, the QKV GEMM, the attention, the per-tensor quantizer, the residual GEMMs --
    whose outputs the 480p-shape tests compare with the oracle.  (The oracle's whole block at this size
    would take minutes: the per-tensor scales of O and GELU couple every token.)  Then zero gates leave
    the values of x unchanged at this size."""
    w = W.WORKLOADS["trim_stack42_480p"]
    L, d, H = w.L, w.d, w.n_heads
    say("480p block vs its steps", L, d, H)
    x = W.activations(w, 0)
    bw = _gpu_weights(W.block_weights(w, 0, 0), w)
    idx, cnt = W.block_mask(w, 0, 0)
    idx_d, cnt_d = i32_dev(idx), i32_dev(cnt)
    mod = Q.adaln_project(999.0, fp16_dev(W.adaln_basis(w, 0)), fp16_dev(W.adaln_proj(w, 0, 0)))

    xb = bf16_dev(x)
    Q.dit_block_forward(bw, mod, xb, idx_d, cnt_d)

    xs = bf16_dev(x)
    h1, s1 = Q.adaln_modulate(xs, mod, 0)
    q8, k8, vt, qs, ks = Q.gemm_fp8(h1, s1, bw.w["qkv"], bw.s["qkv"], mode=_lib.QVD_EPI_QKV, n_heads=H)
    o = Q.sparse_attn_vt(q8, qs, k8, ks, Q.vt_unify(vt), idx_d, cnt_d)
    o8, so = Q.quant_fp8_per_tensor(o.reshape(L, d))
    Q.gemm_fp8(o8, so, bw.w["o"], bw.s["o"], mode=_lib.QVD_EPI_RESID_GATE, out=xs, resid=xs, gate=mod[2])
    h2, s2 = Q.adaln_modulate(xs, mod, 1)
    g = Q.gemm_fp8(h2, s2, bw.w["up"], bw.s["up"], mode=_lib.QVD_EPI_GELU)
    g8, sg = Q.quant_fp8_per_tensor(g)
    Q.gemm_fp8(g8, sg, bw.w["down"], bw.s["down"], mode=_lib.QVD_EPI_RESID_GATE, out=xs, resid=xs,
               gate=mod[5])
    got, steps = host_bits(xb), host_bits(xs)
    say("480p block: differing outputs", int(np.count_nonzero(got != steps)), "of", got.size)
    np.testing.assert_array_equal(got, steps)
    assert not np.array_equal(got, x), "the block left x unchanged"

    mod0 = mod.clone()
    mod0[2].zero_()
    mod0[5].zero_()
    xz = bf16_dev(x)
    Q.dit_block_forward(bw, mod0, xz, idx_d, cnt_d)
    # x + 0 * y: a negative zero of x plus +0 rounds to +0, so compare values, not bits
    np.testing.assert_array_equal(OC.bf16_to_f64(host_bits(xz)), OC.bf16_to_f64(x))


@pytest.mark.parametrize("fmt", ["w4a8_static", "w4a4"])
def test_block_768p_4bit_full_size_equals_its_steps(fmt):
    """The 768p block at full size with MXFP4 weights (85,696 tokens, the last query tile of 64 rows,
    135 of 670 key tiles kept), as the 768p report times it: W4A8 with static E4M3 activation scales,
    and W4A4.  dit_block_forward must equal, bit for bit, the block computed through the exported
    steps, each of which has its own oracle tests."""
    w = W.WORKLOADS["block_768p_mxfp4"]
    L, d, H = w.L, w.d, w.n_heads
    say("768p block vs its steps", fmt, L, d, H)
    x = W.activations(w, 0)
    gfmt = _lib.QVD_W_MXFP4 if fmt == "w4a8_static" else _lib.QVD_W_MXFP4_A4
    act = np.array([1.6, 4.0, 1.4, 600.0], np.float32) if fmt == "w4a8_static" else None
    bw = _gpu_weights(W.block_weights(w, 0, 0), w, gfmt, act)
    idx, cnt = W.block_mask(w, 0, 0)
    idx_d, cnt_d = i32_dev(idx), i32_dev(cnt)
    mod = Q.adaln_project(999.0, fp16_dev(W.adaln_basis(w, 0)), fp16_dev(W.adaln_proj(w, 0, 0)))

    xb = bf16_dev(x)
    Q.dit_block_forward(bw, mod, xb, idx_d, cnt_d)

    xs = bf16_dev(x)
    wq = {s: (bw.w[s], bw.e8[s]) for s in ("qkv", "o", "up", "down")}
    rg = dict(mode=_lib.QVD_EPI_RESID_GATE, out=xs, resid=xs)
    if fmt == "w4a4":
        hp, he = Q.adaln_modulate_mxfp4(xs, mod, 0)
        q8, k8, vt, qs, ks = Q.gemm_mxfp4_w4a4(hp, he, *wq["qkv"], mode=_lib.QVD_EPI_QKV, n_heads=H)
        op, oe = Q.sparse_attn_vt_mxfp4(q8, qs, k8, ks, Q.vt_unify(vt), idx_d, cnt_d)
        Q.gemm_mxfp4_w4a4(op, oe, *wq["o"], gate=mod[2], **rg)
        hp, he = Q.adaln_modulate_mxfp4(xs, mod, 1)
        gp, ge = Q.gemm_mxfp4_w4a4(hp, he, *wq["up"], mode=_lib.QVD_EPI_GELU_MXFP4)
        Q.gemm_mxfp4_w4a4(gp, ge, *wq["down"], gate=mod[5], **rg)
    else:
        a = bw.act_scale
        h, s = Q.adaln_modulate(xs, mod, 0, act_scale=a[0:1])
        q8, k8, vt, qs, ks = Q.gemm_mxfp4(h, s, *wq["qkv"], mode=_lib.QVD_EPI_QKV, n_heads=H)
        o8 = Q.sparse_attn_vt_e4m3(q8, qs, k8, ks, Q.vt_unify(vt), idx_d, cnt_d, a[1:2])
        Q.gemm_mxfp4(o8.reshape(L, d), a[1:2], *wq["o"], gate=mod[2], **rg)
        h, s = Q.adaln_modulate(xs, mod, 1, act_scale=a[2:3])
        g8 = Q.gemm_mxfp4(h, s, *wq["up"], mode=_lib.QVD_EPI_GELU_E4M3, out_scale=a[3:4])
        Q.gemm_mxfp4(g8, a[3:4], *wq["down"], gate=mod[5], **rg)
    got, steps = host_bits(xb), host_bits(xs)
    say("768p block: differing outputs", int(np.count_nonzero(got != steps)), "of", got.size)
    np.testing.assert_array_equal(got, steps)
    assert not np.array_equal(got, x), "the block left x unchanged"
