"""GPU parity of the sampler around the stack (qvd_sampler_start / qvd_sampler_step) against the
oracle's sampler, step by step from the GPU's own state, and the eight-step loop around a real block
stack with the state carried between steps."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from oracle import codecs as OC, sampler as OS
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, host, host_bits

pytestmark = pytest.mark.gpu


def _bound(a, x, b, s0, v, c, p):
    """fp32 evaluation of a x + b x0_hat + c p with x0_hat = x - s0 v formed in fp32 first (its error is
    relative to |x| + s0 |v|, not to the possibly cancelled x0_hat); coefficients rounded to fp32."""
    return 2.0 ** -20 * (np.abs(a * x) + np.abs(b) * (np.abs(x) + s0 * np.abs(v)) + np.abs(c * p)) + 1e-30


def _check_step(smp, i, x, v_bits, p, x_gpu, h_gpu, xin_gpu, L_video):
    """The GPU's step i from state x (fp32 as float64), velocity v (bf16) and previous estimate p."""
    v = OC.bf16_to_f64(v_bits)
    for rows, s in ((slice(0, L_video), smp.shift_video), (slice(L_video, None), smp.shift_audio)):
        sig = OS.sigmas(s)
        want, want_h = OS.step(x[rows], v[rows], p[rows], sig, i)
        s0, a, b, c = OS.step_coefficients(sig, i)
        np.testing.assert_array_less(np.abs(h_gpu[rows] - want_h), 2.0 ** -22 * (np.abs(x[rows]) + s0 * np.abs(v[rows])) + 1e-30)
        np.testing.assert_array_less(np.abs(x_gpu[rows] - want), _bound(a, x[rows], b, s0, v[rows], c, p[rows]))
    # the next stack input is the state rounded once to bf16
    np.testing.assert_array_equal(xin_gpu, OC.f64_to_bf16(x_gpu))


@pytest.mark.parametrize("L,L_video,d", [(300, 250, 256), (1100, 1024, 2688), (64, 64, 128)])
def test_sampler_steps_vs_oracle(L, L_video, d):
    """Every step of the pages' schedule from the GPU's own state and a random velocity; video rows
    (shift 10) and audio rows (shift 3)."""
    rng = np.random.default_rng(L)
    smp = Q.Sampler(L_video=L_video)
    eps = W.normal_bf16((L, d), seed=L + 1)
    xin = smp.start(bf16_dev(eps))
    x = host(smp.x_state).astype(np.float64)
    sv, sa = OS.sigmas(10.0), OS.sigmas(3.0)
    e = OC.bf16_to_f64(eps)
    np.testing.assert_array_equal(x[:L_video], (np.float32(sv[0]) * e[:L_video].astype(np.float32)))
    np.testing.assert_array_equal(x[L_video:], (np.float32(sa[0]) * e[L_video:].astype(np.float32)))
    np.testing.assert_array_equal(host_bits(xin), OC.f64_to_bf16(x))
    p = np.zeros_like(x)
    for i in range(8):
        v_bits = W.normal_bf16((L, d), seed=100 * L + i, scale=float(rng.uniform(0.5, 2.0)))
        vd = bf16_dev(v_bits)
        xin = smp.step(i, vd)                          # in place: the next input replaces v
        x_gpu, h_gpu = host(smp.x_state).astype(np.float64), host(smp.x0_hat).astype(np.float64)
        _check_step(smp, i, x, v_bits, p, x_gpu, h_gpu, host_bits(xin), L_video)
        x, p = x_gpu, h_gpu
    # after the last step the state is the final estimate
    np.testing.assert_array_equal(host(smp.x_state), host(smp.x0_hat))


def test_sampler_loop_around_a_block_stack():
    """The eight-step loop around a two-block toy stack (the stack works in place on the bf16 input;
    the sampler keeps the fp32 state): at every step the stack's input is bf16 of the state, and the
    state advances as the oracle's step from the GPU's state and the stack's output.  Two blocks of the
    toy workload, 256 tokens of which the last 56 are audio rows."""
    w = W.WORKLOADS["toy_d256_L256"]
    L, L_video = w.L, 200
    Bb = W.adaln_basis(w, 3)
    bws, projs, masks = [], [], []
    for b in range(2):
        wb = {k: bf16_dev(v) for k, v in W.block_weights(w, 3, b).items()}
        bws.append(Q.quantize_block_weights(wb, w.d, w.n_heads, w.mlp))
        projs.append(W.adaln_proj(w, 3, b))
        idx, cnt = W.block_mask(w, 3, b)
        masks.append((i32_dev(idx), i32_dev(cnt)))
    proj = fp16_dev(np.stack(projs))
    smp = Q.Sampler(L_video=L_video)
    eps = W.activations(w, 3)
    xin = smp.start(bf16_dev(eps))
    p = np.zeros((L, w.d))
    for i, t in enumerate(OS.timesteps()):
        x = host(smp.x_state).astype(np.float64)
        np.testing.assert_array_equal(host_bits(xin), OC.f64_to_bf16(x))
        mods = Q.adaln_project(float(t), fp16_dev(Bb), proj)
        for b in range(2):
            Q.dit_block_forward(bws[b], mods[b], xin, *masks[b])
        v_bits = host_bits(xin)
        assert not np.array_equal(v_bits, OC.f64_to_bf16(x)), "the stack left its input unchanged"
        xin = smp.step(i, xin)
        x_gpu, h_gpu = host(smp.x_state).astype(np.float64), host(smp.x0_hat).astype(np.float64)
        _check_step(smp, i, x, v_bits, p, x_gpu, h_gpu, host_bits(xin), L_video)
        p = h_gpu
    final = host(smp.x_state)
    assert np.isfinite(final).all()
    say("sampler loop: final latent RMS", float(np.sqrt(np.mean(final.astype(np.float64) ** 2))))
