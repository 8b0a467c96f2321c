"""HIP-graph capture of the hot path (Q.capture_graph).  A captured stack step replays to the bits of the
same step run eagerly, replay after replay, with other eager work (a step at another timestep, which
overwrites the input, the workspace and the modulation) and synchronisations between the replays.  The
eight-step sampler loop captured as one graph per timestep (the stack and the sampler update) reaches
the eager loop's final latent bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from _gpu_util import say, bf16_dev, fp16_dev, f32_dev, i32_dev, host, host_bits

pytestmark = pytest.mark.gpu


class Stack:
    """n_blocks seeded blocks of workload w at L tokens, one shared workspace; step(t) runs x <- x0,
    the AdaLN projection for timestep t and the blocks in order (x updated in place)."""

    def __init__(self, w, L, seed, n_blocks, fmt=_lib.QVD_W_FP8, act_scale=None):
        self.n = n_blocks
        self.basis = fp16_dev(W.adaln_basis(w, seed))
        self.bws, projs, self.masks = [], [], []
        for b in range(n_blocks):
            wb = {k: bf16_dev(v) for k, v in W.block_weights(w, seed, b).items()}
            bw = Q.quantize_block_weights(wb, w.d, w.n_heads, w.mlp, fmt=fmt)
            if act_scale is not None:
                bw.act_scale = f32_dev(act_scale)
            self.bws.append(bw)
            projs.append(W.adaln_proj(w, seed, b))
            idx, cnt = W.block_mask(w, seed, b, L=L)
            self.masks.append((i32_dev(idx), i32_dev(cnt)))
        self.proj = fp16_dev(np.stack(projs))
        self.ws = torch.empty(Q.block_ws_bytes(self.bws[0], L), dtype=torch.uint8, device="cuda")
        self.x0 = bf16_dev(W.activations(w, seed, L=L))
        self.x = torch.empty_like(self.x0)

    def blocks(self, t):
        mods = Q.adaln_project(float(t), self.basis, self.proj)
        for b in range(self.n):
            Q.dit_block_forward(self.bws[b], mods[b], self.x, *self.masks[b], self.ws)

    def step(self, t):
        self.x.copy_(self.x0)
        self.blocks(t)


def _check_replays(st, name, t=999.0, t_other=125.0, replays=3):
    st.step(t)
    torch.cuda.synchronize()
    ref = host_bits(st.x)
    g = Q.capture_graph(lambda: st.step(t))
    for r in range(replays):
        st.step(t_other)                                  # eager work between the replays
        torch.cuda.synchronize()
        assert not np.array_equal(host_bits(st.x), ref), f"{name}: the other timestep gave the same output"
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(st.x), ref, err_msg=f"{name}: replay {r}")
    say(f"{name}: {replays} replays bit-exact")


def test_graph_toy_stack_fp8():
    w = W.WORKLOADS["toy_d256_L256"]
    _check_replays(Stack(w, w.L, seed=1, n_blocks=2), "toy 2 blocks FP8")


def test_graph_trim_width_stack_fp8_ragged_sparse():
    w = W.WORKLOADS["trim_block_L4096"]
    _check_replays(Stack(w, 1100, seed=2, n_blocks=3), "Trim width L=1100, 3 blocks, FP8")


def test_graph_trim_width_w4a4_and_static_w4a8():
    w = W.WORKLOADS["trim_block_L4096"]
    _check_replays(Stack(w, 1100, seed=3, n_blocks=2, fmt=_lib.QVD_W_MXFP4_A4), "Trim width W4A4")
    act = np.array([0.1, 0.002, 0.1, 0.008], np.float32)
    _check_replays(Stack(w, 1100, seed=3, n_blocks=2, fmt=_lib.QVD_W_MXFP4, act_scale=act),
                   "Trim width W4A8 static scales")


def test_graph_sampler_loop_matches_eager():
    """One graph per timestep (stack + sampler update), replayed in order after an eager start, against
    the eager loop: every step's state and the final latent bit for bit."""
    w = W.WORKLOADS["toy_d256_L256"]
    st = Stack(w, w.L, seed=4, n_blocks=2)
    smp = Q.Sampler(L_video=200)
    ts = [int(t) for t in W.SAMPLER_TIMESTEPS]

    def iteration(i):
        st.blocks(ts[i])
        smp.step(i, st.x)

    smp.start(st.x0, x_in=st.x)
    # the graphs hold the state tensors' addresses: the second pass restores the start state into the
    # same tensors (start() would allocate new ones)
    start = (smp.x_state.clone(), smp.x0_hat.clone(), st.x.clone())
    states = []
    for i in range(len(ts)):
        iteration(i)
        torch.cuda.synchronize()
        states.append(host(smp.x_state).copy())
    graphs = [Q.capture_graph(lambda i=i: iteration(i)) for i in range(len(ts))]
    for rep in range(2):
        for dst, src in zip((smp.x_state, smp.x0_hat, st.x), start):
            dst.copy_(src)
        for i, g in enumerate(graphs):
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(smp.x_state), states[i], err_msg=f"pass {rep}, step {i}")
    say(f"sampler loop: {len(ts)} graphs, 2 passes bit-exact; final latent RMS "
        f"{float(np.sqrt(np.mean(states[-1].astype(np.float64) ** 2))):.4f}")


def test_capture_refuses_with_timing_on():
    Q.timing_enable(True)
    try:
        with pytest.raises(RuntimeError, match="timing"):
            Q.capture_graph(lambda: None)
    finally:
        Q.timing_enable(False)
        Q.timing_report()
