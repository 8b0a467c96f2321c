"""Teacher-forced stage-by-stage parity of dit_block_forward (FP8 block, dynamic scales) against the
oracle: every stage is fed the GPU block's own inputs and scales (see _block_stages.py for the bars).
The toy and Trim-width blocks are checked on every row; the 480p blocks of the 42-block stack (blocks
0, 20 and 41 at the timesteps 999 and 125, each with its own weights, mask and modulation, fed the
seeded 480p input) on three token tiles: the first, one in the middle and the ragged last one
(120 rows)."""
import numpy as np
import pytest

import workloads as W
import quantized_video_diffusion_amd as Q
from oracle import block as OB
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, f32_dev, host
from _block_stages import run_stages, check_block_stages

pytestmark = pytest.mark.gpu


def _gpu_qw(bw):
    """The GPU block's own weight codes and scales, in the oracle's weight-dict form."""
    qw = {}
    for s in OB.SITES:
        qw["w_" + s] = host(bw.w[s])
        qw["s_" + s] = np.float32(host(bw.s[s])[0])
    return qw


def _run(name, w, L, seed, block=0, t=999.0, sparse=None, gate=None, rows=None):
    x = W.activations(w, seed, L=L)
    wbits = W.block_weights(w, seed, block)
    idx, cnt = W.block_mask(w, seed, block, L=L, sparse=sparse)
    if gate is None:
        mod_d = Q.adaln_project(t, fp16_dev(W.adaln_basis(w, seed)), fp16_dev(W.adaln_proj(w, seed, block)))
    else:
        mod_d = f32_dev(W.random_mod(w.d, seed=seed + 100, tag=w.tag, gate=gate))
    bw = Q.quantize_block_weights({k: bf16_dev(v) for k, v in wbits.items()}, w.d, w.n_heads, w.mlp)
    g = run_stages(bw, mod_d, x, i32_dev(idx), i32_dev(cnt), rows=rows)
    return check_block_stages(name, _gpu_qw(bw), host(mod_d), x, idx, cnt, g, w.n_heads, rows=rows)


def test_stages_toy_t999():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy t=999", w, w.L, seed=0)


def test_stages_toy_gate_one_ragged_sparse():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy gate=1 L=391 sparse", w, 391, seed=1, sparse=True, gate=1.0)


def test_stages_trim_width_L4096_gate_one():
    w = W.WORKLOADS["trim_block_L4096"]
    say("trim width L=4096: all rows")
    _run("trim L=4096 gate=1", w, w.L, seed=0, gate=1.0)


def test_stages_trim_width_L1100_sparse_t125():
    w = W.WORKLOADS["trim_block_L4096"]
    _run("trim L=1100 sparse t=125", w, 1100, seed=3, t=125.0, sparse=True)


@pytest.mark.parametrize("block,t", [(0, 999.0), (20, 999.0), (41, 999.0), (0, 125.0), (20, 125.0),
                                     (41, 125.0)])
def test_stages_480p_stack_blocks_sampled_tiles(block, t):
    w = W.WORKLOADS["trim_stack42_480p"]
    T = w.n_tiles
    rows = np.concatenate([np.arange(i * 128, min(w.L, (i + 1) * 128)) for i in (0, T // 2, T - 1)])
    say(f"480p block {block} t={t}: {len(rows)} rows of {w.L}")
    _run(f"480p block {block} t={t:g}", w, w.L, seed=0, block=block, t=t, rows=rows)
