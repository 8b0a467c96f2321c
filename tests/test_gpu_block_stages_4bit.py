"""Teacher-forced stage-by-stage parity of the blocks with MXFP4 weights against the oracle: static
E4M3 activation scales (W4A8) and MXFP4 activations (W4A4), the two 768p configurations.  Every stage
is fed the GPU block's own inputs (see _block_stages.py for the bars).  The W4A8 static scales are
calibrated on the block's own input: each is the dynamic scale the same block takes on it (the amax of
that GEMM input / 448).  Toy and Trim-width blocks on every row; the 768p block (85,696 tokens, 135 of
670 key tiles kept, the last query tile of 64 rows) on three token tiles: the first, one in the middle
and the last."""
import numpy as np
import pytest

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, f32_dev, host
from _block_stages import run_stages_4bit, check_block_stages_4bit

pytestmark = pytest.mark.gpu


def _run(name, w, L, seed, block=0, t=999.0, sparse=None, gate=None, rows=None, a4=False):
    x = W.activations(w, seed, L=L)
    idx, cnt = W.block_mask(w, seed, block, L=L, sparse=sparse)
    idx_d, cnt_d = i32_dev(idx), i32_dev(cnt)
    if gate is None:
        mod_d = Q.adaln_project(t, fp16_dev(W.adaln_basis(w, seed)), fp16_dev(W.adaln_proj(w, seed, block)))
    else:
        mod_d = f32_dev(W.random_mod(w.d, seed=seed + 100, tag=w.tag, gate=gate))
    wbits = W.block_weights(w, seed, block)
    bw = Q.quantize_block_weights({k: bf16_dev(v) for k, v in wbits.items()}, w.d, w.n_heads, w.mlp,
                                  fmt=_lib.QVD_W_MXFP4_A4 if a4 else _lib.QVD_W_MXFP4)
    act = None
    if not a4:
        # calibrate on the block's own input: the dynamic-scale run's four per-tensor scales
        ws = Q.block_forward_until(bw, mod_d, bf16_dev(x), idx_d, cnt_d, _lib.QVD_STAGE_ALL)
        act = host(Q.block_intermediates(bw, ws, L)["scales"]).copy()
        del ws
        bw.act_scale = f32_dev(act)
        say(name, "static scales", act.tolist())
    rows = np.arange(L) if rows is None else rows
    g = run_stages_4bit(bw, mod_d, x, idx_d, cnt_d, rows)
    wm = {}
    for s in ("qkv", "o", "up", "down"):
        wm["w_" + s], wm["e8_" + s] = host(bw.w[s]), host(bw.e8[s])
    return check_block_stages_4bit(name, wm, act, host(mod_d), x, idx, cnt, g, w.n_heads, rows)


def test_w4a8_stages_toy():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W4A8", w, w.L, seed=2)


def test_w4a8_stages_toy_gate_one_ragged_sparse():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W4A8 gate=1 L=391 sparse", w, 391, seed=4, sparse=True, gate=1.0)


def test_w4a8_stages_trim_width_L1100_sparse():
    w = W.WORKLOADS["trim_block_L4096"]
    _run("trim W4A8 L=1100 sparse", w, 1100, seed=5, sparse=True, t=125.0)


def _sampled_tiles(w):
    T = w.n_tiles
    return np.concatenate([np.arange(i * 128, min(w.L, (i + 1) * 128)) for i in (0, T // 2, T - 1)])


def test_w4a8_stages_768p_sampled_tiles():
    w = W.WORKLOADS["block_768p_mxfp4"]
    rows = _sampled_tiles(w)
    say(f"768p W4A8 block: {len(rows)} rows of {w.L}")
    _run("768p W4A8", w, w.L, seed=0, rows=rows)


def test_w4a4_stages_toy():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W4A4", w, w.L, seed=2, a4=True)


def test_w4a4_stages_toy_gate_one_ragged_sparse():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W4A4 gate=1 L=391 sparse", w, 391, seed=4, sparse=True, gate=1.0, a4=True)


def test_w4a4_stages_trim_width_L1100_sparse():
    w = W.WORKLOADS["trim_block_L4096"]
    _run("trim W4A4 L=1100 sparse", w, 1100, seed=5, sparse=True, t=125.0, a4=True)


def test_w4a4_stages_768p_sampled_tiles():
    w = W.WORKLOADS["block_768p_mxfp4"]
    rows = _sampled_tiles(w)
    say(f"768p W4A4 block: {len(rows)} rows of {w.L}")
    _run("768p W4A4", w, w.L, seed=0, rows=rows, a4=True)
