"""Teacher-forced stage-by-stage parity against the oracle of the blocks whose producers write the next
GEMM's codes: static E4M3 activation scales with FP8 weights (W8A8, the static-scale 480p stack of the
bench) or MXFP4 weights (W4A8, 768p), and MXFP4 activations (W4A4, 768p).  Every stage is fed the GPU
block's own inputs (see _block_stages.py for the bars).  The static scales are calibrated on the
block's own input: each is the dynamic scale the same block takes on it (the amax of that GEMM input /
448).  Toy and Trim-width blocks on every row; the 480p stack's blocks (33,784 tokens, 53 of 264 key
tiles kept, the last query tile of 120 rows) and the 768p block (85,696 tokens, 135 of 670 key tiles,
the last tile of 64 rows) on three token tiles: the first, one in the middle and the last."""
import numpy as np
import pytest

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, f32_dev, host
from _block_stages import run_stages_fused, check_block_stages_fused

pytestmark = pytest.mark.gpu


def _run(name, w, L, seed, block=0, t=999.0, sparse=None, gate=None, rows=None, fmt=_lib.QVD_W_MXFP4):
    x = W.activations(w, seed, L=L)
    idx, cnt = W.block_mask(w, seed, block, L=L, sparse=sparse)
    idx_d, cnt_d = i32_dev(idx), i32_dev(cnt)
    if gate is None:
        mod_d = Q.adaln_project(t, fp16_dev(W.adaln_basis(w, seed)), fp16_dev(W.adaln_proj(w, seed, block)))
    else:
        mod_d = f32_dev(W.random_mod(w.d, seed=seed + 100, tag=w.tag, gate=gate))
    wbits = W.block_weights(w, seed, block)
    bw = Q.quantize_block_weights({k: bf16_dev(v) for k, v in wbits.items()}, w.d, w.n_heads, w.mlp, fmt=fmt)
    act = None
    if fmt != _lib.QVD_W_MXFP4_A4:
        # calibrate on the block's own input: the dynamic-scale run's four per-tensor scales
        ws = Q.block_forward_until(bw, mod_d, bf16_dev(x), idx_d, cnt_d, _lib.QVD_STAGE_ALL)
        act = host(Q.block_intermediates(bw, ws, L)["scales"]).copy()
        del ws
        bw.act_scale = f32_dev(act)
        say(name, "static scales", act.tolist())
    rows = np.arange(L) if rows is None else rows
    g = run_stages_fused(bw, mod_d, x, idx_d, cnt_d, rows)
    wm = {}
    for s in ("qkv", "o", "up", "down"):
        wm["w_" + s] = host(bw.w[s])
        if fmt == _lib.QVD_W_FP8:
            wm["s_" + s] = np.float32(host(bw.s[s])[0])
        else:
            wm["e8_" + s] = host(bw.e8[s])
    return check_block_stages_fused(name, wm, act, host(mod_d), x, idx, cnt, g, w.n_heads, rows)


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
    _run("toy W4A4", w, w.L, seed=2, fmt=_lib.QVD_W_MXFP4_A4)


def test_w4a4_stages_toy_gate_one_ragged_sparse():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W4A4 gate=1 L=391 sparse", w, 391, seed=4, sparse=True, gate=1.0, fmt=_lib.QVD_W_MXFP4_A4)


def test_w4a4_stages_trim_width_L1100_sparse():
    w = W.WORKLOADS["trim_block_L4096"]
    _run("trim W4A4 L=1100 sparse", w, 1100, seed=5, sparse=True, t=125.0, fmt=_lib.QVD_W_MXFP4_A4)


def test_w4a4_stages_768p_sampled_tiles():
    w = W.WORKLOADS["block_768p_mxfp4"]
    rows = _sampled_tiles(w)
    say(f"768p W4A4 block: {len(rows)} rows of {w.L}")
    _run("768p W4A4", w, w.L, seed=0, rows=rows, fmt=_lib.QVD_W_MXFP4_A4)


def test_w8a8_static_stages_toy():
    w = W.WORKLOADS["toy_d256_L256"]
    _run("toy W8A8 static", w, w.L, seed=6, fmt=_lib.QVD_W_FP8)


def test_w8a8_static_stages_trim_width_L1100_sparse_gate_one():
    w = W.WORKLOADS["trim_block_L4096"]
    _run("trim W8A8 static L=1100 sparse gate=1", w, 1100, seed=7, sparse=True, gate=1.0, fmt=_lib.QVD_W_FP8)


@pytest.mark.parametrize("block,t", [(0, 999.0), (41, 125.0)])
def test_w8a8_static_stages_480p_stack_blocks_sampled_tiles(block, t):
    w = W.WORKLOADS["trim_stack42_480p"]
    rows = _sampled_tiles(w)
    say(f"480p W8A8 static block {block} t={t}: {len(rows)} rows of {w.L}")
    _run(f"480p W8A8 static block {block} t={t:g}", w, w.L, seed=0, block=block, t=t, rows=rows,
         fmt=_lib.QVD_W_FP8)
