"""GPU parity of the sparse-tile selector (qvd_select_tiles) against the oracle: the selected tile
lists must be identical, bit for bit (the rank key is an exact integer times a once-rounded float64
weight on both sides), including the planted cases of the oracle's pins and the 480p / 768p shapes."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from oracle import quant as OQ, selector as OS, block as OB, adaln as OA
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, f32_dev, host, host_bits

pytestmark = pytest.mark.gpu


def _both_codes(qb, kb, L, H):
    """INT8 Q/K on the device and in the oracle from the same bf16 input (bit-exact quantizer): the
    device codes feed the kernel, the oracle's codes feed the oracle."""
    q8, qs = Q.quant_int8_qk(bf16_dev(qb.reshape(L, H * 128)), H)
    k8, ks = Q.quant_int8_qk(bf16_dev(kb.reshape(L, H * 128)), H)
    oq, _ = OQ.quant_int8_qk(qb, L, H)
    ok, oks = OQ.quant_int8_qk(kb, L, H)
    np.testing.assert_array_equal(host(q8), oq)
    np.testing.assert_array_equal(host(k8), ok)
    np.testing.assert_array_equal(host(ks), oks)
    return (q8, k8, ks), (oq, ok, oks)


@pytest.mark.parametrize("L,H,kept", [(300, 2, 2), (1000, 2, 3), (2000, 3, 20), (1, 1, 4), (128 * 37 + 5, 3, 8)])
def test_select_tiles_vs_oracle(L, H, kept):
    say("select", L, H, kept)
    qb, kb, _ = W.qkv_heads(L, H, seed=L + kept)
    dev, orc = _both_codes(qb, kb, L, H)
    idx, cnt = Q.select_tiles(*dev, kept)
    oi, oc = OS.select_tiles(*orc, L, H, kept)
    np.testing.assert_array_equal(host(cnt), oc)
    np.testing.assert_array_equal(host(idx), oi)


def _planted(L, plant, seed):
    rng = np.random.default_rng(seed)
    q = (0.1 * rng.standard_normal((L, 1, 128))).astype(np.float32)
    k = (0.1 * rng.standard_normal((L, 1, 128))).astype(np.float32)
    plant(q, k, rng)
    return W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)


def test_select_tiles_planted_scale_ragged_and_ties():
    """The oracle pins' planted inputs: the key scale decides (tile 6 over 3), the ragged last tile is
    averaged over its own rows (tile 4 over 1), equal scores go to the lower tile (2 over 4)."""
    def p_scale(q, k, rng):
        w = rng.standard_normal((128, 128)).astype(np.float32)
        q[0:128, 0] = w
        k[384:512, 0] = 0.5 * w
        k[768:896, 0] = w

    def p_ragged(q, k, rng):
        u = rng.standard_normal((64, 128)).astype(np.float32)
        q[0:64, 0] = u
        q[64:128, 0] = u
        k[128:192, 0] = u
        k[192:256, 0] = 0.5 * u
        k[512:576, 0] = u

    def p_tie(q, k, rng):
        w = rng.standard_normal((128, 128)).astype(np.float32)
        q[0:128, 0] = w
        for t in (0, 2, 4):
            k[t * 128:(t + 1) * 128, 0] = w

    for L, plant, want in ((1024, p_scale, [0, 6]), (576, p_ragged, [0, 4]), (768, p_tie, [0, 2])):
        qb, kb = _planted(L, plant, L)
        dev, orc = _both_codes(qb, kb, L, 1)
        idx, _ = Q.select_tiles(*dev, 2)
        assert list(host(idx)[0, 0, :2]) == want, (L, host(idx)[0, 0])
        oi, _ = OS.select_tiles(*orc, L, 1, 2)
        np.testing.assert_array_equal(host(idx), oi)


@pytest.mark.parametrize("wl,heads", [("attn_480p", 4), ("block_768p_mxfp4", 2)])
def test_select_tiles_full_length(wl, heads):
    """The 480p (264 tiles, 53 kept) and 768p (670 tiles, 135 kept) token counts, a few heads."""
    w = W.WORKLOADS[wl]
    L, H, kept = w.L, heads, w.kmax
    say("select full", wl, L, H, kept)
    qb, kb, _ = W.qkv_heads(L, H, seed=7)
    dev, orc = _both_codes(qb, kb, L, H)
    idx, cnt = Q.select_tiles(*dev, kept)
    oi, oc = OS.select_tiles(*orc, L, H, kept)
    np.testing.assert_array_equal(host(cnt), oc)
    np.testing.assert_array_equal(host(idx), oi)


def test_block_selects_its_own_mask():
    """dit_block_forward with no mask: the block selects from its own INT8 Q/K.  Against the oracle block
    run with the oracle selector's mask on the oracle's Q/K codes (the same codes but for near-tie flips,
    R20, which here move no selection)."""
    w = W.WORKLOADS["toy_d256_L256"]
    L, kept = 1290, 3
    x = W.activations(w, 11, L=L)
    wbits = W.block_weights(w, 11)
    mod = W.random_mod(w.d, seed=12, tag=w.tag, gate=1.0)
    bw = Q.quantize_block_weights({k: bf16_dev(v) for k, v in wbits.items()}, w.d, w.n_heads, w.mlp)
    xd = bf16_dev(x)
    Q.dit_block_forward(bw, f32_dev(mod), xd, None, None, kmax=kept)
    got = host_bits(xd)
    qw = OB.quantize_block_weights(wbits)
    T = (L + 127) // 128
    dummy_idx = np.tile(np.arange(T, dtype=np.int32), (w.n_heads, T, 1))
    _, it = OB.dit_block(x, mod, qw, dummy_idx, np.full((w.n_heads, T), T, np.int32), w.n_heads, keep=True)
    oi, oc = OS.select_tiles(it["q8"], it["k8"], it["sk"], L, w.n_heads, kept)
    want = OB.dit_block(x, mod, qw, oi, oc, w.n_heads)
    from test_gpu_block import _check
    _check(x, got, want, "block with selected mask")


def test_w4a4_block_selects_its_own_mask():
    """W4A4 block with no mask passed: the selector runs on the block's INT8 Q/K between the QKV GEMM
    and the attention, as in the FP8 block."""
    w = W.WORKLOADS["toy_d256_L256"]
    L, kept = 1290, 3
    x = W.activations(w, 13, L=L)
    wbits = W.block_weights(w, 13)
    mod = W.random_mod(w.d, seed=14, tag=w.tag, gate=1.0)
    bw = Q.quantize_block_weights({k: bf16_dev(v) for k, v in wbits.items()}, w.d, w.n_heads, w.mlp,
                                  fmt=_lib.QVD_W_MXFP4_A4)
    xd = bf16_dev(x)
    Q.dit_block_forward(bw, f32_dev(mod), xd, None, None, kmax=kept)
    got = host_bits(xd)
    qm = {}
    for site in OB.SITES:
        qm["w_" + site], qm["e8_" + site] = OQ.quant_mxfp4_weight(wbits["w_" + site])
    T = (L + 127) // 128
    dummy_idx = np.tile(np.arange(T, dtype=np.int32), (w.n_heads, T, 1))
    _, it = OB.dit_block(x, mod, qm, dummy_idx, np.full((w.n_heads, T), T, np.int32), w.n_heads,
                         fmt="w4a4", keep=True)
    oi, oc = OS.select_tiles(it["q8"], it["k8"], it["sk"], L, w.n_heads, kept)
    want = OB.dit_block(x, mod, qm, oi, oc, w.n_heads, fmt="w4a4")
    from test_gpu_block import _check
    _check(x, got, want, "w4a4 block with selected mask", a4=True)


def test_select_kept_at_least_tiles_and_single_tile():
    """kept >= T keeps every tile in order; L <= 128 (one tile) keeps the diagonal only."""
    for L, kept in ((700, 9), (100, 3)):
        qb, kb, _ = W.qkv_heads(L, 2, seed=kept)
        dev, orc = _both_codes(qb, kb, L, 2)
        idx, cnt = Q.select_tiles(*dev, kept)
        oi, oc = OS.select_tiles(*orc, L, 2, kept)
        np.testing.assert_array_equal(host(idx), oi)
        np.testing.assert_array_equal(host(cnt), oc)
