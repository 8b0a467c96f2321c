"""The seeded workloads carry the numbers the pages print (tests/golden/page_constants.json)."""
import json
import os

import numpy as np

import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_page_constants_in_workloads():
    assert list(W.SAMPLER_TIMESTEPS) == GOLD["sampler_timesteps"]["value"]
    assert W.N_BLOCKS_TRIM == GOLD["blocks_trim"]["value"]
    assert GOLD["blocks_base"]["value"] - GOLD["blocks_removed"]["value"] == W.N_BLOCKS_TRIM
    assert W.ADALN_RANK == GOLD["shared_basis_rank"]["value"]
    assert W.N_MOD == GOLD["modulation_vectors"]["value"]
    for name in ("trim_block_L4096", "attn_480p", "trim_stack42_480p", "block_768p_mxfp4"):
        assert W.WORKLOADS[name].d == GOLD["time_embedding_dim"]["value"]
    a, b, c = GOLD["pruning_measurements"]["factors"]
    assert a * b * c == GOLD["pruning_measurements"]["value"]
    assert W.N_BLOCKS_TRIM * GOLD["calibrated_layers_trim"]["per_block"] == \
        GOLD["calibrated_layers_trim"]["value"]


def test_token_counts_and_sparsity():
    assert W.TOKENS_480P == 32760 + 1024 == 33784
    assert W.TOKENS_768P == 84672 + 1024 == 85696
    w = W.WORKLOADS["attn_480p"]
    assert (w.n_tiles, w.kmax, w.L - 128 * (w.n_tiles - 1)) == (264, 53, 120)
    w = W.WORKLOADS["block_768p_mxfp4"]
    assert (w.n_tiles, w.kmax, w.L - 128 * (w.n_tiles - 1)) == (670, 135, 64)
    sp = GOLD["attention_sparsity"]["value"]
    for T in (264, 670):
        kept = W.kept_tiles_per_row(T)
        assert abs(kept / T - (1 - sp)) < 0.002


def test_generators_are_deterministic_and_shaped():
    w = W.WORKLOADS["toy_d256_L256"]
    a, b = W.activations(w, 3), W.activations(w, 3)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, W.activations(w, 4))
    wt = W.WORKLOADS["trim_block_L4096"]
    x = W.bf16_bits_to_f32(W.activations(wt, 0, L=64))
    ch = W.outlier_channels(wt.d, 0, wt.tag)
    assert len(ch) == 3
    assert np.abs(x[:, ch]).mean() > 10 * np.abs(np.delete(x, ch, axis=1)).mean()
    wq = W.linear_weight(w, "w_qkv")
    assert wq.shape == (768, 256) and wq.dtype == np.uint16
    lim = np.sqrt(6 / (768 + 256))
    assert np.abs(W.bf16_bits_to_f32(wq)).max() <= lim * (1 + 2 ** -8)
    codes = W.random_e4m3_codes(100000)
    assert not np.isin(codes, [0x7F, 0xFF]).any()
