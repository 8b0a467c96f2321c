"""Pins of the sparse-tile selector oracle (oracle/selector.py) against exact rational arithmetic and
the structure the selection must have."""
from fractions import Fraction

import numpy as np

import workloads as W
from oracle import quant as Q, selector as S


def _codes(L, H, seed):
    qb, kb, _ = W.qkv_heads(L, H, seed=seed)
    q8, qs = Q.quant_int8_qk(qb, L, H)
    k8, ks = Q.quant_int8_qk(kb, L, H)
    return q8, qs, k8, ks


def test_selector_matches_exact_rational_pooled_scores():
    """Exact rationals: pooled means of the dequantized codes (code x fp32 scale, averaged over the tile's
    existing rows) and their dot product; the kept set is the diagonal plus the top kept - 1 by that
    exact score (lower index on ties), sorted."""
    L, H, kept = 1000, 2, 3                      # T = 8, last tile 104 rows
    q8, qs, k8, ks = _codes(L, H, 21)
    T = 8
    idx, cnt = S.select_tiles(q8, k8, ks, L, H, kept)
    assert np.all(cnt == kept)
    for h in range(H):
        means = {}
        for name, c8, sc in (("q", q8, qs), ("k", k8, ks)):
            for t in range(T):
                rows = range(t * 128, min(L, (t + 1) * 128))
                tot = [sum(int(c8[r, h, e]) for r in rows) for e in range(128)]
                f = Fraction(float(sc[h, t])) / len(rows)
                means[name, t] = [f * v for v in tot]
        for i in range(T):
            score = {j: sum(a * b for a, b in zip(means["q", i], means["k", j])) for j in range(T) if j != i}
            ranked = sorted(score, key=lambda j: (-score[j], j))
            assert score[ranked[kept - 2]] != score[ranked[kept - 1]]     # no tie at the cut here
            want = sorted([i] + ranked[:kept - 1])
            assert list(idx[h, i, :kept]) == want, (h, i)


def test_selector_structure_and_limits():
    L, H = 2000, 3                                # T = 16, last tile 80 rows
    q8, qs, k8, ks = _codes(L, H, 5)
    T = 16
    for kept in (1, 4, 16, 20):
        idx, cnt = S.select_tiles(q8, k8, ks, L, H, kept)
        c = min(kept, T)
        assert idx.shape == (H, T, kept) and np.all(cnt == c)
        assert np.all(idx[:, :, c:] == -1)
        sel = idx[:, :, :c]
        assert np.all(np.diff(sel, axis=-1) > 0)                          # sorted, distinct
        assert np.all((sel == np.arange(T)[None, :, None]).any(-1))       # diagonal kept
        assert sel.min() >= 0 and sel.max() < T
        if kept >= T:
            assert np.all(sel == np.arange(T)[None, None, :])


def test_selector_prefers_aligned_key_tile_and_ignores_uniform_key_scale():
    """A key tile whose rows repeat the query tile's rows (times 2) outranks random tiles; scaling every
    key scale by the same power of two changes no selection (the rank key scales uniformly)."""
    L, H = 1280, 1
    qb, kb, _ = W.qkv_heads(L, H, seed=8)
    kf = W.bf16_bits_to_f32(kb)
    kf[5 * 128:6 * 128] = 2.0 * W.bf16_bits_to_f32(qb)[2 * 128:3 * 128]
    kb = W.f32_to_bf16_bits(kf)
    q8, qs = Q.quant_int8_qk(qb, L, H)
    k8, ks = Q.quant_int8_qk(kb, L, H)
    idx, _ = S.select_tiles(q8, k8, ks, L, H, 2)
    assert list(idx[0, 2, :2]) == [2, 5]
    idx2, _ = S.select_tiles(q8, k8, (ks * np.float32(4.0)).astype(np.float32), L, H, 5)
    idx5, _ = S.select_tiles(q8, k8, ks, L, H, 5)
    np.testing.assert_array_equal(idx2, idx5)


def _planted(L, rows_fn, seed):
    """Q and K bf16 [L][1][128]: noise x 0.1 everywhere, then the planted rows (dict row -> f32 [128])."""
    rng = np.random.default_rng(seed)
    q = (0.1 * rng.standard_normal((L, 1, 128))).astype(np.float32)
    k = (0.1 * rng.standard_normal((L, 1, 128))).astype(np.float32)
    rows_fn(q, k, rng)
    return W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)


def test_selector_uses_each_key_tiles_scale():
    """Key tiles 3 and 6 hold the same rows up to an exact factor 2: identical INT8 codes, scales 1 : 2.
    Query tile 0 is aligned with them, so tile 6 must win (a rank that ignored the key scale would tie
    and take tile 3)."""
    L = 1024

    def plant(q, k, rng):
        w = rng.standard_normal((128, 128)).astype(np.float32)
        q[0:128, 0] = w
        k[3 * 128:4 * 128, 0] = 0.5 * w
        k[6 * 128:7 * 128, 0] = w

    qb, kb = _planted(L, plant, 3)
    q8, qs = Q.quant_int8_qk(qb, L, 1)
    k8, ks = Q.quant_int8_qk(kb, L, 1)
    np.testing.assert_array_equal(k8[3 * 128:4 * 128], k8[6 * 128:7 * 128])
    assert ks[0, 6] == 2 * ks[0, 3]
    idx, _ = S.select_tiles(q8, k8, ks, L, 1, 2)
    assert list(idx[0, 0, :2]) == [0, 6]


def test_selector_averages_over_existing_rows_of_the_last_tile():
    """L = 576: the last key tile (4) has 64 rows equal to u; tile 1 holds u and 0.5 u (same scale).
    Mean-pooled, tile 4 scores 4/3 of tile 1 against a query tile made of u; pooled over 128 rows it
    would score 2/3 of it."""
    L = 576

    def plant(q, k, rng):
        u = rng.standard_normal((64, 128)).astype(np.float32)
        q[0:64, 0] = u
        q[64:128, 0] = u
        k[128:192, 0] = u
        k[192:256, 0] = 0.5 * u
        k[512:576, 0] = u

    qb, kb = _planted(L, plant, 4)
    q8, qs = Q.quant_int8_qk(qb, L, 1)
    k8, ks = Q.quant_int8_qk(kb, L, 1)
    assert ks[0, 1] == ks[0, 4]
    idx, _ = S.select_tiles(q8, k8, ks, L, 1, 2)
    assert list(idx[0, 0, :2]) == [0, 4]


def test_selector_ties_take_the_lower_tile_and_the_diagonal_never_counts_twice():
    """Key tiles 0 (the diagonal), 2 and 4 hold the query tile's own rows: tiles 2 and 4 tie exactly and
    the lower one is kept; the diagonal, though it scores as high, does not take the other slot."""
    L = 768

    def plant(q, k, rng):
        w = rng.standard_normal((128, 128)).astype(np.float32)
        q[0:128, 0] = w
        for t in (0, 2, 4):
            k[t * 128:(t + 1) * 128, 0] = w

    qb, kb = _planted(L, plant, 5)
    q8, qs = Q.quant_int8_qk(qb, L, 1)
    k8, ks = Q.quant_int8_qk(kb, L, 1)
    idx, cnt = S.select_tiles(q8, k8, ks, L, 1, 2)
    assert list(idx[0, 0, :2]) == [0, 2] and cnt[0, 0] == 2
    idx3, _ = S.select_tiles(q8, k8, ks, L, 1, 3)
    assert list(idx3[0, 0, :3]) == [0, 2, 4]
