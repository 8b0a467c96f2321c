"""Sparse-tile selector: which key tiles each query tile attends to (test infrastructure only).

[TRIM] "Trim 改变了什么", training bullet: the model runs with 80% attention sparsity.  The pages give
the sparsity and nothing of how the kept tiles are chosen.  Reading (a plain content-based rule):

  per head h and 128-row query tile i, every key tile j is scored by the dot product of the
  mean-pooled query tile and the mean-pooled key tile, both dequantized from their INT8 codes:
      score(h, i, j) = (sq[h][i] / n_i) (sk[h][j] / n_j) sum_e Qsum[h][i][e] Ksum[h][j][e]
  with Qsum / Ksum the sums of the INT8 codes over the tile's existing rows (n_i, n_j of them);
  the diagonal tile is always kept, and the kept - 1 other tiles of highest score join it (equal
  scores: the lower tile index first); the list is sorted by tile index.

The positive factor sq[h][i] / n_i is common to a row and cannot change its ranking, so the rank is
taken on D(h, i, j) * w(h, j) with D = sum_e Qsum Ksum the exact integer (|D| < 2^36) and
w = float64(sk[h][j]) / n_j, each operation rounded once in float64: a definition that both sides can
evaluate to the same bits.
"""
from __future__ import annotations

import numpy as np

TILE = 128


def tile_sums(codes, L: int, H: int, tile: int = TILE) -> np.ndarray:
    """INT8 codes [L][H][D] -> int64 [H][T][D]: per (head, tile) sum of the codes over existing rows."""
    c = np.asarray(codes, dtype=np.int64)
    T = (L + tile - 1) // tile
    out = np.zeros((H, T, c.shape[-1]), dtype=np.int64)
    for t in range(T):
        out[:, t, :] = c[t * tile:min(L, (t + 1) * tile)].sum(axis=0)
    return out


def tile_rows(L: int, tile: int = TILE) -> np.ndarray:
    T = (L + tile - 1) // tile
    return np.array([min(L, (t + 1) * tile) - t * tile for t in range(T)], dtype=np.int64)


def pooled_scores(q8, k8, k_scale, L: int, H: int) -> np.ndarray:
    """float64 [H][T][T]: D(h, i, j) * w(h, j), the ranking key of key tile j for query tile i."""
    qs = tile_sums(q8, L, H)
    ks = tile_sums(k8, L, H)
    n = tile_rows(L).astype(np.float64)
    w = np.asarray(k_scale, dtype=np.float32).astype(np.float64) / n[None, :]     # [H][T]
    D = np.einsum("hie,hje->hij", qs, ks)                                         # exact int64
    return D.astype(np.float64) * w[:, None, :]


def select_tiles(q8, k8, k_scale, L: int, H: int, kept: int):
    """-> (kv_idx int32 [H][T][kept] (-1 past the count), kv_cnt int32 [H][T])."""
    T = (L + TILE - 1) // TILE
    S = pooled_scores(q8, k8, k_scale, L, H)
    cnt = min(kept, T)
    idx = np.full((H, T, kept), -1, dtype=np.int32)
    for h in range(H):
        for i in range(T):
            others = np.array([j for j in range(T) if j != i], dtype=np.int64)
            order = np.lexsort((others, -S[h, i, others]))       # score descending, then j ascending
            chosen = np.sort(np.concatenate([[i], others[order[:cnt - 1]]]))
            idx[h, i, :cnt] = chosen
    return idx, np.full((H, T), cnt, dtype=np.int32)
