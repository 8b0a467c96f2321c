"""Block-sparse attention with INT8 query/key scores (test infrastructure only).

[TRIM] "Trim 改变了什么", training bullet: the model runs with 80% attention sparsity.
[TRIM] "运行速度如何", note under the table: query and key are quantized to INT8 for the score
computation.

Plain definition, per head h and 128-row query tile i:
  keys(h, i)  = the rows of the kept key tiles kv_idx[h][i][:kv_cnt[h][i]] that exist (< L);
  S[r][c]     = sum_e q[r][h][e] * k[c][h][e]                      (exact integer)
  s[r][c]     = S[r][c] * q_scale[h][i] * k_scale[h][tile(c)] * sm_scale
  out[r][h][:] = sum_c softmax_c(s[r][:]) * v[c][h][:]
with V taken as the bf16 values it is given in, and everything after the integer scores in float64
(the row maximum is subtracted before exponentiating; that changes nothing but the range).
Readings: a key tile not in the list weighs zero (it is skipped, not attended with -inf after the
fact); key rows >= L do not exist; sm_scale = 1/sqrt(head_dim) with the natural exponential.  The
pages give no precision for softmax.V, so the oracle fixes none: it is the exact softmax attention
of the quantized scores, and an implementation's own rounding of the weights or of V is a deviation
to be bounded, not part of the definition.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64

TILE = 128


def kept_keys(kv_idx, kv_cnt, h: int, i: int, L: int) -> tuple[np.ndarray, np.ndarray]:
    """Key row indices of query tile i of head h, and the key tile each row belongs to."""
    tiles = np.asarray(kv_idx[h, i, : int(kv_cnt[h, i])], dtype=np.int64)
    rows = [np.arange(j * TILE, min(L, (j + 1) * TILE)) for j in tiles]
    tile_of = [np.full(len(r), j) for r, j in zip(rows, tiles)]
    if not rows:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(rows), np.concatenate(tile_of)


def sparse_attn_tile(q, q_scale, k, k_scale, v_bits, kv_idx, kv_cnt, h: int, i: int,
                     sm_scale: float) -> np.ndarray:
    """Output rows of query tile i of head h, float64 [rows][head_dim] (zeros for a row with no
    kept key)."""
    L = q.shape[0]
    rows = np.arange(i * TILE, min(L, (i + 1) * TILE))
    keys, key_tile = kept_keys(kv_idx, kv_cnt, h, i, L)
    if keys.size == 0:
        return np.zeros((len(rows), q.shape[2]))
    # exact: |S| <= 128 * 127 * 127 < 2^53, so the float64 library product is the integer sum
    S = q[rows, h, :].astype(np.float64) @ k[keys, h, :].astype(np.float64).T
    fac = (np.float64(q_scale[h, i]) * np.asarray(k_scale[h], dtype=np.float64)[key_tile]
           * sm_scale)
    s = S * fac[None, :]
    e = np.exp(s - s.max(axis=1, keepdims=True))
    V = bf16_to_f64(v_bits[keys, h, :])
    return (e @ V) / e.sum(axis=1, keepdims=True)


def sparse_attn(q, q_scale, k, k_scale, v_bits, kv_idx, kv_cnt, sm_scale=None,
                tiles=None) -> np.ndarray:
    """out float64 [L][H][head_dim].  ``tiles`` restricts the work to a list of (h, i) pairs
    (the other rows are returned as NaN)."""
    L, H, D = q.shape
    sm_scale = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    T = (L + TILE - 1) // TILE
    out = np.full((L, H, D), np.nan)
    pairs = [(h, i) for h in range(H) for i in range(T)] if tiles is None else tiles
    for h, i in pairs:
        out[i * TILE: min(L, (i + 1) * TILE), h, :] = sparse_attn_tile(
            q, q_scale, k, k_scale, v_bits, kv_idx, kv_cnt, h, i, sm_scale)
    return out
