"""Seeded synthetic inputs for the quantized DiT-block forward.

Both the CPU oracle (``oracle/``) and the HIP path take their inputs from here, and from nowhere
else. This module holds none of the method's arithmetic: it draws random numbers, stores them in the
formats the method consumes (bf16 activations and master weights, fp16 AdaLN factors, int32
tile lists), and fixes the shapes of the workloads.

Shapes and value distributions follow the FastH3 Trim pages:
* comfyui-wiki "FastH3 Trim: pruned 8-step MiniMax H3 for 8 GB GPUs", section "What Trim
  changes": the 42-block transformer, the 2,688-dim time embedding, the shared 2,688->16 basis
  plus a per-block projection stored in fp16, 80% attention sparsity and the eight sampler
  timesteps 999 ... 125;
* same page, section "How fast is it", caption of the timing table: clips are 832x480, 5 s, with
  audio.  The latent token counts below (21 frames x 30 x 52 video + 1,024 audio at 480p;
  21 x 48 x 84 + 1,024 at 768p) are the workload definitions this build measures on; the pages
  do not print them.

Every generator is a pure function of (seed, workload, block, tensor id), through
``numpy.random.SeedSequence``; the same call returns the same bits on any machine.
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np

TILE = 128          # query/key tile edge of the block-sparse mask and of the INT8 Q/K scales
HEAD_DIM = 128
ADALN_RANK = 16     # width of the shared timestep basis
N_MOD = 6           # shift1, scale1, gate1, shift2, scale2, gate2
SAMPLER_TIMESTEPS = (999, 874, 749, 624, 500, 375, 250, 125)
N_BLOCKS_TRIM = 42

# token counts: video latent frames x rows x cols, then the audio tokens
AUDIO_TOKENS = 1024
TOKENS_480P = 21 * 30 * 52 + AUDIO_TOKENS      # 33,784
TOKENS_768P = 21 * 48 * 84 + AUDIO_TOKENS      # 85,696


@dataclass(frozen=True)
class Workload:
    name: str
    tag: int            # stable id mixed into every seed
    d: int
    n_heads: int
    mlp: int
    L: int
    sparse: bool        # keep 20% of key tiles per query tile (+ diagonal) instead of all
    outliers: bool      # 0.1% of channels of the block input scaled x30
    n_blocks: int = 1
    weight_format: str = "fp8"   # "fp8" (E4M3 per tensor) or "mxfp4" (E2M1 + E8M0 per 32)

    @property
    def head_dim(self) -> int:
        return HEAD_DIM

    @property
    def n_tiles(self) -> int:
        return (self.L + TILE - 1) // TILE

    @property
    def L_video(self) -> int:
        """Video tokens (they come first); the last AUDIO_TOKENS are audio at the 480p and 768p
        token counts, and every token is video in the other workloads."""
        return self.L - AUDIO_TOKENS if self.L in (TOKENS_480P, TOKENS_768P) else self.L

    @property
    def kmax(self) -> int:
        return kept_tiles_per_row(self.n_tiles) if self.sparse else self.n_tiles


WORKLOADS = {
    w.name: w
    for w in (
        # toy block: width 256, 2 heads x 128, MLP 1024, 256 tokens, dense attention
        Workload("toy_d256_L256", 1, d=256, n_heads=2, mlp=1024, L=256, sparse=False,
                 outliers=False),
        # one block at Trim width, 4,096 tokens, dense attention
        Workload("trim_block_L4096", 2, d=2688, n_heads=21, mlp=10752, L=4096, sparse=False,
                 outliers=True),
        # attention alone at the 480p token count, 80% block-sparse
        Workload("attn_480p", 3, d=2688, n_heads=21, mlp=10752, L=TOKENS_480P, sparse=True,
                 outliers=False),
        # the 42-block Trim stack, one denoising step at the 480p token count
        Workload("trim_stack42_480p", 4, d=2688, n_heads=21, mlp=10752, L=TOKENS_480P,
                 sparse=True, outliers=True, n_blocks=N_BLOCKS_TRIM),
        # one block at the 768p token count with MXFP4 weights and static activation scales
        Workload("block_768p_mxfp4", 5, d=2688, n_heads=21, mlp=10752, L=TOKENS_768P,
                 sparse=True, outliers=True, weight_format="mxfp4"),
    )
}


def kept_tiles_per_row(n_tiles: int) -> int:
    """Key tiles kept per query tile under 80% sparsity: floor(0.2*T) drawn tiles + the diagonal."""
    drawn = min((2 * n_tiles) // 10, n_tiles - 1)
    return drawn + 1


# ---------------------------------------------------------------------------------------------
# seeding

_TENSOR_IDS = {
    "x": 1, "w_qkv": 2, "w_o": 3, "w_up": 4, "w_down": 5, "basis": 6, "proj": 7, "mask": 8,
    "q": 9, "k": 10, "v": 11, "codes_a": 12, "codes_b": 13, "mod": 14, "calib": 15, "vec": 16,
    "outlier_ch": 17, "bias": 18, "scales": 19,
}


def rng_for(seed: int, tag: int, block: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, block, _TENSOR_IDS[tensor]]))


# ---------------------------------------------------------------------------------------------
# storage formats of the inputs (not the method's roundings: these only fix how a drawn number is
# handed over)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bf16 (ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------------------------
# generators

def outlier_channels(d: int, seed: int, tag: int) -> np.ndarray:
    """round(0.001*d) channel indices (3 at d = 2688, none at d = 256)."""
    n = int(round(0.001 * d))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng_for(seed, tag, 0, "outlier_ch").choice(d, size=n, replace=False))


def activations(w: Workload, seed: int = 0, block: int = 0, L: int | None = None) -> np.ndarray:
    """Block input x: N(0,1), outlier channels x30 when the workload has them -> bf16 [L, d]."""
    L = w.L if L is None else L
    x = rng_for(seed, w.tag, block, "x").standard_normal((L, w.d), dtype=np.float32)
    if w.outliers:
        x[:, outlier_channels(w.d, seed, w.tag)] *= np.float32(30.0)
    return f32_to_bf16_bits(x)


def glorot_uniform(n_out: int, n_in: int, rng: np.random.Generator) -> np.ndarray:
    a = np.float32(np.sqrt(6.0 / (n_in + n_out)))
    u = rng.random((n_out, n_in), dtype=np.float32)
    u *= np.float32(2.0) * a
    u -= a
    return u


def linear_weight(w: Workload, name: str, seed: int = 0, block: int = 0) -> np.ndarray:
    """Master weight [N][K] (K contiguous), Glorot-uniform, as bf16 bits."""
    n_out, n_in = weight_shape(w, name)
    return f32_to_bf16_bits(glorot_uniform(n_out, n_in, rng_for(seed, w.tag, block, name)))


def weight_shape(w: Workload, name: str) -> tuple[int, int]:
    d, f = w.d, w.mlp
    return {"w_qkv": (3 * d, d), "w_o": (d, d), "w_up": (f, d), "w_down": (d, f)}[name]


def block_weights(w: Workload, seed: int = 0, block: int = 0) -> dict:
    return {n: linear_weight(w, n, seed, block) for n in ("w_qkv", "w_o", "w_up", "w_down")}


def adaln_basis(w: Workload, seed: int = 0) -> np.ndarray:
    """Shared basis B [16][d] (fp16 bits), Glorot-uniform; one per model, shared by all blocks."""
    return f32_to_fp16_bits(glorot_uniform(ADALN_RANK, w.d, rng_for(seed, w.tag, 0, "basis")))


def adaln_proj(w: Workload, seed: int = 0, block: int = 0) -> np.ndarray:
    """Per-block projection P_k [6d][16] (fp16 bits), Glorot-uniform."""
    return f32_to_fp16_bits(glorot_uniform(N_MOD * w.d, ADALN_RANK,
                                           rng_for(seed, w.tag, block, "proj")))


def random_mod(d: int, seed: int = 0, tag: int = 0, gate: float | None = None) -> np.ndarray:
    """A synthetic modulation table [6][d] fp32 (for testing the modulate step on its own)."""
    m = rng_for(seed, tag, 0, "mod").standard_normal((N_MOD, d), dtype=np.float32)
    m *= np.float32(0.5)
    if gate is not None:
        m[2] = gate
        m[5] = gate
    return m


def block_mask(w: Workload, seed: int = 0, block: int = 0, L: int | None = None,
               sparse: bool | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Block-sparse 128x128 mask as sorted kept-key-tile lists.

    Returns kv_idx int32 [H][T][kmax] (ascending, padded with -1) and kv_cnt int32 [H][T].
    Sparse: per (head, query tile) independently, floor(0.2*T) distinct non-diagonal key tiles
    drawn uniformly without replacement, plus the diagonal tile. Dense: all T tiles.
    """
    L = w.L if L is None else L
    sparse = w.sparse if sparse is None else sparse
    H, T = w.n_heads, (L + TILE - 1) // TILE
    if not sparse:
        idx = np.broadcast_to(np.arange(T, dtype=np.int32), (H, T, T)).copy()
        return idx, np.full((H, T), T, dtype=np.int32)
    k = kept_tiles_per_row(T) - 1
    r = rng_for(seed, w.tag, block, "mask").random((H, T, T))
    diag = np.arange(T)
    r[:, diag, diag] = np.inf                       # the diagonal is never drawn
    drawn = np.argsort(r, axis=-1, kind="stable")[..., :k]
    idx = np.concatenate([drawn, np.broadcast_to(diag[None, :, None], (H, T, 1))], axis=-1)
    idx = np.sort(idx, axis=-1).astype(np.int32)
    return idx, np.full((H, T), k + 1, dtype=np.int32)


def qkv_heads(L: int, n_heads: int, seed: int = 0, tag: int = 0) -> tuple:
    """Q, K, V ~ N(0,1) as bf16 bits [L][H][128] (attention-only workloads)."""
    out = []
    for name in ("q", "k", "v"):
        g = rng_for(seed, tag, 0, name).standard_normal((L, n_heads, HEAD_DIM), dtype=np.float32)
        out.append(f32_to_bf16_bits(g))
    return tuple(out)


def normal_bf16(shape, seed: int = 0, tag: int = 0, scale: float = 1.0,
                tensor: str = "vec") -> np.ndarray:
    g = rng_for(seed, tag, 0, tensor).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        g *= np.float32(scale)
    return f32_to_bf16_bits(g)


def random_e4m3_codes(shape, seed: int = 0, tag: int = 0, tensor: str = "codes_a") -> np.ndarray:
    """Uniformly drawn finite E4M3 byte patterns (0x7F and 0xFF, the NaN patterns, excluded)."""
    c = rng_for(seed, tag, 0, tensor).integers(0, 254, size=shape, dtype=np.int32)
    c = c + (c >= 0x7F)                              # skip 0x7F
    return c.astype(np.uint8)


def calibration_batch(d_in: int, b: int, seed: int = 0, tag: int = 5, site: int = 0,
                      tokens: int = 1024) -> np.ndarray:
    """Batch ``b`` of heavy-tailed activations at one calibration site: Student-t (nu = 3), fp32
    [tokens][d_in].  Each batch has its own seed, so held-out batches are reproducible too."""
    g = np.random.default_rng(np.random.SeedSequence([seed, tag, site, _TENSOR_IDS["calib"], b]))
    return g.standard_t(3.0, size=(tokens, d_in)).astype(np.float32)


def outlier_spec(d_in: int, ratio: float, seed: int = 0, tag: int = 5, site: int = 0,
                 n_batches: int = 64, tokens: int = 1024) -> tuple[np.ndarray, np.float32, float]:
    """Outlier channels of a calibration site and the factor that puts them at ``ratio`` x A0.

    round(0.001*d_in) channels (at least one) are drawn; A0 is the amax of the site's first
    ``n_batches`` batches without outliers (the magnitude of a typical layer), and the factor
    rescales the drawn channels so that their amax over the same batches is ratio*A0.
    Returns (channels, factor, A0).
    """
    n_ch = max(1, int(round(0.001 * d_in)))
    ch = np.sort(rng_for(seed, tag, site, "outlier_ch").choice(d_in, size=n_ch, replace=False))
    base = 0.0
    ch_max = 0.0
    for b in range(n_batches):
        a = np.abs(calibration_batch(d_in, b, seed, tag, site, tokens))
        base = max(base, float(a.max()))
        ch_max = max(ch_max, float(a[:, ch].max()))
    return ch, np.float32(ratio * base / ch_max), base


def _device_seed(*key) -> int:
    return int(np.random.SeedSequence(list(key)).generate_state(1)[0])


def calibration_batch_device(d_in: int, b: int, seed: int = 0, tag: int = 5, site: int = 0,
                             tokens: int = 1024, device: str = "cuda"):
    """Batch ``b`` of heavy-tailed activations drawn on the GPU (full-size calibration runs): Student-t
    with nu = 3 built from its definition, Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3), from torch's seeded
    normal generator; fp32 [tokens][d_in].  A different stream from ``calibration_batch``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(seed, tag, site, _TENSOR_IDS["calib"], b, 1))
    z = torch.randn((4, tokens, d_in), generator=g, device=device)
    return z[0] / torch.sqrt((z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0)


def outlier_channels_device(d_in: int, seed: int = 0, tag: int = 5, site: int = 0, device: str = "cuda"):
    """round(0.001 d_in) (at least one) distinct channels of a site, drawn on the GPU, ascending."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(seed, tag, site, _TENSOR_IDS["outlier_ch"], 1))
    n_ch = max(1, int(round(0.001 * d_in)))
    return torch.sort(torch.randperm(d_in, generator=g, device=device)[:n_ch]).values


def apply_outliers(batch: np.ndarray, channels: np.ndarray, factor: np.float32) -> np.ndarray:
    out = batch.copy()
    out[:, channels] *= factor
    return out
