/*
 * qvd.h -- C ABI of the MI355X (gfx950) quantized DiT-block forward.
 *
 * The hot path of the FastH3 / FastH3 Trim pages: one diffusion-transformer block that denoises
 * video and audio latents, with
 *   - AdaLN modulation from a 2,688->16 timestep basis shared by all blocks plus a small per-block
 *     projection, both stored in fp16 (comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步
 *     MiniMax H3", section "Trim 改变了什么", timestep-conditioning bullet);
 *   - FP8 linear layers with one scale per tensor, the scales applied to the matmul output in the
 *     same kernel, and query/key quantized to INT8 for the attention scores (same page, section
 *     "运行速度如何", the note under the timing table);
 *   - 80% block-sparse attention (same page, "Trim 改变了什么", training bullet);
 *   - 4-bit weights with calibrated static activation scales (news.farwalk.ai FastH3 story,
 *     post 6/8; comfyui-wiki page, section "ComfyUI 重打包包含什么").
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never frees them.
 *     Scalars that the device produces (scales, amax) stay on the device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; nothing is synchronised or read back.
 *   - Return value: QVD_OK or a negative status.  Argument errors are detected on the host before
 *     anything is enqueued, and leave every buffer untouched.  qvd_last_error() then returns a
 *     message (per thread).  A failing launch returns QVD_EHIP.  Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Tensors must be 16-byte aligned (QVD_EALIGN otherwise); head_dim and tile are 128; d is a
 *     multiple of 128.
 *   - Results are deterministic: the same inputs give the same bits on every run.
 *   - bf16 and fp16 tensors are passed as their 16-bit patterns (uint16_t).  E4M3 codes follow the
 *     OCP OFP8 E4M3 ("FN") encoding; INT8 codes are symmetric in [-127, 127].
 *   - Workspaces (`ws`) are caller-allocated device memory of at least the size the matching
 *     qvd_*_ws_bytes() returns; their contents on entry do not matter.
 *   - Calls that share a workspace or an output must be ordered on one stream.
 */
#ifndef QVD_H
#define QVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QVD_ABI_VERSION 2

enum qvd_status {
    QVD_OK = 0,
    QVD_EINVAL = -1,       /* null pointer or out-of-range scalar                               */
    QVD_ESHAPE = -2,       /* unsupported or inconsistent sizes                                 */
    QVD_EALIGN = -3,       /* a tensor pointer is not 16-byte aligned                           */
    QVD_EWORKSPACE = -4,   /* workspace missing or smaller than the matching qvd_*_ws_bytes()  */
    QVD_EUNSUPPORTED = -5, /* the current device is not gfx950                                  */
    QVD_EHIP = -6          /* a HIP runtime call or kernel launch failed                        */
};

/* Version of this ABI (QVD_ABI_VERSION). */
int qvd_abi_version(void);

/* Message describing the last failure on the calling thread ("" if none).  The pointer stays
 * valid until the next failing call on the same thread. */
const char* qvd_last_error(void);

/* Checks that the current HIP device is gfx950.  Every other entry point performs the same check
 * on first use per device; calling it early only reports the result up front.
 * Returns QVD_OK, QVD_EUNSUPPORTED or QVD_EHIP. */
int qvd_init(void);

/* Failure injection for the error paths of callers (testing support, not part of the method): the
 * launch `after` launches from now (0: the next one) on the calling thread reports QVD_EHIP, as when
 * the runtime rejects a launch -- the kernel itself still runs -- and the entry point that made it
 * returns QVD_EHIP with "injected failure" in qvd_last_error().  after = -1 cancels a pending
 * injection; below -1 is QVD_EINVAL.  Only the calling thread's launches count. */
int qvd_inject_launch_failure(int32_t after);

/* ------------------------------------------------------------------------------------------
 * Per-tensor FP8 (E4M3) quantization -- "运行速度如何" note: one scale per tensor.
 *   x         : n bf16 values (any shape, contiguous).
 *   scale_in  : NULL -> dynamic scale: amax = max|x|, s = amax/448 (fp32, correctly rounded),
 *               q = E4M3(fp32(x * fp32(448/amax))); amax = 0 gives s = 1.
 *               non-NULL -> static scale read from device memory: s = *scale_in,
 *               q = E4M3(fp32(x * fp32(1/s))).
 *   q         : n E4M3 codes (round to nearest even; magnitudes above 448 saturate to 448).
 *   scale_out : one device fp32 receiving s.
 *   ws        : qvd_quant_ws_bytes(n) bytes (per-block partial maxima); unused for static scales.
 * n may be 0 (then only *scale_out is written: s = 1, or *scale_in). */
size_t qvd_quant_ws_bytes(int64_t n);
int quant_fp8_per_tensor(const uint16_t* x, int64_t n, const float* scale_in, uint8_t* q,
                         float* scale_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * INT8 query/key quantization -- "运行速度如何" note: Q and K are quantized to INT8 for the score
 * computation.  One symmetric scale per (head, tile of 128 tokens):
 *   a = max |x| over the tile's rows that exist (< L), s = a/127, q = clamp(rint(x * 127/a), +-127)
 *   (fp32 products, round half to even); a = 0 gives s = 1 and zero codes.
 *   x     : bf16 [L][H][head_dim] (token-major, heads interleaved; row stride = row_stride
 *           elements, >= H*head_dim; pass H*head_dim for a dense tensor).
 *   q     : int8 [L][H][head_dim], dense.
 *   scale : fp32 [H][ceil(L/tile)].
 * head_dim and tile must be 128; L >= 0. */
int quant_int8_qk(const uint16_t* x, int32_t L, int32_t H, int32_t head_dim, int32_t tile,
                  int64_t row_stride, int8_t* q, float* scale, void* stream);

/* ------------------------------------------------------------------------------------------
 * AdaLN projection -- "Trim 改变了什么", timestep-conditioning bullet.
 *   e(t) = [cos(t f_i), sin(t f_i)], f_i = 10000^(-i/(dt/2)), i < dt/2   (float64)
 *   c    = B e(t)                (B: fp16 [16][dt], the basis shared by all blocks)
 *   mod  = P c (+ b)             (P: fp16 [6d][16] per block; b: fp16 [6d] or NULL)
 * written as fp32 [6][d]: shift1, scale1, gate1, shift2, scale2, gate2.  All arithmetic is
 * float64, rounded once to fp32.  dt must be even and <= 16384; d a multiple of 128.
 * The _stack form does n_blocks blocks in one launch: proj [n_blocks][6d][16],
 * bias [n_blocks][6d] or NULL, mod [n_blocks][6][d]. */
int qvd_adaln_project(float t, const uint16_t* basis, int32_t dt, const uint16_t* proj,
                      const uint16_t* bias, int32_t d, float* mod, void* stream);
int qvd_adaln_project_stack(float t, const uint16_t* basis, int32_t dt, const uint16_t* proj,
                            const uint16_t* bias, int32_t d, int32_t n_blocks, float* mod,
                            void* stream);

/* ------------------------------------------------------------------------------------------
 * Modulated LayerNorm + per-tensor FP8 -- same bullet (the modulation it applies):
 *   y = fp32(LN(x) * (1 + scale) + shift), LN without affine parameters, biased variance,
 *   statistics and the affine map in float64; then the per-tensor E4M3 quantization above
 *   (dynamic, or static when act_scale_in is non-NULL).
 *   x   : bf16 [L][d];  mod: fp32 [6][d];  half = 0 uses rows (0 shift1, 1 scale1),
 *         half = 1 uses rows (3 shift2, 4 scale2).
 *   q   : E4M3 [L][d];  act_scale_out: one device fp32.
 *   ws  : qvd_adaln_modulate_ws_bytes(L, d) bytes.
 * d must be a multiple of 128 and at most 4096. */
size_t qvd_adaln_modulate_ws_bytes(int32_t L, int32_t d);
int adaln_modulate(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                   float eps, const float* act_scale_in, uint8_t* q, float* act_scale_out,
                   void* ws, size_t ws_bytes, void* stream);
/* adaln_modulate for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation and results, with no ws argument.
 * The dynamic scale's workspace (row statistics and partial maxima) is a 4 MiB array inside the
 * library, one per GPU, held until the process ends; its device address is looked up once per
 * device on the first call there.  Dynamic scales (act_scale_in == NULL) therefore accept
 * L <= 261,872 tokens (QVD_EWORKSPACE beyond, with nothing launched); a static scale needs no
 * workspace and takes any L.  The call allocates nothing (no hipMalloc/hipFree, no timer events:
 * the library's opt-in per-kernel timer skips it).  Every call on one GPU uses that GPU's single
 * array: calls that overlap on one GPU (concurrent streams or threads) race and must be serialized
 * by the caller.  Nothing in the array needs clearing between calls. */
int adaln_modulate_noalloc(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                           float eps, const float* act_scale_in, uint8_t* q, float* act_scale_out,
                           void* stream);
/* The same modulated LayerNorm with MXFP4 output (W4A4 blocks: the 4-bit transformer of the
 * news.farwalk.ai FastH3 story, post 6/8, in OCP MX form): y as above, then per token row and 32
 * consecutive channels X = 2^(floor(log2 max|y|) - 2) (all-zero block: X = 1), codes E2M1(y / X),
 * round to nearest even, saturating at 6.  packed: uint8 [L][d/2] (channel 2j in the low nibble of
 * byte j); e8m0: uint8 [L][d/32].  One pass; no workspace. */
int adaln_modulate_mxfp4(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                         float eps, uint8_t* packed, uint8_t* e8m0, void* stream);
/* The values the modulate quantizers encode, for calibration: y fp32 [L][d] =
 * fp32(LN(x)(1 + scale) + shift) with the statistics and the affine map in float64, rounded once
 * (the same y as adaln_modulate).  No workspace. */
int adaln_layernorm_modulate_f32(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                                 float eps, float* y, void* stream);

/* ------------------------------------------------------------------------------------------
 * Block-sparse attention with INT8 scores -- "Trim 改变了什么" training bullet (80% sparsity)
 * and the "运行速度如何" note (INT8 Q/K).  For head h and query tile i (128 rows):
 *   keys   = rows of the key tiles kv_idx[h][i][0 .. kv_cnt[h][i]-1] that exist (< L)
 *   s      = (Q8 K8^T)[exact int32] * q_scale[h][i] * k_scale[h][j] * sm_scale
 *   out    = softmax over the kept keys of s, times V (bf16 values)  per query row, as bf16.
 *   q, k   : int8 [L][H][head_dim];  q_scale, k_scale: fp32 [H][T], T = ceil(L/128).
 *   v      : bf16 [L][H][head_dim];  out: bf16 [L][H][head_dim].
 *   kv_idx : int32 [H][T][kmax], 1 <= kmax <= 1024; kv_cnt: int32 [H][T].  Entries outside [0, T) and counts outside
 *            [0, kmax] are ignored (clamped), so device data can never send the kernel out of
 *            bounds; a row with no kept key outputs zeros.  Tile lists are expected ascending
 *            with the diagonal present; another order changes the result only at the level of
 *            bf16/fp32 rounding.
 *   out_amax_partials : NULL, or fp32 [H][T] receiving max|out| of each (h, i) tile (feeds the
 *            dynamic FP8 quantization of the attention output without another pass).
 *   ws     : qvd_sparse_attn_ws_bytes(L, H) bytes: V transposed to fp16 with one power-of-two
 *            scale per head (as the QKV GEMM epilogue and qvd_vt_unify write it), and its exponents.
 * Arithmetic: INT8 MFMA scores (exact int32); one pass over the kept tiles with a reference
 * maximum m per row, moved (and the fp32 sums rescaled) only when a tile's row maximum exceeds it
 * by more than 8 in log2 units: numerators exp2((s - m) log2 e) <= 2^8 rounded to fp16, fp16 MFMA
 * P.V and numerator sums with fp32 accumulation, normalised by the sum of the rounded numerators.
 * Each weight is the exact one up to a relative 2^-11 (the numerator's fp16 rounding) and fp32
 * arithmetic.  V enters at any finite bf16 magnitude: fp16 V 2^-E per head, exact for every
 * element within 2^28 of the head's max|V|, and the output is multiplied back by 2^E. */
size_t qvd_sparse_attn_ws_bytes(int32_t L, int32_t H);
int sparse_attn(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                const uint16_t* v, int32_t L, int32_t H, int32_t head_dim,
                const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                uint16_t* out, float* out_amax_partials, void* ws, size_t ws_bytes, void* stream);
/* bf16 V [L][H][128] -> fp16 V^T [H][128][T*128] (columns L.. zeroed) with one exponent per
 * (head, 128-token tile) in tile_exp [H][T], by the rule of the QKV epilogue (QVD_EPI_QKV): the
 * transpose sparse_attn runs on its V, exported for callers that hold V token-major. */
int qvd_vt_from_bf16(const uint16_t* v, int32_t L, int32_t H, uint16_t* vt, int32_t* tile_exp, void* stream);

/* One V scale per head, in place: vt fp16 [H][128][T*128] holds each (head, 128-token tile) j as
 * fp16(v 2^-tile_exp[h][j]) (the QKV GEMM epilogue's output).  Writes head_exp[h] = E = the largest
 * of the head's tile exponents and rescales every tile with a smaller exponent e by 2^(e - E), so the
 * head holds fp16(v 2^-E) (exact wherever that is an fp16 normal; a value more than 2^28 below the
 * head's max|v| may round to the fp16 subnormal grid).  Tiles already at E are not touched.
 * tile_exp: int32 [H][T]; head_exp: int32 [H]. */
int qvd_vt_unify(uint16_t* vt, int32_t L, int32_t H, const int32_t* tile_exp, int32_t* head_exp,
                 void* stream);

/* The same attention with V already transposed: vt fp16 [H][128][T*128] holding V 2^-v_exp[h]
 * (keys contiguous per (head, dim) row; columns L .. T*128-1 must hold finite values, e.g. zeros),
 * v_exp int32 [H].  This is the layout the QKV GEMM epilogue and qvd_vt_unify write. */
int qvd_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k,
                       const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L, int32_t H,
                       const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                       uint16_t* out, float* out_amax_partials, void* stream);

/* The same attention over fp16 V^T (and its head exponents) writing, instead of bf16 O, the E4M3 codes
 *   out_q[l][h][d] = E4M3(bf16(O[l][h][d]) * fp32(1 / *out_scale))
 * that quant_fp8_per_tensor computes from bf16 O with scale_in = out_scale (a static, calibrated
 * per-tensor scale > 0), without writing O: the attention output enters the out-projection GEMM
 * directly.  out_q: uint8 [L][H][128], 16-byte aligned. */
int qvd_sparse_attn_vt_e4m3(const int8_t* q, const float* q_scale, const int8_t* k,
                            const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L, int32_t H,
                            const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                            const float* out_scale, uint8_t* out_q, void* stream);
/* The same attention writing the MXFP4 codes of bf16 O (W4A4 blocks), per (token, head) and 32
 * consecutive dims exactly as qvd_quant_mxfp4 quantizes the bf16 tensor O viewed as [L][H*128]:
 * out_packed uint8 [L][H][64] (dim 2j in the low nibble of byte j; 16-byte aligned), out_e8m0
 * uint8 [L][H][4] (4-byte aligned).  O itself is not written. */
int qvd_sparse_attn_vt_mxfp4(const int8_t* q, const float* q_scale, const int8_t* k,
                             const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L, int32_t H,
                             const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                             uint8_t* out_packed, uint8_t* out_e8m0, void* stream);

/* ------------------------------------------------------------------------------------------
 * Sparse-tile selector -- "Trim 改变了什么", training bullet (80% attention sparsity; the pages do
 * not say how the kept tiles are chosen).  The rule: per head h and 128-token query tile i, key
 * tile j is ranked by the dot product of the mean-pooled, dequantized query and key tiles,
 *   score(h, i, j) = (sq[h][i] / n_i)(sk[h][j] / n_j) sum_e Qsum[h][i][e] Ksum[h][j][e]
 * (Qsum, Ksum: sums of the INT8 codes over the tile's n rows that exist); the diagonal is always
 * kept and the kept - 1 best other tiles join it (equal scores: lower j first).  The rank is taken
 * on D * w, D the exact integer dot of the code sums and w = double(sk[h][j]) / n_j, each rounded
 * once in float64, so it is reproducible bit for bit.
 *   q, k    : int8 [L][H][128] (the INT8 Q/K of quant_int8_qk or the QKV epilogue), 16-byte aligned
 *   k_scale : fp32 [H][T]
 *   kv_idx  : int32 [H][T][kept], out: the kept tiles in ascending order, then -1
 *   kv_cnt  : int32 [H][T], out: min(kept, T)
 *   ws      : qvd_select_tiles_ws_bytes(L, H) bytes (the code sums and the [H][T][T] scores)
 * L <= 131,072 (T <= 1024), 1 <= kept <= 1024. */
size_t qvd_select_tiles_ws_bytes(int32_t L, int32_t H);
int qvd_select_tiles(const int8_t* q, const int8_t* k, const float* k_scale, int32_t L, int32_t H,
                     int32_t kept, int32_t* kv_idx, int32_t* kv_cnt, void* ws, size_t ws_bytes,
                     void* stream);

/* Exact INT32 accumulators Q8[rows of tile i] . K8[rows of tile j]^T of head h, computed by the
 * same INT8 MFMA tile routine the attention kernel uses, into out int32 [128][128]
 * (out[r][c] = query row i*128+r, key row j*128+c; rows/keys >= L are written as 0). */
int qvd_qk_int32_tile(const int8_t* q, const int8_t* k, int32_t L, int32_t H, int32_t h,
                      int32_t i, int32_t j, int32_t* out, void* stream);

/* ------------------------------------------------------------------------------------------
 * FP8 GEMM with the per-tensor output scale fused into the epilogue -- "运行速度如何" note:
 *   acc[m][n] = sum_k E4M3(a[m][k]) * E4M3(w[n][k])   (MFMA, fp32 accumulation)
 *   y[m][n]   = acc * fp32(s_a * s_w) + bias[n]        (bias NULL = 0)
 * a: E4M3 [M][K], w: E4M3 [N][K] (both K-contiguous); s_a, s_w: device fp32 scalars.
 * M >= 0, N and K multiples of 128.  The epilogue is chosen by `epi`: */
enum qvd_epilogue_mode {
    QVD_EPI_F32 = 0,        /* out_f32[m][n] = y                                               */
    QVD_EPI_BF16 = 1,       /* out_bf16[m][n] = bf16(y)                                        */
    QVD_EPI_RESID_GATE = 2, /* out_bf16[m][n] = bf16(resid[m][n] + gate[n] * y); out may alias
                               resid (in-place residual update)                                 */
    QVD_EPI_GELU = 3,       /* out_bf16[m][n] = bf16(GELU(y)) (erf form); amax_partials, if
                               non-NULL, receives per-output-tile max|out| (see below)          */
    QVD_EPI_QKV = 4,        /* N = 3*H*128: columns [Q | K | V].  y is rounded to bf16; the Q and
                               K parts are then quantized per (head, 128-token tile) exactly as
                               quant_int8_qk does, into q8/k8 int8 [M][H][128] with scales
                               q_scale/k_scale [H][ceil(M/128)]; the V part (bf16 values) is
                               written transposed in fp16 into v as [H][128][ceil(M/128)*128],
                               columns M.. of the last tile zeroed, each (head, 128-token tile)
                               as fp16(v 2^-e) with its exponent e in v_exp [H][ceil(M/128)]:
                               e = 0 while the tile's max|v| is in [2^-6, 2^15), else
                               floor(log2 max|v|) - 14 (exact wherever v 2^-e is an fp16
                               normal).  qvd_vt_unify then gives the head one exponent, the
                               layout qvd_sparse_attn_vt reads                                  */
    QVD_EPI_GELU_E4M3 = 5,  /* out_e4m3[m][n] = E4M3(bf16(GELU(y)) * fp32(1 / *out_scale)): the
                               GELU output quantized with a static per-tensor scale exactly as
                               quant_fp8_per_tensor does with scale_in = out_scale, without the
                               bf16 tensor (static scales: the calibrated path)                 */
    QVD_EPI_GELU_MXFP4 = 6  /* bf16(GELU(y)) quantized to MXFP4 per row and 32 consecutive columns
                               exactly as qvd_quant_mxfp4 does from the bf16 tensor, without
                               writing it: out_e2m1 [M][N/2] (column 2j in the low nibble of byte
                               j), out_e8m0 [M][N/32] (W4A4 blocks: the down-projection's input) */
};
typedef struct {
    int32_t mode;               /* qvd_epilogue_mode                                           */
    int32_t n_heads;            /* QVD_EPI_QKV                                                 */
    float* out_f32;             /* QVD_EPI_F32                                                 */
    uint16_t* out_bf16;         /* QVD_EPI_BF16, QVD_EPI_RESID_GATE, QVD_EPI_GELU              */
    const uint16_t* resid;      /* QVD_EPI_RESID_GATE                                          */
    const float* gate;          /* QVD_EPI_RESID_GATE: fp32 [N]                                */
    float* amax_partials;       /* QVD_EPI_GELU (optional): fp32 [qvd_gemm_tiles(M, N)]        */
    int8_t* q8;                 /* QVD_EPI_QKV                                                 */
    int8_t* k8;
    uint16_t* v;                /* QVD_EPI_QKV: fp16 V^T [H][128][ceil(M/128)*128]               */
    float* q_scale;
    float* k_scale;
    int32_t* v_exp;             /* QVD_EPI_QKV: int32 [H][ceil(M/128)] V tile exponents          */
    uint8_t* out_e4m3;          /* QVD_EPI_GELU_E4M3: E4M3 codes [M][N]                          */
    const float* out_scale;     /* QVD_EPI_GELU_E4M3: device fp32 static scale s (> 0)           */
    uint8_t* out_e2m1;          /* QVD_EPI_GELU_MXFP4: packed E2M1 [M][N/2], 16-byte aligned     */
    uint8_t* out_e8m0;          /* QVD_EPI_GELU_MXFP4: E8M0 [M][N/32]                            */
} qvd_epilogue;
int64_t qvd_gemm_tiles(int32_t M, int32_t N);
int qvd_gemm_fp8(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                 const float* bias, int32_t M, int32_t N, int32_t K, const qvd_epilogue* epi,
                 void* stream);
/* The same GEMM with 4-bit weights (news.farwalk.ai FastH3 story, post 6/8, in OCP MX form):
 *   acc[m][n] = sum_k E4M3(a[m][k]) * E2M1(w[n][k]) * 2^(e8m0[n][k/32] - 127)  (block-scaled MFMA)
 *   y[m][n]   = acc * s_a + bias[n]
 * w_packed: uint8 [N][K/2], element 2j in the low nibble of byte j; e8m0: uint8 [N][K/32]. */
int qvd_gemm_mxfp4(const uint8_t* a, const float* s_a, const uint8_t* w_packed,
                   const uint8_t* e8m0, const float* bias, int32_t M, int32_t N, int32_t K,
                   const qvd_epilogue* epi, void* stream);
/* Both operands 4-bit (W4A4; the same story's NVFP4 transformer, in OCP MX form): activations
 * quantized per 32 consecutive K exactly as qvd_quant_mxfp4 quantizes weights, then
 *   acc[m][n] = sum_k E2M1(a[m][k]) 2^(a_e8m0[m][k/32] - 127) * E2M1(w[n][k]) 2^(w_e8m0[n][k/32] - 127)
 *   y[m][n]   = acc + bias[n]              (no per-tensor factor; every epilogue mode applies)
 * a_packed: uint8 [M][K/2], a_e8m0: uint8 [M][K/32]; w_packed, w_e8m0 as in qvd_gemm_mxfp4 (element
 * 2j in the low nibble of byte j).  Packed operands 16-byte aligned, scale arrays 4-byte aligned.
 * Accumulation is fp32 in the matrix cores' own order.  Shapes and errors as qvd_gemm_fp8. */
int qvd_gemm_mxfp4_w4a4(const uint8_t* a_packed, const uint8_t* a_e8m0, const uint8_t* w_packed,
                        const uint8_t* w_e8m0, const float* bias, int32_t M, int32_t N, int32_t K,
                        const qvd_epilogue* epi, void* stream);

/* ------------------------------------------------------------------------------------------
 * One DiT block forward -- the reading of the block (pre-norm adaLN-Zero DiT block):
 *   h1 = FP8(LN(x)(1+scale1) + shift1);  [Q|K|V] = bf16(h1 W_qkv^T s s + b)
 *   Q8, K8 = INT8 per (head, 128-token tile);  O = sparse_attn(Q8, K8, V)
 *   x1 = bf16(x + gate1 * (FP8(O) W_o^T s s + b))
 *   h2 = FP8(LN(x1)(1+scale2) + shift2);  g = bf16(GELU(h2 W_up^T s s + b))
 *   x2 = bf16(x1 + gate2 * (FP8(g) W_down^T s s + b))
 * Weights are [N][K] (K contiguous).  weight_format QVD_W_FP8: E4M3 codes with per-tensor fp32
 * scales s_*.  QVD_W_MXFP4: packed E2M1 (element 2j in the low nibble of byte j) with E8M0
 * scales e8m0_* [N][K/32]; s_* are ignored.  act_scale: NULL (dynamic scales) or fp32 [4] static
 * scales of the QKV, out, up and down GEMM inputs (with MXFP4 weights too; NULL there gives dynamic
 * per-tensor E4M3 activations, the calibration configuration).  QVD_W_MXFP4_A4 (W4A4):
 * the weights as for QVD_W_MXFP4 and every GEMM input MXFP4 too -- h1 and h2 from
 * adaln_modulate_mxfp4, O from qvd_sparse_attn_vt_mxfp4, g from the QVD_EPI_GELU_MXFP4 epilogue --
 * each with a dynamic E8M0 scale per token row and 32 channels; act_scale is ignored.  Biases may
 * be NULL. */
enum qvd_weight_format { QVD_W_FP8 = 0, QVD_W_MXFP4 = 1, QVD_W_MXFP4_A4 = 2 };
typedef struct {
    int32_t version;            /* QVD_ABI_VERSION                                             */
    int32_t d, n_heads, head_dim, mlp, weight_format;
    const void *w_qkv, *w_o, *w_up, *w_down;
    const uint8_t *e8m0_qkv, *e8m0_o, *e8m0_up, *e8m0_down;
    const float *s_qkv, *s_o, *s_up, *s_down;
    const float *b_qkv, *b_o, *b_up, *b_down;
    const float* act_scale;
    float ln_eps;
} qvd_block_params;

/* Workspace of dit_block_forward for L tokens. */
size_t qvd_block_ws_bytes(const qvd_block_params* p, int32_t L);
/* x: bf16 [L][d], read and overwritten with the block output.  mod: fp32 [6][d] of this block at
 * this timestep (qvd_adaln_project).  kv_idx/kv_cnt/kmax: the block's sparse mask as in
 * sparse_attn; or kv_idx = kv_cnt = NULL: the block selects min(kmax, T) key tiles per query tile
 * from its own INT8 Q/K by the qvd_select_tiles rule, in the workspace.  Sizes: head_dim 128,
 * d = 128 n_heads <= 4096, mlp a positive multiple of 256, kmax 1..1024, and every GEMM input and V^T
 * below 4 GiB (L max(d, mlp) < 2^32 and 2 d 128 ceil(L/128) < 2^32: L < 399,457 at d = 2,688,
 * mlp = 10,752); QVD_ESHAPE otherwise, QVD_EINVAL for NULL or inconsistent pointers, QVD_EALIGN,
 * QVD_EWORKSPACE below qvd_block_ws_bytes. */
int dit_block_forward(const qvd_block_params* p, const float* mod, uint16_t* x, int32_t L,
                      const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, void* ws,
                      size_t ws_bytes, void* stream);

/* Stage-by-stage inspection of the same block (for parity tests that feed each stage's GPU inputs to
 * a reference of the next stage).  qvd_block_forward_until runs dit_block_forward's own launches, with
 * the same arguments, and returns after `stage`; the intermediates are then in the workspace (and x),
 * at the offsets qvd_block_ws_layout gives.  After:
 *   QVD_STAGE_MODULATE1 : h = h1 codes (E4M3 [L][d], or packed E2M1 [L][d/2] + h_e8m0 [L][d/32] in
 *                         W4A4), scales[0] = s1 (dynamic FP8)
 *   QVD_STAGE_QKV       : q8, k8 [L][H][128], q_scale, k_scale [H][T]; vt fp16 [H][128][T*128] with
 *                         vt_tile_exp [H][T] (the QVD_EPI_QKV outputs)
 *   QVD_STAGE_VT        : vt with one exponent per head, vt_head_exp [H] (qvd_vt_unify)
 *   QVD_STAGE_ATTN      : o bf16 [L][d] (dynamic FP8); with static scales or W4A4 the attention writes
 *                         the codes of O into h directly, as at QVD_STAGE_OQUANT
 *   QVD_STAGE_OQUANT    : h = codes of O, scales[1] = s_O (dynamic FP8)
 *   QVD_STAGE_OPROJ     : x = x1
 *   QVD_STAGE_MODULATE2 : h = h2 codes (+ h_e8m0), scales[2] = s2
 *   QVD_STAGE_UP        : g bf16 [L][F] (dynamic FP8); static scales or W4A4: the codes of g, as at
 *                         QVD_STAGE_GQUANT
 *   QVD_STAGE_GQUANT    : g8 = codes of g (E4M3 [L][F], or packed E2M1 [L][F/2] + g_e8m0 [L][F/32]),
 *                         scales[3] = s_g (dynamic FP8)
 *   QVD_STAGE_ALL       : x = x2 (the whole block, as dit_block_forward)
 * Later stages overwrite h and x.  Errors as dit_block_forward; QVD_EINVAL for an unknown stage. */
enum qvd_block_stage {
    QVD_STAGE_MODULATE1 = 1, QVD_STAGE_QKV = 2, QVD_STAGE_VT = 3, QVD_STAGE_ATTN = 4, QVD_STAGE_OQUANT = 5,
    QVD_STAGE_OPROJ = 6, QVD_STAGE_MODULATE2 = 7, QVD_STAGE_UP = 8, QVD_STAGE_GQUANT = 9, QVD_STAGE_ALL = 10
};
int qvd_block_forward_until(const qvd_block_params* p, const float* mod, uint16_t* x, int32_t L,
                            const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, int32_t stage,
                            void* ws, size_t ws_bytes, void* stream);
/* Byte offsets, in dit_block_forward's workspace for L tokens, of its intermediates: offsets[i] for
 * i in qvd_block_ws_slot.  Slots the configuration does not use (o and g with static scales or W4A4,
 * the E8M0 arrays outside W4A4) have zero-length regions.  scales: fp32 [4] (s1, s_O, s2, s_g). */
enum qvd_block_ws_slot {
    QVD_WS_H = 0, QVD_WS_Q8, QVD_WS_K8, QVD_WS_VT, QVD_WS_VT_TILE_EXP, QVD_WS_VT_HEAD_EXP, QVD_WS_O, QVD_WS_G,
    QVD_WS_G8, QVD_WS_H_E8M0, QVD_WS_G_E8M0, QVD_WS_Q_SCALE, QVD_WS_K_SCALE, QVD_WS_SCALES, QVD_WS_SEL_IDX,
    QVD_WS_SEL_CNT, QVD_WS_SLOT_COUNT
};
int qvd_block_ws_layout(const qvd_block_params* p, int32_t L, int64_t* offsets);

/* ------------------------------------------------------------------------------------------
 * MXFP4 weights and static-scale calibration -- farwalk post 6/8 (calibrated 4-bit layers).
 * qvd_quant_mxfp4: bf16 [N][K] -> packed E2M1 [N][K/2] + E8M0 [N][K/32], per 32 consecutive K:
 *   X = 2^(floor(log2 amax) - 2) (all-zero block: X = 1), element = E2M1(w / X), RNE, saturating
 *   at 6.  K must be a multiple of 32.
 * qvd_amax_update: *amax = max(*amax, max|x|) over n fp32 values (running calibration amax; the
 *   caller zeroes *amax once before the first batch).
 * qvd_clip_count: *count += #{ |x| > s*448 } (exact comparison in float64) over n fp32 values,
 *   s = *scale; *count is a device uint64 the caller zeroes.
 * qvd_calibrated_scale: the static per-tensor scale of each of n calibration maxima (the farwalk
 *   post's calibrated 4-bit layers; the rule is this library's reading): scale[i] = fp32(amax[i]/448),
 *   raised by one fp32 ulp when 448 scale[i] (exact) would fall below amax[i], so that no value of
 *   the calibration set clips; amax[i] = 0 gives 1.  amax, scale: device fp32 [n]. */
int qvd_quant_mxfp4(const uint16_t* w, int32_t N, int32_t K, uint8_t* packed, uint8_t* e8m0,
                    void* stream);
int qvd_amax_update(const float* x, int64_t n, float* amax, void* stream);
int qvd_clip_count(const float* x, int64_t n, const float* scale, uint64_t* count, void* stream);
/* The same two reductions over n bf16 values (activations the block holds in bf16: O and GELU(g)). */
int qvd_amax_update_bf16(const uint16_t* x, int64_t n, float* amax, void* stream);
int qvd_clip_count_bf16(const uint16_t* x, int64_t n, const float* scale, uint64_t* count, void* stream);
int qvd_calibrated_scale(const float* amax, float* scale, int32_t n, void* stream);

/* ------------------------------------------------------------------------------------------
 * The sampler around the stack -- comfyui-wiki page, "Trim 改变了什么" training bullet (eight steps
 * at t = 999, 874, 749, 624, 500, 375, 250, 125) and "在 ComfyUI 中运行" (8 steps of res_multistep,
 * simple schedule, sigma shift 10 on video and 3 on audio).  Readings this library takes:
 *   sigma = t / 1000, rectified flow x_sigma = (1 - sigma) x0 + sigma eps; per modality the time
 *   shift sigma' = s sigma / (1 + (s - 1) sigma) (s = shift_video for rows < L_video, shift_audio for
 *   the rest) and a final sigma' = 0;
 *   the stack's output is the velocity v, so x0_hat = x - sigma' v (the latent head is the identity:
 *   the latent is the token sequence itself);
 *   res_multistep: the two-step exponential Adams-Bashforth step of the refined exponential solver in
 *   lambda = log((1 - sigma) / sigma), h = lambda_next - lambda:
 *     x_next = (sigma_next / sigma) x + alpha_next [(1 - e^-h) x0_hat + (h - 1 + e^-h) / h_prev
 *              (x0_hat - x0_hat_prev)]
 *   (first order at step 0; the last step, to sigma' = 0, returns x0_hat).
 * Coefficients are computed in double precision on the host; the state is fp32.
 * timesteps: NULL for the pages' eight (n_steps = 8: rint(999 - 999 i / n_steps)), or a host array
 * of n_steps values, strictly decreasing, in (0, 1000). */
#define QVD_SAMPLER_MAX_STEPS 64
typedef struct {
    int32_t n_steps;
    const float* timesteps;
    float shift_video, shift_audio;
    int32_t L_video;
} qvd_sampler_config;
/* The n_steps + 1 noise levels of modality 0 (video) or 1 (audio) into host doubles. */
int qvd_sampler_sigmas(const qvd_sampler_config* c, int32_t modality, double* sigmas);
/* Start from noise: eps bf16 [L][d] -> x_state fp32 [L][d] = sigma'_0 eps (per modality), and
 * x_in bf16 [L][d] = bf16(x_state), the first step's stack input.  d a multiple of 8; 16-byte aligned. */
int qvd_sampler_start(const qvd_sampler_config* c, const uint16_t* eps, int32_t L, int32_t d, float* x_state,
                      uint16_t* x_in, void* stream);
/* Step `step` (0 .. n_steps-1) after the stack has run at its timestep: v bf16 [L][d] is the stack's
 * output for the input bf16(x_state).  Updates x_state (fp32) to the next state; x0_hat (fp32 [L][d])
 * holds the previous step's estimate on entry (unused at step 0) and this step's on return; writes
 * x_in = bf16(new state), the next step's stack input.  x_in may be the same buffer as v (the stack
 * works in place).  After the last step x_state holds the final latent. */
int qvd_sampler_step(const qvd_sampler_config* c, int32_t step, const uint16_t* v, float* x_state, float* x0_hat,
                     uint16_t* x_in, int32_t L, int32_t d, void* stream);

/* ------------------------------------------------------------------------------------------
 * Matrix-core rate probe (measurement support, not part of the method): `workgroups` workgroups of
 * four waves each run `iters` iterations of four independent MFMAs of one kind, alternating two sets
 * of random operands, entirely in registers; out (device fp32 [workgroups * 256]) receives one sum per
 * thread, and clocks (NULL, or device uint64 [2 * workgroups]) each workgroup's elapsed shader-clock
 * count and constant-rate ("wall") count over its loop, whose ratio times the wall-clock rate
 * (hipDeviceAttributeWallClockRate) is the clock the loop ran at.  The caller times the launch;
 * qvd_mfma_probe_flops gives its flop count (ops for INT8).
 * Kinds: the FP8 GEMMs' 32x32x64 E4M3, the W4A4 GEMMs' 32x32x64 E2M1, INT8 16x16x64, fp16 16x16x32,
 * INT8 32x32x32, fp16 32x32x16 and E4M3 16x16x128. */
enum qvd_probe_kind {
    QVD_PROBE_FP8 = 0, QVD_PROBE_FP4 = 1, QVD_PROBE_INT8 = 2, QVD_PROBE_F16 = 3,
    QVD_PROBE_INT8_32 = 4, QVD_PROBE_F16_32 = 5, QVD_PROBE_FP8_16 = 6
};
int qvd_mfma_probe(int32_t kind, int32_t iters, int32_t workgroups, float* out, uint64_t* clocks,
                   void* stream);
double qvd_mfma_probe_flops(int32_t kind, int32_t iters, int32_t workgroups);
/* The current device's constant wall-clock rate in kHz (QVD_EHIP on a runtime error). */
int32_t qvd_wall_clock_khz(void);

/* ------------------------------------------------------------------------------------------
 * Per-kernel timing (off by default).  While enabled, each kernel launch the library makes is
 * bracketed by a pair of HIP events recorded on the launch's own stream.  qvd_timing_report waits
 * for the recorded work, writes {"<kernel key>": {"count": n, "total_ms": t}, ...} (NUL-terminated
 * JSON) into buf and clears the records.  Keys: "sparse_attn", "adaln_modulate", "adaln_project",
 * "adaln_modulate_mxfp4", "quant_fp8", "amax_bf16", "quant_int8_qk", "select_tiles", "vt_unify", "vt_from_bf16",
 * "sampler", "gemm_<fp8|mxfp4|w4a4>_<epilogue>_<M>x<N>x<K>".
 * Returns QVD_EINVAL if len is too small (the records are then lost), QVD_EHIP on event errors. */
int qvd_timing_enable(int on);
int qvd_timing_report(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* QVD_H */
