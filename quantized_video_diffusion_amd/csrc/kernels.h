// Internal launchers shared between the translation units of the library (not part of the ABI).
#pragma once

#include "common.h"

namespace qvd {

constexpr int AMAX_PARTIALS_MAX = 1024;

int launch_amax_bf16(const uint16_t* x, int64_t n, float* partials, int* np_out, hipStream_t st);
int launch_quant_fp8(const uint16_t* x, int64_t n, const float* scale_in, const float* partials,
                     int np, uint8_t* q, float* scale_out, hipStream_t st);

size_t adaln_ws_bytes(int L, int d);
int launch_modulate(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                    const float* scale_in, uint8_t* q, float* scale_out, void* ws, hipStream_t st);
// modulated LayerNorm -> MXFP4 activations: packed E2M1 [L][d/2] + E8M0 [L][d/32]
int launch_modulate_mx(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                       uint8_t* packed, uint8_t* e8m0, hipStream_t st);
int launch_adaln_project(float t, const uint16_t* basis, int dt, const uint16_t* proj,
                         const uint16_t* bias, int d, int nb, float* mod, hipStream_t st);

int64_t gemm_tiles(int M, int N);
// FP8 x FP8 (w_fmt = QVD_W_FP8, s_w per tensor) or E4M3 x MXFP4 (w_fmt = QVD_W_MXFP4, w packed
// E2M1 [N][K/2], e8 [N][K/32], s_w ignored).
int launch_gemm(const uint8_t* a, const float* s_a, const void* w, const uint8_t* e8, const float* s_w,
                int w_fmt, const float* bias, int M, int N, int K, const qvd_epilogue& epi,
                hipStream_t st);
// MXFP4 x MXFP4: a packed E2M1 [M][K/2] + a_e8 [M][K/32], w packed E2M1 [N][K/2] + w_e8 [N][K/32]
int launch_gemm_w4a4(const uint8_t* a, const uint8_t* a_e8, const uint8_t* w, const uint8_t* w_e8,
                     const float* bias, int M, int N, int K, const qvd_epilogue& epi, hipStream_t st);

// attention over fp16 V^T [H][128][ceil(L/128)*128] holding V 2^-v_exp[h] (one exponent per head)
int launch_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                          const uint16_t* vt, const int32_t* v_exp, int L, int H, const int32_t* kv_idx,
                          const int32_t* kv_cnt, int kmax, float sm_scale, uint16_t* out,
                          float* amax_partials, hipStream_t st);
// the same attention writing the E4M3 codes of bf16 O under the static scale *out_scale
int launch_sparse_attn_vt_e4m3(const int8_t* q, const float* q_scale, const int8_t* k,
                               const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int L, int H,
                               const int32_t* kv_idx, const int32_t* kv_cnt, int kmax, float sm_scale,
                               const float* out_scale, uint8_t* out_q, hipStream_t st);
// ... and the MXFP4 codes of bf16 O: packed E2M1 [L][H][64] + E8M0 [L][H][4]
int launch_sparse_attn_vt_mxfp4(const int8_t* q, const float* q_scale, const int8_t* k,
                                const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int L, int H,
                                const int32_t* kv_idx, const int32_t* kv_cnt, int kmax, float sm_scale,
                                uint8_t* out_packed, uint8_t* out_e8m0, hipStream_t st);
// V^T tiles stored with per-(head, tile) exponents tile_exp [H][T] -> one exponent per head head_exp [H]
int launch_vt_unify(uint16_t* vt, int L, int H, const int32_t* tile_exp, int32_t* head_exp, hipStream_t st);
size_t vt_bytes(int L, int H);

// sparse-tile selector: kv_idx [H][T][kept] (-1 past the count), kv_cnt [H][T]
size_t select_ws_bytes(int L, int H);
int launch_select_tiles(const int8_t* q8, const int8_t* k8, const float* k_scale, int L, int H, int kept,
                        int32_t* kv_idx, int32_t* kv_cnt, void* ws, hipStream_t st);

}  // namespace qvd
