// Host-side driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the library's C ABI
// (test infrastructure).  Every call below either fails argument validation -- fake, never dereferenced
// device pointers -- or is pure host code (sizes, layouts, the sampler schedule), so it runs without a
// GPU; the sanitizers watch the validation and error-reporting code itself.  Exit status 0 and no
// sanitizer report means clean.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <cstdint>

#include "qvd.h"

static int g_failed = 0;

#define EXPECT(call, want)                                                                         \
    do {                                                                                           \
        const int got_ = (call);                                                                   \
        if (got_ != (want)) {                                                                      \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, \
                         (int)(want), qvd_last_error());                                           \
            ++g_failed;                                                                            \
        }                                                                                          \
    } while (0)

#define EXPECT_TRUE(cond)                                                                          \
    do {                                                                                           \
        if (!(cond)) {                                                                             \
            std::fprintf(stderr, "line %d: %s is false\n", __LINE__, #cond);                       \
            ++g_failed;                                                                            \
        }                                                                                          \
    } while (0)

template <class T>
static T* fake(uintptr_t a = 0x10000) { return reinterpret_cast<T*>(a); }

int main() {
    void* st = nullptr;
    uint16_t* fb = fake<uint16_t>();
    uint8_t* fu = fake<uint8_t>();
    int8_t* fi8 = fake<int8_t>();
    float* ff = fake<float>();
    int32_t* fi = fake<int32_t>();
    uint16_t* mis = fake<uint16_t>(0x10001);

    EXPECT(qvd_abi_version(), QVD_ABI_VERSION);
    // device check: no GPU here -> the HIP error maps to QVD_EHIP (a GPU host -> QVD_OK)
    {
        const int s = qvd_init();
        EXPECT_TRUE(s == QVD_EHIP || s == QVD_OK);
        if (s == QVD_EHIP) EXPECT_TRUE(std::strstr(qvd_last_error(), "hipGetDevice") != nullptr);
    }
    EXPECT(qvd_inject_launch_failure(-2), QVD_EINVAL);
    EXPECT(qvd_inject_launch_failure(-1), QVD_OK);

    // quantizers
    EXPECT(quant_fp8_per_tensor(fb, -1, nullptr, fu, ff, fu, 4096, st), QVD_ESHAPE);
    EXPECT(quant_fp8_per_tensor(fb, 16, nullptr, fu, nullptr, fu, 4096, st), QVD_EINVAL);
    EXPECT_TRUE(std::strstr(qvd_last_error(), "scale_out") != nullptr);
    EXPECT(quant_fp8_per_tensor(mis, 16, nullptr, fu, ff, fu, 4096, st), QVD_EALIGN);
    EXPECT(quant_fp8_per_tensor(fb, 16, nullptr, fu, ff, fu, 16, st), QVD_EWORKSPACE);
    EXPECT_TRUE(qvd_quant_ws_bytes(10) >= 4096);
    EXPECT(quant_int8_qk(fb, 10, 2, 64, 128, 256, fi8, ff, st), QVD_ESHAPE);
    EXPECT(quant_int8_qk(fb, 10, 2, 128, 128, 100, fi8, ff, st), QVD_ESHAPE);
    EXPECT(quant_int8_qk(nullptr, 10, 2, 128, 128, 256, fi8, ff, st), QVD_EINVAL);
    EXPECT(quant_int8_qk(fb, 0, 2, 128, 128, 256, nullptr, nullptr, st), QVD_OK);
    EXPECT(qvd_quant_mxfp4(fb, 4, 33, fu, fu, st), QVD_ESHAPE);
    EXPECT(qvd_amax_update(ff, -1, ff, st), QVD_ESHAPE);
    EXPECT(qvd_clip_count(ff, 5, nullptr, fake<uint64_t>(), st), QVD_EINVAL);
    EXPECT(qvd_amax_update_bf16(fb, -1, ff, st), QVD_ESHAPE);
    EXPECT(qvd_clip_count_bf16(fb, 5, ff, nullptr, st), QVD_EINVAL);
    EXPECT(qvd_calibrated_scale(nullptr, ff, 4, st), QVD_EINVAL);
    EXPECT(qvd_calibrated_scale(ff, ff, -1, st), QVD_ESHAPE);

    // AdaLN
    EXPECT(qvd_adaln_project(1.0f, fb, 7, fb, nullptr, 256, ff, st), QVD_ESHAPE);
    EXPECT(qvd_adaln_project(1.0f, fb, 256, fb, nullptr, 200, ff, st), QVD_ESHAPE);
    EXPECT(qvd_adaln_project_stack(1.0f, fb, 256, fb, nullptr, 256, 0, ff, st), QVD_ESHAPE);
    EXPECT(adaln_modulate(fb, 4, 256, ff, 2, 1e-6f, nullptr, fu, ff, fu, 1 << 20, st), QVD_EINVAL);
    EXPECT(adaln_modulate(fb, 4, 8192, ff, 0, 1e-6f, nullptr, fu, ff, fu, 1 << 20, st), QVD_ESHAPE);
    EXPECT(adaln_modulate(fb, 4, 256, ff, 0, 1e-6f, nullptr, fu, ff, fu, 8, st), QVD_EWORKSPACE);
    EXPECT(adaln_modulate_mxfp4(fb, 4, 200, ff, 0, 1e-6f, fu, fu, st), QVD_ESHAPE);
    EXPECT(adaln_modulate_mxfp4(fb, 4, 256, ff, 0, 1e-6f, fu, nullptr, st), QVD_EINVAL);
    EXPECT(adaln_layernorm_modulate_f32(fb, 4, 256, ff, 3, 1e-6f, ff, st), QVD_EINVAL);
    EXPECT(adaln_modulate_noalloc(fb, 4, 200, ff, 0, 1e-6f, nullptr, fu, ff, st), QVD_ESHAPE);

    // attention
    const size_t big = size_t(1) << 30;
    EXPECT(sparse_attn(fi8, ff, fi8, ff, fb, 300, 2, 64, fi, fi, 3, 0.1f, fb, nullptr, fu, big, st), QVD_ESHAPE);
    EXPECT(sparse_attn(fi8, ff, fi8, ff, fb, 300, 2, 128, fi, fi, 0, 0.1f, fb, nullptr, fu, big, st), QVD_ESHAPE);
    EXPECT(sparse_attn(fi8, ff, fi8, ff, fb, 300, 2, 128, nullptr, fi, 3, 0.1f, fb, nullptr, fu, big, st), QVD_EINVAL);
    EXPECT(sparse_attn(fi8, ff, fi8, ff, fb, 300, 2, 128, fi, fi, 3, 0.1f, fb, nullptr, fu, 16, st), QVD_EWORKSPACE);
    EXPECT(sparse_attn(fi8, ff, fi8, ff, fb, 0, 2, 128, nullptr, nullptr, 3, 0.1f, nullptr, nullptr, nullptr, 0, st), QVD_OK);
    EXPECT_TRUE(qvd_sparse_attn_ws_bytes(300, 2) == 2u * 128 * 384 * 2 + 256 + 8);
    EXPECT(qvd_sparse_attn_vt(fi8, ff, fi8, ff, mis, fi, 300, 2, fi, fi, 3, 0.1f, fb, nullptr, st), QVD_EALIGN);
    EXPECT(qvd_sparse_attn_vt(fi8, ff, fi8, ff, fb, nullptr, 300, 2, fi, fi, 3, 0.1f, fb, nullptr, st), QVD_EINVAL);
    EXPECT(qvd_sparse_attn_vt_e4m3(fi8, ff, fi8, ff, fb, fi, 300, 2, fi, fi, 3, 0.1f, nullptr, fu, st), QVD_EINVAL);
    EXPECT(qvd_sparse_attn_vt_mxfp4(fi8, ff, fi8, ff, fb, fi, 300, 2, fi, fi, 3, 0.1f, fu, nullptr, st), QVD_EINVAL);
    EXPECT(qvd_vt_unify(fb, 300, 0, fi, fi, st), QVD_ESHAPE);
    EXPECT(qvd_vt_unify(fb, 300, 2, nullptr, fi, st), QVD_EINVAL);
    EXPECT(qvd_vt_from_bf16(fb, 300, 2, fb, nullptr, st), QVD_EINVAL);
    EXPECT(qvd_vt_from_bf16(fb, 0, 2, nullptr, nullptr, st), QVD_OK);
    EXPECT(qvd_select_tiles(fi8, fi8, ff, 300, 2, 0, fi, fi, fu, big, st), QVD_ESHAPE);
    EXPECT(qvd_select_tiles(fi8, fi8, ff, 300, 2, 4, fi, nullptr, fu, big, st), QVD_EINVAL);
    EXPECT(qvd_select_tiles(fi8, fi8, ff, 300, 2, 4, fi, fi, fu, 16, st), QVD_EWORKSPACE);
    EXPECT(qvd_qk_int32_tile(fi8, fi8, 300, 2, 2, 0, 0, fi, st), QVD_EINVAL);

    // GEMMs
    qvd_epilogue e;
    std::memset(&e, 0, sizeof(e));
    e.mode = QVD_EPI_F32;
    EXPECT(qvd_gemm_fp8(fu, ff, fu, ff, nullptr, 10, 100, 128, &e, st), QVD_ESHAPE);
    EXPECT(qvd_gemm_fp8(fu, ff, fu, ff, nullptr, 10, 128, 128, &e, st), QVD_EINVAL);
    e.mode = 9;
    e.out_f32 = ff;
    EXPECT(qvd_gemm_fp8(fu, ff, fu, ff, nullptr, 10, 128, 128, &e, st), QVD_EINVAL);
    EXPECT(qvd_gemm_fp8(fu, ff, fu, ff, nullptr, 10, 128, 128, nullptr, st), QVD_EINVAL);
    e.mode = QVD_EPI_QKV;
    e.n_heads = 2;
    EXPECT(qvd_gemm_fp8(fu, ff, fu, ff, nullptr, 10, 512, 128, &e, st), QVD_ESHAPE);
    EXPECT_TRUE(qvd_gemm_tiles(33784, 8064) == 132 * 32);
    e.mode = QVD_EPI_F32;
    EXPECT(qvd_gemm_mxfp4(fu, ff, fu, nullptr, nullptr, 10, 128, 128, &e, st), QVD_EINVAL);
    EXPECT(qvd_gemm_mxfp4_w4a4(fu, fu, fu, fu, nullptr, 10, 128, 96, &e, st), QVD_ESHAPE);
    EXPECT(qvd_gemm_mxfp4_w4a4(fu, fake<uint8_t>(0x10002), fu, fu, nullptr, 10, 128, 128, &e, st), QVD_EALIGN);

    // block
    qvd_block_params p;
    std::memset(&p, 0, sizeof(p));
    p.version = 99;
    EXPECT(dit_block_forward(&p, ff, fb, 10, fi, fi, 1, fu, 1, st), QVD_EINVAL);
    p.version = QVD_ABI_VERSION;
    p.d = 256; p.n_heads = 2; p.head_dim = 128; p.mlp = 1024;
    p.w_qkv = p.w_o = p.w_up = p.w_down = fu;
    p.s_qkv = p.s_o = p.s_up = p.s_down = ff;
    const size_t ws = qvd_block_ws_bytes(&p, 256);
    EXPECT_TRUE(ws > 0);
    EXPECT(dit_block_forward(&p, ff, fb, 256, fi, fi, 2, fu, 16, st), QVD_EWORKSPACE);
    EXPECT(qvd_block_forward_until(&p, ff, fb, 256, fi, fi, 2, 0, fu, ws, st), QVD_EINVAL);
    EXPECT(qvd_block_forward_until(&p, ff, fb, 256, fi, fi, 2, 11, fu, ws, st), QVD_EINVAL);
    int64_t offs[QVD_WS_SLOT_COUNT];
    EXPECT(qvd_block_ws_layout(&p, 256, offs), QVD_OK);
    for (int i = 0; i < QVD_WS_SLOT_COUNT; ++i) EXPECT_TRUE(offs[i] >= 0 && (size_t)offs[i] <= ws);
    p.weight_format = 3;
    EXPECT(dit_block_forward(&p, ff, fb, 256, fi, fi, 2, fu, ws, st), QVD_EINVAL);
    p.weight_format = QVD_W_FP8;
    p.d = 300;
    EXPECT(dit_block_forward(&p, ff, fb, 256, fi, fi, 2, fu, ws, st), QVD_ESHAPE);

    // sampler schedule (host arithmetic) and its validation
    qvd_sampler_config c;
    std::memset(&c, 0, sizeof(c));
    c.n_steps = 8;
    c.shift_video = 10.0f;
    c.shift_audio = 3.0f;
    c.L_video = 100;
    double sg[QVD_SAMPLER_MAX_STEPS + 1];
    for (int m = 0; m < 2; ++m) {
        EXPECT(qvd_sampler_sigmas(&c, m, sg), QVD_OK);
        for (int i = 0; i < 8; ++i) EXPECT_TRUE(sg[i] > sg[i + 1] && sg[i] < 1.0);
        EXPECT_TRUE(sg[8] == 0.0);
    }
    c.n_steps = QVD_SAMPLER_MAX_STEPS;
    EXPECT(qvd_sampler_sigmas(&c, 0, sg), QVD_OK);
    c.n_steps = QVD_SAMPLER_MAX_STEPS + 1;
    EXPECT(qvd_sampler_sigmas(&c, 0, sg), QVD_EINVAL);
    c.n_steps = 8;
    EXPECT(qvd_sampler_sigmas(&c, 2, sg), QVD_EINVAL);
    const float bad_ts[3] = {900.0f, 950.0f, 100.0f};    // not decreasing
    c.n_steps = 3;
    c.timesteps = bad_ts;
    EXPECT(qvd_sampler_sigmas(&c, 0, sg), QVD_EINVAL);
    c.timesteps = nullptr;
    c.n_steps = 8;
    EXPECT(qvd_sampler_start(&c, fb, 10, 12, ff, fb, st), QVD_ESHAPE);
    EXPECT(qvd_sampler_step(&c, 8, fb, ff, ff, fb, 10, 16, st), QVD_EINVAL);

    // timing report into a too-small buffer
    char tiny[2];
    EXPECT(qvd_timing_report(tiny, sizeof(tiny)), QVD_EINVAL);
    EXPECT_TRUE(qvd_mfma_probe_flops(0, 10, 10) > 0.0 && qvd_mfma_probe_flops(99, 10, 10) == 0.0);

    if (g_failed) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failed);
        return 1;
    }
    std::printf("validation driver: all checks passed\n");
    return 0;
}
