// One DiT block forward: host-side orchestration of the kernels on one stream, with the caller's
// workspace carved into the block's intermediate tensors.
//
// The block (a pre-norm adaLN-Zero DiT block; the pages name its parts, not its wiring):
//   comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么"
//   (a transformer that denoises the video and audio latents together; six AdaLN modulation
//   vectors per block; 80% attention sparsity) and section "运行速度如何", note under the table
//   (per-tensor FP8 linear layers with the scales applied to the output; INT8 query/key).
//
//   adaln_modulate(x, shift1, scale1)             -> h (E4M3) + s_h
//   GEMM h . W_qkv^T, epilogue: bf16 Q|K|V, INT8 Q/K per (head, 128-token tile), V^T in fp16 with
//                                                    one power-of-two scale per (head, tile)
//   vt_unify                                      -> one V scale per head
//   sparse_attn                                   -> O (bf16) + per-tile max|O|
//   per-tensor FP8 of O (amax from those partials) -> O8
//   GEMM O8 . W_o^T, epilogue: x += gate1 * y      (in place)
//   adaln_modulate(x, shift2, scale2)             -> h
//   GEMM h . W_up^T, epilogue: g = bf16(GELU(y)) + per-tile max|g|
//   per-tensor FP8 of g                           -> g8
//   GEMM g8 . W_down^T, epilogue: x += gate2 * y   (in place)
// Dynamic scales never leave the device: every amax is reduced from per-workgroup partial maxima
// written by the producing kernel.  With static (calibrated) scales the two per-tensor FP8 steps
// are fused into their producers: the attention writes the E4M3 codes of O and the up-projection's
// epilogue the E4M3 codes of g, with the same arithmetic as the standalone quantizer, so neither
// bf16 tensor is written or read back.
// W4A4 (QVD_W_MXFP4_A4; the 4-bit transformer of the news.farwalk.ai FastH3 story, post 6/8, in
// OCP MX form): every GEMM input is MXFP4 with one E8M0 scale per token row and 32 channels.  The
// modulate kernel writes h in MXFP4, the attention writes the MXFP4 codes of bf16 O and the
// up-projection's epilogue those of bf16 GELU; all four GEMMs take both operands in E2M1.  Block
// scales are dynamic and local, so nothing is reduced across the tensor and no scale is passed.
#include "common.h"
#include "kernels.h"

namespace qvd {

namespace {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BlockWs {
    uint8_t* h;          // E4M3 [L][d]: modulated LN output, then the FP8 attention output
    int8_t* q8;          // [L][d]
    int8_t* k8;          // [L][d]
    uint16_t* v;         // fp16 V^T [H][128][T*128]
    int32_t* v_texp;     // [H][T] V tile exponents (QKV epilogue)
    int32_t* v_hexp;     // [H] V head exponents (vt_unify)
    uint16_t* o;         // bf16 [L][d] (dynamic scales only)
    uint16_t* g;         // bf16 [L][F] (dynamic scales only)
    uint8_t* g8;         // E4M3 [L][F] (W4A4: packed E2M1 [L][F/2])
    uint8_t* h_e8;       // W4A4: E8M0 [L][d/32] of h, then of O
    uint8_t* g_e8;       // W4A4: E8M0 [L][F/32] of g
    float* qs;           // [H][T]
    float* ks;           // [H][T]
    float* attn_part;    // [H][T]
    float* gelu_part;    // [tiles of the up GEMM]
    float* scales;       // [4]: s_h1, s_o, s_h2, s_g
    void* ln_ws;         // adaln_modulate workspace
    int32_t* sel_idx;    // selected mask [H][T][min(kmax, T)] (when the caller passes none)
    int32_t* sel_cnt;    // [H][T]
    void* sel_ws;        // selector workspace
    size_t total;
};

BlockWs carve(const qvd_block_params* p, int L, uint8_t* base) {
    const size_t Ld = (size_t)L * p->d, LF = (size_t)L * p->mlp;
    const int T = (L + 127) / 128;
    const size_t HT = (size_t)p->n_heads * T;
    BlockWs w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        uint8_t* ptr = base ? base + off : nullptr;
        off += align256(bytes);
        return ptr;
    };
    w.h = take(Ld);
    w.q8 = (int8_t*)take(Ld);
    w.k8 = (int8_t*)take(Ld);
    w.v = (uint16_t*)take(vt_bytes(L, p->n_heads));
    w.v_texp = (int32_t*)take(4 * HT);
    w.v_hexp = (int32_t*)take(4 * (size_t)p->n_heads);
    const bool a4 = p->weight_format == QVD_W_MXFP4_A4;
    // static scales or W4A4: O and g exist only as codes
    const bool stat = p->act_scale != nullptr || a4;
    w.o = (uint16_t*)take(stat ? 0 : 2 * Ld);
    w.g = (uint16_t*)take(stat ? 0 : 2 * LF);
    w.g8 = take(LF);
    w.h_e8 = take(a4 ? Ld / 32 : 0);
    w.g_e8 = take(a4 ? LF / 32 : 0);
    w.qs = (float*)take(4 * HT);
    w.ks = (float*)take(4 * HT);
    w.attn_part = (float*)take(4 * HT);
    w.gelu_part = (float*)take(4 * (size_t)gemm_tiles(L, p->mlp));
    w.scales = (float*)take(4 * 4);
    w.ln_ws = take(adaln_ws_bytes(L, p->d));
    w.sel_idx = (int32_t*)take(4 * HT * (size_t)T);
    w.sel_cnt = (int32_t*)take(4 * HT);
    w.sel_ws = take(select_ws_bytes(L, p->n_heads));
    w.total = off;
    return w;
}

int validate(const qvd_block_params* p, int L) {
    QVD_PTR(p);
    QVD_REQUIRE(p->version == QVD_ABI_VERSION, QVD_EINVAL, "qvd_block_params.version = %d, expected %d",
                p->version, QVD_ABI_VERSION);
    QVD_REQUIRE(p->head_dim == 128, QVD_ESHAPE, "block: head_dim = %d (must be 128)", p->head_dim);
    QVD_REQUIRE(p->n_heads >= 1 && p->d == 128 * p->n_heads, QVD_ESHAPE,
                "block: d = %d must equal 128 * n_heads (n_heads = %d)", p->d, p->n_heads);
    QVD_REQUIRE(p->d <= 4096, QVD_ESHAPE, "block: d = %d (at most 4096)", p->d);
    QVD_REQUIRE(p->mlp >= 128 && p->mlp % 256 == 0, QVD_ESHAPE,
                "block: mlp = %d (positive multiple of 256)", p->mlp);
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "block: L = %d", L);
    // the GEMM operand and V^T DMAs address their buffers with 32-bit offsets
    const double widest = (double)(p->mlp > p->d ? p->mlp : p->d);
    QVD_REQUIRE((double)L * widest < 4294967296.0 && 2.0 * p->d * 128.0 * ((L + 127) / 128) < 4294967296.0,
                QVD_ESHAPE, "block: L = %d too large (every GEMM input and V^T must stay below 4 GiB)", L);
    QVD_REQUIRE(p->weight_format == QVD_W_FP8 || p->weight_format == QVD_W_MXFP4 ||
                    p->weight_format == QVD_W_MXFP4_A4,
                QVD_EINVAL, "block: weight_format = %d", p->weight_format);
    QVD_REQUIRE(p->ln_eps >= 0.0f, QVD_EINVAL, "block: ln_eps < 0");
    QVD_PTR(p->w_qkv);
    QVD_PTR(p->w_o);
    QVD_PTR(p->w_up);
    QVD_PTR(p->w_down);
    QVD_ALIGN(p->w_qkv);
    QVD_ALIGN(p->w_o);
    QVD_ALIGN(p->w_up);
    QVD_ALIGN(p->w_down);
    if (p->weight_format == QVD_W_FP8) {
        QVD_PTR(p->s_qkv);
        QVD_PTR(p->s_o);
        QVD_PTR(p->s_up);
        QVD_PTR(p->s_down);
    } else {
        QVD_PTR(p->e8m0_qkv);
        QVD_PTR(p->e8m0_o);
        QVD_PTR(p->e8m0_up);
        QVD_PTR(p->e8m0_down);
    }
    const float* b[4] = {p->b_qkv, p->b_o, p->b_up, p->b_down};
    for (int i = 0; i < 4; ++i)
        if (b[i]) QVD_ALIGN(b[i]);
    return QVD_OK;
}

}  // namespace

}  // namespace qvd

using namespace qvd;

extern "C" {

size_t qvd_block_ws_bytes(const qvd_block_params* p, int32_t L) {
    if (!p || L < 0 || p->d <= 0 || p->mlp <= 0 || p->n_heads <= 0) return 0;
    return carve(p, L, nullptr).total;
}

}  // extern "C"

namespace {

// The block, ending after stage `stop` (QVD_STAGE_*; QVD_STAGE_ALL runs it whole).  Every partial run
// executes exactly the kernels and arguments of the whole block up to that stage.
int block_forward(const char* fn, const qvd_block_params* p, const float* mod, uint16_t* x, int32_t L,
                  const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, void* ws, size_t ws_bytes,
                  int stop, hipStream_t st) {
    int s = validate(p, L);
    if (s) return s;
    if (L == 0) return QVD_OK;
    QVD_PTR(mod);
    QVD_PTR(x);
    const bool select = kv_idx == nullptr && kv_cnt == nullptr;   // the block chooses its mask
    if (!select) {
        QVD_PTR(kv_idx);
        QVD_PTR(kv_cnt);
    }
    QVD_PTR(ws);
    QVD_ALIGN(mod);
    QVD_ALIGN(x);
    QVD_ALIGN(ws);
    QVD_REQUIRE(kmax >= 1 && kmax <= 1024, QVD_ESHAPE, "%s: kmax = %d (1 .. 1024)", fn, kmax);
    QVD_REQUIRE(!select || L <= 131072, QVD_ESHAPE,
                "%s: L = %d; the block selects its mask for L <= 131,072 only", fn, L);
    const size_t need = carve(p, L, nullptr).total;
    QVD_REQUIRE(ws_bytes >= need, QVD_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    QVD_DEVICE_OK();

    const BlockWs w = carve(p, L, (uint8_t*)ws);
    const int d = p->d, F = p->mlp, H = p->n_heads;
    const int T = (L + 127) / 128;
    const int fmt = p->weight_format;
    const float* act = p->act_scale;           // NULL: dynamic
    const float* shift_scale_gate = mod;       // [6][d]
    const float sm_scale = 0.08838834764831845f;   // 1/sqrt(128)
    // with no mask given, the selector picks min(kmax, T) tiles per row from the block's own INT8 Q/K
    // (after the QKV GEMM) into the workspace; its row length is then the attention's kmax
    if (select) kmax = kmax < T ? kmax : T;
    auto select_mask = [&]() -> int {
        if (!select) return QVD_OK;
        kv_idx = w.sel_idx;
        kv_cnt = w.sel_cnt;
        return launch_select_tiles(w.q8, w.k8, w.ks, L, H, kmax, w.sel_idx, w.sel_cnt, w.sel_ws, st);
    };
    if (fmt == QVD_W_MXFP4_A4) {
        s = launch_modulate_mx(x, L, d, mod, 0, p->ln_eps, w.h, w.h_e8, st);
        if (s || stop <= QVD_STAGE_MODULATE1) return s;
        qvd_epilogue e{};
        e.mode = QVD_EPI_QKV;
        e.n_heads = H;
        e.q8 = w.q8;
        e.k8 = w.k8;
        e.v = w.v;
        e.q_scale = w.qs;
        e.k_scale = w.ks;
        e.v_exp = w.v_texp;
        s = launch_gemm_w4a4(w.h, w.h_e8, (const uint8_t*)p->w_qkv, p->e8m0_qkv, p->b_qkv, L, 3 * d, d, e, st);
        if (s || stop <= QVD_STAGE_QKV) return s;
        s = launch_vt_unify(w.v, L, H, w.v_texp, w.v_hexp, st);
        if (s || stop <= QVD_STAGE_VT) return s;
        s = select_mask();
        if (s) return s;
        s = launch_sparse_attn_vt_mxfp4(w.q8, w.qs, w.k8, w.ks, w.v, w.v_hexp, L, H, kv_idx, kv_cnt, kmax,
                                        sm_scale, w.h, w.h_e8, st);
        if (s || stop <= QVD_STAGE_OQUANT) return s;
        e = qvd_epilogue{};
        e.mode = QVD_EPI_RESID_GATE;
        e.out_bf16 = x;
        e.resid = x;
        e.gate = shift_scale_gate + 2 * d;
        s = launch_gemm_w4a4(w.h, w.h_e8, (const uint8_t*)p->w_o, p->e8m0_o, p->b_o, L, d, d, e, st);
        if (s || stop <= QVD_STAGE_OPROJ) return s;
        s = launch_modulate_mx(x, L, d, mod, 1, p->ln_eps, w.h, w.h_e8, st);
        if (s || stop <= QVD_STAGE_MODULATE2) return s;
        e = qvd_epilogue{};
        e.mode = QVD_EPI_GELU_MXFP4;
        e.out_e2m1 = w.g8;
        e.out_e8m0 = w.g_e8;
        s = launch_gemm_w4a4(w.h, w.h_e8, (const uint8_t*)p->w_up, p->e8m0_up, p->b_up, L, F, d, e, st);
        if (s || stop <= QVD_STAGE_GQUANT) return s;
        e = qvd_epilogue{};
        e.mode = QVD_EPI_RESID_GATE;
        e.out_bf16 = x;
        e.resid = x;
        e.gate = shift_scale_gate + 5 * d;
        return launch_gemm_w4a4(w.g8, w.g_e8, (const uint8_t*)p->w_down, p->e8m0_down, p->b_down, L, d, F, e,
                                st);
    }

    // attention branch
    s = launch_modulate(x, L, d, mod, 0, p->ln_eps, act ? act + 0 : nullptr, w.h, w.scales + 0, w.ln_ws, st);
    if (s || stop <= QVD_STAGE_MODULATE1) return s;
    qvd_epilogue e{};
    e.mode = QVD_EPI_QKV;
    e.n_heads = H;
    e.q8 = w.q8;
    e.k8 = w.k8;
    e.v = w.v;
    e.q_scale = w.qs;
    e.k_scale = w.ks;
    e.v_exp = w.v_texp;
    s = launch_gemm(w.h, w.scales + 0, p->w_qkv, p->e8m0_qkv, p->s_qkv, fmt, p->b_qkv, L, 3 * d, d, e, st);
    if (s || stop <= QVD_STAGE_QKV) return s;
    s = launch_vt_unify(w.v, L, H, w.v_texp, w.v_hexp, st);
    if (s || stop <= QVD_STAGE_VT) return s;
    s = select_mask();
    if (s) return s;
    if (act) {
        s = launch_sparse_attn_vt_e4m3(w.q8, w.qs, w.k8, w.ks, w.v, w.v_hexp, L, H, kv_idx, kv_cnt, kmax,
                                       sm_scale, act + 1, w.h, st);
    } else {
        s = launch_sparse_attn_vt(w.q8, w.qs, w.k8, w.ks, w.v, w.v_hexp, L, H, kv_idx, kv_cnt, kmax, sm_scale,
                                  w.o, w.attn_part, st);
        if (s || stop <= QVD_STAGE_ATTN) return s;
        s = launch_quant_fp8(w.o, (int64_t)L * d, nullptr, w.attn_part, H * T, w.h, w.scales + 1, st);
    }
    if (s || stop <= QVD_STAGE_OQUANT) return s;
    e = qvd_epilogue{};
    e.mode = QVD_EPI_RESID_GATE;
    e.out_bf16 = x;
    e.resid = x;
    e.gate = shift_scale_gate + 2 * d;
    s = launch_gemm(w.h, act ? act + 1 : w.scales + 1, p->w_o, p->e8m0_o, p->s_o, fmt, p->b_o, L, d, d, e,
                    st);
    if (s || stop <= QVD_STAGE_OPROJ) return s;

    // MLP branch
    s = launch_modulate(x, L, d, mod, 1, p->ln_eps, act ? act + 2 : nullptr, w.h, w.scales + 2, w.ln_ws, st);
    if (s || stop <= QVD_STAGE_MODULATE2) return s;
    e = qvd_epilogue{};
    if (act) {
        e.mode = QVD_EPI_GELU_E4M3;
        e.out_e4m3 = w.g8;
        e.out_scale = act + 3;
    } else {
        e.mode = QVD_EPI_GELU;
        e.out_bf16 = w.g;
        e.amax_partials = w.gelu_part;
    }
    s = launch_gemm(w.h, w.scales + 2, p->w_up, p->e8m0_up, p->s_up, fmt, p->b_up, L, F, d, e, st);
    if (s || stop <= QVD_STAGE_UP) return s;
    if (!act) {
        s = launch_quant_fp8(w.g, (int64_t)L * F, nullptr, w.gelu_part, (int)gemm_tiles(L, F), w.g8,
                             w.scales + 3, st);
        if (s) return s;
    }
    if (stop <= QVD_STAGE_GQUANT) return QVD_OK;
    e = qvd_epilogue{};
    e.mode = QVD_EPI_RESID_GATE;
    e.out_bf16 = x;
    e.resid = x;
    e.gate = shift_scale_gate + 5 * d;
    return launch_gemm(w.g8, act ? act + 3 : w.scales + 3, p->w_down, p->e8m0_down, p->s_down, fmt,
                       p->b_down, L, d, F, e, st);
}

}  // namespace

extern "C" {

int dit_block_forward(const qvd_block_params* p, const float* mod, uint16_t* x, int32_t L,
                      const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, void* ws,
                      size_t ws_bytes, void* stream) {
    return block_forward("dit_block_forward", p, mod, x, L, kv_idx, kv_cnt, kmax, ws, ws_bytes,
                         QVD_STAGE_ALL, (hipStream_t)stream);
}

int qvd_block_forward_until(const qvd_block_params* p, const float* mod, uint16_t* x, int32_t L,
                            const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, int32_t stage,
                            void* ws, size_t ws_bytes, void* stream) {
    QVD_REQUIRE(stage >= QVD_STAGE_MODULATE1 && stage <= QVD_STAGE_ALL, QVD_EINVAL,
                "qvd_block_forward_until: stage = %d", stage);
    return block_forward("qvd_block_forward_until", p, mod, x, L, kv_idx, kv_cnt, kmax, ws, ws_bytes, stage,
                         (hipStream_t)stream);
}

int qvd_block_ws_layout(const qvd_block_params* p, int32_t L, int64_t* offsets) {
    QVD_PTR(p);
    QVD_PTR(offsets);
    QVD_REQUIRE(L >= 0 && p->d > 0 && p->mlp > 0 && p->n_heads > 0, QVD_ESHAPE, "qvd_block_ws_layout: shape");
    // offsets from a carve at a stand-in base address (carve gives NULL pointers for a NULL base)
    uint8_t* base = reinterpret_cast<uint8_t*>(static_cast<uintptr_t>(0x100));
    const BlockWs b = carve(p, L, base);
    auto off = [&](const void* ptr) { return (int64_t)(static_cast<const uint8_t*>(ptr) - base); };
    offsets[QVD_WS_H] = off(b.h);
    offsets[QVD_WS_Q8] = off(b.q8);
    offsets[QVD_WS_K8] = off(b.k8);
    offsets[QVD_WS_VT] = off(b.v);
    offsets[QVD_WS_VT_TILE_EXP] = off(b.v_texp);
    offsets[QVD_WS_VT_HEAD_EXP] = off(b.v_hexp);
    offsets[QVD_WS_O] = off(b.o);
    offsets[QVD_WS_G] = off(b.g);
    offsets[QVD_WS_G8] = off(b.g8);
    offsets[QVD_WS_H_E8M0] = off(b.h_e8);
    offsets[QVD_WS_G_E8M0] = off(b.g_e8);
    offsets[QVD_WS_Q_SCALE] = off(b.qs);
    offsets[QVD_WS_K_SCALE] = off(b.ks);
    offsets[QVD_WS_SCALES] = off(b.scales);
    offsets[QVD_WS_SEL_IDX] = off(b.sel_idx);
    offsets[QVD_WS_SEL_CNT] = off(b.sel_cnt);
    return QVD_OK;
}

}  // extern "C"
