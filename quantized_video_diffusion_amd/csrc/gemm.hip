// FP8 (E4M3) GEMM on the gfx950 matrix cores with the per-tensor output scale fused into the
// epilogue, and its E4M3 x MXFP4 variant.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3", section "运行速度如何", note
// under the table: the FP8 path computes each linear layer as one matmul of per-tensor-scaled FP8
// operands and applies the scales to the matmul output in the same kernel, instead of per-token /
// per-channel FP8 scaling.  The 4-bit weights stand in for the pages' NVFP4 layers (news.farwalk.ai
// FastH3 story, post 6/8) in the OCP MX form gfx950 executes natively.
//
// Design (gfx950): C^T tiles are computed as W . A^T with v_mfma_f32_16x16x128_f8f6f4, so each lane
// ends up holding four consecutive output columns of one token row -- the shape every epilogue
// wants (8-byte bf16 stores, per-column bias/gate vectors, per-head INT8 quantization).
//   workgroup tile 256 (tokens) x 256 (outputs) x 128 (K), four waves of 128 x 128;
//   both operands K-contiguous, staged through LDS (double buffered, 16-byte chunks XOR-swizzled by
//   row so the 16-row MFMA fragment reads are bank-conflict free);
//   tile order: contiguous tile ranges per XCD (workgroup b runs on XCD b % 8) and groups of 8 token
//   tiles sweeping the output tiles, so an XCD's L2 holds the operands its tiles share.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr int BM = 256, BN = 256, BK = 128;

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* w;
    const uint8_t* e8;
    const float* s_a;
    const float* s_w;
    const float* bias;
    int M, N, K;
    int tiles_m, tiles_n;
    qvd_epilogue epi;
};

int64_t gemm_tiles(int M, int N) {
    return (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
}

QVD_DEV void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    const int xcd = pid & 7, local = pid >> 3;
    const int per = T >> 3, rem = T & 7;
    const int id = xcd * per + (xcd < rem ? xcd : rem) + local;
    constexpr int GM = 8;
    const int group_size = GM * tiles_n;
    const int grp = id / group_size;
    const int first_m = grp * GM;
    const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int in = id - grp * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

QVD_DEV float gelu_erf(float y) { return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f)); }

// 32-byte MFMA fragment of row r (16-byte chunks 2g and 2g+1 of a 128-byte, XOR-swizzled row)
QVD_DEV v8i frag_fp8(const uint8_t* tile, int r, int g) {
    const int p0 = (2 * g) ^ (r & 7);
    const v4i lo = *reinterpret_cast<const v4i*>(tile + r * 128 + (p0 << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + r * 128 + ((p0 ^ 1) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// FP8 fragment that pairs with an FP4 fragment in the mixed-format MFMA: for 16x16x128 with an E2M1
// operand, lane group g's 32 FP4 elements meet the FP8 bytes of 16-byte chunks g and g + 4 of the
// other operand (measured on gfx950 with identity operands), so the FP8 side gathers those chunks
// and every 32-element E2M1 block keeps its own E8M0 scale.
QVD_DEV v8i frag_fp8_for_fp4(const uint8_t* tile, int r, int g) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + r * 128 + ((g ^ (r & 7)) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + r * 128 + (((g + 4) ^ (r & 7)) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 16-byte FP4 fragment (32 elements) of row r of a 64-byte row; chunks swizzled by (r >> 2) & 3
QVD_DEV v8i frag_fp4(const uint8_t* tile, int r, int g) {
    const int p = g ^ ((r >> 2) & 3);
    const v4i v = *reinterpret_cast<const v4i*>(tile + r * 64 + (p << 4));
    const v4i z = {0, 0, 0, 0};
    return __builtin_shufflevector(v, z, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int WFMT>
struct TileCfg {
    static constexpr int W_BYTES = WFMT == QVD_W_MXFP4 ? BN * BK / 2 : BN * BK;
    static constexpr int E_BYTES = WFMT == QVD_W_MXFP4 ? BN * 4 : 0;
    static constexpr int STAGE = BM * BK + W_BYTES + E_BYTES;
};

template <int EPI, int WFMT>
__global__ void __launch_bounds__(256, 1) k_gemm(GemmArgs g) {
    using Cfg = TileCfg<WFMT>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Cfg::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    int tm, tn;
    tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;

    // ---- global -> register staging -------------------------------------------------------------
    // A (and FP8 W): thread t moves 16-byte chunk (t & 7) of rows (t >> 3) + 32 j, j < 8.
    // MXFP4 W (64-byte rows): chunk (t & 3) of rows (t >> 2) + 64 j, j < 4; E8M0: row t, 4 bytes.
    const int ld_row = tid >> 3, ld_ch = tid & 7;
    constexpr int WJ = WFMT == QVD_W_MXFP4 ? 4 : 8;
    constexpr int WSTEP = WFMT == QVD_W_MXFP4 ? 64 : 32;
    const int wld_row = WFMT == QVD_W_MXFP4 ? (tid >> 2) : ld_row;
    const int wld_ch = WFMT == QVD_W_MXFP4 ? (tid & 3) : ld_ch;
    const int64_t w_row_bytes = WFMT == QVD_W_MXFP4 ? K / 2 : K;
    const uint8_t* a_base = g.a + ld_ch * 16;
    const uint8_t* w_base = g.w + wld_ch * 16;
    int a_off[8], w_off[WJ];          // row offsets (bytes / 16) of the clamped rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int r = m0 + ld_row + 32 * j;
        r = r < M ? r : M - 1;
        a_off[j] = r;
    }
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
        int r = n0 + wld_row + WSTEP * j;
        r = r < N ? r : N - 1;
        w_off[j] = r;
    }
    const uint8_t* e_src = nullptr;
    if (WFMT == QVD_W_MXFP4) {
        int r = n0 + tid;
        r = r < N ? r : N - 1;
        e_src = g.e8 + (int64_t)r * (K / 32);
    }

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    u32x4 ra[8], rw[WJ];
    u32 re = 0;
#define QVD_GLOAD(k0)                                                                              \
    do {                                                                                           \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) ra[j] =                                      \
            *reinterpret_cast<const u32x4*>(a_base + (int64_t)a_off[j] * K + (k0));                \
        _Pragma("unroll") for (int j = 0; j < WJ; ++j) rw[j] = *reinterpret_cast<const u32x4*>(    \
            w_base + (int64_t)w_off[j] * w_row_bytes + (WFMT == QVD_W_MXFP4 ? (k0) / 2 : (k0)));    \
        if (WFMT == QVD_W_MXFP4) re = *reinterpret_cast<const u32*>(e_src + (k0) / 32);            \
    } while (0)
#define QVD_LSTORE(buf)                                                                            \
    do {                                                                                           \
        uint8_t* As_ = smem + (buf) * Cfg::STAGE;                                                  \
        uint8_t* Ws_ = As_ + BM * BK;                                                              \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                            \
            const int r = ld_row + 32 * j;                                                         \
            *reinterpret_cast<u32x4*>(As_ + r * 128 + ((ld_ch ^ (r & 7)) << 4)) = ra[j];           \
        }                                                                                          \
        if (WFMT == QVD_W_MXFP4) {                                                                 \
            _Pragma("unroll") for (int j = 0; j < WJ; ++j) {                                       \
                const int r = wld_row + WSTEP * j;                                                 \
                *reinterpret_cast<u32x4*>(Ws_ + r * 64 + ((wld_ch ^ ((r >> 2) & 3)) << 4)) = rw[j]; \
            }                                                                                      \
            reinterpret_cast<u32*>(Ws_ + Cfg::W_BYTES)[tid] = re;                                  \
        } else {                                                                                   \
            _Pragma("unroll") for (int j = 0; j < WJ; ++j) {                                       \
                const int r = ld_row + 32 * j;                                                     \
                *reinterpret_cast<u32x4*>(Ws_ + r * 128 + ((ld_ch ^ (r & 7)) << 4)) = rw[j];       \
            }                                                                                      \
        }                                                                                          \
    } while (0)

    const int KT = K / BK;
    QVD_GLOAD(0);
    QVD_LSTORE(0);
    __syncthreads();
    const int fr = lane & 15, fg = lane >> 4;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) QVD_GLOAD((kt + 1) * BK);
        const uint8_t* As = smem + buf * Cfg::STAGE;
        const uint8_t* Ws = As + BM * BK;
        v8i bfr[8];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
            bfr[mb] = WFMT == QVD_W_MXFP4 ? frag_fp8_for_fp4(As, 128 * wm + 16 * mb + fr, fg)
                                          : frag_fp8(As, 128 * wm + 16 * mb + fr, fg);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int r = 128 * wn + 16 * nb + fr;
            if (WFMT == QVD_W_MXFP4) {
                const v8i af = frag_fp4(Ws, r, fg);
                const int sc = (int)(reinterpret_cast<const u32*>(Ws + Cfg::W_BYTES)[r] >> (8 * fg));
#pragma unroll
                for (int mb = 0; mb < 8; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af, bfr[mb], acc[nb][mb], 4, 0, 0, sc, 0, 127);
            } else {
                const v8i af = frag_fp8(Ws, r, fg);
#pragma unroll
                for (int mb = 0; mb < 8; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af, bfr[mb], acc[nb][mb], 0, 0, 0, 0, 0, 0);
            }
        }
        if (kt + 1 < KT) QVD_LSTORE(buf ^ 1);
        __syncthreads();
    }
#undef QVD_GLOAD
#undef QVD_LSTORE

    // ---- epilogue: lane holds C[m][n .. n+3], m = mrow(mb), n = ncol(nb) ----------------------------
    const float alpha = WFMT == QVD_W_MXFP4 ? *g.s_a : (*g.s_a) * (*g.s_w);
    const int mw0 = m0 + 128 * wm, nw0 = n0 + 128 * wn;
    const bool wave_live = nw0 < N && mw0 < M;
    const qvd_epilogue& ep = g.epi;

    if (EPI == QVD_EPI_GELU) {
        __shared__ float red[4];
        float amax = 0.0f;
        if (wave_live) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int n = nw0 + 16 * nb + 4 * fg;
                float4 b = g.bias ? *reinterpret_cast<const float4*>(g.bias + n)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    const int m = mw0 + 16 * mb + fr;
                    if (m < M) {
                        const v4f c = acc[nb][mb];
                        const u32 p0 = pack_bf16x2(gelu_erf(c[0] * alpha + b.x), gelu_erf(c[1] * alpha + b.y));
                        const u32 p1 = pack_bf16x2(gelu_erf(c[2] * alpha + b.z), gelu_erf(c[3] * alpha + b.w));
                        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16lo(p0)), fabsf(bf16hi(p0))),
                                                 fmaxf(fabsf(bf16lo(p1)), fabsf(bf16hi(p1)))));
                        *reinterpret_cast<uint2*>(ep.out_bf16 + (int64_t)m * N + n) = make_uint2(p0, p1);
                    }
                }
            }
        }
        if (ep.amax_partials) {
            amax = block_max_nonneg<4>(amax, red);
            if (tid == 0) ep.amax_partials[blockIdx.x] = amax;
        }
        return;
    }
    if (!wave_live) return;

    if (EPI == QVD_EPI_QKV) {
        const int dm = N / 3;
        const int part = nw0 / dm;                     // 0 Q, 1 K, 2 V
        const int head = (nw0 - part * dm) >> 7;
        const int Tm = (M + 127) >> 7;
        if (part == 2) {
            // V: bf16 rounding, then fp16 (exact for 2^-14 <= |v| <= 65504; larger saturate),
            // stored transposed as V^T[head][dim][token] with tokens M .. Lp-1 zeroed
            const int64_t Lp = (int64_t)Tm * 128;
            uint16_t* vt = ep.v + (int64_t)head * 128 * Lp;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int n = nw0 + 16 * nb + 4 * fg;
                float4 b = g.bias ? *reinterpret_cast<const float4*>(g.bias + n)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
                const int dd = 16 * nb + 4 * fg;
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    const int m = mw0 + 16 * mb + fr;
                    const v4f c = acc[nb][mb];
                    float y[4] = {c[0] * alpha + b.x, c[1] * alpha + b.y, c[2] * alpha + b.z,
                                  c[3] * alpha + b.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float vb = bf16lo(pack_bf16x2(y[r], 0.0f));
                        const float vc = fminf(fmaxf(vb, -65504.0f), 65504.0f);
                        const uint16_t h16 = m < M ? __builtin_bit_cast(uint16_t, (_Float16)vc) : (uint16_t)0;
                        vt[(int64_t)(dd + r) * Lp + m] = h16;
                    }
                }
            }
            return;
        }
        // Q or K: round to bf16, then one symmetric INT8 scale over this (128-token tile, head)
        float amax = 0.0f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int n = nw0 + 16 * nb + 4 * fg;
            float4 b = g.bias ? *reinterpret_cast<const float4*>(g.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const int m = mw0 + 16 * mb + fr;
                const v4f c = acc[nb][mb];
                const u32 p0 = pack_bf16x2(c[0] * alpha + b.x, c[1] * alpha + b.y);
                const u32 p1 = pack_bf16x2(c[2] * alpha + b.z, c[3] * alpha + b.w);
                if (m < M)
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16lo(p0)), fabsf(bf16hi(p0))),
                                             fmaxf(fabsf(bf16lo(p1)), fabsf(bf16hi(p1)))));
            }
        }
        amax = wave_max(amax);
        const float inv = amax == 0.0f ? 1.0f : __fdiv_rn(127.0f, amax);
        int8_t* dst = part == 0 ? ep.q8 : ep.k8;
        float* sdst = part == 0 ? ep.q_scale : ep.k_scale;
        if (lane == 0) sdst[head * Tm + (mw0 >> 7)] = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 127.0f);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int n = nw0 + 16 * nb + 4 * fg;
            float4 b = g.bias ? *reinterpret_cast<const float4*>(g.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const int m = mw0 + 16 * mb + fr;
                if (m < M) {
                    const v4f c = acc[nb][mb];
                    const u32 p0 = pack_bf16x2(c[0] * alpha + b.x, c[1] * alpha + b.y);
                    const u32 p1 = pack_bf16x2(c[2] * alpha + b.z, c[3] * alpha + b.w);
                    const u32 q = (u32)(int8_encode(bf16lo(p0), inv) & 0xFF) |
                                  ((u32)(int8_encode(bf16hi(p0), inv) & 0xFF) << 8) |
                                  ((u32)(int8_encode(bf16lo(p1), inv) & 0xFF) << 16) |
                                  ((u32)(int8_encode(bf16hi(p1), inv) & 0xFF) << 24);
                    *reinterpret_cast<u32*>(dst + (int64_t)m * dm + (n - part * dm)) = q;
                }
            }
        }
        return;
    }

#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int n = nw0 + 16 * nb + 4 * fg;
        float4 b = g.bias ? *reinterpret_cast<const float4*>(g.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 gt = make_float4(0.f, 0.f, 0.f, 0.f);
        if (EPI == QVD_EPI_RESID_GATE) gt = *reinterpret_cast<const float4*>(ep.gate + n);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int m = mw0 + 16 * mb + fr;
            if (m >= M) continue;
            const v4f c = acc[nb][mb];
            const float y0 = c[0] * alpha + b.x, y1 = c[1] * alpha + b.y;
            const float y2 = c[2] * alpha + b.z, y3 = c[3] * alpha + b.w;
            const int64_t off = (int64_t)m * N + n;
            if (EPI == QVD_EPI_F32) {
                *reinterpret_cast<float4*>(ep.out_f32 + off) = make_float4(y0, y1, y2, y3);
            } else if (EPI == QVD_EPI_BF16) {
                *reinterpret_cast<uint2*>(ep.out_bf16 + off) =
                    make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            } else if (EPI == QVD_EPI_RESID_GATE) {
                const uint2 xr = *reinterpret_cast<const uint2*>(ep.resid + off);
                *reinterpret_cast<uint2*>(ep.out_bf16 + off) =
                    make_uint2(pack_bf16x2(bf16lo(xr.x) + gt.x * y0, bf16hi(xr.x) + gt.y * y1),
                               pack_bf16x2(bf16lo(xr.y) + gt.z * y2, bf16hi(xr.y) + gt.w * y3));
            }
        }
    }
}

template <int WFMT>
static int launch_fmt(const GemmArgs& g, hipStream_t st) {
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), blk(256);
    switch (g.epi.mode) {
        case QVD_EPI_F32: hipLaunchKernelGGL((k_gemm<QVD_EPI_F32, WFMT>), grid, blk, 0, st, g); break;
        case QVD_EPI_BF16: hipLaunchKernelGGL((k_gemm<QVD_EPI_BF16, WFMT>), grid, blk, 0, st, g); break;
        case QVD_EPI_RESID_GATE:
            hipLaunchKernelGGL((k_gemm<QVD_EPI_RESID_GATE, WFMT>), grid, blk, 0, st, g);
            break;
        case QVD_EPI_GELU: hipLaunchKernelGGL((k_gemm<QVD_EPI_GELU, WFMT>), grid, blk, 0, st, g); break;
        case QVD_EPI_QKV: hipLaunchKernelGGL((k_gemm<QVD_EPI_QKV, WFMT>), grid, blk, 0, st, g); break;
        default: return fail(QVD_EINVAL, "gemm: epilogue mode %d", g.epi.mode);
    }
    return launch_status("gemm");
}

int launch_gemm(const uint8_t* a, const float* s_a, const void* w, const uint8_t* e8, const float* s_w,
                int w_fmt, const float* bias, int M, int N, int K, const qvd_epilogue& epi,
                hipStream_t st) {
    if (M == 0) return QVD_OK;
    GemmArgs g;
    g.a = a;
    g.w = (const uint8_t*)w;
    g.e8 = e8;
    g.s_a = s_a;
    g.s_w = s_w;
    g.bias = bias;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = (M + BM - 1) / BM;
    g.tiles_n = (N + BN - 1) / BN;
    g.epi = epi;
    static const char* epi_name[] = {"f32", "bf16", "resid_gate", "gelu", "qkv"};
    char key[96];
    snprintf(key, sizeof(key), "gemm_%s_%s_%dx%dx%d", w_fmt == QVD_W_MXFP4 ? "mxfp4" : "fp8",
             (epi.mode >= 0 && epi.mode < 5) ? epi_name[epi.mode] : "?", M, N, K);
    TimingScope ts(key, st);
    return w_fmt == QVD_W_MXFP4 ? launch_fmt<QVD_W_MXFP4>(g, st) : launch_fmt<QVD_W_FP8>(g, st);
}

}  // namespace qvd

using namespace qvd;

static int validate_gemm(const char* fn, const uint8_t* a, const float* s_a, const void* w,
                         const float* bias, int32_t M, int32_t N, int32_t K, const qvd_epilogue* epi) {
    QVD_REQUIRE(epi != nullptr, QVD_EINVAL, "%s: epi is NULL", fn);
    QVD_REQUIRE(M >= 0 && N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0, QVD_ESHAPE,
                "%s: M = %d, N = %d, K = %d (N, K: positive multiples of 128)", fn, M, N, K);
    QVD_REQUIRE(gemm_tiles(M, N) < (1ll << 31), QVD_ESHAPE, "%s: too many tiles", fn);
    QVD_REQUIRE(s_a != nullptr && w != nullptr, QVD_EINVAL, "%s: s_a or w is NULL", fn);
    QVD_REQUIRE(aligned16(w) && (!bias || aligned16(bias)), QVD_EALIGN, "%s: w/bias not 16-byte aligned", fn);
    if (M > 0) QVD_REQUIRE(a && aligned16(a), QVD_EINVAL, "%s: a is NULL or misaligned", fn);
    switch (epi->mode) {
        case QVD_EPI_F32:
            QVD_REQUIRE(epi->out_f32 && aligned16(epi->out_f32), QVD_EINVAL, "%s: out_f32 NULL/misaligned", fn);
            break;
        case QVD_EPI_BF16:
        case QVD_EPI_GELU:
            QVD_REQUIRE(epi->out_bf16 && aligned16(epi->out_bf16), QVD_EINVAL, "%s: out_bf16 NULL/misaligned", fn);
            break;
        case QVD_EPI_RESID_GATE:
            QVD_REQUIRE(epi->out_bf16 && epi->resid && epi->gate, QVD_EINVAL, "%s: out/resid/gate NULL", fn);
            QVD_REQUIRE(aligned16(epi->out_bf16) && aligned16(epi->resid) && aligned16(epi->gate),
                        QVD_EALIGN, "%s: out/resid/gate not 16-byte aligned", fn);
            break;
        case QVD_EPI_QKV:
            QVD_REQUIRE(epi->n_heads >= 1 && N == 3 * 128 * epi->n_heads, QVD_ESHAPE,
                        "%s: QKV epilogue needs N = 3*128*n_heads (N = %d, n_heads = %d)", fn, N,
                        epi->n_heads);
            QVD_REQUIRE(epi->q8 && epi->k8 && epi->v && epi->q_scale && epi->k_scale, QVD_EINVAL,
                        "%s: QKV outputs NULL", fn);
            QVD_REQUIRE(aligned16(epi->q8) && aligned16(epi->k8) && aligned16(epi->v), QVD_EALIGN,
                        "%s: QKV outputs not 16-byte aligned", fn);
            break;
        default:
            return fail(QVD_EINVAL, "%s: unknown epilogue mode %d", fn, epi->mode);
    }
    return QVD_OK;
}

extern "C" {

int64_t qvd_gemm_tiles(int32_t M, int32_t N) {
    return (M < 0 || N < 0) ? 0 : gemm_tiles(M, N);
}

int qvd_gemm_fp8(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                 const float* bias, int32_t M, int32_t N, int32_t K, const qvd_epilogue* epi,
                 void* stream) {
    int s = validate_gemm("qvd_gemm_fp8", a, s_a, w, bias, M, N, K, epi);
    if (s) return s;
    QVD_PTR(s_w);
    QVD_DEVICE_OK();
    return launch_gemm(a, s_a, w, nullptr, s_w, QVD_W_FP8, bias, M, N, K, *epi, (hipStream_t)stream);
}

int qvd_gemm_mxfp4(const uint8_t* a, const float* s_a, const uint8_t* w_packed,
                   const uint8_t* e8m0, const float* bias, int32_t M, int32_t N, int32_t K,
                   const qvd_epilogue* epi, void* stream) {
    int s = validate_gemm("qvd_gemm_mxfp4", a, s_a, w_packed, bias, M, N, K, epi);
    if (s) return s;
    QVD_PTR(e8m0);
    QVD_DEVICE_OK();
    return launch_gemm(a, s_a, w_packed, e8m0, nullptr, QVD_W_MXFP4, bias, M, N, K, *epi,
                       (hipStream_t)stream);
}

}  // extern "C"
