// FP8 (E4M3) GEMM on the gfx950 matrix cores with the per-tensor output scale fused into the
// epilogue, and its E4M3 x MXFP4 variant.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3", section "运行速度如何", note
// under the table: the FP8 path computes each linear layer as one matmul of per-tensor-scaled FP8
// operands and applies the scales to the matmul output in the same kernel, instead of per-token /
// per-channel FP8 scaling.  The 4-bit weights stand in for the pages' NVFP4 layers (news.farwalk.ai
// FastH3 story, post 6/8) in the OCP MX form gfx950 executes natively.
//
// Design (gfx950): C^T tiles are computed as W . A^T with v_mfma_scale_f32_32x32x64_f8f6f4, so each
// lane ends up holding four consecutive output columns of one token row -- the shape every epilogue
// wants (8-byte bf16 stores, per-column bias/gate vectors, per-head INT8 quantization).
//   workgroup tile 256 (tokens) x 256 (outputs), eight waves (two per SIMD) of 128 x 64 outputs;
//   K in stages of 128: both operands K-contiguous, moved HBM/L2 -> LDS by buffer_load_dwordx4 ... lds
//   into two 64 KB stage buffers (stage s+2 lands while stage s is multiplied), 16-byte chunks
//   XOR-swizzled by row so the 32-row MFMA fragment reads are bank-conflict free;
//   tile order: contiguous tile ranges per XCD (workgroup b runs on XCD b % 8) and groups of 8 token
//   tiles sweeping the output tiles, so an XCD's L2 holds the operands its tiles share.
// The E4M3 x MXFP4 and MXFP4 x MXFP4 kernels further down keep the same tiles and schedule.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr int BM = 256, BN = 256;

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* w;
    const uint8_t* e8;
    const uint8_t* a_e8;     // E8M0 scales of MXFP4 activations (W4A4), else NULL
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

// GELU(y) = y Phi(y) = max(y, 0) - |y| h, h = erfc(z) / 2, z = |y|/sqrt 2 (Phi(y) is h for y < 0 and
// 1 - h for y >= 0).  erfc in the form of the approximation of W. H. Press et al., Numerical Recipes,
// section 6.2 (function erfcc): erfc(z) / 2 = t 2^(-z^2 log2 e + P(t)), t = 1/(1 + z/2), with P a
// degree-7 polynomial refitted (minimax, gelu_erfc_fit.py beside this file) over z in [0, 9.5], past
// which the output is 0 or y in fp32: relative error 6.3e-7 of erfc, a ratio that holds in the tail too,
// where a form built on 1 - erf would lose the small values that a static E4M3 scale can still resolve.
// z enters through |y| (t = 1/(1 + |y|/(2 sqrt 2)), z^2 log2(e) = |y|^2 log2(e)/2).  |y| t < 2 sqrt 2
// always; the bound keeps GELU(+inf) = +inf (inf * 0 would make a NaN).  max(y, 0) is taken as -0 for
// y < 0, so that a negative input whose GELU underflows gives -0, the sign that y Phi(y) has (the
// MXFP4 and E4M3 codes of -0 and +0 differ).
QVD_DEV float gelu_erf(float y) {
    const float ay = fabsf(y);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.35355339059327373f, ay, 1.0f));
    float p = fmaf(-0.26331817f, t, 1.05167408f);
    p = fmaf(p, t, -1.38636225f);
    p = fmaf(p, t, 0.45005937f);
    p = fmaf(p, t, -0.0276269704f);
    p = fmaf(p, t, 0.559243484f);
    p = fmaf(p, t, 1.44212113f);
    p = fmaf(p, t, -2.82579158f);
    const float arg = fmaf(-(ay * 0.72134752044448170f), ay, p);
    const float at = fminf(ay * t, 2.8284271247461903f);
    return fmaf(-at, __builtin_amdgcn_exp2f(arg), y >= 0.0f ? y : -0.0f);
}

// Running max of |v| over the bf16 halves of packed pairs, kept as two 16-bit magnitudes: for finite
// bf16 values the order of |v| is the order of (bits & 0x7FFF) as unsigned integers, so one packed
// 16-bit max per pair does what two extractions and float maxima would.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
QVD_DEV u32 absmax_bf16x2(u32 m, u32 p) {
    return __builtin_bit_cast(u32, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                             __builtin_bit_cast(u16x2, p & 0x7FFF7FFFu)));
}

typedef __attribute__((address_space(3))) void lds_void;

// Operand DMA: buffer loads to LDS (MUBUF, raw resource over the whole 32-bit offset range; the
// launcher keeps every operand below 4 GiB), the lane's offset in a VGPR and the stage's K offset in
// the scalar offset.  Not global_load_lds: a FLAT instruction that may write LDS counts, for the
// compiler, as an LDS access that completes out of order, so with one in flight every wait on a
// fragment read becomes lgkmcnt(0), including the reads issued for the next step; a buffer load
// counts on vmcnt only.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A wait the compiler sees (lgkmcnt(0), no vmcnt or expcnt wait), once before the main loop: no scalar
// load (the kernel arguments the epilogue reads) is then in flight where the loop is entered, which
// would otherwise make the first fragment wait of every stage lgkmcnt(0), since scalar loads may
// return out of order.
QVD_DEV void lgkm_settle() { __builtin_amdgcn_s_waitcnt(0xC07F); }

QVD_DEV rsrc_t raw_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
}

// 16 (4) bytes per lane from byte offset soff + voff of the buffer at base; lane l's bytes land at slot l
QVD_DEV void dma_lds16(const void* base, uint32_t voff, uint32_t soff, void* lds_slot_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(base), (lds_void*)lds_slot_base, 16, voff, soff, 0, 0);
}
QVD_DEV void dma_lds4(const void* base, uint32_t voff, uint32_t soff, void* lds_slot_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(base), (lds_void*)lds_slot_base, 4, voff, soff, 0, 0);
}

// ---- accumulator layout ----------------------------------------------------------------------------
// The MFMAs compute C^T = W . A^T, so a lane holds runs of 4 consecutive output columns (n) of one token
// row (m).  v_mfma_f32_32x32x64 over a 128 x 64 wave tile: acc[nb][mb] (nb in 0..1, mb in 0..3, 16
// values each); value 4g + i of lane l is C[32 mb + l%32][32 nb + 8 g + 4 (l/32) + i].  The epilogue
// walks it as NCG column groups of 4 x MR row blocks of RB rows.
struct Layout32N64 {
    static constexpr int NCG = 8, MR = 4, RB = 32;
    typedef v16f Acc[2][4];
    QVD_DEV static int ncol(int cg, int lane) { return 32 * (cg >> 2) + 8 * (cg & 3) + 4 * (lane >> 5); }
    QVD_DEV static int mrow(int r, int lane) { return 32 * r + (lane & 31); }
    QVD_DEV static v4f get(const Acc& a, int cg, int r) {
        const v16f& v = a[cg >> 2][r];
        const int b = 4 * (cg & 3);
        return (v4f){v[b], v[b + 1], v[b + 2], v[b + 3]};
    }
};

QVD_DEV float4 load_bias4(const float* bias, int n) {
    return bias ? *reinterpret_cast<const float4*>(bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---- fused epilogues: y = acc * alpha + bias, then the mode's output ---------------------------------
// The wave owns the 128 x WN block at (mw0, nw0) = (m0 + 128 wm, n0 + WN wn) of a workgroup of NWV
// waves.  Results go through a 16 KB LDS region of the wave (stage), in rounds of rows, so that every
// global store is 16 bytes per lane over whole rows (bf16, fp32 and INT8 token rows; V^T head-
// dimension rows).  16-byte chunks are XOR-swizzled by row.  red: NWV floats of LDS.
QVD_DEV void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int EPI, class LY, int WN, int NWV>
QVD_DEV void gemm_epilogue(const GemmArgs& g, const typename LY::Acc& acc, float alpha, int m0, int n0,
                           int wm, int wn, float* red, uint8_t* stage) {
    static_assert(WN == 64 || WN == 128, "wave tile width");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int M = g.M, N = g.N;
    const int mw0 = m0 + 128 * wm, nw0 = n0 + WN * wn;
    const bool wave_live = nw0 < N && mw0 < M;
    const qvd_epilogue& ep = g.epi;

    // bf16 token rows of 2 WN bytes, R rows per round; RESID first brings the x rows in
    constexpr int BC = WN / 8;                           // 16-byte chunks per row
    constexpr int BR = 16384 / (2 * WN);                 // rows per round
    auto bslot = [&](int ml, int c) { return stage + ml * (2 * WN) + ((c ^ (ml & (BC - 1))) << 4); };
    auto bf16_rounds = [&](auto mode, float& amax) {
        constexpr int MODE = decltype(mode)::value;      // 0 plain, 1 GELU, 2 x += gate y
        constexpr int RPR = BR / LY::RB;
        u32 amb = 0u;                                    // MODE 1: packed |bf16| maxima
#pragma unroll
        for (int rd = 0; rd < 128 / BR; ++rd) {
            if (MODE == 2) {
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const int idx = 64 * it + lane, ml = idx / BC, c = idx % BC;
                    const int m = mw0 + BR * rd + ml;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (m < M) v = *reinterpret_cast<const u32x4*>(ep.resid + (int64_t)m * N + nw0 + 8 * c);
                    *reinterpret_cast<u32x4*>(bslot(ml, c)) = v;
                }
                lds_wait();
            }
#pragma unroll
            for (int cg = 0; cg < LY::NCG; ++cg) {
                const int nl = LY::ncol(cg, lane);
                const float4 b = load_bias4(g.bias, nw0 + nl);
                float4 gt = make_float4(0.f, 0.f, 0.f, 0.f);
                if (MODE == 2) gt = *reinterpret_cast<const float4*>(ep.gate + nw0 + nl);
#pragma unroll
                for (int rr = 0; rr < RPR; ++rr) {
                    const int r = rd * RPR + rr;
                    const int ml = LY::mrow(r, lane) - BR * rd;
                    const v4f c = LY::get(acc, cg, r);
                    float y[4] = {c[0] * alpha + b.x, c[1] * alpha + b.y, c[2] * alpha + b.z, c[3] * alpha + b.w};
                    u32x2* slot = reinterpret_cast<u32x2*>(bslot(ml, nl >> 3) + ((nl >> 2) & 1) * 8);
                    u32 p0, p1;
                    if (MODE == 2) {
                        const u32x2 xr = *slot;
                        p0 = pack_bf16x2(bf16lo(xr[0]) + gt.x * y[0], bf16hi(xr[0]) + gt.y * y[1]);
                        p1 = pack_bf16x2(bf16lo(xr[1]) + gt.z * y[2], bf16hi(xr[1]) + gt.w * y[3]);
                    } else {
                        if (MODE == 1) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) y[i] = gelu_erf(y[i]);
                        }
                        p0 = pack_bf16x2(y[0], y[1]);
                        p1 = pack_bf16x2(y[2], y[3]);
                        if (MODE == 1 && mw0 + BR * rd + ml < M) amb = absmax_bf16x2(absmax_bf16x2(amb, p0), p1);
                    }
                    *slot = (u32x2){p0, p1};
                }
            }
            lds_wait();
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int idx = 64 * it + lane, ml = idx / BC, c = idx % BC;
                const u32x4 v = *reinterpret_cast<const u32x4*>(bslot(ml, c));
                const int m = mw0 + BR * rd + ml;
                if (m < M) *reinterpret_cast<u32x4*>(ep.out_bf16 + (int64_t)m * N + nw0 + 8 * c) = v;
            }
            lds_wait();
        }
        if (MODE == 1) amax = fmaxf(amax, fmaxf(bf16lo(amb), bf16hi(amb)));
    };

    if (EPI == QVD_EPI_GELU) {
        float amax = 0.0f;
        if (wave_live) bf16_rounds(std::integral_constant<int, 1>{}, amax);
        if (ep.amax_partials) {
            amax = block_max_nonneg<NWV>(amax, red);
            if (tid == 0) ep.amax_partials[blockIdx.x] = amax;
        }
        return;
    }

    if (EPI == QVD_EPI_GELU_E4M3) {
        // GELU, bf16 rounding, then E4M3 with the static scale: the standalone static quantizer's
        // arithmetic (one fp32 product by the correctly rounded 1/s, saturating encode).  LDS: 128
        // token rows of WN codes, stored as whole 16-byte chunks of the rows.
        if (!wave_live) return;
        const float inv_s = __fdiv_rn(1.0f, *ep.out_scale);
        constexpr int QC = WN / 16;
#pragma unroll
        for (int cg = 0; cg < LY::NCG; ++cg) {
            const int nl = LY::ncol(cg, lane);
            const float4 b = load_bias4(g.bias, nw0 + nl);
#pragma unroll
            for (int r = 0; r < LY::MR; ++r) {
                const int ml = LY::mrow(r, lane);
                const v4f c = LY::get(acc, cg, r);
                const u32 p0 = pack_bf16x2(gelu_erf(c[0] * alpha + b.x), gelu_erf(c[1] * alpha + b.y));
                const u32 p1 = pack_bf16x2(gelu_erf(c[2] * alpha + b.z), gelu_erf(c[3] * alpha + b.w));
                const u32 q = e4m3_encode2(bf16lo(p0) * inv_s, bf16hi(p0) * inv_s) |
                              (e4m3_encode2(bf16lo(p1) * inv_s, bf16hi(p1) * inv_s) << 16);
                *reinterpret_cast<u32*>(stage + ml * WN + (((nl >> 4) ^ (ml & (QC - 1))) << 4) + (nl & 15)) = q;
            }
        }
        lds_wait();
#pragma unroll
        for (int it = 0; it < 2 * QC; ++it) {
            const int idx = 64 * it + lane, ml = idx / QC, c = idx % QC;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + ml * WN + ((c ^ (ml & (QC - 1))) << 4));
            const int m = mw0 + ml;
            if (m < M) *reinterpret_cast<u32x4*>(ep.out_e4m3 + (int64_t)m * N + nw0 + 16 * c) = v;
        }
        return;
    }

    if (EPI == QVD_EPI_GELU_MXFP4) {
        // GELU and bf16 rounding as in the GELU epilogue, the wave's 128 x WN bf16 block staged in LDS
        // (one round: 128 rows of 2 WN bytes), then each lane quantizes whole 32-column blocks of a
        // row with the standalone quantizer's arithmetic: 16 code bytes and one scale byte per block.
        static_assert(BR == 128, "one staging round");
        if (!wave_live) return;
        constexpr int QB = WN / 32;                      // 32-column blocks per row
#pragma unroll
        for (int cg = 0; cg < LY::NCG; ++cg) {
            const int nl = LY::ncol(cg, lane);
            const float4 b = load_bias4(g.bias, nw0 + nl);
#pragma unroll
            for (int r = 0; r < LY::MR; ++r) {
                const int ml = LY::mrow(r, lane);
                const v4f c = LY::get(acc, cg, r);
                const u32 p0 = pack_bf16x2(gelu_erf(c[0] * alpha + b.x), gelu_erf(c[1] * alpha + b.y));
                const u32 p1 = pack_bf16x2(gelu_erf(c[2] * alpha + b.z), gelu_erf(c[3] * alpha + b.w));
                *reinterpret_cast<u32x2*>(bslot(ml, nl >> 3) + ((nl >> 2) & 1) * 8) = (u32x2){p0, p1};
            }
        }
        lds_wait();
        const int Nh = N / 2, Nb = N / 32;
#pragma unroll
        for (int it = 0; it < 2 * QB; ++it) {
            const int idx = 64 * it + lane, ml = idx / QB, bk = idx % QB;
            u32 ws[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(bslot(ml, 4 * bk + q));
                ws[4 * q] = v.x; ws[4 * q + 1] = v.y; ws[4 * q + 2] = v.z; ws[4 * q + 3] = v.w;
            }
            u32 amb = 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) amb = absmax_bf16x2(amb, ws[j]);
            const int k = mx_exponent(fmaxf(bf16lo(amb), bf16hi(amb)));
            u32 o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = e2m1_encode8_bf16(ws + 4 * j, k);
            const int m = mw0 + ml;
            if (m < M) {
                *reinterpret_cast<u32x4*>(ep.out_e2m1 + (int64_t)m * Nh + (nw0 + 32 * bk) / 2) =
                    (u32x4){o[0], o[1], o[2], o[3]};
                ep.out_e8m0[(int64_t)m * Nb + nw0 / 32 + bk] = (uint8_t)(k + 127);
            }
        }
        return;
    }

    if (EPI == QVD_EPI_QKV) {
        const int dm = N / 3;
        // The V columns start at 2 dm = 256 H, a tile boundary, so a workgroup's waves are either all
        // in Q|K or all in V (the exchange barrier below is taken by all of them or by none).
        const bool v_tile = n0 >= 2 * dm;
        const int part = v_tile ? 2 : nw0 / dm;        // 0 Q, 1 K, 2 V
        const int hc = nw0 - part * dm;                // column of this wave inside its part
        const int head = hc >> 7;
        const int Tm = (M + 127) >> 7;
        if (v_tile) {
            // V: rounded to bf16, then stored in fp16, transposed as V^T[head][dim][token] with tokens
            // M .. Lp-1 zeroed, scaled by 2^-e with one exponent e per (head, 128-token tile):
            // vt_tile_exponent of the tile's max|V| (0 for the usual range, else the power of two that
            // brings the maximum into [2^14, 2^15)).  The fp16 value is the bf16 value times 2^-e
            // exactly wherever it is an fp16 normal.  The two waves of a head meet in LDS (every wave
            // of the workgroup is a V wave, so all take the barrier).  LDS: WN dimension rows of TR
            // tokens per round.
            float amax = 0.0f;
            if (wave_live) {
                u32 amb = 0u;
#pragma unroll
                for (int cg = 0; cg < LY::NCG; ++cg) {
                    const float4 b = load_bias4(g.bias, nw0 + LY::ncol(cg, lane));
#pragma unroll
                    for (int r = 0; r < LY::MR; ++r) {
                        const int m = mw0 + LY::mrow(r, lane);
                        const v4f c = LY::get(acc, cg, r);
                        const u32 p0 = pack_bf16x2(c[0] * alpha + b.x, c[1] * alpha + b.y);
                        const u32 p1 = pack_bf16x2(c[2] * alpha + b.z, c[3] * alpha + b.w);
                        if (m < M) amb = absmax_bf16x2(absmax_bf16x2(amb, p0), p1);
                    }
                }
                amax = fmaxf(bf16lo(amb), bf16hi(amb));
            }
            amax = wave_max(amax);
            if (lane == 0) red[wv] = amax;
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            amax = fmaxf(amax, red[wv ^ 2]);
            if (!wave_live) return;
            const int ve = vt_tile_exponent(amax);
            if (lane == 0 && (hc & 127) == 0) ep.v_exp[head * Tm + (mw0 >> 7)] = ve;
            constexpr int TR = 16384 / (2 * WN);
            constexpr int CT = TR / 8;
            constexpr int RPR = TR / LY::RB;
            const int64_t Lp = (int64_t)Tm * 128;
            uint16_t* vt = ep.v + ((int64_t)head * 128 + (hc & 127)) * Lp;
#pragma unroll
            for (int rd = 0; rd < 128 / TR; ++rd) {
#pragma unroll
                for (int cg = 0; cg < LY::NCG; ++cg) {
                    const int dd = LY::ncol(cg, lane);
                    const float4 b = load_bias4(g.bias, nw0 + dd);
#pragma unroll
                    for (int rr = 0; rr < RPR; ++rr) {
                        const int r = rd * RPR + rr;
                        const int ml = LY::mrow(r, lane) - TR * rd;
                        const bool ok = mw0 + TR * rd + ml < M;
                        const v4f c = LY::get(acc, cg, r);
                        const float y[4] = {c[0] * alpha + b.x, c[1] * alpha + b.y, c[2] * alpha + b.z,
                                            c[3] * alpha + b.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint16_t h16 = ok ? f16_scaled(bf16lo(pack_bf16x2(y[i], 0.0f)), ve) : (uint16_t)0;
                            const int row = dd + i;
                            *reinterpret_cast<uint16_t*>(stage + row * (2 * TR) + (((ml >> 3) ^ (row & (CT - 1))) << 4) +
                                                         (ml & 7) * 2) = h16;
                        }
                    }
                }
                lds_wait();
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const int idx = 64 * it + lane, row = idx / CT, c = idx % CT;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * (2 * TR) + ((c ^ (row & (CT - 1))) << 4));
                    *reinterpret_cast<u32x4*>(vt + (int64_t)row * Lp + mw0 + TR * rd + 8 * c) = v;
                }
                lds_wait();
            }
            return;
        }
        // Q or K: round to bf16, then one symmetric INT8 scale over this (128-token tile, head); a
        // 64-wide wave shares the head with its neighbour (wn ^ 1) and their maxima meet in LDS.
        // LDS: 128 token rows of WN codes.
        float amax = 0.0f;
        if (wave_live) {
            u32 amb = 0u;
#pragma unroll
            for (int cg = 0; cg < LY::NCG; ++cg) {
                const float4 b = load_bias4(g.bias, nw0 + LY::ncol(cg, lane));
#pragma unroll
                for (int r = 0; r < LY::MR; ++r) {
                    const int m = mw0 + LY::mrow(r, lane);
                    const v4f c = LY::get(acc, cg, r);
                    const u32 p0 = pack_bf16x2(c[0] * alpha + b.x, c[1] * alpha + b.y);
                    const u32 p1 = pack_bf16x2(c[2] * alpha + b.z, c[3] * alpha + b.w);
                    if (m < M) amb = absmax_bf16x2(absmax_bf16x2(amb, p0), p1);
                }
            }
            amax = fmaxf(bf16lo(amb), bf16hi(amb));
        }
        amax = wave_max(amax);
        if (WN == 64) {                                // every wave takes part: the barrier is shared
            if (lane == 0) red[wv] = amax;
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            amax = fmaxf(amax, red[wv ^ 2]);
        }
        if (!wave_live) return;
        const float inv = amax == 0.0f ? 1.0f : __fdiv_rn(127.0f, amax);
        int8_t* dst = part == 0 ? ep.q8 : ep.k8;
        float* sdst = part == 0 ? ep.q_scale : ep.k_scale;
        if (lane == 0 && (hc & 127) == 0) sdst[head * Tm + (mw0 >> 7)] = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 127.0f);
        constexpr int QC = WN / 16;                    // 16-byte chunks per token row
#pragma unroll
        for (int cg = 0; cg < LY::NCG; ++cg) {
            const int nl = LY::ncol(cg, lane);
            const float4 b = load_bias4(g.bias, nw0 + nl);
#pragma unroll
            for (int r = 0; r < LY::MR; ++r) {
                const int ml = LY::mrow(r, lane);
                const v4f c = LY::get(acc, cg, r);
                const u32 p0 = pack_bf16x2(c[0] * alpha + b.x, c[1] * alpha + b.y);
                const u32 p1 = pack_bf16x2(c[2] * alpha + b.z, c[3] * alpha + b.w);
                const u32 q = (u32)(int8_encode(bf16lo(p0), inv) & 0xFF) |
                              ((u32)(int8_encode(bf16hi(p0), inv) & 0xFF) << 8) |
                              ((u32)(int8_encode(bf16lo(p1), inv) & 0xFF) << 16) |
                              ((u32)(int8_encode(bf16hi(p1), inv) & 0xFF) << 24);
                *reinterpret_cast<u32*>(stage + ml * WN + (((nl >> 4) ^ (ml & (QC - 1))) << 4) + (nl & 15)) = q;
            }
        }
        lds_wait();
#pragma unroll
        for (int it = 0; it < 2 * QC; ++it) {
            const int idx = 64 * it + lane, ml = idx / QC, c = idx % QC;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + ml * WN + ((c ^ (ml & (QC - 1))) << 4));
            const int m = mw0 + ml;
            if (m < M) *reinterpret_cast<u32x4*>(dst + (int64_t)m * dm + hc + 16 * c) = v;
        }
        return;
    }

    if (!wave_live) return;
    if (EPI == QVD_EPI_BF16 || EPI == QVD_EPI_RESID_GATE) {
        float unused = 0.0f;
        bf16_rounds(std::integral_constant<int, EPI == QVD_EPI_RESID_GATE ? 2 : 0>{}, unused);
        return;
    }

    // fp32 output: token rows of 4 WN bytes
    constexpr int FC = WN / 4;
    constexpr int FR = 16384 / (4 * WN);
    constexpr int RPR = FR / LY::RB > 0 ? FR / LY::RB : 1;
#pragma unroll
    for (int rd = 0; rd < 128 / FR; ++rd) {
#pragma unroll
        for (int cg = 0; cg < LY::NCG; ++cg) {
            const int nl = LY::ncol(cg, lane);
            const float4 b = load_bias4(g.bias, nw0 + nl);
#pragma unroll
            for (int rr = 0; rr < RPR; ++rr) {
                const int r = rd * RPR + rr;
                const int ml = LY::mrow(r, lane) - FR * rd;
                const v4f c = LY::get(acc, cg, r);
                const float4 y = make_float4(c[0] * alpha + b.x, c[1] * alpha + b.y, c[2] * alpha + b.z,
                                             c[3] * alpha + b.w);
                *reinterpret_cast<float4*>(stage + ml * (4 * WN) + (((nl >> 2) ^ (ml & (FC - 1))) << 4)) = y;
            }
        }
        lds_wait();
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int idx = 64 * it + lane, ml = idx / FC, c = idx % FC;
            const float4 y = *reinterpret_cast<const float4*>(stage + ml * (4 * WN) + ((c ^ (ml & (FC - 1))) << 4));
            const int m = mw0 + FR * rd + ml;
            if (m < M) *reinterpret_cast<float4*>(ep.out_f32 + (int64_t)m * N + nw0 + 4 * c) = y;
        }
        lds_wait();
    }
}

// ================================================================================================
// E4M3 x E4M3: 256 x 256 tiles, v_mfma_f32_32x32x64_f8f6f4, eight waves (two per SIMD) of 128 x 64
// outputs each.
//
// Operands move HBM/L2 -> LDS by buffer loads to LDS in stages of 128 K (two LDS buffers of
// 64 KB): one DMA instruction fills 8 whole 128-byte rows, so every request is a full cache line.
// The MFMAs run in K-steps of 64 (half a stage) on fragments already in registers while the next
// step's 6 fragments are read from LDS.  One s_barrier per stage, at the start of the stage's second
// step: stage s+1 has landed (its first fragments are read during that step) and every wave is done
// with stage s-1, whose buffer then receives stage s+2 -- two steps of lead for the DMA.
// Two waves per SIMD matter here: a single wave draws fragments from LDS at about half the rate that
// two do, and the MFMA work of one wave covers the other's waits.
// Stage layout: A rows and W rows of 128 bytes; 16-byte chunk c of row r sits at chunk c ^ ((r>>1)&7),
// so rows r .. r+15 at one logical chunk land on 16 distinct bank quads of the 64 LDS banks.
constexpr int BKS = 128;                          // K per stage
constexpr int NBUF8 = 2;
constexpr int STAGE8 = (BM + BN) * BKS;           // 64 KB
constexpr int NWAVE8 = 8;

// DMA instruction u of wave w's share of a stage (0..3: A row blocks 4w+u; 4..7: W row blocks
// 4w+u-4; 8 rows each)
QVD_DEV void dma_f8(const GemmArgs& g, uint8_t* smem, int buf, int k0, int wv, const uint32_t* a_off,
                    const uint32_t* w_off, int u) {
    uint8_t* dst = smem + buf * STAGE8 + (u < 4 ? 0 : BM * BKS) + (4 * wv + (u & 3)) * 1024;
    if (u < 4) dma_lds16(g.a, a_off[u & 3], (uint32_t)k0, dst);
    else dma_lds16(g.w, w_off[u & 3], (uint32_t)k0, dst);
}

QVD_DEV void stage_f8(const GemmArgs& g, uint8_t* smem, int buf, int k0, int wv, const uint32_t* a_off,
                      const uint32_t* w_off) {
#pragma unroll
    for (int u = 0; u < 8; ++u) dma_f8(g, smem, buf, k0, wv, a_off, w_off, u);
}

// 32-byte MFMA operand of rows 32 b .. 32 b + 31 of a 128-byte-row tile, K half h: lane l reads row
// l%32, logical chunks 4h + 2(l/32) and 4h + 2(l/32) + 1 (row offsets precomputed in lo/hi per half)
QVD_DEV v8i frag32(const uint8_t* tile, int b, uint32_t lo, uint32_t hi) {
    const v4i x = *reinterpret_cast<const v4i*>(tile + b * 4096 + lo);
    const v4i y = *reinterpret_cast<const v4i*>(tile + b * 4096 + hi);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int V> using IC = std::integral_constant<int, V>;

template <int EPI>
__global__ void __launch_bounds__(512, 1) k_gemm_f8(GemmArgs g) {
    // one LDS object: the two stage buffers and, past them, the epilogue's reduction slots (a second
    // __shared__ array makes the compiler wait for every DMA before each LDS read)
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF8 * STAGE8 + 4 * NWAVE8];
    float* red = reinterpret_cast<float*>(smem + NBUF8 * STAGE8);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    int tm, tn;
    tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;

    // DMA: wave w's A (W) instruction u fills rows (4w+u)*8 .. +7 of the tile; lane l lands in row
    // r = (4w+u)*8 + l/8, slot l%8, and fetches chunk (l%8) ^ ((r>>1)&7) of its row.
    // Rows past M (N) repeat the last row; their results are never stored.
    uint32_t a_off[4], w_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = (4 * wv + u) * 8 + (lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
        const int ra = m0 + r < M ? m0 + r : M - 1;
        const int rw = n0 + r < N ? n0 + r : N - 1;
        a_off[u] = (uint32_t)ra * (uint32_t)K + 16u * c;
        w_off[u] = (uint32_t)rw * (uint32_t)K + 16u * c;
    }
    // fragment reads, per K half h: row l%32 of a 32-row block, logical chunks 4h + 2(l/32) (+1)
    const uint32_t fs = (uint32_t)(((lane & 31) >> 1) & 7);
    const uint32_t rb = (uint32_t)(lane & 31) * 128u, cg0 = 2u * (uint32_t)(lane >> 5);
    const uint32_t flo0 = rb + 16u * (cg0 ^ fs), fhi0 = rb + 16u * ((cg0 + 1u) ^ fs);
    const uint32_t flo1 = rb + 16u * ((cg0 + 4u) ^ fs), fhi1 = rb + 16u * ((cg0 + 5u) ^ fs);
    const int a_blk = 4 * wm, w_blk = 2 * wn;    // first 32-row block of this wave's A / W rows

    Layout32N64::Acc acc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // K is a multiple of 128: S stages, 2 S steps (an even count, so the register sets alternate in
    // pairs: even steps use set 0, odd steps set 1)
    const int S = K / BKS;
    stage_f8(g, smem, 0, 0, wv, a_off, w_off);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (S > 1) stage_f8(g, smem, 1, BKS, wv, a_off, w_off);

    v8i fr[2][6];                                // [set][W blocks 0..1, A blocks 2..5]
#pragma unroll
    for (int i = 0; i < 2; ++i) fr[0][i] = frag32(smem + BM * BKS, w_blk + i, flo0, fhi0);
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[0][2 + i] = frag32(smem, a_blk + i, flo0, fhi0);
    lgkm_settle();

    // Stage s, half h, on register set h.  Half 0 reads the fragments of half 1 (same buffer).  Half 1
    // first waits for stage s+1: after that barrier every wave has also finished reading stage s (its
    // halves were read during the two previous steps), so stage s's buffer takes stage s+2 while the
    // fragments of stage s+1, half 0 are read from the other buffer.
    auto kstep = [&](auto H, int s, bool bar, bool refill) {
        constexpr int h = decltype(H)::value;
        if (h == 1 && bar) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // fragments of the next step: stage s half 1, or stage s+1 half 0 (a stale buffer after the
        // last step, never used)
        const uint8_t* As = smem + ((h == 0 ? s : s + 1) & 1) * STAGE8;
        const uint8_t* Ws = As + BM * BKS;
        const uint32_t lo = h == 0 ? flo1 : flo0, hi = h == 0 ? fhi1 : fhi0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fr[h][q >> 2], fr[h][2 + (q & 3)], acc[q >> 2][q & 3], 0, 0, 0, 0, 0, 0);
            if (h == 1 && refill) dma_f8(g, smem, s & 1, (s + 2) * BKS, wv, a_off, w_off, q);
            if (q < 6) fr[h ^ 1][q] = q < 2 ? frag32(Ws, w_blk + q, lo, hi) : frag32(As, a_blk + q - 2, lo, hi);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int s = 0; s < S; ++s) {
        kstep(IC<0>{}, s, false, false);
        kstep(IC<1>{}, s, s + 1 < S, s + 2 < S);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stages are free
    gemm_epilogue<EPI, Layout32N64, 64, NWAVE8>(g, acc, (*g.s_a) * (*g.s_w), m0, n0, wm, wn, red,
                                                smem + wv * 16384);
}

// ================================================================================================
// E4M3 activations x MXFP4 weights: the tiles, eight waves, 128-K stages and barrier schedule of the
// E4M3 x E4M3 kernel, with v_mfma_scale_f32_32x32x64_f8f6f4 taking the E2M1 operand (cbsz = 4) and
// one E8M0 scale per lane.
// Operand pairing of that MFMA with E2M1 x E4M3 (measured on gfx950 with one-hot operands): lane half h
// of the E2M1 operand holds k = 32h .. 32h+31 of its row in order -- 16 bytes, exactly one 32-element
// block, whose scale the lane supplies -- and lane half h of the E4M3 operand holds k = 16h .. 16h+15
// in its first 16 bytes and k = 32+16h .. 32+16h+15 in its last 16.
// Stage layout (48 KB): A rows of 128 bytes as in the E4M3 kernel; W rows of 64 bytes (128 packed E2M1
// values), 16-byte chunk c of row r at c ^ ((r>>2)&3), so rows r .. r+15 at one logical chunk cover
// 16 distinct bank quads.  The W scales come in chunks of 8 stages (below).
// E8M0 scales of the block-scaled kernels travel in chunks of 8 stages: per operand 256 rows x 32
// bytes (the 4 bytes of each of the 8 stages), two chunk buffers.  A row's 32 bytes are contiguous
// in the [rows][K/32] array, so a DMA of 8 lanes per row covers 8 consecutive rows in a few cache
// lines; loading each stage's 4 bytes for 64 rows instead touched a line per row and cost the W4A4
// kernel 15-25%.  Each stage's refill adds one 32-row slice: stage s loads slice (s+1) % 8 of chunk
// (s+1)/8 + 1 (the prologue loads chunk 0 and slice 0 of chunk 1), so chunk c is complete at stage
// 8c - 2 and first read, for stage 8c, after the barrier of stage 8c - 1.
constexpr int SC_STAGES = 8;                       // stages per scale chunk
constexpr int SC_ROW = 4 * SC_STAGES;              // bytes per row per chunk
constexpr int SC_BUF = BN * SC_ROW;                // one operand's chunk (BM == BN)

// One wave's part of scale slice sl of chunk ch: rows 32 sl + 8 part .. +7 of the tile (base ..),
// 8 lanes per row, 4 bytes each, into the chunk buffer at sc + (ch & 1) * stride.  Chunks past the
// last re-read the last one (never used); columns past K/32 read the row's first word; rows past the
// matrix its last row.
QVD_DEV void dma_scale_slice(const uint8_t* src, int base, int lim, int kb, int nch, uint8_t* sc, int stride,
                             int ch, int sl, int part, int lane) {
    const int chc = ch < nch ? ch : nch - 1;
    int row = base + 32 * sl + 8 * part + (lane >> 3);
    row = row < lim ? row : lim - 1;
    int col = SC_ROW * chc + 4 * (lane & 7);
    col = col < kb ? col : 0;
    dma_lds4(src, (uint32_t)row * (uint32_t)kb + (uint32_t)col, 0u,
               sc + (ch & 1) * stride + (32 * sl + 8 * part) * SC_ROW);
}

// the word of stage t of row r from the chunk buffers at sc (stride between the two)
QVD_DEV uint32_t scale_word(const uint8_t* sc, int stride, int r, int t) {
    return *reinterpret_cast<const uint32_t*>(sc + ((t >> 3) & 1) * stride + r * SC_ROW + 4 * (t & 7));
}

constexpr int W4_OFF = BM * BKS;                  // W rows of a stage
constexpr int STAGE_MX = W4_OFF + BN * BKS / 2;
constexpr int MX_SC_OFF = 2 * STAGE_MX;           // W scale chunks
constexpr int MX_MAIN = MX_SC_OFF + 2 * SC_BUF;
constexpr int SMEM_MX = MX_MAIN > NWAVE8 * 16384 ? MX_MAIN : NWAVE8 * 16384;

// DMA instruction u of wave w's share of a stage: 0..3 A row blocks 4w+u (8 rows of 128 bytes each),
// 4..5 W row blocks 2w+u-4 (16 rows of 64 bytes each)
QVD_DEV void dma_mx(const GemmArgs& g, uint8_t* smem, int buf, int k0, int wv, const uint32_t* a_off,
                    const uint32_t* w_off, int u) {
    uint8_t* st = smem + buf * STAGE_MX;
    if (u < 4) dma_lds16(g.a, a_off[u], (uint32_t)k0, st + (4 * wv + u) * 1024);
    else dma_lds16(g.w, w_off[u - 4], (uint32_t)(k0 / 2), st + W4_OFF + (2 * wv + u - 4) * 1024);
}

QVD_DEV void stage_mx(const GemmArgs& g, uint8_t* smem, int buf, int k0, int wv, const uint32_t* a_off,
                      const uint32_t* w_off) {
#pragma unroll
    for (int u = 0; u < 6; ++u) dma_mx(g, smem, buf, k0, wv, a_off, w_off, u);
}

// 16-byte E2M1 operand (32 elements) of rows 32 b .. 32 b + 31 of a 64-byte-row tile; the MFMA reads
// only the low four registers
QVD_DEV v8i frag_e2m1(const uint8_t* tile, int b, uint32_t off) {
    const v4i x = *reinterpret_cast<const v4i*>(tile + b * 2048 + off);
    const v4i z = {0, 0, 0, 0};
    return __builtin_shufflevector(x, z, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int EPI>
__global__ void __launch_bounds__(512, 1) k_gemm_mx(GemmArgs g) {
    // one LDS object (see k_gemm_f8): stage buffers, which the epilogue then reuses as 16 KB per wave,
    // and the reduction slots
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_MX + 4 * NWAVE8];
    float* red = reinterpret_cast<float*>(smem + SMEM_MX);

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 1, wn = wv >> 1;
    int tm, tn;
    tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;

    // DMA sources.  A as in k_gemm_f8.  W instruction u: lane l lands in row r = (2w+u)*16 + l/4, slot
    // l%4, and fetches chunk (l%4) ^ ((r>>2)&3) of the row's 64 stage bytes.  Rows past M (N) repeat
    // the last row; their results are never stored.  Scale slices: waves w and w+4 load the same part
    // w%4 (the same bytes), which keeps the code free of branches.
    uint32_t a_off[4], w_off[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = (4 * wv + u) * 8 + (lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
        const int ra = m0 + r < M ? m0 + r : M - 1;
        a_off[u] = (uint32_t)ra * (uint32_t)K + 16u * c;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = (2 * wv + u) * 16 + (lane >> 2);
        const uint32_t c = (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
        const int rw = n0 + r < N ? n0 + r : N - 1;
        w_off[u] = (uint32_t)rw * (uint32_t)(K / 2) + 16u * c;
    }
    const int kb = K / 32, S = K / BKS, nch = (S + SC_STAGES - 1) / SC_STAGES;
    uint8_t* const sc = smem + MX_SC_OFF;
    // fragment offsets per K step j of a stage.  A (E4M3): row l%32, logical chunks 4j + h and
    // 4j + 2 + h for lane half h.  W (E2M1): row l%32, logical chunk 2j + h.  Scale word: row l%32.
    const int lr = lane & 31, hl = lane >> 5;
    const uint32_t fs = (uint32_t)((lr >> 1) & 7), rb = (uint32_t)lr * 128u;
    const uint32_t alo0 = rb + 16u * ((uint32_t)hl ^ fs), ahi0 = rb + 16u * ((2u + hl) ^ fs);
    const uint32_t alo1 = rb + 16u * ((4u + hl) ^ fs), ahi1 = rb + 16u * ((6u + hl) ^ fs);
    const uint32_t ws = (uint32_t)((lr >> 2) & 3), rw64 = (uint32_t)lr * 64u;
    const uint32_t wo0 = rw64 + 16u * ((uint32_t)hl ^ ws), wo1 = rw64 + 16u * ((2u + hl) ^ ws);
    const int a_blk = 4 * wm, w_blk = 2 * wn;

    Layout32N64::Acc acc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // K is a multiple of 128: S stages, 2 S steps
    stage_mx(g, smem, 0, 0, wv, a_off, w_off);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) dma_scale_slice(g.e8, n0, N, kb, nch, sc, SC_BUF, 0, sl, wv & 3, lane);
    dma_scale_slice(g.e8, n0, N, kb, nch, sc, SC_BUF, 1, 0, wv & 3, lane);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    stage_mx(g, smem, 1, S > 1 ? BKS : 0, wv, a_off, w_off);

    v8i fw[2][2], fa[2][4];                      // [set][W blocks] / [set][A blocks]
    uint32_t scw[2], scw_next[2];                // E8M0 words of this stage, shifted to the lane half's block
#pragma unroll
    for (int i = 0; i < 2; ++i) fw[0][i] = frag_e2m1(smem + W4_OFF, w_blk + i, wo0);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = frag32(smem, a_blk + i, alo0, ahi0);
#pragma unroll
    for (int i = 0; i < 2; ++i) scw[i] = scale_word(sc, SC_BUF, 32 * (w_blk + i) + lr, 0) >> (8 * hl);
    lgkm_settle();

    // The step schedule of k_gemm_f8, with step bodies free of branches: with the refill and the E8M0
    // loads of waves 0..3 behind branches, the compiler moved every MFMA of the loop behind the last
    // of them (out of its interleave with the fragment reads) and spilled.  So the main loop always
    // refills, the last two stages never do, step 1 always waits at the barrier (once more than
    // needed, in the last stage), and all eight waves load scale slices.  Step 0 of a stage uses blocks
    // h of the stage (byte h of the shifted words), step 1 blocks 2 + h (byte 2); the words of stage
    // s+1 are read at the start of step 1 of stage s.
    auto kstep = [&](auto H, auto REFILL, int s) {
        constexpr int h = decltype(H)::value;
        constexpr bool refill = decltype(REFILL)::value == 1;
        if (h == 1) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int nbuf = (h == 0 ? s : s + 1) & 1;
        const uint8_t* As = smem + nbuf * STAGE_MX;
        const uint8_t* Ws = As + W4_OFF;
        const uint32_t lo = h == 0 ? alo1 : alo0, hi = h == 0 ? ahi1 : ahi0, wo = h == 0 ? wo1 : wo0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int sw = (int)(h == 0 ? scw[q >> 2] : scw[q >> 2] >> 16);
            acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fw[h][q >> 2], fa[h][q & 3], acc[q >> 2][q & 3], 4, 0, 0, sw, 0, 127);
            if (h == 1 && refill && q < 6) dma_mx(g, smem, s & 1, (s + 2) * BKS, wv, a_off, w_off, q);
            if (h == 1 && refill && q == 6)
                dma_scale_slice(g.e8, n0, N, kb, nch, sc, SC_BUF, ((s + 1) >> 3) + 1, (s + 1) & 7, wv & 3, lane);
            if (h == 1 && q == 0) {             // first, so that LDS (which answers in order) has
#pragma unroll                                  // them back before the fragments
                for (int i = 0; i < 2; ++i)
                    scw_next[i] = scale_word(sc, SC_BUF, 32 * (w_blk + i) + lr, s + 1) >> (8 * hl);
            }
            if (q < 2)
                fw[h ^ 1][q] = frag_e2m1(Ws, w_blk + q, wo);
            else if (q < 6)
                fa[h ^ 1][q - 2] = frag32(As, a_blk + q - 2, lo, hi);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (h == 1) {
            scw[0] = scw_next[0];
            scw[1] = scw_next[1];
        }
    };
    int s = 0;
    for (; s < S - 2; ++s) {
        kstep(IC<0>{}, IC<0>{}, s);
        kstep(IC<1>{}, IC<1>{}, s);
    }
    for (; s < S; ++s) {
        kstep(IC<0>{}, IC<0>{}, s);
        kstep(IC<1>{}, IC<0>{}, s);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stages are free
    gemm_epilogue<EPI, Layout32N64, 64, NWAVE8>(g, acc, *g.s_a, m0, n0, wm, wn, red, smem + wv * 16384);
}

// ================================================================================================
// MXFP4 activations x MXFP4 weights (W4A4): v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1
// (cbsz = blgp = 4), each lane supplying the E8M0 scale of its row's 32-element block for both.
// Measured on gfx950 with one-hot and all-ones operands: lane half h of either E2M1 operand holds
// k = 32h .. 32h+31 of its row in order, and lane l's scale byte applies to row l%32, block l/32.
// Tiles, waves, 128-K stages and the branch-free step schedule are those of k_gemm_mx.  Stage
// (32 KB): A and W rows of 64 bytes (chunk c of row r at c ^ ((r>>2)&3)).
// E8M0 scales of both operands in chunks of 8 stages, as in k_gemm_mx: buffer (ch & 1) of operand o
// at W4A4_SC_OFF + ((ch & 1) * 2 + o) * SC_BUF.
constexpr int W4A4_W_OFF = BM * BKS / 2;
constexpr int STAGE_W4A4 = W4A4_W_OFF + BN * BKS / 2;
constexpr int W4A4_SC_OFF = 2 * STAGE_W4A4;
constexpr int W4A4_MAIN = W4A4_SC_OFF + 4 * SC_BUF;
constexpr int SMEM_W4A4 = W4A4_MAIN > NWAVE8 * 16384 ? W4A4_MAIN : NWAVE8 * 16384;

// DMA instruction u of wave w's share of a stage: 0..1 A row blocks 2w+u, 2..3 W row blocks 2w+u-2
// (16 rows of 64 bytes each)
QVD_DEV void dma_w4a4(const GemmArgs& g, uint8_t* smem, int buf, int k0, int wv, const uint32_t* a_off,
                      const uint32_t* w_off, int u) {
    uint8_t* st = smem + buf * STAGE_W4A4;
    if (u < 2) dma_lds16(g.a, a_off[u], (uint32_t)(k0 / 2), st + (2 * wv + u) * 1024);
    else dma_lds16(g.w, w_off[u - 2], (uint32_t)(k0 / 2), st + W4A4_W_OFF + (2 * wv + u - 2) * 1024);
}

// one wave's part of a scale slice: operand o (waves 0..3 A, 4..7 W), part w % 4
QVD_DEV void dma_w4a4_scales(const uint8_t* src, int base, int lim, int kb, int nch, uint8_t* smem, int ch,
                             int sl, int part, int o, int lane) {
    dma_scale_slice(src, base, lim, kb, nch, smem + W4A4_SC_OFF + o * SC_BUF, 2 * SC_BUF, ch, sl, part, lane);
}

template <int EPI>
__global__ void __launch_bounds__(512, 1) k_gemm_w4a4(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_W4A4 + 4 * NWAVE8];
    float* red = reinterpret_cast<float*>(smem + SMEM_W4A4);

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 1, wn = wv >> 1;
    int tm, tn;
    tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;

    // DMA sources.  A and W instruction u: lane l lands in row r = (2w+u)*16 + l/4, slot l%4, and
    // fetches chunk (l%4) ^ ((r>>2)&3) of the row's 64 stage bytes.  Rows past M (N) repeat the last
    // row; their results are never stored.
    uint32_t a_off[2], w_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = (2 * wv + u) * 16 + (lane >> 2);
        const uint32_t c = (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
        const int ra = m0 + r < M ? m0 + r : M - 1;
        const int rw = n0 + r < N ? n0 + r : N - 1;
        a_off[u] = (uint32_t)ra * (uint32_t)(K / 2) + 16u * c;
        w_off[u] = (uint32_t)rw * (uint32_t)(K / 2) + 16u * c;
    }
    const int so = wv >> 2, spart = wv & 3;               // scale DMA: operand and part of this wave
    const uint8_t* e_src = so == 0 ? g.a_e8 : g.e8;
    const int e_base = so == 0 ? m0 : n0, e_lim = so == 0 ? M : N;
    const int S = K / BKS, kb = K / 32, nch = (S + SC_STAGES - 1) / SC_STAGES;

    // fragment offsets per K step j: row l%32 of a 32-row block, logical chunk 2j + h (lane half h)
    const int lr = lane & 31, hl = lane >> 5;
    const uint32_t sw4 = (uint32_t)((lr >> 2) & 3), r64 = (uint32_t)lr * 64u;
    const uint32_t fo0 = r64 + 16u * ((uint32_t)hl ^ sw4), fo1 = r64 + 16u * ((2u + hl) ^ sw4);
    const int a_blk = 4 * wm, w_blk = 2 * wn;
    // scale word of stage t for fragment row block b of operand o: chunk buffer (t/8)&1, word t%8
    auto sc_word = [&](int o, int b, int t) {
        return scale_word(smem + W4A4_SC_OFF + o * SC_BUF, 2 * SC_BUF, 32 * b + lr, t);
    };

    Layout32N64::Acc acc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

#pragma unroll
    for (int u = 0; u < 4; ++u) dma_w4a4(g, smem, 0, 0, wv, a_off, w_off, u);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) dma_w4a4_scales(e_src, e_base, e_lim, kb, nch, smem, 0, sl, spart, so, lane);
    dma_w4a4_scales(e_src, e_base, e_lim, kb, nch, smem, 1, 0, spart, so, lane);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_w4a4(g, smem, 1, S > 1 ? BKS : 0, wv, a_off, w_off, u);

    v8i fw[2][2], fa[2][4];
    uint32_t scw[2], sca[4], scw_n[2], sca_n[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) fw[0][i] = frag_e2m1(smem + W4A4_W_OFF, w_blk + i, fo0);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = frag_e2m1(smem, a_blk + i, fo0);
#pragma unroll
    for (int i = 0; i < 2; ++i) scw[i] = sc_word(1, w_blk + i, 0) >> (8 * hl);
#pragma unroll
    for (int i = 0; i < 4; ++i) sca[i] = sc_word(0, a_blk + i, 0) >> (8 * hl);
    lgkm_settle();

    // the step schedule of k_gemm_mx: step 0 of a stage uses blocks h (byte h of the shifted words),
    // step 1 blocks 2 + h (byte 2); the words of stage s+1 are read at the start of step 1 of stage s
    auto kstep = [&](auto H, auto REFILL, int s) {
        constexpr int h = decltype(H)::value;
        constexpr bool refill = decltype(REFILL)::value == 1;
        if (h == 1) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int nbuf = (h == 0 ? s : s + 1) & 1;
        const uint8_t* As = smem + nbuf * STAGE_W4A4;
        const uint8_t* Ws = As + W4A4_W_OFF;
        const uint32_t fo = h == 0 ? fo1 : fo0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int swv = (int)(h == 0 ? scw[q >> 2] : scw[q >> 2] >> 16);
            const int sav = (int)(h == 0 ? sca[q & 3] : sca[q & 3] >> 16);
            acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fw[h][q >> 2], fa[h][q & 3], acc[q >> 2][q & 3], 4, 4, 0, swv, 0, sav);
            if (h == 1 && refill && q < 4)
                dma_w4a4(g, smem, s & 1, (s + 2) * BKS, wv, a_off, w_off, q);
            if (h == 1 && refill && q == 4)
                dma_w4a4_scales(e_src, e_base, e_lim, kb, nch, smem, ((s + 1) >> 3) + 1, (s + 1) & 7, spart, so,
                                lane);
            if (h == 1 && q == 0) {   // raw words: shifting here would wait for the reads in flight
#pragma unroll
                for (int i = 0; i < 2; ++i) scw_n[i] = sc_word(1, w_blk + i, s + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) sca_n[i] = sc_word(0, a_blk + i, s + 1);
            }
            if (q < 2)
                fw[h ^ 1][q] = frag_e2m1(Ws, w_blk + q, fo);
            else if (q < 6)
                fa[h ^ 1][q - 2] = frag_e2m1(As, a_blk + q - 2, fo);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (h == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i) scw[i] = scw_n[i] >> (8 * hl);
#pragma unroll
            for (int i = 0; i < 4; ++i) sca[i] = sca_n[i] >> (8 * hl);
        }
    };
    int s = 0;
    for (; s < S - 2; ++s) {
        kstep(IC<0>{}, IC<0>{}, s);
        kstep(IC<1>{}, IC<1>{}, s);
    }
    for (; s < S; ++s) {
        kstep(IC<0>{}, IC<0>{}, s);
        kstep(IC<1>{}, IC<0>{}, s);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stages are free
    gemm_epilogue<EPI, Layout32N64, 64, NWAVE8>(g, acc, 1.0f, m0, n0, wm, wn, red, smem + wv * 16384);
}

template <template <int> class KERN>
static int launch_epi(const GemmArgs& g, hipStream_t st) {
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), blk(KERN<QVD_EPI_F32>::threads);
    switch (g.epi.mode) {
        case QVD_EPI_F32: hipLaunchKernelGGL(KERN<QVD_EPI_F32>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_BF16: hipLaunchKernelGGL(KERN<QVD_EPI_BF16>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_RESID_GATE: hipLaunchKernelGGL(KERN<QVD_EPI_RESID_GATE>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_GELU: hipLaunchKernelGGL(KERN<QVD_EPI_GELU>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_QKV: hipLaunchKernelGGL(KERN<QVD_EPI_QKV>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_GELU_E4M3: hipLaunchKernelGGL(KERN<QVD_EPI_GELU_E4M3>::fn, grid, blk, 0, st, g); break;
        case QVD_EPI_GELU_MXFP4: hipLaunchKernelGGL(KERN<QVD_EPI_GELU_MXFP4>::fn, grid, blk, 0, st, g); break;
        default: return fail(QVD_EINVAL, "gemm: epilogue mode %d", g.epi.mode);
    }
    return launch_status("gemm");
}
template <int EPI> struct KF8 { static constexpr auto fn = k_gemm_f8<EPI>; static constexpr unsigned threads = 64 * NWAVE8; };
template <int EPI> struct KMX { static constexpr auto fn = k_gemm_mx<EPI>; static constexpr unsigned threads = 64 * NWAVE8; };
template <int EPI> struct KW4A4 { static constexpr auto fn = k_gemm_w4a4<EPI>; static constexpr unsigned threads = 64 * NWAVE8; };

static const char* epi_name(int mode) {
    static const char* names[] = {"f32", "bf16", "resid_gate", "gelu", "qkv", "gelu_e4m3", "gelu_mxfp4"};
    return (mode >= 0 && mode < 7) ? names[mode] : "?";
}

int launch_gemm(const uint8_t* a, const float* s_a, const void* w, const uint8_t* e8, const float* s_w,
                int w_fmt, const float* bias, int M, int N, int K, const qvd_epilogue& epi,
                hipStream_t st) {
    if (M == 0) return QVD_OK;
    GemmArgs g;
    g.a = a;
    g.w = (const uint8_t*)w;
    g.e8 = e8;
    g.a_e8 = nullptr;
    g.s_a = s_a;
    g.s_w = s_w;
    g.bias = bias;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = (M + BM - 1) / BM;
    g.tiles_n = (N + BN - 1) / BN;
    g.epi = epi;
    char key[96];
    snprintf(key, sizeof(key), "gemm_%s_%s_%dx%dx%d", w_fmt == QVD_W_MXFP4 ? "mxfp4" : "fp8",
             epi_name(epi.mode), M, N, K);
    TimingScope ts(key, st);
    return w_fmt == QVD_W_MXFP4 ? launch_epi<KMX>(g, st) : launch_epi<KF8>(g, st);
}

int launch_gemm_w4a4(const uint8_t* a, const uint8_t* a_e8, const uint8_t* w, const uint8_t* w_e8,
                     const float* bias, int M, int N, int K, const qvd_epilogue& epi, hipStream_t st) {
    if (M == 0) return QVD_OK;
    GemmArgs g;
    g.a = a;
    g.w = w;
    g.e8 = w_e8;
    g.a_e8 = a_e8;
    g.s_a = nullptr;
    g.s_w = nullptr;
    g.bias = bias;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = (M + BM - 1) / BM;
    g.tiles_n = (N + BN - 1) / BN;
    g.epi = epi;
    char key[96];
    snprintf(key, sizeof(key), "gemm_w4a4_%s_%dx%dx%d", epi_name(epi.mode), M, N, K);
    TimingScope ts(key, st);
    return launch_epi<KW4A4>(g, st);
}

}  // namespace qvd

using namespace qvd;

static int validate_gemm(const char* fn, const uint8_t* a, const void* s_a, const void* w,
                         const float* bias, int32_t M, int32_t N, int32_t K, const qvd_epilogue* epi) {
    QVD_REQUIRE(epi != nullptr, QVD_EINVAL, "%s: epi is NULL", fn);
    QVD_REQUIRE(M >= 0 && N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0, QVD_ESHAPE,
                "%s: M = %d, N = %d, K = %d (N, K: positive multiples of 128)", fn, M, N, K);
    QVD_REQUIRE(gemm_tiles(M, N) < (1ll << 31), QVD_ESHAPE, "%s: too many tiles", fn);
    QVD_REQUIRE((double)M * K < 4294967296.0 && (double)N * K < 4294967296.0, QVD_ESHAPE,
                "%s: operands must stay below 4 GiB (M = %d, N = %d, K = %d)", fn, M, N, K);
    QVD_REQUIRE(w != nullptr, QVD_EINVAL, "%s: w is NULL", fn);
    QVD_REQUIRE(aligned16(w) && (!bias || aligned16(bias)), QVD_EALIGN, "%s: w/bias not 16-byte aligned", fn);
    if (M > 0) {
        QVD_REQUIRE(a && aligned16(a), QVD_EINVAL, "%s: a is NULL or misaligned", fn);
        QVD_REQUIRE(s_a != nullptr, QVD_EINVAL, "%s: activation scale is NULL", fn);
    }
    QVD_REQUIRE(epi->mode >= QVD_EPI_F32 && epi->mode <= QVD_EPI_GELU_MXFP4, QVD_EINVAL,
                "%s: unknown epilogue mode %d", fn, epi->mode);
    if (M == 0) return QVD_OK;   // nothing is read or written
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
        case QVD_EPI_GELU_E4M3:
            QVD_REQUIRE(epi->out_e4m3 && aligned16(epi->out_e4m3) && epi->out_scale, QVD_EINVAL,
                        "%s: out_e4m3 NULL/misaligned or out_scale NULL", fn);
            break;
        case QVD_EPI_GELU_MXFP4:
            QVD_REQUIRE(epi->out_e2m1 && aligned16(epi->out_e2m1) && epi->out_e8m0, QVD_EINVAL,
                        "%s: out_e2m1 NULL/misaligned or out_e8m0 NULL", fn);
            break;
        case QVD_EPI_QKV:
            QVD_REQUIRE(epi->n_heads >= 1 && N == 3 * 128 * epi->n_heads, QVD_ESHAPE,
                        "%s: QKV epilogue needs N = 3*128*n_heads (N = %d, n_heads = %d)", fn, N,
                        epi->n_heads);
            QVD_REQUIRE(epi->q8 && epi->k8 && epi->v && epi->q_scale && epi->k_scale && epi->v_exp, QVD_EINVAL,
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
    QVD_REQUIRE(((uintptr_t)e8m0 & 3u) == 0, QVD_EALIGN, "qvd_gemm_mxfp4: e8m0 must be 4-byte aligned");
    QVD_DEVICE_OK();
    return launch_gemm(a, s_a, w_packed, e8m0, nullptr, QVD_W_MXFP4, bias, M, N, K, *epi,
                       (hipStream_t)stream);
}

int qvd_gemm_mxfp4_w4a4(const uint8_t* a_packed, const uint8_t* a_e8m0, const uint8_t* w_packed,
                        const uint8_t* w_e8m0, const float* bias, int32_t M, int32_t N, int32_t K,
                        const qvd_epilogue* epi, void* stream) {
    int s = validate_gemm("qvd_gemm_mxfp4_w4a4", a_packed, a_e8m0, w_packed, bias, M, N, K, epi);
    if (s) return s;
    QVD_PTR(w_e8m0);
    QVD_REQUIRE(((uintptr_t)a_e8m0 & 3u) == 0 && ((uintptr_t)w_e8m0 & 3u) == 0, QVD_EALIGN,
                "qvd_gemm_mxfp4_w4a4: a_e8m0 and w_e8m0 must be 4-byte aligned");
    QVD_DEVICE_OK();
    return launch_gemm_w4a4(a_packed, a_e8m0, w_packed, w_e8m0, bias, M, N, K, *epi, (hipStream_t)stream);
}

}  // extern "C"
