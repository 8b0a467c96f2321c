// AdaLN timestep conditioning: the shared-basis projection and the modulated LayerNorm that feeds
// the per-tensor FP8 GEMMs.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3", section "Trim 改变了什么",
// timestep-conditioning bullet: the time embedding (2,688 wide) is mapped to six modulation vectors
// per block through a 2,688->16 basis shared by all blocks and a small per-block projection, both
// stored in fp16.
//
// The LayerNorm statistics and the affine map run in float64 and round once to fp32, so the FP8
// codes do not depend on the summation order of the row statistics (the fp64 sum of bf16 values is
// exact at these widths).  The kernel is bound by HBM traffic: one wave owns a row, keeps it in
// registers, and stores its codes as 16-bit pairs.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr int RANK = 16;

QVD_DEV double fp16_to_f64(uint16_t b) { return (double)__builtin_bit_cast(_Float16, b); }

// ---------------------------------------------------------------------------------------------
// projection: every workgroup recomputes c = B e(t) (16 x dt MACs, float64) and then produces 256
// entries of its block's modulation table.

__global__ void __launch_bounds__(256) k_adaln_project(float t, const uint16_t* __restrict__ basis,
                                                       int dt, const uint16_t* __restrict__ proj,
                                                       const uint16_t* __restrict__ bias, int d,
                                                       float* __restrict__ mod) {
    __shared__ double red[4][RANK];
    __shared__ double c[RANK];
    const int half = dt / 2;
    const double ln1e4 = 9.210340371976184;        // ln(10000), correctly rounded
    double acc[RANK];
#pragma unroll
    for (int r = 0; r < RANK; ++r) acc[r] = 0.0;
    for (int i = threadIdx.x; i < dt; i += 256) {
        const int fi = i < half ? i : i - half;
        const double f = exp((-ln1e4 * (double)fi) / (double)half);
        const double arg = (double)t * f;
        const double e = i < half ? cos(arg) : sin(arg);
#pragma unroll
        for (int r = 0; r < RANK; ++r) {
            const double b = fp16_to_f64(basis[r * dt + i]);
            acc[r] = fma(b, e, acc[r]);
        }
    }
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < RANK; ++r) {
        const double s = wave_sum_f64(acc[r]);
        if ((threadIdx.x & 63) == 0) red[w][r] = s;
    }
    __syncthreads();
    if (threadIdx.x < RANK)
        c[threadIdx.x] = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                         (red[2][threadIdx.x] + red[3][threadIdx.x]);
    __syncthreads();
    const int blk = blockIdx.y;
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= 6 * d) return;
    const uint16_t* P = proj + ((int64_t)blk * 6 * d + o) * RANK;
    double m = 0.0;
#pragma unroll
    for (int r = 0; r < RANK; ++r) m = fma(fp16_to_f64(P[r]), c[r], m);
    if (bias) m += fp16_to_f64(bias[(int64_t)blk * 6 * d + o]);
    mod[(int64_t)blk * 6 * d + o] = (float)m;
}

// ---------------------------------------------------------------------------------------------
// modulated LayerNorm.  One wave per row; NW = d/128 32-bit words (bf16 pairs) per lane, lane l owns
// words l + 64 j, i.e. columns 2(l + 64 j) and 2(l + 64 j) + 1.  The per-column modulation sits in
// LDS as float4 (a0, b0, a1, b1) per column pair, so registers hold the row and little else.

template <int NW>
struct Row {
    u32 x[NW];
};

// The compiler may not reuse values derived from the row across this point (it would otherwise keep
// float64 copies of every element live between the loops and run out of registers).
template <int NW>
QVD_DEV void row_fence(Row<NW>& R) {
#pragma unroll
    for (int j = 0; j < NW; ++j) asm volatile("" : "+v"(R.x[j]));
}

// mean and 1/sqrt(var + eps) of one row (float64), all lanes get the result
template <int NW>
QVD_DEV void row_stats(Row<NW>& R, int nw, int d, double eps, double& mu, double& rstd) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < NW; ++j)
        if (j < nw) s += (double)bf16lo(R.x[j]) + (double)bf16hi(R.x[j]);
    mu = wave_sum_f64(s) / (double)d;
    row_fence<NW>(R);
    double v = 0.0;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        if (j < nw) {
            const double a = (double)bf16lo(R.x[j]) - mu;
            const double b = (double)bf16hi(R.x[j]) - mu;
            v = fma(a, a, v);
            v = fma(b, b, v);
        }
    }
    const double var = wave_sum_f64(v) / (double)d;
    rstd = 1.0 / sqrt(var + eps);
    row_fence<NW>(R);
}

// y = fp32(((x - mu) * rstd) * (1 + scale) + shift), each float64 operation rounded separately
QVD_DEV float modulate_one(float x, double mu, double rstd, float scale, float shift) {
#pragma clang fp contract(off)
    const double t = ((double)x - mu) * rstd;
    const double y = t * (1.0 + (double)scale) + (double)shift;
    return (float)y;
}

// x - mu for a bf16 x, in fp32 with mu split into mu_hi = fp32(mu) and mu_lo = fp32(mu - mu_hi): when x is
// within a factor two of mu_hi, x - mu_hi is exact (Sterbenz) and the one rounding left is that of the
// subtraction of mu_lo; otherwise |x - mu| is not small next to |mu| and each of the two roundings is
// within 2^-24 of it.  Within a few fp32 ulps of fp32(x - mu) computed in float64, without a float64
// instruction per element.
QVD_DEV float centered(float x, float mu_hi, float mu_lo) { return (x - mu_hi) - mu_lo; }

// LDS table of the modulation: tab[p] = (a(2p), b(2p), a(2p+1), b(2p+1)) with a = scale, b = shift
// (raw), or, with inv given, a = (1 + scale) inv and b = shift inv
QVD_DEV void load_mod_table(float4* tab, const float* __restrict__ mod, int half, int d, bool fold, float inv) {
    const float* shift = mod + (3 * half) * d;
    const float* scale = mod + (3 * half + 1) * d;
    for (int p = threadIdx.x; p < d / 2; p += blockDim.x) {
        const float2 sh = *reinterpret_cast<const float2*>(shift + 2 * p);
        const float2 sc = *reinterpret_cast<const float2*>(scale + 2 * p);
        tab[p] = fold ? make_float4((1.0f + sc.x) * inv, sh.x * inv, (1.0f + sc.y) * inv, sh.y * inv)
                      : make_float4(sc.x, sh.x, sc.y, sh.y);
    }
    __syncthreads();
}

// pass 1 (dynamic scales): row statistics to ws, per-workgroup max |y| to partials.
// max |y| is the float64 modulation's, rounded to fp32, exactly: every element is first evaluated in
// fp32 as fma(centered(x), fp32(rstd) fp32(1 + scale), shift), which is within 6 * 2^-24 (|y| + |shift|)
// < 2^-21 (|y| + |shift|) of it; only elements within 2^-19 (max + max|shift|) of the row's fp32
// maximum can hold the exact maximum, and those (usually one) are evaluated in float64.
// EXACT: d = 128 NW, so every word loop runs whole and the loads carry no branches (the compiler can
// then count the next row's loads in flight instead of waiting for all of them).
template <int NW, bool EXACT>
__global__ void __launch_bounds__(256) k_ln_stats(const uint16_t* __restrict__ x, int L, int d,
                                                  const float* __restrict__ mod, int half, float eps,
                                                  double2* __restrict__ stats,
                                                  float* __restrict__ partials) {
    __shared__ float4 tab[4096 / 2];
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nw = EXACT ? NW : d >> 7;
    load_mod_table(tab, mod, half, d, false, 1.0f);
    float shmax = 0.0f;
    for (int p = threadIdx.x; p < d / 2; p += 256)
        shmax = fmaxf(shmax, fmaxf(fabsf(tab[p].y), fabsf(tab[p].w)));
    shmax = block_max_nonneg<4>(shmax, red);
    float m = 0.0f;
    // the next row's loads are issued before this row is reduced, so their latency is covered
    auto load_row = [&](Row<NW>& D, int r) {
        const u32* xr = reinterpret_cast<const u32*>(x + (int64_t)r * d);
#pragma unroll
        for (int j = 0; j < NW; ++j)
            if (j < nw) D.x[j] = __builtin_nontemporal_load(xr + lane + 64 * j);
    };
    const int stride = gridDim.x * 4;
    Row<NW> R, Rn;
    int row = blockIdx.x * 4 + wv;
    if (row < L) load_row(R, row);
    for (; row < L; row += stride) {
        load_row(Rn, row + stride < L ? row + stride : L - 1);     // past the end: a row never used
        double mu, rstd;
        row_stats<NW>(R, nw, d, (double)eps, mu, rstd);
        if (lane == 0) stats[row] = make_double2(mu, rstd);
        const float rs = (float)rstd;
        const float mu_hi = (float)mu, mu_lo = (float)(mu - (double)mu_hi);
        float aw[NW];                             // per word: the larger fp32 |y| of its two elements
        float m32 = 0.0f;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < nw) {
                const float4 c = tab[lane + 64 * j];
                aw[j] = fmaxf(fabsf(fmaf(centered(bf16lo(R.x[j]), mu_hi, mu_lo), rs * (1.0f + c.x), c.y)),
                              fabsf(fmaf(centered(bf16hi(R.x[j]), mu_hi, mu_lo), rs * (1.0f + c.z), c.w)));
                m32 = fmaxf(m32, aw[j]);
            }
        }
        m32 = wave_max(m32);
        row_fence<NW>(R);
        const float thr = m32 - 0x1p-19f * (m32 + shmax);
        // both elements of a candidate word in float64: the maximum over any set of exact |y| that
        // holds every candidate is the row's exact maximum
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < nw && aw[j] >= thr) {
                const float4 c = tab[lane + 64 * j];
                m = fmaxf(m, fabsf(modulate_one(bf16lo(R.x[j]), mu, rstd, c.x, c.y)));
                m = fmaxf(m, fabsf(modulate_one(bf16hi(R.x[j]), mu, rstd, c.z, c.w)));
            }
        }
        R = Rn;
    }
    m = block_max_nonneg<4>(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// pass 2: codes.  Dynamic: stats from pass 1 and the amax of the partials; static: stats computed
// here and the scale read from scale_in.  The codes are E4M3(y * inv) with y * inv formed in fp32 as
// fma(centered(x), rstd (1 + scale) inv, shift inv): x - mu keeps its accuracy under cancellation (see
// centered); the result is within a few fp32 ulps of the float64 modulation, which moves a code only
// where the value lies that close to a rounding midpoint.  The next row is loaded while this one is
// encoded (EXACT as in k_ln_stats).
template <int NW, bool EXACT>
__global__ void __launch_bounds__(256) k_ln_quant(const uint16_t* __restrict__ x, int L, int d,
                                                  const float* __restrict__ mod, int half, float eps,
                                                  const double2* __restrict__ stats,
                                                  const float* __restrict__ partials, int np,
                                                  const float* __restrict__ scale_in,
                                                  uint8_t* __restrict__ q,
                                                  float* __restrict__ scale_out) {
    __shared__ float4 tab[4096 / 2];
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nw = EXACT ? NW : d >> 7;
    float s, inv;
    if (scale_in) {
        s = *scale_in;
        inv = __fdiv_rn(1.0f, s);
    } else {
        float a = 0.0f;
        for (int i = threadIdx.x; i < np; i += 256) a = fmaxf(a, partials[i]);
        a = block_max_nonneg<4>(a, red);
        if (a == 0.0f) {
            s = 1.0f;
            inv = 1.0f;
        } else {
            s = __fdiv_rn(a, 448.0f);
            inv = __fdiv_rn(448.0f, a);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    load_mod_table(tab, mod, half, d, true, inv);
    auto load_row = [&](Row<NW>& D, int r) {
        const u32* xr = reinterpret_cast<const u32*>(x + (int64_t)r * d);
#pragma unroll
        for (int j = 0; j < NW; ++j)
            if (j < nw) D.x[j] = __builtin_nontemporal_load(xr + lane + 64 * j);
    };
    const int stride = gridDim.x * 4;
    Row<NW> R, Rn;
    int row = blockIdx.x * 4 + wv;
    if (row < L) load_row(R, row);
    for (; row < L; row += stride) {
        load_row(Rn, row + stride < L ? row + stride : L - 1);     // past the end: a row never used
        double mu, rstd;
        if (scale_in) {
            row_stats<NW>(R, nw, d, (double)eps, mu, rstd);
        } else {
            const double2 st = stats[row];
            mu = st.x;
            rstd = st.y;
        }
        const float rs = (float)rstd;
        const float mu_hi = (float)mu, mu_lo = (float)(mu - (double)mu_hi);
        uint16_t* qr = reinterpret_cast<uint16_t*>(q + (int64_t)row * d);
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < nw) {
                const float4 c = tab[lane + 64 * j];
                const float v0 = fmaf(centered(bf16lo(R.x[j]), mu_hi, mu_lo), rs * c.x, c.y);
                const float v1 = fmaf(centered(bf16hi(R.x[j]), mu_hi, mu_lo), rs * c.z, c.w);
                qr[lane + 64 * j] = (uint16_t)e4m3_encode2(v0, v1);
            }
        }
        R = Rn;
    }
}

// MXFP4 activations (no per-tensor scale, so one pass): y = modulate_one, the float64 modulation
// rounded once to fp32; then per 32 consecutive channels -- the 16 lanes of one row of the wave at
// one word column j -- the shared exponent and the E2M1 codes.  packed [L][d/2]: lane l writes byte
// l + 64 j of its row (channels 2(l + 64 j), +1); e8m0 [L][d/32]: the first lane of each 16-lane
// row writes block 4 j + l/16.
template <int NW>
__global__ void __launch_bounds__(256) k_ln_mx(const uint16_t* __restrict__ x, int L, int d,
                                               const float* __restrict__ mod, int half, float eps,
                                               uint8_t* __restrict__ packed, uint8_t* __restrict__ e8m0) {
    __shared__ float4 tab[64 * NW];            // sized for the row width: more workgroups per CU
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nw = d >> 7;
    load_mod_table(tab, mod, half, d, false, 1.0f);
    Row<NW> R;
    for (int row = blockIdx.x * 4 + wv; row < L; row += gridDim.x * 4) {
        const u32* xr = reinterpret_cast<const u32*>(x + (int64_t)row * d);
#pragma unroll
        for (int j = 0; j < NW; ++j)
            if (j < nw) R.x[j] = __builtin_nontemporal_load(xr + lane + 64 * j);
        double mu, rstd;
        row_stats<NW>(R, nw, d, (double)eps, mu, rstd);
        uint8_t* pr = packed + (int64_t)row * (d / 2);
        uint8_t* er = e8m0 + (int64_t)row * (d / 32);
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < nw) {
                const float4 c = tab[lane + 64 * j];
                const float y0 = modulate_one(bf16lo(R.x[j]), mu, rstd, c.x, c.y);
                const float y1 = modulate_one(bf16hi(R.x[j]), mu, rstd, c.z, c.w);
                const int k = mx_exponent(max16_nonneg(fmaxf(fabsf(y0), fabsf(y1))));
                pr[lane + 64 * j] = (uint8_t)e2m1_encode2(y0, y1, k);
                if ((lane & 15) == 0) er[4 * j + (lane >> 4)] = (uint8_t)(k + 127);
            }
        }
    }
}

// The modulated LayerNorm values themselves, y = modulate_one (the float64 modulation rounded once to
// fp32, the values every quantizer of this file encodes), for calibration: y fp32 [L][d].
template <int NW>
__global__ void __launch_bounds__(256) k_ln_f32(const uint16_t* __restrict__ x, int L, int d,
                                                const float* __restrict__ mod, int half, float eps,
                                                float* __restrict__ y) {
    __shared__ float4 tab[64 * NW];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nw = d >> 7;
    load_mod_table(tab, mod, half, d, false, 1.0f);
    Row<NW> R;
    for (int row = blockIdx.x * 4 + wv; row < L; row += gridDim.x * 4) {
        const u32* xr = reinterpret_cast<const u32*>(x + (int64_t)row * d);
#pragma unroll
        for (int j = 0; j < NW; ++j)
            if (j < nw) R.x[j] = __builtin_nontemporal_load(xr + lane + 64 * j);
        double mu, rstd;
        row_stats<NW>(R, nw, d, (double)eps, mu, rstd);
        float2* yr = reinterpret_cast<float2*>(y + (int64_t)row * d);
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < nw) {
                const float4 c = tab[lane + 64 * j];
                yr[lane + 64 * j] = make_float2(modulate_one(bf16lo(R.x[j]), mu, rstd, c.x, c.y),
                                                modulate_one(bf16hi(R.x[j]), mu, rstd, c.z, c.w));
            }
        }
    }
}

template <int NW>
static int launch_ln_f32_nw(const uint16_t* x, int L, int d, const float* mod, int half, float eps, float* y,
                            hipStream_t st) {
    int g = (L + 3) / 4;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(k_ln_f32<NW>, dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, y);
    return launch_status("adaln_layernorm_modulate_f32");
}

int launch_ln_f32(const uint16_t* x, int L, int d, const float* mod, int half, float eps, float* y,
                  hipStream_t st) {
    if (L == 0) return QVD_OK;
    switch (d >> 7) {
        case 2: return launch_ln_f32_nw<2>(x, L, d, mod, half, eps, y, st);
        case 21: return launch_ln_f32_nw<21>(x, L, d, mod, half, eps, y, st);
        default:
            if ((d >> 7) <= 8) return launch_ln_f32_nw<8>(x, L, d, mod, half, eps, y, st);
            return launch_ln_f32_nw<32>(x, L, d, mod, half, eps, y, st);
    }
}

template <int NW>
static int launch_modulate_mx_nw(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                                 uint8_t* packed, uint8_t* e8m0, hipStream_t st) {
    TimingScope ts("adaln_modulate_mxfp4", st);
    int g = (L + 3) / 4;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(k_ln_mx<NW>, dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, packed, e8m0);
    return launch_status("adaln_modulate_mxfp4");
}

int launch_modulate_mx(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                       uint8_t* packed, uint8_t* e8m0, hipStream_t st) {
    if (L == 0) return QVD_OK;
    switch (d >> 7) {
        case 2: return launch_modulate_mx_nw<2>(x, L, d, mod, half, eps, packed, e8m0, st);
        case 21: return launch_modulate_mx_nw<21>(x, L, d, mod, half, eps, packed, e8m0, st);
        default:
            if ((d >> 7) <= 8) return launch_modulate_mx_nw<8>(x, L, d, mod, half, eps, packed, e8m0, st);
            return launch_modulate_mx_nw<32>(x, L, d, mod, half, eps, packed, e8m0, st);
    }
}

constexpr int LN_GRID_STATS = 1024;
constexpr int LN_GRID_QUANT = 1024;

size_t adaln_ws_bytes(int L, int d) {
    (void)d;
    return (size_t)L * sizeof(double2) + LN_GRID_STATS * sizeof(float) + 256;
}

template <int NW>
static int launch_modulate_nw(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                              const float* scale_in, uint8_t* q, float* scale_out, void* ws,
                              hipStream_t st) {
    double2* stats = (double2*)ws;
    float* partials = (float*)((char*)ws + (((size_t)L * sizeof(double2) + 255) & ~(size_t)255));
    int np = 0;
    const int rows_per_pass = 4;
    TimingScope ts("adaln_modulate", st);
    if (!scale_in) {
        int g = (L + rows_per_pass - 1) / rows_per_pass;
        g = g < 1 ? 1 : (g > LN_GRID_STATS ? LN_GRID_STATS : g);
        if ((d >> 7) == NW)
            hipLaunchKernelGGL((k_ln_stats<NW, true>), dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, stats,
                               partials);
        else
            hipLaunchKernelGGL((k_ln_stats<NW, false>), dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, stats,
                               partials);
        np = g;
        int s = launch_status("adaln_modulate stats");
        if (s) return s;
    }
    // 1,024 workgroups (about 8 rows per wave at 480p): each builds the modulation table once, and a
    // grid of 4,096 ran the pass about 7% slower
    int g = (L + rows_per_pass - 1) / rows_per_pass;
    g = g < 1 ? 1 : (g > LN_GRID_QUANT ? LN_GRID_QUANT : g);
    if ((d >> 7) == NW)
        hipLaunchKernelGGL((k_ln_quant<NW, true>), dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, stats,
                           partials, np, scale_in, q, scale_out);
    else
        hipLaunchKernelGGL((k_ln_quant<NW, false>), dim3(g), dim3(256), 0, st, x, L, d, mod, half, eps, stats,
                           partials, np, scale_in, q, scale_out);
    return launch_status("adaln_modulate quant");
}

int launch_modulate(const uint16_t* x, int L, int d, const float* mod, int half, float eps,
                    const float* scale_in, uint8_t* q, float* scale_out, void* ws, hipStream_t st) {
    switch (d >> 7) {
        case 2: return launch_modulate_nw<2>(x, L, d, mod, half, eps, scale_in, q, scale_out, ws, st);
        case 21: return launch_modulate_nw<21>(x, L, d, mod, half, eps, scale_in, q, scale_out, ws, st);
        default:
            if ((d >> 7) <= 8)
                return launch_modulate_nw<8>(x, L, d, mod, half, eps, scale_in, q, scale_out, ws, st);
            return launch_modulate_nw<32>(x, L, d, mod, half, eps, scale_in, q, scale_out, ws, st);
    }
}

int launch_adaln_project(float t, const uint16_t* basis, int dt, const uint16_t* proj,
                         const uint16_t* bias, int d, int nb, float* mod, hipStream_t st) {
    TimingScope ts("adaln_project", st);
    hipLaunchKernelGGL(k_adaln_project, dim3((6 * d + 255) / 256, nb), dim3(256), 0, st, t, basis, dt,
                       proj, bias, d, mod);
    return launch_status("adaln_project");
}

}  // namespace qvd

using namespace qvd;

extern "C" {

int qvd_adaln_project_stack(float t, const uint16_t* basis, int32_t dt, const uint16_t* proj,
                            const uint16_t* bias, int32_t d, int32_t n_blocks, float* mod,
                            void* stream) {
    QVD_REQUIRE(dt >= 2 && dt % 2 == 0 && dt <= 16384, QVD_ESHAPE,
                "qvd_adaln_project: dt = %d (even, 2..16384)", dt);
    QVD_REQUIRE(d >= 128 && d % 128 == 0 && d <= 65536, QVD_ESHAPE,
                "qvd_adaln_project: d = %d (multiple of 128)", d);
    QVD_REQUIRE(n_blocks >= 1 && n_blocks <= 65535, QVD_ESHAPE, "qvd_adaln_project: n_blocks = %d",
                n_blocks);
    QVD_REQUIRE(t == t, QVD_EINVAL, "qvd_adaln_project: t is NaN");
    QVD_PTR(basis);
    QVD_PTR(proj);
    QVD_PTR(mod);
    QVD_ALIGN(mod);
    QVD_DEVICE_OK();
    return launch_adaln_project(t, basis, dt, proj, bias, d, n_blocks, mod, (hipStream_t)stream);
}

int qvd_adaln_project(float t, const uint16_t* basis, int32_t dt, const uint16_t* proj,
                      const uint16_t* bias, int32_t d, float* mod, void* stream) {
    return qvd_adaln_project_stack(t, basis, dt, proj, bias, d, 1, mod, stream);
}

size_t qvd_adaln_modulate_ws_bytes(int32_t L, int32_t d) {
    return L < 0 ? 0 : adaln_ws_bytes(L, d);
}

int adaln_modulate(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                   float eps, const float* act_scale_in, uint8_t* q, float* act_scale_out,
                   void* ws, size_t ws_bytes, void* stream) {
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "adaln_modulate: L = %d", L);
    QVD_REQUIRE(d >= 128 && d % 128 == 0 && d <= 4096, QVD_ESHAPE,
                "adaln_modulate: d = %d (multiple of 128, at most 4096)", d);
    QVD_REQUIRE(half == 0 || half == 1, QVD_EINVAL, "adaln_modulate: half = %d (0 or 1)", half);
    QVD_REQUIRE(eps >= 0.0f, QVD_EINVAL, "adaln_modulate: eps < 0");
    QVD_PTR(mod);
    QVD_PTR(act_scale_out);
    QVD_ALIGN(mod);
    if (L > 0) {
        QVD_PTR(x);
        QVD_PTR(q);
        QVD_ALIGN(x);
        QVD_ALIGN(q);
    }
    QVD_PTR(ws);
    QVD_ALIGN(ws);
    QVD_REQUIRE(ws_bytes >= adaln_ws_bytes(L, d), QVD_EWORKSPACE,
                "adaln_modulate: workspace %zu < %zu bytes", ws_bytes, adaln_ws_bytes(L, d));
    QVD_DEVICE_OK();
    return launch_modulate(x, L, d, mod, half, eps, act_scale_in, q, act_scale_out, ws,
                           (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Allocation-free modulate: the dynamic scale's row statistics and partial maxima (the workspace of
// adaln_modulate) live in this file-scope device array, one copy per GPU for the life of the
// process.  In host code `scratch` names a host-side stand-in, never its device memory: the device
// address comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t MODULATE_SCRATCH_BYTES = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[MODULATE_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_ptr_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QVD_EHIP, "adaln_modulate_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    QVD_REQUIRE(dev >= 0 && dev < MAX_DEVICES, QVD_EUNSUPPORTED, "adaln_modulate_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(QVD_EHIP, "adaln_modulate_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QVD_OK;
}

}  // namespace

extern "C" {

int adaln_modulate_noalloc(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                           float eps, const float* act_scale_in, uint8_t* q, float* act_scale_out,
                           void* stream) {
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "adaln_modulate_noalloc: L = %d", L);
    QVD_REQUIRE(d >= 128 && d % 128 == 0 && d <= 4096, QVD_ESHAPE,
                "adaln_modulate_noalloc: d = %d (multiple of 128, at most 4096)", d);
    QVD_REQUIRE(half == 0 || half == 1, QVD_EINVAL, "adaln_modulate_noalloc: half = %d (0 or 1)", half);
    QVD_REQUIRE(eps >= 0.0f, QVD_EINVAL, "adaln_modulate_noalloc: eps < 0");
    QVD_PTR(mod);
    QVD_PTR(act_scale_out);
    QVD_ALIGN(mod);
    if (L > 0) {
        QVD_PTR(x);
        QVD_PTR(q);
        QVD_ALIGN(x);
        QVD_ALIGN(q);
    }
    QVD_REQUIRE(act_scale_in != nullptr || adaln_ws_bytes(L, d) <= MODULATE_SCRATCH_BYTES, QVD_EWORKSPACE,
                "adaln_modulate_noalloc: L = %d needs %zu bytes of scratch; the library holds %zu per device "
                "(dynamic scales up to L = %d)", L, adaln_ws_bytes(L, d), MODULATE_SCRATCH_BYTES,
                (int)((MODULATE_SCRATCH_BYTES - adaln_ws_bytes(0, d)) / sizeof(double2)));
    QVD_DEVICE_OK();
    void* ws = nullptr;
    int s = scratch_ptr_current_device(&ws);
    if (s) return s;
    TimingOff no_events;
    return launch_modulate(x, L, d, mod, half, eps, act_scale_in, q, act_scale_out, ws, (hipStream_t)stream);
}

int adaln_layernorm_modulate_f32(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                                 float eps, float* y, void* stream) {
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "adaln_layernorm_modulate_f32: L = %d", L);
    QVD_REQUIRE(d >= 128 && d % 128 == 0 && d <= 4096, QVD_ESHAPE,
                "adaln_layernorm_modulate_f32: d = %d (multiple of 128, at most 4096)", d);
    QVD_REQUIRE(half == 0 || half == 1, QVD_EINVAL, "adaln_layernorm_modulate_f32: half = %d (0 or 1)", half);
    QVD_REQUIRE(eps >= 0.0f, QVD_EINVAL, "adaln_layernorm_modulate_f32: eps < 0");
    QVD_PTR(mod);
    QVD_ALIGN(mod);
    if (L == 0) return QVD_OK;
    QVD_PTR(x);
    QVD_PTR(y);
    QVD_ALIGN(x);
    QVD_ALIGN(y);
    QVD_DEVICE_OK();
    return launch_ln_f32(x, L, d, mod, half, eps, y, (hipStream_t)stream);
}

int adaln_modulate_mxfp4(const uint16_t* x, int32_t L, int32_t d, const float* mod, int32_t half,
                         float eps, uint8_t* packed, uint8_t* e8m0, void* stream) {
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "adaln_modulate_mxfp4: L = %d", L);
    QVD_REQUIRE(d >= 128 && d % 128 == 0 && d <= 4096, QVD_ESHAPE,
                "adaln_modulate_mxfp4: d = %d (multiple of 128, at most 4096)", d);
    QVD_REQUIRE(half == 0 || half == 1, QVD_EINVAL, "adaln_modulate_mxfp4: half = %d (0 or 1)", half);
    QVD_REQUIRE(eps >= 0.0f, QVD_EINVAL, "adaln_modulate_mxfp4: eps < 0");
    QVD_PTR(mod);
    QVD_ALIGN(mod);
    if (L > 0) {
        QVD_PTR(x);
        QVD_PTR(packed);
        QVD_PTR(e8m0);
        QVD_ALIGN(x);
    }
    QVD_DEVICE_OK();
    return launch_modulate_mx(x, L, d, mod, half, eps, packed, e8m0, (hipStream_t)stream);
}

}  // extern "C"
