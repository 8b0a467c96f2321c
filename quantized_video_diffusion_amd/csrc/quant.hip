// Quantizers: per-tensor FP8 (E4M3), per-(head, 128-token tile) INT8 for Q/K, MXFP4 weights, and
// the running-amax / clip-count reductions used to calibrate static activation scales.
//
// Per-tensor FP8 and INT8 Q/K: comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3",
// section "运行速度如何", note under the table.  Static calibrated scales and the 4-bit format:
// news.farwalk.ai FastH3 story, post 6/8.
//
// All of these kernels are bound by HBM traffic: they stream 16-byte vectors with grid-stride
// loops sized to a few workgroups per CU, and reduce in registers and LDS.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr int QBLOCK = 256;
constexpr int AMAX_PARTIALS = 1024;   // upper bound on the partial maxima a dynamic quantization uses

// ---------------------------------------------------------------------------------------------
// per-tensor amax: partial maxima per workgroup (no atomics, no zero-initialisation needed)

__global__ void __launch_bounds__(QBLOCK) k_amax_bf16(const uint16_t* __restrict__ x, int64_t n,
                                                      float* __restrict__ partials) {
    __shared__ float red[QBLOCK / 64];
    const int64_t nvec = n >> 3;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * QBLOCK + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * QBLOCK) {
        u32x4 w = __builtin_nontemporal_load(xv + i);
        u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = fmaxf(m, fmaxf(fabsf(bf16lo(ws[j])), fabsf(bf16hi(ws[j]))));
    }
    if (blockIdx.x == 0) {
        for (int64_t i = (nvec << 3) + threadIdx.x; i < n; i += QBLOCK)
            m = fmaxf(m, fabsf(bf16_to_f32(x[i])));
    }
    m = block_max_nonneg<QBLOCK / 64>(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

QVD_DEV float reduce_partials(const float* __restrict__ partials, int np, float* red) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < np; i += blockDim.x) m = fmaxf(m, partials[i]);
    return block_max_nonneg<QBLOCK / 64>(m, red);
}

// (s, inv) from a dynamic amax: s = amax/448, inv = 448/amax, both correctly rounded fp32.
QVD_DEV void fp8_scale_from_amax(float amax, float& s, float& inv) {
    if (amax == 0.0f) {
        s = 1.0f;
        inv = 1.0f;
    } else {
        s = __fdiv_rn(amax, 448.0f);
        inv = __fdiv_rn(448.0f, amax);
    }
}

// Quantize with either a static scale (scale_in != NULL) or the amax of `np` partial maxima.
__global__ void __launch_bounds__(QBLOCK) k_quant_fp8_bf16(const uint16_t* __restrict__ x, int64_t n,
                                                           const float* __restrict__ scale_in,
                                                           const float* __restrict__ partials,
                                                           int np, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale_out) {
    __shared__ float red[QBLOCK / 64];
    float s, inv;
    if (scale_in) {
        s = *scale_in;
        inv = __fdiv_rn(1.0f, s);
    } else {
        fp8_scale_from_amax(reduce_partials(partials, np, red), s, inv);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    const int64_t nvec = n >> 3;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    u32x2* qv = reinterpret_cast<u32x2*>(q);
    // QU independent 16-byte loads in flight per thread before any is consumed: one per thread left
    // the HBM pipe half empty; 8 ran the 480p GELU-sized pass 5% faster than 4, and 16 no faster
    constexpr int QU = 8;
    for (int64_t i0 = (int64_t)blockIdx.x * QBLOCK * QU + threadIdx.x; i0 < nvec;
         i0 += (int64_t)gridDim.x * QBLOCK * QU) {
        u32x4 w[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u)
            if (i0 + u * QBLOCK < nvec) w[u] = __builtin_nontemporal_load(xv + i0 + u * QBLOCK);
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            if (i0 + u * QBLOCK < nvec) {
                const u32 o0 = e4m3_encode2(bf16lo(w[u].x) * inv, bf16hi(w[u].x) * inv) |
                               (e4m3_encode2(bf16lo(w[u].y) * inv, bf16hi(w[u].y) * inv) << 16);
                const u32 o1 = e4m3_encode2(bf16lo(w[u].z) * inv, bf16hi(w[u].z) * inv) |
                               (e4m3_encode2(bf16lo(w[u].w) * inv, bf16hi(w[u].w) * inv) << 16);
                qv[i0 + u * QBLOCK] = (u32x2){o0, o1};
            }
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t i = (nvec << 3) + threadIdx.x; i < n; i += QBLOCK)
            q[i] = (uint8_t)e4m3_encode(bf16_to_f32(x[i]) * inv);
    }
}

static int grid_for(int64_t nvec, int cap) {
    int64_t g = (nvec + QBLOCK * 4 - 1) / (QBLOCK * 4);
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

int launch_quant_fp8(const uint16_t* x, int64_t n, const float* scale_in, const float* partials,
                     int np, uint8_t* q, float* scale_out, hipStream_t st) {
    const int g = grid_for(n >> 3, 2048);
    TimingScope ts("quant_fp8", st);
    hipLaunchKernelGGL(k_quant_fp8_bf16, dim3(g), dim3(QBLOCK), 0, st, x, n, scale_in, partials, np,
                       q, scale_out);
    return launch_status("quant_fp8 kernel");
}

int launch_amax_bf16(const uint16_t* x, int64_t n, float* partials, int* np_out, hipStream_t st) {
    const int g = grid_for(n >> 3, AMAX_PARTIALS);
    TimingScope ts("amax_bf16", st);
    hipLaunchKernelGGL(k_amax_bf16, dim3(g), dim3(QBLOCK), 0, st, x, n, partials);
    *np_out = g;
    return launch_status("amax kernel");
}

// ---------------------------------------------------------------------------------------------
// INT8 Q/K: one workgroup per (token tile, head); the 128 x 128 tile sits in registers between
// the amax reduction and the encode.

__global__ void __launch_bounds__(256) k_quant_int8_qk(const uint16_t* __restrict__ x, int L, int H,
                                                       int64_t row_stride, int8_t* __restrict__ q,
                                                       float* __restrict__ scale) {
    __shared__ float red[4];
    const int i = blockIdx.x, h = blockIdx.y, T = gridDim.x;
    u32x4 v[8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = threadIdx.x + 256 * j;
        const int r = i * 128 + (c >> 4);
        if (r < L) {
            v[j] = *reinterpret_cast<const u32x4*>(x + (int64_t)r * row_stride + h * 128 +
                                                   (c & 15) * 8);
            u32 ws[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                m = fmaxf(m, fmaxf(fabsf(bf16lo(ws[e])), fabsf(bf16hi(ws[e]))));
        }
    }
    const float a = block_max_nonneg<4>(m, red);
    const float inv = a == 0.0f ? 1.0f : __fdiv_rn(127.0f, a);
    if (threadIdx.x == 0) scale[h * T + i] = a == 0.0f ? 1.0f : __fdiv_rn(a, 127.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = threadIdx.x + 256 * j;
        const int r = i * 128 + (c >> 4);
        if (r < L) {
            u32 ws[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            u32 o[2] = {0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32 c0 = (u32)(int8_encode(bf16lo(ws[e]), inv) & 0xFF);
                u32 c1 = (u32)(int8_encode(bf16hi(ws[e]), inv) & 0xFF);
                o[e >> 1] |= (c0 | (c1 << 8)) << ((e & 1) * 16);
            }
            *reinterpret_cast<u32x2*>(q + ((int64_t)r * H + h) * 128 + (c & 15) * 8) =
                (u32x2){o[0], o[1]};
        }
    }
}

// ---------------------------------------------------------------------------------------------
// MXFP4 (weights, or activations per token row): one thread per 32-element block.

__global__ void __launch_bounds__(256) k_quant_mxfp4(const uint16_t* __restrict__ w, int N, int K,
                                                     uint8_t* __restrict__ packed,
                                                     uint8_t* __restrict__ e8) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int kb = K / 32;
    if (b >= (int64_t)N * kb) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(w + b * 32);
    u32 ws[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 t = src[j];
        ws[4 * j] = t.x; ws[4 * j + 1] = t.y; ws[4 * j + 2] = t.z; ws[4 * j + 3] = t.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(ws[j])), fabsf(bf16hi(ws[j]))));
    const int k = mx_exponent(amax);
    e8[b] = (uint8_t)(k + 127);
    u32 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = e2m1_encode8_bf16(ws + 4 * j, k);
    *reinterpret_cast<u32x4*>(packed + b * 16) = (u32x4){o[0], o[1], o[2], o[3]};
}

// ---------------------------------------------------------------------------------------------
// calibration reductions

QVD_DEV float load_f32(const float* x, int64_t i) { return x[i]; }
QVD_DEV float load_f32(const uint16_t* x, int64_t i) { return bf16_to_f32(x[i]); }

template <class T>
__global__ void __launch_bounds__(QBLOCK) k_amax_update(const T* __restrict__ x, int64_t n,
                                                        float* __restrict__ amax) {
    __shared__ float red[QBLOCK / 64];
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * QBLOCK + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * QBLOCK)
        m = fmaxf(m, fabsf(load_f32(x, i)));
    m = block_max_nonneg<QBLOCK / 64>(m, red);
    if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
}

// Static scale from a calibration amax: s = fp32(amax / 448) (correctly rounded), raised to the next
// fp32 value when 448 s (exact in float64) falls below amax, so that no calibration value clips;
// amax = 0 gives 1.
__global__ void __launch_bounds__(256) k_calibrated_scale(const float* __restrict__ amax,
                                                          float* __restrict__ scale, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float a = amax[i];
    float s = 1.0f;
    if (a != 0.0f) {
        s = __fdiv_rn(a, 448.0f);
        if ((double)s * 448.0 < (double)a) s = nextafterf(s, INFINITY);
    }
    scale[i] = s;
}

template <class T>
__global__ void __launch_bounds__(QBLOCK) k_clip_count(const T* __restrict__ x, int64_t n,
                                                       const float* __restrict__ scale,
                                                       unsigned long long* __restrict__ count) {
    __shared__ unsigned long long red[QBLOCK / 64];
    const double thr = (double)(*scale) * 448.0;
    unsigned long long c = 0;
    for (int64_t i = (int64_t)blockIdx.x * QBLOCK + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * QBLOCK)
        c += ((double)fabsf(load_f32(x, i)) > thr) ? 1ull : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < QBLOCK / 64; ++w) t += red[w];
        if (t) atomicAdd(count, t);
    }
}

}  // namespace qvd

using namespace qvd;

extern "C" {

size_t qvd_quant_ws_bytes(int64_t n) {
    (void)n;
    return AMAX_PARTIALS * sizeof(float);
}

int quant_fp8_per_tensor(const uint16_t* x, int64_t n, const float* scale_in, uint8_t* q,
                         float* scale_out, void* ws, size_t ws_bytes, void* stream) {
    QVD_REQUIRE(n >= 0, QVD_ESHAPE, "quant_fp8_per_tensor: n = %lld < 0", (long long)n);
    QVD_PTR(scale_out);
    if (n > 0) {
        QVD_PTR(x);
        QVD_PTR(q);
        QVD_ALIGN(x);
        QVD_ALIGN(q);
    }
    if (!scale_in) {
        QVD_PTR(ws);
        QVD_ALIGN(ws);
        QVD_REQUIRE(ws_bytes >= qvd_quant_ws_bytes(n), QVD_EWORKSPACE,
                    "quant_fp8_per_tensor: workspace %zu < %zu bytes", ws_bytes,
                    qvd_quant_ws_bytes(n));
    }
    QVD_DEVICE_OK();
    hipStream_t st = (hipStream_t)stream;
    int np = 0;
    float* partials = (float*)ws;
    if (!scale_in) {
        int s = launch_amax_bf16(x, n, partials, &np, st);
        if (s) return s;
    }
    return launch_quant_fp8(x, n, scale_in, partials, np, q, scale_out, st);
}

int quant_int8_qk(const uint16_t* x, int32_t L, int32_t H, int32_t head_dim, int32_t tile,
                  int64_t row_stride, int8_t* q, float* scale, void* stream) {
    QVD_REQUIRE(head_dim == 128 && tile == 128, QVD_ESHAPE,
                "quant_int8_qk: head_dim = %d, tile = %d (both must be 128)", head_dim, tile);
    QVD_REQUIRE(L >= 0 && H >= 1 && H <= 65535, QVD_ESHAPE, "quant_int8_qk: L = %d, H = %d", L, H);
    QVD_REQUIRE(row_stride >= (int64_t)H * 128 && row_stride % 8 == 0, QVD_ESHAPE,
                "quant_int8_qk: row_stride = %lld (needs >= H*128 and a multiple of 8)",
                (long long)row_stride);
    if (L == 0) return QVD_OK;
    QVD_PTR(x);
    QVD_PTR(q);
    QVD_PTR(scale);
    QVD_ALIGN(x);
    QVD_ALIGN(q);
    QVD_DEVICE_OK();
    const int T = (L + 127) / 128;
    TimingScope ts("quant_int8_qk", (hipStream_t)stream);
    hipLaunchKernelGGL(k_quant_int8_qk, dim3(T, H), dim3(256), 0, (hipStream_t)stream, x, L, H,
                       row_stride, q, scale);
    return launch_status("quant_int8_qk");
}

int qvd_quant_mxfp4(const uint16_t* w, int32_t N, int32_t K, uint8_t* packed, uint8_t* e8m0,
                    void* stream) {
    QVD_REQUIRE(N >= 0 && K >= 0 && K % 32 == 0, QVD_ESHAPE, "qvd_quant_mxfp4: N = %d, K = %d", N, K);
    if ((int64_t)N * K == 0) return QVD_OK;
    QVD_PTR(w);
    QVD_PTR(packed);
    QVD_PTR(e8m0);
    QVD_ALIGN(w);
    QVD_ALIGN(packed);
    QVD_DEVICE_OK();
    const int64_t nb = (int64_t)N * (K / 32);
    hipLaunchKernelGGL(k_quant_mxfp4, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, w, N, K, packed, e8m0);
    return launch_status("qvd_quant_mxfp4");
}

int qvd_calibrated_scale(const float* amax, float* scale, int32_t n, void* stream) {
    QVD_REQUIRE(n >= 0, QVD_ESHAPE, "qvd_calibrated_scale: n < 0");
    if (n == 0) return QVD_OK;
    QVD_PTR(amax);
    QVD_PTR(scale);
    QVD_DEVICE_OK();
    hipLaunchKernelGGL(k_calibrated_scale, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, amax,
                       scale, n);
    return launch_status("qvd_calibrated_scale");
}

}  // extern "C"

namespace {

template <class T>
int amax_update(const char* fn, const T* x, int64_t n, float* amax, void* stream) {
    QVD_REQUIRE(n >= 0, QVD_ESHAPE, "%s: n < 0", fn);
    if (n == 0) return QVD_OK;
    QVD_PTR(x);
    QVD_PTR(amax);
    QVD_DEVICE_OK();
    hipLaunchKernelGGL(k_amax_update<T>, dim3(grid_for(n / 8, 2048)), dim3(QBLOCK), 0,
                       (hipStream_t)stream, x, n, amax);
    return launch_status(fn);
}

template <class T>
int clip_count(const char* fn, const T* x, int64_t n, const float* scale, uint64_t* count, void* stream) {
    QVD_REQUIRE(n >= 0, QVD_ESHAPE, "%s: n < 0", fn);
    if (n == 0) return QVD_OK;
    QVD_PTR(x);
    QVD_PTR(scale);
    QVD_PTR(count);
    QVD_DEVICE_OK();
    hipLaunchKernelGGL(k_clip_count<T>, dim3(grid_for(n / 8, 2048)), dim3(QBLOCK), 0,
                       (hipStream_t)stream, x, n, scale, (unsigned long long*)count);
    return launch_status(fn);
}

}  // namespace

extern "C" {

int qvd_amax_update(const float* x, int64_t n, float* amax, void* stream) {
    return amax_update("qvd_amax_update", x, n, amax, stream);
}

int qvd_amax_update_bf16(const uint16_t* x, int64_t n, float* amax, void* stream) {
    return amax_update("qvd_amax_update_bf16", x, n, amax, stream);
}

int qvd_clip_count(const float* x, int64_t n, const float* scale, uint64_t* count, void* stream) {
    return clip_count("qvd_clip_count", x, n, scale, count, stream);
}

int qvd_clip_count_bf16(const uint16_t* x, int64_t n, const float* scale, uint64_t* count, void* stream) {
    return clip_count("qvd_clip_count_bf16", x, n, scale, count, stream);
}

}  // extern "C"
