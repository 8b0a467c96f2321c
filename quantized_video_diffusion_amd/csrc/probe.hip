// Matrix-core rate probe: a register-only loop of one MFMA kind, for the achievable peak a
// measurement reports beside the nominal one.  Every wave keeps four independent accumulator chains
// and alternates between two sets of random operands, so consecutive instructions see different
// data (the matrix cores' rate under toggling operands is below the rate on constant ones); nothing
// touches memory until the accumulators are summed into one float per wave at the end.
#include "common.h"
#include "kernels.h"

namespace qvd {

namespace {

QVD_DEV uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int KIND>
struct Mfma;

// E4M3 x E4M3, 32 x 32 x 64 (the FP8 GEMMs' instruction)
template <>
struct Mfma<QVD_PROBE_FP8> {
    typedef v8i Op;
    typedef v16f Acc;
    static constexpr double FLOPS = 2.0 * 32 * 32 * 64;
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// E2M1 x E2M1, 32 x 32 x 64 (the W4A4 GEMMs' instruction; scales 2^0)
template <>
struct Mfma<QVD_PROBE_FP4> {
    typedef v8i Op;
    typedef v16f Acc;
    static constexpr double FLOPS = 2.0 * 32 * 32 * 64;
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, 127, 0, 127);
    }
};

// INT8 x INT8 -> INT32, 16 x 16 x 64 (the attention's QK^T instruction)
template <>
struct Mfma<QVD_PROBE_INT8> {
    typedef v4i Op;
    typedef v4i Acc;
    static constexpr double FLOPS = 2.0 * 16 * 16 * 64;
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }
};

// fp16 x fp16 -> fp32, 16 x 16 x 32 (the attention's P.V instruction)
template <>
struct Mfma<QVD_PROBE_F16> {
    typedef v4i Op;
    typedef v4f Acc;
    static constexpr double FLOPS = 2.0 * 16 * 16 * 32;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0,
                                                     0, 0);
    }
};

// INT8 x INT8 -> INT32, 32 x 32 x 32
template <>
struct Mfma<QVD_PROBE_INT8_32> {
    typedef v4i Op;
    typedef v16i Acc;
    static constexpr double FLOPS = 2.0 * 32 * 32 * 32;
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

// fp16 x fp16 -> fp32, 32 x 32 x 16
template <>
struct Mfma<QVD_PROBE_F16_32> {
    typedef v4i Op;
    typedef v16f Acc;
    static constexpr double FLOPS = 2.0 * 32 * 32 * 16;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0,
                                                     0, 0);
    }
};

// E4M3 x E4M3, 16 x 16 x 128
template <>
struct Mfma<QVD_PROBE_FP8_16> {
    typedef v8i Op;
    typedef v4f Acc;
    static constexpr double FLOPS = 2.0 * 16 * 16 * 128;
    QVD_DEV static Acc run(const Op& a, const Op& b, const Acc& c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

template <class Op>
QVD_DEV Op random_op(uint32_t seed) {
    Op o;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(Op) / 4); ++i) {
        uint32_t r = mix(seed * 0x9e3779b9u + (uint32_t)i);
        o[i] = (int)(r & 0x3F3F3F3Fu);      // finite, moderate magnitudes for every element format
    }
    return o;
}

}  // namespace

template <int KIND>
__global__ void __launch_bounds__(256) k_mfma_probe(int iters, float* __restrict__ out,
                                                    unsigned long long* __restrict__ clocks) {
    typedef Mfma<KIND> M;
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    const unsigned long long c0 = clock64(), w0 = wall_clock64();
    const typename M::Op a0 = random_op<typename M::Op>(4 * t), a1 = random_op<typename M::Op>(4 * t + 1);
    const typename M::Op b0 = random_op<typename M::Op>(4 * t + 2), b1 = random_op<typename M::Op>(4 * t + 3);
    typename M::Acc acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = typename M::Acc{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = M::run((j & 1) ? a1 : a0, (j & 2) ? b1 : b0, acc[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < (int)(sizeof(acc[j]) / 4); ++e) s += (float)acc[j][e];
    out[t] = s;
    // shader-clock and constant-rate counters over the loop: their ratio is the clock the loop ran at
    if (clocks && threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = clock64() - c0;
        clocks[2 * blockIdx.x + 1] = wall_clock64() - w0;
    }
}

}  // namespace qvd

using namespace qvd;

extern "C" {

int32_t qvd_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QVD_EHIP;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return QVD_EHIP;
    return khz;
}

double qvd_mfma_probe_flops(int32_t kind, int32_t iters, int32_t workgroups) {
    double f = 0.0;
    switch (kind) {
        case QVD_PROBE_FP8: f = Mfma<QVD_PROBE_FP8>::FLOPS; break;
        case QVD_PROBE_FP4: f = Mfma<QVD_PROBE_FP4>::FLOPS; break;
        case QVD_PROBE_INT8: f = Mfma<QVD_PROBE_INT8>::FLOPS; break;
        case QVD_PROBE_F16: f = Mfma<QVD_PROBE_F16>::FLOPS; break;
        case QVD_PROBE_INT8_32: f = Mfma<QVD_PROBE_INT8_32>::FLOPS; break;
        case QVD_PROBE_F16_32: f = Mfma<QVD_PROBE_F16_32>::FLOPS; break;
        case QVD_PROBE_FP8_16: f = Mfma<QVD_PROBE_FP8_16>::FLOPS; break;
        default: return 0.0;
    }
    return f * 4.0 * (double)iters * (double)workgroups * 4.0;    // 4 waves x 4 chains per iteration
}

int qvd_mfma_probe(int32_t kind, int32_t iters, int32_t workgroups, float* out, uint64_t* clocks,
                   void* stream) {
    QVD_REQUIRE(kind >= QVD_PROBE_FP8 && kind <= QVD_PROBE_FP8_16, QVD_EINVAL, "qvd_mfma_probe: kind = %d", kind);
    QVD_REQUIRE(iters >= 1 && workgroups >= 1 && workgroups <= 65535, QVD_EINVAL,
                "qvd_mfma_probe: iters = %d, workgroups = %d", iters, workgroups);
    QVD_PTR(out);
    QVD_DEVICE_OK();
    hipStream_t st = (hipStream_t)stream;
    unsigned long long* ck = reinterpret_cast<unsigned long long*>(clocks);
    switch (kind) {
        case QVD_PROBE_FP8: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_FP8>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        case QVD_PROBE_FP4: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_FP4>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        case QVD_PROBE_INT8: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_INT8>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        case QVD_PROBE_F16: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_F16>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        case QVD_PROBE_INT8_32: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_INT8_32>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        case QVD_PROBE_F16_32: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_F16_32>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
        default: hipLaunchKernelGGL(k_mfma_probe<QVD_PROBE_FP8_16>, dim3(workgroups), dim3(256), 0, st, iters, out, ck); break;
    }
    return launch_status("qvd_mfma_probe");
}

}  // extern "C"
