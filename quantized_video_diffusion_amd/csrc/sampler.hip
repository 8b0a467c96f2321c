// The sampler around the 42-block stack: the latent state between the eight denoising steps.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么",
// training bullet (eight sampling steps at t = 999, 874, 749, 624, 500, 375, 250, 125) and section
// "在 ComfyUI 中运行" (8 steps of res_multistep, simple schedule, sigma shift 10 on video and 3 on
// audio).  The readings (the pages name the sampler but do not write it out):
//   sigma = t / 1000 under rectified flow, x_sigma = (1 - sigma) x0 + sigma eps;
//   per modality the time shift sigma' = s sigma / (1 + (s - 1) sigma), then a final sigma' = 0;
//   the stack's output is the velocity v = eps - x0 (the latent head is the identity), so
//   x0_hat = x - sigma' v;
//   res_multistep as the two-step exponential Adams-Bashforth step of the refined exponential solver
//   (Zhang, Tao & Chen 2023) in lambda = log((1 - sigma) / sigma):
//     x_next = (sigma_next / sigma) x + alpha_next [(1 - e^-h) x0_hat + (h - 1 + e^-h) / h_prev
//              (x0_hat - x0_hat_prev)],
//   first order at the first step and at the last (sigma_next = 0: x_next = x0_hat).
// The schedule's coefficients are formed on the host in double precision (a few numbers per step);
// the device pass is elementwise and bound by HBM: per element it reads v (bf16), the fp32 state
// and the previous fp32 estimate, and writes the new state, the new estimate and the bf16 copy of
// the state the next step's stack reads -- 20 bytes.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

namespace {

struct StepCoef {
    float sigma, a, b, c;   // x0_hat = x - sigma v;  x_next = a x + b x0_hat + c x0_hat_prev
};

double shifted(double t, double s) {
    const double sg = t / 1000.0;
    return s * sg / (1.0 + (s - 1.0) * sg);
}

// the n + 1 noise levels of one modality
void schedule(const qvd_sampler_config* c, double s, double* sig) {
    for (int i = 0; i < c->n_steps; ++i) {
        const double t = c->timesteps ? (double)c->timesteps[i]
                                      : std::nearbyint(999.0 - 999.0 * (double)i / (double)c->n_steps);
        sig[i] = shifted(t, s);
    }
    sig[c->n_steps] = 0.0;
}

double lam(double s) { return std::log((1.0 - s) / s); }

StepCoef coefficients(const double* sig, int i) {
    const double s0 = sig[i], s1 = sig[i + 1];
    if (s1 == 0.0) return StepCoef{(float)s0, 0.0f, 1.0f, 0.0f};
    const double h = lam(s1) - lam(s0);
    const double alpha1 = 1.0 - s1;
    double b = alpha1 * (1.0 - std::exp(-h)), c = 0.0;
    if (i > 0) {
        const double k = alpha1 * (h - 1.0 + std::exp(-h)) / (lam(s0) - lam(sig[i - 1]));
        b += k;
        c = -k;
    }
    return StepCoef{(float)s0, (float)(s1 / s0), (float)b, (float)c};
}

int validate_config(const char* fn, const qvd_sampler_config* c) {
    QVD_PTR(c);
    QVD_REQUIRE(c->n_steps >= 1 && c->n_steps <= QVD_SAMPLER_MAX_STEPS, QVD_EINVAL, "%s: n_steps = %d (1 .. %d)",
                fn, c->n_steps, QVD_SAMPLER_MAX_STEPS);
    QVD_REQUIRE(c->shift_video > 0.0f && c->shift_audio > 0.0f, QVD_EINVAL, "%s: shifts must be > 0", fn);
    QVD_REQUIRE(c->L_video >= 0, QVD_EINVAL, "%s: L_video < 0", fn);
    if (c->timesteps) {
        for (int i = 0; i < c->n_steps; ++i) {
            QVD_REQUIRE(c->timesteps[i] > 0.0f && c->timesteps[i] < 1000.0f, QVD_EINVAL,
                        "%s: timesteps[%d] = %g outside (0, 1000)", fn, i, (double)c->timesteps[i]);
            QVD_REQUIRE(i == 0 || c->timesteps[i] < c->timesteps[i - 1], QVD_EINVAL,
                        "%s: timesteps must decrease", fn);
        }
    }
    return QVD_OK;
}

}  // namespace

// x_state = sigma_0 eps (per modality), x_in = bf16(x_state).  8 elements per thread (d % 8 == 0, so
// the 8 lie in one row).
__global__ void __launch_bounds__(256) k_sampler_start(const uint16_t* __restrict__ eps, int64_t nvec, int d,
                                                       int L_video, float s0_video, float s0_audio,
                                                       float* __restrict__ x_state, uint16_t* __restrict__ x_in) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const int64_t e0 = i * 8;
        const float s0 = (e0 / d) < L_video ? s0_video : s0_audio;
        const u32x4 w = *reinterpret_cast<const u32x4*>(eps + e0);
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = s0 * bf16lo(w[k]);
            x[2 * k + 1] = s0 * bf16hi(w[k]);
        }
        float4* xs = reinterpret_cast<float4*>(x_state + e0);
        xs[0] = make_float4(x[0], x[1], x[2], x[3]);
        xs[1] = make_float4(x[4], x[5], x[6], x[7]);
        *reinterpret_cast<u32x4*>(x_in + e0) = (u32x4){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                        pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    }
}

// one step: x0_hat = x - sigma v; x_next = a x + b x0_hat + c x0_hat_prev (fp32); x_in may alias v
// (each element is read before the same thread writes it)
template <bool SECOND>
__global__ void __launch_bounds__(256) k_sampler_step(const uint16_t* v, int64_t nvec, int d, int L_video,
                                                      StepCoef cv, StepCoef ca, float* __restrict__ x_state,
                                                      float* __restrict__ x0_hat, uint16_t* x_in) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const int64_t e0 = i * 8;
        const StepCoef k = (e0 / d) < L_video ? cv : ca;
        const u32x4 vw = *reinterpret_cast<const u32x4*>(v + e0);
        const float4* xs = reinterpret_cast<const float4*>(x_state + e0);
        const float4 x0 = xs[0], x1 = xs[1];
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float pv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (SECOND) {
            const float4* ps = reinterpret_cast<const float4*>(x0_hat + e0);
            const float4 p0 = ps[0], p1 = ps[1];
            pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w;
            pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
        }
        float xh[8], xn[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xh[2 * j] = fmaf(-k.sigma, bf16lo(vw[j]), xv[2 * j]);
            xh[2 * j + 1] = fmaf(-k.sigma, bf16hi(vw[j]), xv[2 * j + 1]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float r = fmaf(k.b, xh[j], k.a * xv[j]);
            if (SECOND) r = fmaf(k.c, pv[j], r);
            xn[j] = r;
        }
        float4* xo = reinterpret_cast<float4*>(x_state + e0);
        xo[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
        xo[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
        float4* ho = reinterpret_cast<float4*>(x0_hat + e0);
        ho[0] = make_float4(xh[0], xh[1], xh[2], xh[3]);
        ho[1] = make_float4(xh[4], xh[5], xh[6], xh[7]);
        *reinterpret_cast<u32x4*>(x_in + e0) = (u32x4){pack_bf16x2(xn[0], xn[1]), pack_bf16x2(xn[2], xn[3]),
                                                        pack_bf16x2(xn[4], xn[5]), pack_bf16x2(xn[6], xn[7])};
    }
}

namespace {

int grid_of(int64_t nvec) {
    int64_t g = (nvec + 255) / 256;
    return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

int validate_tensors(const char* fn, int32_t L, int32_t d, const void* a, const void* b, const void* c) {
    QVD_REQUIRE(L >= 0, QVD_ESHAPE, "%s: L = %d", fn, L);
    QVD_REQUIRE(d >= 8 && d % 8 == 0, QVD_ESHAPE, "%s: d = %d (a positive multiple of 8)", fn, d);
    if (L == 0) return QVD_OK;
    QVD_REQUIRE(a && b && c, QVD_EINVAL, "%s: a required pointer is NULL", fn);
    QVD_REQUIRE(aligned16(a) && aligned16(b) && aligned16(c), QVD_EALIGN, "%s: tensors must be 16-byte aligned", fn);
    return QVD_OK;
}

}  // namespace

}  // namespace qvd

using namespace qvd;

extern "C" {

int qvd_sampler_sigmas(const qvd_sampler_config* c, int32_t modality, double* sigmas) {
    int s = validate_config("qvd_sampler_sigmas", c);
    if (s) return s;
    QVD_PTR(sigmas);
    QVD_REQUIRE(modality == 0 || modality == 1, QVD_EINVAL, "qvd_sampler_sigmas: modality = %d", modality);
    schedule(c, modality == 0 ? c->shift_video : c->shift_audio, sigmas);
    return QVD_OK;
}

int qvd_sampler_start(const qvd_sampler_config* c, const uint16_t* eps, int32_t L, int32_t d, float* x_state,
                      uint16_t* x_in, void* stream) {
    int s = validate_config("qvd_sampler_start", c);
    if (s) return s;
    s = validate_tensors("qvd_sampler_start", L, d, eps, x_state, x_in);
    if (s || L == 0) return s;
    QVD_DEVICE_OK();
    double sv[QVD_SAMPLER_MAX_STEPS + 1], sa[QVD_SAMPLER_MAX_STEPS + 1];
    schedule(c, c->shift_video, sv);
    schedule(c, c->shift_audio, sa);
    const int64_t nvec = (int64_t)L * d / 8;
    hipStream_t st = (hipStream_t)stream;
    TimingScope ts("sampler", st);
    hipLaunchKernelGGL(k_sampler_start, dim3(grid_of(nvec)), dim3(256), 0, st, eps, nvec, d, c->L_video,
                       (float)sv[0], (float)sa[0], x_state, x_in);
    return launch_status("qvd_sampler_start");
}

int qvd_sampler_step(const qvd_sampler_config* c, int32_t step, const uint16_t* v, float* x_state, float* x0_hat,
                     uint16_t* x_in, int32_t L, int32_t d, void* stream) {
    int s = validate_config("qvd_sampler_step", c);
    if (s) return s;
    QVD_REQUIRE(step >= 0 && step < c->n_steps, QVD_EINVAL, "qvd_sampler_step: step = %d (0 .. %d)", step,
                c->n_steps - 1);
    s = validate_tensors("qvd_sampler_step", L, d, v, x_state, x_in);
    if (s || L == 0) return s;
    QVD_PTR(x0_hat);
    QVD_ALIGN(x0_hat);
    QVD_DEVICE_OK();
    double sv[QVD_SAMPLER_MAX_STEPS + 1], sa[QVD_SAMPLER_MAX_STEPS + 1];
    schedule(c, c->shift_video, sv);
    schedule(c, c->shift_audio, sa);
    const StepCoef cv = coefficients(sv, step), ca = coefficients(sa, step);
    const int64_t nvec = (int64_t)L * d / 8;
    hipStream_t st = (hipStream_t)stream;
    TimingScope ts("sampler", st);
    if (cv.c != 0.0f || ca.c != 0.0f)
        hipLaunchKernelGGL(k_sampler_step<true>, dim3(grid_of(nvec)), dim3(256), 0, st, v, nvec, d, c->L_video,
                           cv, ca, x_state, x0_hat, x_in);
    else
        hipLaunchKernelGGL(k_sampler_step<false>, dim3(grid_of(nvec)), dim3(256), 0, st, v, nvec, d, c->L_video,
                           cv, ca, x_state, x0_hat, x_in);
    return launch_status("qvd_sampler_step");
}

}  // extern "C"
