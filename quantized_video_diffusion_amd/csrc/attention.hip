// Block-sparse attention with INT8 query/key scores on the gfx950 matrix cores.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么",
// training bullet (the model runs with 80% attention sparsity) and section "运行速度如何", note under
// the table (query and key are quantized to INT8 for the score computation).
//
// One workgroup per (query tile of 128 rows, head); four waves of 32 query rows.  Two passes over
// the kept key tiles:
//   pass 1: stage K (int8, 16 KB, XOR-swizzled 16-byte chunks) in LDS, S^T = K . Q^T with
//           v_mfma_i32_16x16x64_i8 (exact int32; Q fragments stay in registers), keep each query
//           row's maximum of S * sQ*sK*sm_scale*log2(e);
//   pass 2: stage K and V (transposed, fp16, rows padded to 264 bytes), recompute S^T, numerators
//           exp2(s - m) rounded to fp16 against the final row maximum, their sum, and
//           O^T += V^T . P^T with v_mfma_f32_16x16x32_f16 (fp32 accumulation).
// Rounding the numerators against the final maximum (rather than a running one) makes every
// rounding decision a function of the scores alone, so the result reproduces the reading the
// oracle states: fp16 numerators, exact normalisation by their sum.
// P.V runs in fp16 rather than bf16: P lies in [0, 1], where fp16 keeps 3 more significand bits than
// bf16, and V (bf16, 8 significant bits) converts to fp16 exactly inside fp16's normal range.
// Computing the transposed products makes every lane own one query row in both MFMA outputs, so the
// row statistics never move between lanes except for the 4-way sum/max across lane groups.
// Masked key tiles are never loaded or multiplied.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr int VT_STRIDE = 132;                 // bf16 elements per transposed-V row (128 + 4 pad)
constexpr float LOG2E = 1.4426950408889634f;

struct AttnSmem {
    int8_t k[128 * 128];
    uint16_t vt[128 * VT_STRIDE];     // fp16 bit patterns
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// two bf16 values -> packed fp16 pair (exact for 2^-14 <= |v| <= 65504; larger magnitudes saturate)
QVD_DEV u32 bf16pair_to_f16pair(float a, float b) {
    a = fminf(fmaxf(a, -65504.0f), 65504.0f);
    b = fminf(fmaxf(b, -65504.0f), 65504.0f);
    return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(a, b));
}

QVD_DEV u32 pack_f16x2(float lo, float hi) {
    v2h r;
    r.x = (_Float16)lo;
    r.y = (_Float16)hi;
    return __builtin_bit_cast(u32, r);
}
QVD_DEV float f16lo(u32 w) { return (float)__builtin_bit_cast(v2h, w).x; }
QVD_DEV float f16hi(u32 w) { return (float)__builtin_bit_cast(v2h, w).y; }

// Q fragments of this wave (B operand): qf[qb][ks] = Q[q0 + 16 qb + fr][h][64 ks + 16 fg .. +15]
QVD_DEV void load_q_frags(const int8_t* __restrict__ q, int L, int H, int h, int q0, int fr, int fg,
                          v4i qf[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int row = q0 + 16 * qb + fr;
        row = row < L ? row : L - 1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            qf[qb][ks] = *reinterpret_cast<const v4i*>(q + ((int64_t)row * H + h) * 128 + 64 * ks + 16 * fg);
    }
}

// K tile j -> LDS (rows past L repeat row L-1; their scores are masked)
QVD_DEV void stage_k(AttnSmem& sm, const int8_t* __restrict__ k, int L, int H, int h, int j, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = tid + 256 * u;
        const int row = c >> 3, ch = c & 7;
        int kr = j * 128 + row;
        kr = kr < L ? kr : L - 1;
        const v4i val = *reinterpret_cast<const v4i*>(k + ((int64_t)kr * H + h) * 128 + 16 * ch);
        *reinterpret_cast<v4i*>(sm.k + row * 128 + ((ch ^ (row & 7)) << 4)) = val;
    }
}

// V tile j -> LDS transposed and converted to fp16: vt[dim][key].  Thread t handles key pair (t & 63) and dim chunks
// (t >> 6) + 4u of 8 dims; each 32-bit LDS write holds (key 2p, key 2p+1) of one dim.
QVD_DEV void stage_v(AttnSmem& sm, const uint16_t* __restrict__ v, int L, int H, int h, int j, int tid) {
    const int kp = tid & 63, c0 = tid >> 6;
    int r0 = j * 128 + 2 * kp, r1 = r0 + 1;
    r0 = r0 < L ? r0 : L - 1;
    r1 = r1 < L ? r1 : L - 1;
    const uint16_t* v0 = v + ((int64_t)r0 * H + h) * 128;
    const uint16_t* v1 = v + ((int64_t)r1 * H + h) * 128;
    u32* vt = reinterpret_cast<u32*>(sm.vt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int cc = c0 + 4 * u;
        const u32x4 a = *reinterpret_cast<const u32x4*>(v0 + 8 * cc);
        const u32x4 b = *reinterpret_cast<const u32x4*>(v1 + 8 * cc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 8 * cc + 2 * e;
            vt[(d * VT_STRIDE + 2 * kp) >> 1] = bf16pair_to_f16pair(bf16lo(a[e]), bf16lo(b[e]));
            vt[((d + 1) * VT_STRIDE + 2 * kp) >> 1] = bf16pair_to_f16pair(bf16hi(a[e]), bf16hi(b[e]));
        }
    }
}

// S^T = K . Q^T for this wave: s[qb][kb][r] = score(query q0 + 16 qb + fr, key 16 kb + 4 fg + r)
QVD_DEV void qk_scores(const AttnSmem& sm, const v4i qf[2][2], int fr, int fg, v4i s[2][8]) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int row = 16 * kb + fr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const v4i kf = *reinterpret_cast<const v4i*>(sm.k + row * 128 + (((4 * ks + fg) ^ (row & 7)) << 4));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const v4i c = ks == 0 ? (v4i){0, 0, 0, 0} : s[qb][kb];
                s[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qf[qb][ks], c, 0, 0, 0);
            }
        }
    }
}

template <bool WRITE_AMAX>
__global__ void __launch_bounds__(256, 2) k_sparse_attn(
    const int8_t* __restrict__ q, const float* __restrict__ q_scale, const int8_t* __restrict__ k,
    const float* __restrict__ k_scale, const uint16_t* __restrict__ v, int L, int H,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int kmax, float c_log2,
    uint16_t* __restrict__ out, float* __restrict__ amax_partials) {
    __shared__ AttnSmem sm;
    __shared__ float red[4];
    const int i = blockIdx.x, h = blockIdx.y, T = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const int q0 = i * 128 + 32 * wv;

    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    const float qsc = q_scale[h * T + i] * c_log2;
    int cnt = kv_cnt[h * T + i];
    cnt = cnt < 0 ? 0 : (cnt > kmax ? kmax : cnt);
    const int32_t* list = kv_idx + ((int64_t)h * T + i) * kmax;

    // pass 1: the maximum of every query row over all kept keys (scores only, K staged alone)
    float m[2] = {-INFINITY, -INFINITY};
    for (int t = 0; t < cnt; ++t) {
        const int j = list[t];
        if (j < 0 || j >= T) continue;
        __syncthreads();
        stage_k(sm, k, L, H, h, j, tid);
        __syncthreads();
        v4i s[2][8];
        qk_scores(sm, qf, fr, fg, s);
        const float c = qsc * k_scale[h * T + j];
        const bool ragged = (j == T - 1) && (L & 127);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            int mx = INT_MIN;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = !ragged || (j * 128 + 16 * kb + 4 * fg + r) < L;
                    mx = ok ? max(mx, s[qb][kb][r]) : mx;
                }
            if (mx != INT_MIN) m[qb] = fmaxf(m[qb], (float)mx * c);
        }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        m[qb] = fmaxf(m[qb], __shfl_xor(m[qb], 16, 64));
        m[qb] = fmaxf(m[qb], __shfl_xor(m[qb], 32, 64));
    }

    // pass 2: numerators exp2(s - m) rounded to fp16, their sum, and P.V
    float l[2] = {0.0f, 0.0f};
    v4f o[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) o[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < cnt; ++t) {
        const int j = list[t];
        if (j < 0 || j >= T) continue;
        __syncthreads();                       // the previous tile's LDS reads are done
        stage_k(sm, k, L, H, h, j, tid);
        stage_v(sm, v, L, H, h, j, tid);
        __syncthreads();

        v4i s[2][8];
        qk_scores(sm, qf, fr, fg, s);

        const float c = qsc * k_scale[h * T + j];
        const bool ragged = (j == T - 1) && (L & 127);
        v8h pb[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mq = m[qb];
            float lsum = 0.0f;
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                u32 w[4];
#pragma unroll
                for (int hlf = 0; hlf < 2; ++hlf) {
                    const int kb = 2 * kp + hlf;
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool ok = !ragged || (j * 128 + 16 * kb + 4 * fg + r) < L;
                        p[r] = ok ? __builtin_amdgcn_exp2f(fmaf((float)s[qb][kb][r], c, -mq)) : 0.0f;
                    }
                    const u32 w0 = pack_f16x2(p[0], p[1]);
                    const u32 w1 = pack_f16x2(p[2], p[3]);
                    lsum += (f16lo(w0) + f16hi(w0)) + (f16lo(w1) + f16hi(w1));
                    w[2 * hlf] = w0;
                    w[2 * hlf + 1] = w1;
                }
                const v4i pw = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                pb[qb][kp] = __builtin_bit_cast(v8h, pw);
            }
            l[qb] += lsum;
        }

#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const uint16_t* vrow = sm.vt + (16 * db + fr) * VT_STRIDE;
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                const v2i lo = *reinterpret_cast<const v2i*>(vrow + 32 * kp + 4 * fg);
                const v2i hi = *reinterpret_cast<const v2i*>(vrow + 32 * kp + 16 + 4 * fg);
                const v4i vw = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
                const v8h vf = __builtin_bit_cast(v8h, vw);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[qb][kp], o[qb][db], 0, 0, 0);
            }
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float lt = l[qb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int row = q0 + 16 * qb + fr;
        if (row < L) {
            uint16_t* orow = out + ((int64_t)row * H + h) * 128;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const v4f c = o[qb][db];
                const u32 w0 = pack_bf16x2(c[0] * inv, c[1] * inv);
                const u32 w1 = pack_bf16x2(c[2] * inv, c[3] * inv);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16lo(w0)), fabsf(bf16hi(w0))),
                                         fmaxf(fabsf(bf16lo(w1)), fabsf(bf16hi(w1)))));
                *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * fg) = (u32x2){w0, w1};
            }
        }
    }
    if (WRITE_AMAX) {
        amax = block_max_nonneg<4>(amax, red);
        if (tid == 0) amax_partials[h * T + i] = amax;
    }
}

// The INT32 accumulators of one (query tile, key tile) pair through the same tile routines.
__global__ void __launch_bounds__(256) k_qk_tile(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                 int L, int H, int h, int i, int j,
                                                 int32_t* __restrict__ out) {
    __shared__ AttnSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const int q0 = i * 128 + 32 * wv;
    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    stage_k(sm, k, L, H, h, j, tid);
    __syncthreads();
    v4i s[2][8];
    qk_scores(sm, qf, fr, fg, s);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 32 * wv + 16 * qb + fr, cc = 16 * kb + 4 * fg + r;
                const bool ok = (i * 128 + rr) < L && (j * 128 + cc) < L;
                out[rr * 128 + cc] = ok ? s[qb][kb][r] : 0;
            }
}

int launch_sparse_attn(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                       const uint16_t* v, int L, int H, const int32_t* kv_idx, const int32_t* kv_cnt,
                       int kmax, float sm_scale, uint16_t* out, float* amax_partials, hipStream_t st) {
    if (L == 0) return QVD_OK;
    const int T = (L + 127) / 128;
    const float c = sm_scale * LOG2E;
    TimingScope ts("sparse_attn", st);
    if (amax_partials)
        hipLaunchKernelGGL(k_sparse_attn<true>, dim3(T, H), dim3(256), 0, st, q, q_scale, k, k_scale, v,
                           L, H, kv_idx, kv_cnt, kmax, c, out, amax_partials);
    else
        hipLaunchKernelGGL(k_sparse_attn<false>, dim3(T, H), dim3(256), 0, st, q, q_scale, k, k_scale, v,
                           L, H, kv_idx, kv_cnt, kmax, c, out, amax_partials);
    return launch_status("sparse_attn");
}

}  // namespace qvd

using namespace qvd;

extern "C" {

int sparse_attn(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                const uint16_t* v, int32_t L, int32_t H, int32_t head_dim,
                const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                uint16_t* out, float* out_amax_partials, void* stream) {
    QVD_REQUIRE(head_dim == 128, QVD_ESHAPE, "sparse_attn: head_dim = %d (must be 128)", head_dim);
    QVD_REQUIRE(L >= 0 && H >= 1 && H <= 65535, QVD_ESHAPE, "sparse_attn: L = %d, H = %d", L, H);
    QVD_REQUIRE(L <= (1 << 30) / 128 * 128, QVD_ESHAPE, "sparse_attn: L = %d too large", L);
    QVD_REQUIRE(kmax >= 1, QVD_ESHAPE, "sparse_attn: kmax = %d", kmax);
    QVD_REQUIRE(sm_scale > 0.0f && sm_scale < 1e30f, QVD_EINVAL, "sparse_attn: sm_scale out of range");
    if (L == 0) return QVD_OK;
    QVD_PTR(q);
    QVD_PTR(q_scale);
    QVD_PTR(k);
    QVD_PTR(k_scale);
    QVD_PTR(v);
    QVD_PTR(kv_idx);
    QVD_PTR(kv_cnt);
    QVD_PTR(out);
    QVD_ALIGN(q);
    QVD_ALIGN(k);
    QVD_ALIGN(v);
    QVD_ALIGN(out);
    QVD_DEVICE_OK();
    return launch_sparse_attn(q, q_scale, k, k_scale, v, L, H, kv_idx, kv_cnt, kmax, sm_scale, out,
                              out_amax_partials, (hipStream_t)stream);
}

int qvd_qk_int32_tile(const int8_t* q, const int8_t* k, int32_t L, int32_t H, int32_t h,
                      int32_t i, int32_t j, int32_t* out, void* stream) {
    QVD_REQUIRE(L >= 1 && H >= 1, QVD_ESHAPE, "qvd_qk_int32_tile: L = %d, H = %d", L, H);
    const int T = (L + 127) / 128;
    QVD_REQUIRE(h >= 0 && h < H && i >= 0 && i < T && j >= 0 && j < T, QVD_EINVAL,
                "qvd_qk_int32_tile: (h, i, j) = (%d, %d, %d) outside (%d, %d, %d)", h, i, j, H, T, T);
    QVD_PTR(q);
    QVD_PTR(k);
    QVD_PTR(out);
    QVD_ALIGN(q);
    QVD_ALIGN(k);
    QVD_DEVICE_OK();
    hipLaunchKernelGGL(k_qk_tile, dim3(1), dim3(256), 0, (hipStream_t)stream, q, k, L, H, h, i, j, out);
    return launch_status("qvd_qk_int32_tile");
}

}  // extern "C"
