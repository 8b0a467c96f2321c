// Shared device helpers and host-side argument checking for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "../../include/qvd.h"

// ---------------------------------------------------------------------------------------------
// vector types for MFMA operands

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define QVD_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------------
// bf16

QVD_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((u32)b) << 16); }
QVD_DEV float bf16lo(u32 w) { return __uint_as_float(w << 16); }
QVD_DEV float bf16hi(u32 w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
QVD_DEV u32 pack_bf16x2(float lo, float hi) {
    v2bf r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(u32, r);
}

// ---------------------------------------------------------------------------------------------
// V in fp16 for the attention's P.V product.  One (head, 128-token tile) of V is stored as fp16 of
// v 2^-e, with e = 0 while the tile's max|v| lies in [2^-6, 2^15) (fp16's normal range then holds
// everything down to 2^-20 of the maximum), else e = floor(log2 max|v|) - 14, which brings the
// maximum into [2^14, 2^15), below fp16's largest value 65,504.  An all-zero or non-finite maximum
// takes e = 0.  A bf16 value scaled by a power of two converts to fp16 exactly while it stays an fp16
// normal (bf16 has 8 significant bits, fp16 11).

QVD_DEV int vt_tile_exponent(float amax) {
    if (!(amax > 0.0f) || !(amax < 3.0e38f) || (amax >= 0x1p-6f && amax < 32768.0f)) return 0;
    int k;
    frexpf(amax, &k);                      // amax = f 2^k, f in [0.5, 1): floor(log2 amax) = k - 1
    return k - 15;
}

QVD_DEV uint16_t f16_scaled(float v, int e) {
    return __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v, -e));
}

// ---------------------------------------------------------------------------------------------
// E4M3 ("FN") encoding.
// fp32 -> E4M3 (OCP "FN"): round to nearest even, finite values beyond 448 saturate to +-448, NaN -> 0x7F.
// The gfx950 converter rounds to nearest even; clamping to +-448 first makes it saturate (the pair
// agrees with a direct implementation of the rule on all 2^32 fp32 inputs, checked on the device).
QVD_DEV u32 e4m3_encode2(float a, float b) {
    const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    u32 r = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (a != a) r = (r & 0xFF00u) | 0x7Fu;
    if (b != b) r = (r & 0x00FFu) | 0x7F00u;
    return r;
}

QVD_DEV u32 e4m3_encode(float v) { return e4m3_encode2(v, v) & 0xFFu; }

QVD_DEV int int8_encode(float x, float inv) {
    float p = x * inv;                                     // one fp32 product (no contraction)
    float r = __builtin_rintf(p);
    r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
    return (int)r;
}

// ---------------------------------------------------------------------------------------------
// MXFP4 (OCP MX v1.0 elements E2M1 with one E8M0 scale per 32 consecutive values).  The block scale
// is X = 2^k with k = floor(log2 amax) - 2 (2 is the exponent of E2M1's largest value, 6), clamped to
// E8M0's [-127, 127]; an all-zero block takes k = 0.  Elements are E2M1(v / X): round to nearest
// even on the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6, saturating at 6; sign in bit 3.

QVD_DEV int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e;
    frexpf(amax, &e);                      // amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
    const int k = e - 3;
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// The gfx950 converter v_cvt_scalef32_pk_fp4_f32 turns two fp32 values into two E2M1 codes (value /
// scale, round to nearest even, saturating at 6, first value in the low nibble) and writes them into
// the selected byte of a 32-bit register.  Called with scale 1 on values already multiplied by 2^-k
// (ldexp is exact here: a result below 2^-126 codes to zero either way), it agrees with the rounding
// rule above on every finite fp32 input (checked exhaustively on the device).

// two elements of one block -> one byte (first element in the low nibble)
QVD_DEV u32 e2m1_encode2(float a, float b, int k) {
    return (u32)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ldexpf(a, -k), ldexpf(b, -k), 1.0f, 0) & 0xFFu;
}

// eight consecutive elements of one block (bf16 pairs w[0..3]) -> one word (element i in bits 4i..4i+3)
QVD_DEV u32 e2m1_encode8_bf16(const u32* w, int k) {
    u32 r = 0u;
    r = (u32)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(bf16lo(w[0]), -k), ldexpf(bf16hi(w[0]), -k), 1.0f, 0);
    r = (u32)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(bf16lo(w[1]), -k), ldexpf(bf16hi(w[1]), -k), 1.0f, 1);
    r = (u32)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(bf16lo(w[2]), -k), ldexpf(bf16hi(w[2]), -k), 1.0f, 2);
    r = (u32)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(bf16lo(w[3]), -k), ldexpf(bf16hi(w[3]), -k), 1.0f, 3);
    return r;
}

// max of non-negative floats over each row of 16 lanes (DPP: swap neighbours, swap pairs, then the
// half-row and row mirrors)
QVD_DEV float max16_nonneg(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// ---------------------------------------------------------------------------------------------
// wave / block reductions (wave64)

QVD_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
QVD_DEV double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// max of non-negative floats over the block; every thread gets the result.  `red` holds one
// float per wave.
template <int NWAVES>
QVD_DEV float block_max_nonneg(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) m = fmaxf(m, red[i]);
    return m;
}

// ---------------------------------------------------------------------------------------------
// host side

namespace qvd {

void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
int check_device();                       // gfx950 check, cached per device
int launch_status(const char* what);      // hipGetLastError after a launch -> QVD_OK / QVD_EHIP

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }

}  // namespace qvd

#define QVD_REQUIRE(cond, status, ...)                              \
    do {                                                            \
        if (!(cond)) return qvd::fail((status), __VA_ARGS__);       \
    } while (0)

#define QVD_PTR(p) QVD_REQUIRE((p) != nullptr, QVD_EINVAL, "%s: %s is NULL", __func__, #p)
#define QVD_ALIGN(p) \
    QVD_REQUIRE(qvd::aligned16(p), QVD_EALIGN, "%s: %s is not 16-byte aligned", __func__, #p)
#define QVD_DEVICE_OK()                              \
    do {                                             \
        int _s = qvd::check_device();                \
        if (_s != QVD_OK) return _s;                 \
    } while (0)
