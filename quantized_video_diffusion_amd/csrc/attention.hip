// Block-sparse attention with INT8 query/key scores on the gfx950 matrix cores.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么",
// training bullet (the model runs with 80% attention sparsity) and section "运行速度如何", note under
// the table (query and key are quantized to INT8 for the score computation).
//
// One workgroup per (query tile of 128 rows, head); four waves of 32 query rows.  Two passes over
// the kept key tiles (masked tiles are never loaded or multiplied):
//   pass 1: K tile -> LDS; S^T = K . Q^T with v_mfma_i32_16x16x64_i8 (exact int32, Q fragments in
//           registers); each query row keeps its maximum of S * sQ*sK*sm_scale*log2(e);
//   pass 2: K and V^T tiles -> LDS; S^T again; numerators exp2(s - max) rounded to fp16 against the
//           final row maximum; O^T += V^T . P^T with v_mfma_f32_16x16x32_f16 and the numerator
//           sum as ones . P^T on the same unit (fp32 accumulation).
// Rounding against the final maximum makes every rounding decision a function of the scores alone:
// the result is the oracle's reading (fp16 numerators, exact normalisation by their sum) up to the
// fp32 accumulation order.
//
// Staging: tiles move HBM/L2 -> LDS with global_load_lds_dwordx4 (no register round trip).  Each
// lane picks the global 16-byte chunk that belongs at its LDS slot, which applies an XOR swizzle:
// K rows (128 B) swizzle chunks by row & 7, V^T rows (256 B, fp16, keys contiguous) by row & 15,
// so the 16-row MFMA fragment reads hit distinct banks.  V arrives transposed and in fp16 from the
// QKV GEMM epilogue (or from a conversion pass for bf16 callers).  Computing the transposed products
// makes each lane own one query row in both MFMA outputs.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr float LOG2E = 1.4426950408889634f;

constexpr int MAX_KEPT = 1024;      // longest kept-tile list a workgroup takes (kmax bound)

struct AttnSmem {
    int8_t k[2][128 * 128];         // 2 x 16 KB: double-buffered K tiles
    uint16_t vt[128 * 128];         // 32 KB, fp16 bit patterns
    int tiles[MAX_KEPT];            // the valid entries of this row's kept-tile list, in order
    int wcount[4];
    float red[4];                   // block reduction of max|O|
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

QVD_DEV u32 pack_f16x2(float lo, float hi) {
    v2h r;
    r.x = (_Float16)lo;
    r.y = (_Float16)hi;
    return __builtin_bit_cast(u32, r);
}

QVD_DEV void dma16(const void* g, void* lds_slot_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_slot_base, 16, 0, 0);
}

QVD_DEV void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// wait until at most 4 DMA/vector loads are outstanding (the 4 K-tile loads issued last)
QVD_DEV void dma_wait_but_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }

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

// K tile j -> LDS.  Wave w, instruction u fills LDS rows (4w + u)*8 .. +7; lane l lands in row
// r = (4w+u)*8 + l/8, slot l%8, and fetches chunk (l%8) ^ (r & 7) of key row j*128 + r (clamped).
QVD_DEV void stage_k(int8_t* kbuf, const int8_t* __restrict__ k, int L, int H, int h, int j,
                     int wv, int lane) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int blk = 4 * wv + u;
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        int kr = j * 128 + r;
        kr = kr < L ? kr : L - 1;
        const uint32_t off = ((uint32_t)kr * (uint32_t)H + (uint32_t)h) * 128u + (uint32_t)(16 * c);
        dma16(k + off, kbuf + blk * 1024);
    }
}

// V^T tile j -> LDS.  vt rows are (head, dim), Lp keys each.  Wave w, instruction u fills LDS rows
// (8w + u)*4 .. +3 (256 B each); lane l lands in row d = (8w+u)*4 + l/16, slot l%16, and fetches
// chunk (l%16) ^ (d & 15) of keys j*128 .. j*128+127.
// (32-bit offsets: H*128*Lp*2 bytes stays far below 2^32 for every L the launcher accepts)
QVD_DEV void stage_vt(AttnSmem& sm, const uint16_t* __restrict__ vt, int Lp, int h, int j,
                      int wv, int lane) {
    const char* base = reinterpret_cast<const char*>(vt) + (size_t)j * 256u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int blk = 8 * wv + u;
        const int d = blk * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (d & 15);
        const uint32_t off = ((uint32_t)(h * 128 + d) * (uint32_t)Lp + (uint32_t)(8 * c)) * 2u;
        dma16(base + off, sm.vt + blk * 512);
    }
}

// S^T = K . Q^T for this wave: s[qb][kb][r] = score(query q0 + 16 qb + fr, key 16 kb + 4 fg + r)
QVD_DEV void qk_scores(const int8_t* kbuf, const v4i qf[2][2], int fr, int fg, v4i s[2][8]) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int row = 16 * kb + fr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const v4i kf = *reinterpret_cast<const v4i*>(kbuf + row * 128 + (((4 * ks + fg) ^ (row & 7)) << 4));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const v4i c = ks == 0 ? (v4i){0, 0, 0, 0} : s[qb][kb];
                s[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qf[qb][ks], c, 0, 0, 0);
            }
        }
    }
}

// pass-1 body: running row maxima (in log2 units) of this tile's scores
template <bool RAGGED>
QVD_DEV void tile_max(const v4i s[2][8], float c, int key0, int L, int fg, float m[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int mx = INT_MIN;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (RAGGED && key0 + 16 * kb + 4 * fg + r >= L) continue;
                mx = max(mx, s[qb][kb][r]);
            }
        if (!RAGGED || mx != INT_MIN) m[qb] = fmaxf(m[qb], (float)mx * c);
    }
}

// pass-2 body: fp16 numerators of this tile as the B operand of the P.V MFMA
template <bool RAGGED>
QVD_DEV void tile_numerators(const v4i s[2][8], float c, const float m[2], int key0, int L, int fg,
                             v8h pb[2][4]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
            u32 w[4];
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const int kb = 2 * kp + hlf;
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(fmaf((float)s[qb][kb][r], c, -m[qb]));
                    if (RAGGED && key0 + 16 * kb + 4 * fg + r >= L) p[r] = 0.0f;
                }
                w[2 * hlf] = pack_f16x2(p[0], p[1]);
                w[2 * hlf + 1] = pack_f16x2(p[2], p[3]);
            }
            const v4i pw = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            pb[qb][kp] = __builtin_bit_cast(v8h, pw);
        }
    }
}

// The valid entries (0 <= j < T) of the first `cnt` list elements, in list order, into sm.tiles;
// returns their number.  Ballot-based prefix sums keep the order deterministic.
QVD_DEV int compact_tiles(AttnSmem& sm, const int32_t* __restrict__ list, int cnt, int T, int tid,
                          int lane, int wv) {
    int total = 0;
    for (int base = 0; base < cnt; base += 256) {
        const int t = base + tid;
        const int j = t < cnt ? list[t] : -1;
        const bool ok = j >= 0 && j < T;
        const unsigned long long mask = __ballot(ok);
        const int pos = __popcll(mask & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) sm.wcount[wv] = __popcll(mask);
        __syncthreads();
        int off = total;
        for (int w = 0; w < wv; ++w) off += sm.wcount[w];
        if (ok) sm.tiles[off + pos] = j;
        total += sm.wcount[0] + sm.wcount[1] + sm.wcount[2] + sm.wcount[3];
    }
    __syncthreads();
    return total;
}

template <bool WRITE_AMAX>
__global__ void __launch_bounds__(256, 2) k_sparse_attn(
    const int8_t* __restrict__ q, const float* __restrict__ q_scale, const int8_t* __restrict__ k,
    const float* __restrict__ k_scale, const uint16_t* __restrict__ vt, int L, int H,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int kmax, float c_log2,
    uint16_t* __restrict__ out, float* __restrict__ amax_partials) {
    // a single LDS object: with a second __shared__ array the compiler waits for every DMA before
    // each LDS read
    __shared__ __attribute__((aligned(16))) AttnSmem sm;
    const int i = blockIdx.x, h = blockIdx.y, T = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const int q0 = i * 128 + 32 * wv;
    const int Lp = T * 128;
    const bool ragged_L = (L & 127) != 0;

    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    const float qsc = q_scale[h * T + i] * c_log2;
    int cnt = kv_cnt[h * T + i];
    cnt = cnt < 0 ? 0 : (cnt > kmax ? kmax : cnt);
    const int32_t* list = kv_idx + ((int64_t)h * T + i) * kmax;
    const int n = compact_tiles(sm, list, cnt, T, tid, lane, wv);

    // pass 1: the maximum of every query row over all kept keys; K double-buffered, the next tile
    // loading while this one is multiplied
    float m[2] = {-INFINITY, -INFINITY};
    if (n > 0) stage_k(sm.k[0], k, L, H, h, sm.tiles[0], wv, lane);
    for (int t = 0; t < n; ++t) {
        const int j = sm.tiles[t];
        dma_wait();
        __syncthreads();                       // K(t) is in LDS; everyone is done with K(t-1)
        if (t + 1 < n) stage_k(sm.k[(t + 1) & 1], k, L, H, h, sm.tiles[t + 1], wv, lane);
        v4i s[2][8];
        qk_scores(sm.k[t & 1], qf, fr, fg, s);
        const float c = qsc * k_scale[h * T + j];
        if (ragged_L && j == T - 1) tile_max<true>(s, c, j * 128, L, fg, m);
        else tile_max<false>(s, c, j * 128, L, fg, m);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        m[qb] = fmaxf(m[qb], __shfl_xor(m[qb], 16, 64));
        m[qb] = fmaxf(m[qb], __shfl_xor(m[qb], 32, 64));
    }

    // pass 2: fp16 numerators, their sum (ones . P^T) and P.V.  V^T(t) loads under QK(t) and the
    // numerators; K(t+1) loads under P.V(t).
    v4f o[2][8], lacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        lacc[a] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 8; ++b) o[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    const v8h ones = {1, 1, 1, 1, 1, 1, 1, 1};

    __syncthreads();                           // pass 1's last reads of sm.k are done
    if (n > 0) stage_k(sm.k[0], k, L, H, h, sm.tiles[0], wv, lane);
    for (int t = 0; t < n; ++t) {
        const int j = sm.tiles[t];
        dma_wait();
        __syncthreads();                       // K(t) in LDS; P.V(t-1) and QK(t-1) are done
        stage_vt(sm, vt, Lp, h, j, wv, lane);
        const bool more = t + 1 < n;
        if (more) stage_k(sm.k[(t + 1) & 1], k, L, H, h, sm.tiles[t + 1], wv, lane);

        v4i s[2][8];
        qk_scores(sm.k[t & 1], qf, fr, fg, s);
        const float c = qsc * k_scale[h * T + j];
        v8h pb[2][4];
        if (ragged_L && j == T - 1) tile_numerators<true>(s, c, m, j * 128, L, fg, pb);
        else tile_numerators<false>(s, c, m, j * 128, L, fg, pb);

#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[qb][kp], lacc[qb], 0, 0, 0);
        if (more) dma_wait_but_4();            // V^T(t) landed (K(t+1) may still be in flight)
        else dma_wait();
        __syncthreads();                       // every wave's part of V^T(t) is in LDS
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int d = 16 * db + fr;
            const uint16_t* vrow = sm.vt + d * 128;
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                const int c0 = (4 * kp + (fg >> 1)) ^ (d & 15);
                const int c1 = (4 * kp + 2 + (fg >> 1)) ^ (d & 15);
                const v2i lo = *reinterpret_cast<const v2i*>(vrow + 8 * c0 + 4 * (fg & 1));
                const v2i hi = *reinterpret_cast<const v2i*>(vrow + 8 * c1 + 4 * (fg & 1));
                const v8h vf = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[qb][kp], o[qb][db], 0, 0, 0);
            }
            // keep the V fragment reads of one 16-dim block next to their MFMAs (bounds the
            // registers the scheduler may spend on reads hoisted ahead)
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = lacc[qb][0];
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int row = q0 + 16 * qb + fr;
        if (row < L) {
            uint16_t* orow = out + ((int64_t)row * H + h) * 128;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const v4f cc = o[qb][db];
                const u32 w0 = pack_bf16x2(cc[0] * inv, cc[1] * inv);
                const u32 w1 = pack_bf16x2(cc[2] * inv, cc[3] * inv);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16lo(w0)), fabsf(bf16hi(w0))),
                                         fmaxf(fabsf(bf16lo(w1)), fabsf(bf16hi(w1)))));
                *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * fg) = (u32x2){w0, w1};
            }
        }
    }
    if (WRITE_AMAX) {
        amax = block_max_nonneg<4>(amax, sm.red);
        if (tid == 0) amax_partials[h * T + i] = amax;
    }
}

// bf16 V [L][H][128] -> fp16 V^T [H][128][T*128] (zeros past L).  One workgroup per (token tile,
// head): the tile goes through LDS so both the reads and the writes are 16-byte coalesced.
__global__ void __launch_bounds__(256) k_vt_from_bf16(const uint16_t* __restrict__ v, int L, int H,
                                                      uint16_t* __restrict__ vt) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[128][136];   // [dim][token], fp16
    const int j = blockIdx.x, h = blockIdx.y, T = gridDim.x;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = tid + 256 * u;               // 2048 chunks of 8 dims
        const int tok = c >> 4, d0 = (c & 15) * 8;
        const int row = j * 128 + tok;
        u32x4 w = {0, 0, 0, 0};
        if (row < L) w = *reinterpret_cast<const u32x4*>(v + ((int64_t)row * H + h) * 128 + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = fminf(fmaxf(bf16lo(w[e]), -65504.0f), 65504.0f);
            const float b = fminf(fmaxf(bf16hi(w[e]), -65504.0f), 65504.0f);
            tile[d0 + 2 * e][tok] = __builtin_bit_cast(uint16_t, (_Float16)a);
            tile[d0 + 2 * e + 1][tok] = __builtin_bit_cast(uint16_t, (_Float16)b);
        }
    }
    __syncthreads();
    const int64_t Lp = (int64_t)T * 128;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = tid + 256 * u;
        const int d = c >> 4, t0 = (c & 15) * 8;
        *reinterpret_cast<u32x4*>(vt + ((int64_t)h * 128 + d) * Lp + j * 128 + t0) =
            *reinterpret_cast<const u32x4*>(&tile[d][t0]);
    }
}

// The INT32 accumulators of one (query tile, key tile) pair through the same tile routines.
__global__ void __launch_bounds__(256) k_qk_tile(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                 int L, int H, int h, int i, int j,
                                                 int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) AttnSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const int q0 = i * 128 + 32 * wv;
    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    stage_k(sm.k[0], k, L, H, h, j, wv, lane);
    dma_wait();
    __syncthreads();
    v4i s[2][8];
    qk_scores(sm.k[0], qf, fr, fg, s);
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

int launch_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                          const uint16_t* vt, int L, int H, const int32_t* kv_idx, const int32_t* kv_cnt,
                          int kmax, float sm_scale, uint16_t* out, float* amax_partials, hipStream_t st) {
    if (L == 0) return QVD_OK;
    const int T = (L + 127) / 128;
    const float c = sm_scale * LOG2E;
    TimingScope ts("sparse_attn", st);
    if (amax_partials)
        hipLaunchKernelGGL(k_sparse_attn<true>, dim3(T, H), dim3(256), 0, st, q, q_scale, k, k_scale, vt,
                           L, H, kv_idx, kv_cnt, kmax, c, out, amax_partials);
    else
        hipLaunchKernelGGL(k_sparse_attn<false>, dim3(T, H), dim3(256), 0, st, q, q_scale, k, k_scale, vt,
                           L, H, kv_idx, kv_cnt, kmax, c, out, amax_partials);
    return launch_status("sparse_attn");
}

size_t vt_bytes(int L, int H) { return (size_t)H * 128 * (size_t)((L + 127) / 128) * 128 * 2; }

}  // namespace qvd

using namespace qvd;

namespace {

int validate_attn(const char* fn, const int8_t* q, const float* q_scale, const int8_t* k,
                  const float* k_scale, const void* v, int32_t L, int32_t H, const int32_t* kv_idx,
                  const int32_t* kv_cnt, int32_t kmax, float sm_scale, uint16_t* out) {
    QVD_REQUIRE(L >= 0 && H >= 1 && H <= 65535, QVD_ESHAPE, "%s: L = %d, H = %d", fn, L, H);
    QVD_REQUIRE((double)H * 128.0 * ((L + 127) / 128) * 128.0 * 2.0 < 4294967296.0, QVD_ESHAPE,
                "%s: L = %d, H = %d too large (V^T must stay below 4 GiB)", fn, L, H);
    QVD_REQUIRE(kmax >= 1 && kmax <= MAX_KEPT, QVD_ESHAPE, "%s: kmax = %d (1 .. %d)", fn, kmax, MAX_KEPT);
    QVD_REQUIRE(sm_scale > 0.0f && sm_scale < 1e30f, QVD_EINVAL, "%s: sm_scale out of range", fn);
    if (L == 0) return QVD_OK;
    QVD_REQUIRE(q && q_scale && k && k_scale && v && kv_idx && kv_cnt && out, QVD_EINVAL,
                "%s: a required pointer is NULL", fn);
    QVD_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), QVD_EALIGN,
                "%s: q, k, v and out must be 16-byte aligned", fn);
    return QVD_OK;
}

}  // namespace

extern "C" {

size_t qvd_sparse_attn_ws_bytes(int32_t L, int32_t H) {
    return (L < 0 || H < 1) ? 0 : vt_bytes(L, H);
}

int qvd_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k,
                       const float* k_scale, const uint16_t* vt, int32_t L, int32_t H,
                       const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                       uint16_t* out, float* out_amax_partials, void* stream) {
    int s = validate_attn("qvd_sparse_attn_vt", q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt, kmax,
                          sm_scale, out);
    if (s || L == 0) return s;
    QVD_DEVICE_OK();
    return launch_sparse_attn_vt(q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt, kmax, sm_scale, out,
                                 out_amax_partials, (hipStream_t)stream);
}

int sparse_attn(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                const uint16_t* v, int32_t L, int32_t H, int32_t head_dim,
                const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                uint16_t* out, float* out_amax_partials, void* ws, size_t ws_bytes, void* stream) {
    QVD_REQUIRE(head_dim == 128, QVD_ESHAPE, "sparse_attn: head_dim = %d (must be 128)", head_dim);
    int s = validate_attn("sparse_attn", q, q_scale, k, k_scale, v, L, H, kv_idx, kv_cnt, kmax,
                          sm_scale, out);
    if (s || L == 0) return s;
    QVD_PTR(ws);
    QVD_ALIGN(ws);
    QVD_REQUIRE(ws_bytes >= vt_bytes(L, H), QVD_EWORKSPACE, "sparse_attn: workspace %zu < %zu bytes",
                ws_bytes, vt_bytes(L, H));
    QVD_DEVICE_OK();
    hipStream_t st = (hipStream_t)stream;
    uint16_t* vt = (uint16_t*)ws;
    {
        TimingScope ts("vt_from_bf16", st);
        hipLaunchKernelGGL(k_vt_from_bf16, dim3((L + 127) / 128, H), dim3(256), 0, st, v, L, H, vt);
        s = launch_status("sparse_attn (V conversion)");
        if (s) return s;
    }
    return launch_sparse_attn_vt(q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt, kmax, sm_scale, out,
                                 out_amax_partials, st);
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
