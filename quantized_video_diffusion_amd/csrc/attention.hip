// Block-sparse attention with INT8 query/key scores on the gfx950 matrix cores.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么",
// training bullet (the model runs with 80% attention sparsity) and section "运行速度如何", note under
// the table (query and key are quantized to INT8 for the score computation).
//
// One workgroup per (query tile of 128 rows, head); four waves of 32 query rows; two workgroups per
// CU.  One pass over the kept key tiles (masked tiles are never loaded or multiplied):
//   S^T = K . Q^T with v_mfma_i32_16x16x64_i8 (exact int32, Q fragments in registers);
//   running row maxima m of S * sQ*sK*sm_scale*log2(e); numerators exp2(s - m) rounded to fp16;
//   the fp32 sums so far are multiplied by exp2(m_old - m_new) (every tile, branch-free);
//   numerator sums (ones . P^T) and O^T += V^T . P^T with v_mfma_f32_16x16x32_f16, fp32 accumulation.
// A numerator rounded against the running maximum and later rescaled differs from the one rounded
// against the final maximum by at most one fp16 rounding (relative 2^-11); the output is normalised by
// the sum of the numerators actually used.
//
// Staging: tiles move HBM/L2 -> LDS with global_load_lds_dwordx4 (no register round trip).  The K
// tile's rows are permuted (key_of_row) so that each lane's 8 numerators of a 32-key block are 8
// consecutive keys, read from V^T in one 16-byte access.  Each lane picks the global 16-byte chunk
// that belongs at its LDS slot, which applies an XOR swizzle:
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

// Barriers with explicit waits: this wave's DMA (all of it, or all but the 4 K-tile instructions
// issued last) has landed and its LDS reads are done, then every wave meets.  (__syncthreads() would
// also wait for the K prefetch, which is meant to stay in flight.)
QVD_DEV void dma_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
QVD_DEV void dma_barrier_but_4() { asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Key (0..127 within its tile) held by row rho of the LDS K tile.  Row rho = 16 kb + 4 g + r is the
// score-block row that lane group g receives as element r of block kb; the map gives lane group g the
// keys 32 (kb/2) + 8 g + 4 (kb%2) + r, i.e. 8 consecutive keys across blocks 2 kp and 2 kp + 1, which
// one 16-byte read of a V^T row then matches.
QVD_DEV int key_of_row(int rho) {
    const int kb = rho >> 4, g = (rho >> 2) & 3, r = rho & 3;
    return 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
}

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
// r = (4w+u)*8 + l/8, slot l%8, and fetches chunk (l%8) ^ (r & 7) of key row j*128 + key_of_row(r)
// (clamped to L-1).
QVD_DEV void stage_k(int8_t* kbuf, const int8_t* __restrict__ k, int L, int H, int h, int j,
                     int wv, int lane) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int blk = 4 * wv + u;
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        int kr = j * 128 + key_of_row(r);
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

// S^T = K . Q^T for this wave: s[qb][kb][r] = score(query q0 + 16 qb + fr, key key_of_row(16 kb + 4 fg + r))
QVD_DEV void qk_scores(const int8_t* kbuf, const v4i qf[2][2], int fr, int fg, v4i s[2][8]) {
    // steps (ks, half): 4 key blocks x 2 query blocks; an accumulator's next MFMA comes 16 later, and
    // the next step's K fragments are read while this step multiplies
    auto kfrag = [&](int kb, int ks) {
        const int row = 16 * kb + fr;
        return *reinterpret_cast<const v4i*>(kbuf + row * 128 + (((4 * ks + fg) ^ (row & 7)) << 4));
    };
    v4i kcur[4], knext[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) kcur[b] = kfrag(b, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int ks = st >> 1, hf = st & 1;
        if (st + 1 < 4) {
#pragma unroll
            for (int b = 0; b < 4; ++b) knext[b] = kfrag(4 * ((st + 1) & 1) + b, (st + 1) >> 1);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int kb = 4 * hf + b;
                const v4i c = ks == 0 ? (v4i){0, 0, 0, 0} : s[qb][kb];
                s[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kcur[b], qf[qb][ks], c, 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) kcur[b] = knext[b];
    }
}

// running row maxima (in log2 units) of this tile's scores, this lane's share
template <bool RAGGED>
QVD_DEV void tile_max(const v4i s[2][8], float c, int key0, int L, int fg, float m[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int mx = INT_MIN;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (RAGGED && key0 + key_of_row(16 * kb + 4 * fg + r) >= L) continue;
                mx = max(mx, s[qb][kb][r]);
            }
        if (!RAGGED || mx != INT_MIN) m[qb] = fmaxf(m[qb], (float)mx * c);
    }
}

// fp16 numerators of this tile against the running maxima, as the B operand of the P.V MFMA
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
                    if (RAGGED && key0 + key_of_row(16 * kb + 4 * fg + r) >= L) p[r] = 0.0f;
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

    // running row maxima (log2 units) of the tiles seen so far
    float m[2] = {-INFINITY, -INFINITY};

    // per tile: V^T(t) loads under QK(t) and the numerators; K(t+1) loads under P.V(t)
    v4f o[2][8], lacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        lacc[a] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 8; ++b) o[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    const v8h ones = {1, 1, 1, 1, 1, 1, 1, 1};

    if (n > 0) stage_k(sm.k[0], k, L, H, h, sm.tiles[0], wv, lane);
    for (int t = 0; t < n; ++t) {
        const int j = sm.tiles[t];
        dma_barrier();                         // K(t) in LDS; P.V(t-1) and QK(t-1) are done
        stage_vt(sm, vt, Lp, h, j, wv, lane);
        const bool more = t + 1 < n;
        if (more) stage_k(sm.k[(t + 1) & 1], k, L, H, h, sm.tiles[t + 1], wv, lane);

        v4i s[2][8];
        qk_scores(sm.k[t & 1], qf, fr, fg, s);
        const float c = qsc * k_scale[h * T + j];
        // new running maxima; the sums so far are rescaled to them (every tile, without a branch)
        float tmax[2] = {-INFINITY, -INFINITY};
        if (ragged_L && j == T - 1) tile_max<true>(s, c, j * 128, L, fg, tmax);
        else tile_max<false>(s, c, j * 128, L, fg, tmax);
        float alpha[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            tmax[qb] = fmaxf(tmax[qb], __shfl_xor(tmax[qb], 16, 64));
            tmax[qb] = fmaxf(tmax[qb], __shfl_xor(tmax[qb], 32, 64));
            const float mnew = fmaxf(m[qb], tmax[qb]);
            alpha[qb] = m[qb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[qb] - mnew);
            m[qb] = mnew;
        }
        v8h pb[2][4];
        if (ragged_L && j == T - 1) tile_numerators<true>(s, c, m, j * 128, L, fg, pb);
        else tile_numerators<false>(s, c, m, j * 128, L, fg, pb);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            lacc[qb] *= alpha[qb];
#pragma unroll
            for (int db = 0; db < 8; ++db) o[qb][db] *= alpha[qb];
        }

        if (more) dma_barrier_but_4();         // every wave's V^T(t) landed; K(t+1) may be in flight
        else dma_barrier();
        // O^T += V^T . P^T; lane group g's 8 numerators meet keys 32 kp + 8 g .. +7 of V^T row d,
        // one 16-byte chunk.  Steps (kp, half of the 16-dim blocks): an accumulator's next MFMA comes
        // 16 later, and the next step's fragments are read while this step multiplies.
        auto vfrag = [&](int db, int kp) {
            const int d = 16 * db + fr;
            return *reinterpret_cast<const v8h*>(sm.vt + d * 128 + 8 * ((4 * kp + fg) ^ (d & 15)));
        };
        v8h vcur[4], vnext[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) vcur[b] = vfrag(b, 0);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const int kp = st >> 1, hf = st & 1;
            if (st + 1 < 8) {
#pragma unroll
                for (int b = 0; b < 4; ++b) vnext[b] = vfrag(4 * ((st + 1) & 1) + b, (st + 1) >> 1);
            }
            if (hf == 0) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[qb][kp], lacc[qb], 0, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[qb][4 * hf + b] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(vcur[b], pb[qb][kp], o[qb][4 * hf + b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < 4; ++b) vcur[b] = vnext[b];
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
    dma_barrier();
    v4i s[2][8];
    qk_scores(sm.k[0], qf, fr, fg, s);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 32 * wv + 16 * qb + fr, cc = key_of_row(16 * kb + 4 * fg + r);
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
