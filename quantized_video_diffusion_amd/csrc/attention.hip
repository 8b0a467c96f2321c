// Block-sparse attention with INT8 query/key scores on the gfx950 matrix cores.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3": section "Trim 改变了什么",
// training bullet (the model runs with 80% attention sparsity) and section "运行速度如何", note under
// the table (query and key are quantized to INT8 for the score computation).
//
// Work item: one (query tile of 128 rows, head); four waves of 32 query rows each.  A workgroup of
// eight waves (one per CU, two per SIMD) holds two work items, one per group of four waves, and runs
// them in alternating phases separated by workgroup barriers: while one group multiplies (MFMA) the
// other computes its softmax numerators (VALU), so the matrix cores and the vector ALUs of each SIMD
// work at the same time.  Per item, over the kept key tiles t (masked tiles are never loaded or
// multiplied):
//   MFMA phase t:  O^T += V^T(t-1) . P^T(t-1) and the numerator sums (ones . P^T) with
//                  v_mfma_f32_16x16x32_f16, fp32 accumulation; then S^T = K(t) . Q^T with
//                  v_mfma_i32_16x16x64_i8 (exact int32, Q fragments in registers);
//   VALU phase t:  row maxima of S * sQ*sK*sm_scale*log2(e); numerators P = exp2(s - m) rounded to
//                  fp16 against a reference maximum m per row (scores biased into float patterns,
//                  see SCORE_BIAS).
// The reference m moves only when a tile's row maximum exceeds it by more than 8 (log2 units), and
// then the fp32 sums so far are multiplied by exp2(m_old - m_new); otherwise the numerators stay
// below 2^8.  Each weight is the exact softmax weight up to one fp16 rounding of its numerator
// (relative 2^-11) and fp32 arithmetic; the output is normalised by the sum of the numerators
// actually used.  V arrives in fp16 scaled by one power of two 2^-E[h] per head (vt_tile_exponent,
// k_vt_unify), exact for every element within 2^28 of the head's max|V|, whatever its magnitude;
// the output stage multiplies by 2^E[h].
//
// Staging: tiles move HBM/L2 -> LDS with global_load_lds_dwordx4 (no register round trip).  The K
// tile's rows are permuted (key_of_row) so that each lane's 8 numerators of a 32-key block are 8
// consecutive keys, read from V^T in one 16-byte access.  Each lane picks the global 16-byte chunk
// that belongs at its LDS slot, which applies an XOR swizzle:
// K rows (128 B) swizzle chunks by row & 7, V^T rows (256 B, fp16, keys contiguous) by row & 15,
// so the 16-row MFMA fragment reads hit distinct banks.  V arrives transposed from the QKV GEMM
// epilogue (or from a transpose pass for callers holding V token-major).  Computing the transposed products
// makes each lane own one query row in both MFMA outputs.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

constexpr float LOG2E = 1.4426950408889634f;

constexpr int MAX_KEPT = 1024;      // longest kept-tile list a workgroup takes (kmax bound)

// LDS of one work item (group of four waves)
struct GroupSmem {
    int8_t k[2][128 * 128];         // 2 x 16 KB: double-buffered K tiles
    uint16_t vt[128 * 128];         // 32 KB, fp16 bit patterns
    int tiles[MAX_KEPT];            // the valid entries of the item's kept-tile list, in order
    float tks[MAX_KEPT];            // their K scales
};

struct AttnSmem {
    GroupSmem grp[2];
    int wcount[2][4];
    float wkmax[2][4];              // per-wave maxima of the kept tiles' K scales
    int n[2];                       // kept tiles per group
    float red[8];                   // per-group reductions of max|O|
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// a 32-bit word as two fp16 values, taken by value (a bit_cast applied to a vector element lvalue
// reads element 0)
QVD_DEV v2h as_v2h(u32 w) { return __builtin_bit_cast(v2h, w); }

QVD_DEV u32 pack_f16x2(float lo, float hi) {
    v2h r;
    r.x = (_Float16)lo;
    r.y = (_Float16)hi;
    return __builtin_bit_cast(u32, r);
}

// The tile DMAs are buffer loads to LDS (MUBUF), not global_load_lds: a FLAT instruction that may
// write LDS counts, for the compiler, as an LDS access that completes out of order, so with one in
// flight every wait on an LDS read becomes lgkmcnt(0) and the next step's fragment reads could never
// stay in flight under the current step's MFMAs.  A buffer load counts on vmcnt only.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// raw buffer (stride 0, no swizzle) over the whole 32-bit offset range at base; every offset the
// kernel forms lies inside the operand (the launcher keeps V^T below 4 GiB)
QVD_DEV rsrc_t raw_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
}

// 16 bytes per lane from byte offset soff + voff of the buffer; lane l's bytes land at slot l
QVD_DEV void dma16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds_slot_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_slot_base, 16, voff, soff, 0, 0);
}

// Barriers with explicit waits: this wave's LDS reads are done (and with dma_barrier its DMA has
// landed), then every wave meets.  (__syncthreads() would also wait for DMA that is meant to stay in
// flight across the barrier.)
QVD_DEV void dma_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
QVD_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
        dma16(raw_rsrc(k), off, 0u, kbuf + blk * 1024);
    }
}

// V^T tile j -> LDS.  vt rows are (head, dim), Lp keys each.  Wave w, instruction u fills LDS rows
// (8w + u)*4 .. +3 (256 B each); lane l lands in row d = (8w+u)*4 + l/16, slot l%16, and fetches
// chunk (l%16) ^ (d & 15) of keys j*128 .. j*128+127.
// (32-bit offsets: H*128*Lp*2 bytes stays far below 2^32 for every L the launcher accepts)
QVD_DEV void stage_vt(uint16_t* vbuf, const uint16_t* __restrict__ vt, int Lp, int h, int j,
                      int wv, int lane) {
    const rsrc_t r = raw_rsrc(vt);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int blk = 8 * wv + u;
        const int d = blk * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (d & 15);
        // the lane offset in a VGPR (loop-invariant: the compiler keeps the eight in registers across
        // the tile loop), the tile's in the scalar offset
        const uint32_t off = ((uint32_t)(h * 128 + d) * (uint32_t)Lp + (uint32_t)(8 * c)) * 2u;
        dma16(r, off, (uint32_t)j * 256u, vbuf + blk * 512);
    }
}

// S^T = K . Q^T for this wave: s[qb][kb][r] = s0 + score(query q0 + 16 qb + fr,
// key key_of_row(16 kb + 4 fg + r)) (exact int32 sums)
QVD_DEV void qk_scores(const int8_t* kbuf, const v4i qf[2][2], int fr, int fg, v4i s[2][8], int s0) {
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
        // the reads issue before this step's MFMAs, into registers of their own
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int kb = 4 * hf + b;
                const v4i c = ks == 0 ? (v4i){s0, s0, s0, s0} : s[qb][kb];
                s[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kcur[b], qf[qb][ks], c, 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) kcur[b] = knext[b];
    }
}

// Scores arrive biased: the QK accumulators start at the bit pattern of SCORE_BIAS = 1.5 * 2^23, so
// the int32 result is the bit pattern of the float SCORE_BIAS + s, exactly (|s| <= 128^3 = 2^21 <
// 2^22 keeps it in the binade of SCORE_BIAS, where the float spacing is 1).  The row maximum is then
// an integer maximum of the patterns (positive floats order as their patterns), and the numerator
// argument s c - m is a single fma, fma(SCORE_BIAS + s, c, -(SCORE_BIAS c + m)), with no int -> float
// conversion.
//
// That fma is exact before its one rounding only if the folded constant SCORE_BIAS c + m is itself
// an fp32 number.  The kernel makes it one (ScoreGrid): per work item, G = 2^(ceil(log2 cmax) + 1)
// for the largest factor cmax = |sQ| max|sK| sm_scale log2(e) over its kept tiles; each tile's factor
// c is rounded to a multiple of u = G 2^-22 (so SCORE_BIAS c = 3 (c/u) G is a multiple of G), and the
// reference maxima m are kept on multiples of G.  Then |SCORE_BIAS c + m| <= (3 2^21 + 2^20 + 2) G
// < 2^23 G: an exact multiple of G with fewer than 24 significant bits, which fma(SCORE_BIAS, c, m)
// forms with no rounding.  The tiles' references therefore agree exactly, and the argument's only
// errors are its final fp32 rounding and the rounding of c, |s| u / 2 <= |s c| 2^-23 G / c (a few
// fp32 ulps of the argument when the kept tiles' K scales are alike).
constexpr int SCORE_BIAS_BITS = 0x4B400000;
constexpr float SCORE_BIAS = 12582912.0f;

struct ScoreGrid {
    float g, inv_g;      // G and 1/G
    float u, inv_u;      // u = G 2^-22 and its inverse

    QVD_DEV explicit ScoreGrid(float cmax) {
        int e = 0;
        if (cmax > 0.0f && cmax < 3.0e38f) frexpf(cmax, &e);   // cmax = f 2^e, f in [0.5, 1)
        e = e < -98 ? -98 : (e > 100 ? 100 : e);            // keeps G, u and their inverses normal
        g = ldexpf(1.0f, e + 1);
        inv_g = ldexpf(1.0f, -(e + 1));
        u = ldexpf(1.0f, e + 1 - 22);
        inv_u = ldexpf(1.0f, 22 - (e + 1));
    }
    // the tile's factor on the grid of u (both products are exact power-of-two scalings)
    QVD_DEV float factor(float c) const { return __builtin_rintf(c * inv_u) * u; }
    // the smallest multiple of G at or above x
    QVD_DEV float ceil_g(float x) const { return __builtin_ceilf(x * inv_g) * g; }
};

// Vector elements reach a bit_cast through this by-value helper: a bit_cast applied to a vector
// element lvalue reads element 0.
QVD_DEV float as_float(u32 x) { return __builtin_bit_cast(float, x); }

QVD_DEV float unbias(int bits) { return as_float((u32)bits) - SCORE_BIAS; }

// max over lanes l, l^16, l^32, l^48 with the gfx950 lane swaps (pure VALU: v_permlane16_swap pairs
// lane l with l^16, v_permlane32_swap with l^32), so the softmax phase issues no LDS instruction
QVD_DEV int max_over_lane_groups(int x) {
    const auto a = __builtin_amdgcn_permlane16_swap((u32)x, (u32)x, false, false);
    const int y = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((u32)y, (u32)y, false, false);
    return max((int)b[0], (int)b[1]);
}

// row maxima (log2 units) of this tile's scores: integer maxima of the biased patterns over this
// lane's keys, then over the row's four lane groups
template <bool RAGGED>
QVD_DEV void tile_max(const v4i s[2][8], float c, int key0, int L, int fg, float tmax[2]) {
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
        mx = max_over_lane_groups(mx);         // every row keeps at least one key of a ragged tile
        tmax[qb] = unbias(mx) * c;
    }
}

// fp16 numerators of this tile against the reference maxima, as the B operand of the P.V MFMA.
// c is on the grid of u and m on the grid of G (ScoreGrid), so mb below is exact.
template <bool RAGGED>
QVD_DEV void tile_numerators(const v4i s[2][8], float c, const float m[2], int key0, int L, int fg,
                             v8h pb[2][4]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float mb = fmaf(SCORE_BIAS, c, m[qb]);
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
            u32 w[4];
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const int kb = 2 * kp + hlf;
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(fmaf(as_float((u32)s[qb][kb][r]), c, -mb));
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

// The valid entries (0 <= j < T) of the first `cnt` list elements, in list order, into tiles and their
// K scales into tks; their number into *n_out.  Returns the largest |K scale| of those tiles (ks_row:
// the head's K scales).
// Run by both groups of the workgroup at once (gtid: thread index in the group, wg: wave in the
// group): the iteration count depends on kmax only, so every wave meets the same barriers.
// Ballot-based prefix sums keep the order deterministic.
QVD_DEV float compact_tiles(int* tiles, float* tks, int* wcount, float* wkmax, int* n_out,
                            const int32_t* __restrict__ list, int cnt, int kmax, int T,
                            const float* __restrict__ ks_row, int gtid, int lane, int wg) {
    int total = 0;
    float km = 0.0f;
    for (int base = 0; base < kmax; base += 256) {
        const int t = base + gtid;
        const int j = t < cnt ? list[t] : -1;
        const bool ok = j >= 0 && j < T;
        const float kj = ok ? ks_row[j] : 0.0f;
        km = fmaxf(km, fabsf(kj));
        const unsigned long long mask = __ballot(ok);
        const int pos = __popcll(mask & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) wcount[wg] = __popcll(mask);
        __syncthreads();
        int off = total;
        for (int w = 0; w < wg; ++w) off += wcount[w];
        if (ok) {
            tiles[off + pos] = j;
            tks[off + pos] = kj;
        }
        total += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    }
    km = wave_max(km);
    if (lane == 0) wkmax[wg] = km;
    if (gtid == 0) *n_out = total;
    __syncthreads();
    return fmaxf(fmaxf(wkmax[0], wkmax[1]), fmaxf(wkmax[2], wkmax[3]));
}

// O^T += V^T . P^T and the numerator sums, this wave's share, from the V^T tile in LDS.  Lane group
// g's 8 numerators meet keys 32 kp + 8 g .. +7 of V^T row d, one 16-byte chunk.  Steps (kp, half of
// the 16-dim blocks): an accumulator's next MFMA comes 16 later, and the next step's fragments are
// read while this step multiplies.
QVD_DEV void pv_tile(const uint16_t* vbuf, const v8h pb[2][4], int fr, int fg, v4f o[2][8], v4f lacc[2]) {
    const v8h ones = {1, 1, 1, 1, 1, 1, 1, 1};
    auto vfrag = [&](int db, int kp) {
        const int d = 16 * db + fr;
        return *reinterpret_cast<const v8h*>(vbuf + d * 128 + 8 * ((4 * kp + fg) ^ (d & 15)));
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
        __builtin_amdgcn_sched_barrier(0);
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

constexpr float RESCALE_SLACK = 8.0f;   // log2 units a tile maximum may exceed the reference by


// Numerators of one tile against the reference maxima m (moved, and the sums rescaled, when a row's
// tile maximum exceeds its reference by more than RESCALE_SLACK; the wave takes or skips the rescale
// as a whole).  c is the tile's factor on the grid of u; a moved reference is the tile maximum
// raised to the next multiple of G, so the numerators stay at most 2^8.
QVD_DEV void softmax_tile(const v4i s[2][8], float c, const ScoreGrid& grid, bool ragged, int key0, int L,
                          int fg, float m[2], v4f o[2][8], v4f lacc[2], v8h pb[2][4]) {
    float tmax[2];
    if (ragged) tile_max<true>(s, c, key0, L, fg, tmax);
    else tile_max<false>(s, c, key0, L, fg, tmax);
    float alpha[2];
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const bool u = tmax[qb] > m[qb] + RESCALE_SLACK;
        const float mnew = u ? grid.ceil_g(tmax[qb]) : m[qb];
        alpha[qb] = m[qb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[qb] - mnew);
        m[qb] = mnew;
        up = up || u;
    }
    if (__ballot(up) != 0ull) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            lacc[qb] *= alpha[qb];
#pragma unroll
            for (int db = 0; db < 8; ++db) o[qb][db] *= alpha[qb];
        }
    }
    if (ragged) tile_numerators<true>(s, c, m, key0, L, fg, pb);
    else tile_numerators<false>(s, c, m, key0, L, fg, pb);
}

// Output of the attention kernel: bf16 O; bf16 O and the per-(head, tile) max|O|; or the E4M3 codes
// of bf16 O under a static per-tensor scale, as the standalone static quantizer computes them.
enum AttnOut { OUT_BF16 = 0, OUT_BF16_AMAX = 1, OUT_E4M3 = 2, OUT_MXFP4 = 3 };

template <int OUT>
__global__ void __launch_bounds__(512, 1) k_sparse_attn(
    const int8_t* __restrict__ q, const float* __restrict__ q_scale, const int8_t* __restrict__ k,
    const float* __restrict__ k_scale, const uint16_t* __restrict__ vt, const int32_t* __restrict__ v_exp,
    int L, int H, const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int kmax, float c_log2,
    void* __restrict__ out, float* __restrict__ amax_partials, const float* __restrict__ out_scale,
    uint8_t* __restrict__ out_e8m0) {
    // a single LDS object: with a second __shared__ array the compiler waits for every DMA before
    // each LDS read
    __shared__ __attribute__((aligned(16))) AttnSmem sm;
    const int T = (L + 127) >> 7, total = T * H;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wv >> 2, wg = wv & 3;
    const int fr = lane & 15, fg = lane >> 4;

    // Workgroup b -> pair index -> work items 2 pair + g, head-major (h = id / T, i = id % T).
    // Workgroups are handed to the 8 XCDs round-robin (b % 8), so each XCD is given one contiguous
    // range of pairs: the workgroups resident on an XCD at a time hold neighbouring query tiles of one
    // head, whose ascending tile lists sweep the same K and V^T tiles through the XCD's L2 at about
    // the same time.
    int id;
    {
        const int pairs = (total + 1) >> 1, b = blockIdx.x;
        const int xcd = b & 7, per = pairs >> 3, rem = pairs & 7;
        id = 2 * (xcd * per + (xcd < rem ? xcd : rem) + (b >> 3)) + g;
    }
    const bool valid = id < total;               // an odd item count leaves the last group idle
    const int h = valid ? id / T : 0;
    const int i = valid ? id - h * T : 0;
    const int q0 = i * 128 + 32 * wg;
    const int Lp = T * 128;
    const bool ragged_L = (L & 127) != 0;
    GroupSmem& gs = sm.grp[g];

    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    const float qsc = q_scale[h * T + i] * c_log2;
    int cnt = valid ? kv_cnt[h * T + i] : 0;
    cnt = cnt < 0 ? 0 : (cnt > kmax ? kmax : cnt);
    const int32_t* list = kv_idx + ((int64_t)h * T + i) * kmax;
    const float ks_max = compact_tiles(gs.tiles, gs.tks, sm.wcount[g], sm.wkmax[g], &sm.n[g], list, cnt, kmax, T,
                                       k_scale + (int64_t)h * T, tid & 255, lane, wg);
    const ScoreGrid grid(fabsf(qsc) * ks_max);
    const int n = sm.n[g];
    const int n_other = sm.n[g ^ 1];

    float m[2] = {-INFINITY, -INFINITY};         // reference row maxima (log2 units)
    v4f o[2][8], lacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        lacc[a] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 8; ++b) o[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    v4i s[2][8];                                  // scores of tile t: MFMA phase t -> VALU phase t
    v8h pb[2][4];                                 // numerators of tile t: VALU phase t -> MFMA phase t+1
    float ksc = 0.0f;                             // K scale of the tile the next VALU phase takes

    // Phases p = 0, 1, ... end at workgroup barriers B_p (B_-1 before phase 0).  Group 0 runs MFMA
    // phase t in phase 2t and VALU phase t in phase 2t+1; group 1 one phase later.  Each group runs
    // its own loop, so its scores and numerators are live only where it uses them; the loops meet
    // the same barriers (s_barrier counts waves, not program locations), P + 1 of them in all.
    // Before a group's MFMA phase its waves wait for their DMA (K(t) and V^T(t-1)).
    //   MFMA phase t: K(t+1) -> LDS (its buffer was last read in MFMA phase t-1); P.V(t-1); S(t);
    //                 index and K scale of tile t from LDS.  (The last one, t = n, multiplies a stale K
    //                 buffer into unused scores, which keeps the loop free of register merges.)
    //   VALU phase t: V^T(t) -> LDS (its buffer was last read in MFMA phase t); numerators of tile t.
    //                 No LDS reads: the tile index and its K scale are read in the MFMA phase before,
    //                 so the other group's fragment reads never hold this phase up.
    const int n0 = g == 0 ? n : n_other, n1 = g == 0 ? n_other : n;
    const int P = 2 * n0 + 1 > 2 * n1 + 2 ? 2 * n0 + 1 : 2 * n1 + 2;
    auto mfma_qk = [&](int t) {                   // the QK part of MFMA phase t and its DMA
        if (t + 1 < n) stage_k(gs.k[(t + 1) & 1], k, L, H, h, gs.tiles[t + 1], wg, lane);
        qk_scores(gs.k[t & 1], qf, fr, fg, s, SCORE_BIAS_BITS);
    };
    int j = 0;                                    // tile of the next VALU phase (read in the MFMA phase)
    auto valu_phase = [&]() {
        stage_vt(gs.vt, vt, Lp, h, j, wg, lane);
        softmax_tile(s, grid.factor(qsc * ksc), grid, ragged_L && j == T - 1, j * 128, L, fg, m, o, lacc, pb);
    };

    if (n > 0) stage_k(gs.k[0], k, L, H, h, gs.tiles[0], wg, lane);
    if (g == 1) lds_barrier();                   // group 1: B_-1 (its phase 0 is idle)
    dma_barrier();                                // group 0: B_-1; group 1: B_0
    int passed = 1 + g;                           // barriers passed
    // The next VALU phase's tile index (made wave-uniform for the DMA addresses) and K scale are read
    // from the compacted list in LDS at the end of the MFMA phase, under its last MFMAs.  LDS reads
    // return in order, so the compiler keeps graded waits (lgkmcnt(n)) on the fragment reads, and the
    // next step's fragments load while this step multiplies.  A scalar load of the K scale in flight
    // here made it wait for every outstanding LDS read (lgkmcnt(0)) before each MFMA step, since
    // scalar loads may return out of order; a vector load would make the VALU phase wait for vmcnt,
    // i.e. for the V^T DMA just issued.
    if (n > 0) {
        j = __builtin_amdgcn_readfirstlane(gs.tiles[0]);
        ksc = gs.tks[0];
        mfma_qk(0);
        lds_barrier();
        ++passed;
        for (int t = 0; t < n; ++t) {
            valu_phase();
            dma_barrier();
            // The MFMA phase issues at raised priority: where its instructions and the other group's
            // VALU instructions compete for a SIMD's issue, the matrix core is served first.  Without
            // it the older group (waves 0-3) wins in both phases, which stretched the younger group's
            // MFMA phases by about a fifth and with them every second barrier interval.
            __builtin_amdgcn_s_setprio(2);
            pv_tile(gs.vt, pb, fr, fg, o, lacc);
            mfma_qk(t + 1);
            if (t + 1 < n) {
                j = __builtin_amdgcn_readfirstlane(gs.tiles[t + 1]);
                ksc = gs.tks[t + 1];
            }
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
            passed += 2;
        }
    }
    for (; passed < P + 1; ++passed) lds_barrier();
    const int ve = valid ? v_exp[h] : 0;          // the head's V scale: O = (P.V') 2^ve / sum P

    if (OUT == OUT_MXFP4) {
        // bf16 O, then MXFP4 per (row, head, 32 dims) with the standalone quantizer's arithmetic.  Dims
        // 32 b .. 32 b + 31 of a row are this lane's column blocks 2b and 2b+1 in each of the row's
        // four lanes (fg): the block maximum meets across them before any lane stores.
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float lt = lacc[qb][0];
            const float inv = lt > 0.0f ? ldexpf(1.0f / lt, ve) : 0.0f;
            const int row = q0 + 16 * qb + fr;
            u32 w[8][2];
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const v4f cc = o[qb][db];
                w[db][0] = pack_bf16x2(cc[0] * inv, cc[1] * inv);
                w[db][1] = pack_bf16x2(cc[2] * inv, cc[3] * inv);
            }
            int kx[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float m = 0.0f;
#pragma unroll
                for (int db = 2 * b; db < 2 * b + 2; ++db)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        m = fmaxf(m, fmaxf(fabsf(bf16lo(w[db][u])), fabsf(bf16hi(w[db][u]))));
                kx[b] = mx_exponent(__int_as_float(max_over_lane_groups(__float_as_int(m))));
            }
            if (valid && row < L) {
                const int64_t orow = (int64_t)row * H + h;
                uint8_t* pr = static_cast<uint8_t*>(out) + orow * 64;
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const int k = kx[db >> 1];
                    const u32 c = e2m1_encode2(bf16lo(w[db][0]), bf16hi(w[db][0]), k) |
                                  (e2m1_encode2(bf16lo(w[db][1]), bf16hi(w[db][1]), k) << 8);
                    *reinterpret_cast<uint16_t*>(pr + 8 * db + 2 * fg) = (uint16_t)c;
                }
                if (fg == 0)
                    *reinterpret_cast<u32*>(out_e8m0 + orow * 4) =
                        (u32)(kx[0] + 127) | ((u32)(kx[1] + 127) << 8) | ((u32)(kx[2] + 127) << 16) |
                        ((u32)(kx[3] + 127) << 24);
            }
        }
        return;
    }

    float amax = 0.0f;
    const float inv_s = OUT == OUT_E4M3 ? __fdiv_rn(1.0f, *out_scale) : 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = lacc[qb][0];
        const float inv = lt > 0.0f ? ldexpf(1.0f / lt, ve) : 0.0f;
        const int row = q0 + 16 * qb + fr;
        if (valid && row < L) {
            const int64_t orow = ((int64_t)row * H + h) * 128;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const v4f cc = o[qb][db];
                const u32 w0 = pack_bf16x2(cc[0] * inv, cc[1] * inv);
                const u32 w1 = pack_bf16x2(cc[2] * inv, cc[3] * inv);
                if (OUT == OUT_E4M3) {
                    const u32 c4 = e4m3_encode2(bf16lo(w0) * inv_s, bf16hi(w0) * inv_s) |
                                   (e4m3_encode2(bf16lo(w1) * inv_s, bf16hi(w1) * inv_s) << 16);
                    *reinterpret_cast<u32*>(static_cast<uint8_t*>(out) + orow + 16 * db + 4 * fg) = c4;
                } else {
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16lo(w0)), fabsf(bf16hi(w0))),
                                             fmaxf(fabsf(bf16lo(w1)), fabsf(bf16hi(w1)))));
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow + 16 * db + 4 * fg) =
                        (u32x2){w0, w1};
                }
            }
        }
    }
    if (OUT == OUT_BF16_AMAX) {
        // max over the group's four waves (both groups reduce at once)
        amax = wave_max(amax);
        if (lane == 0) sm.red[wv] = amax;
        __syncthreads();
        if ((tid & 255) == 0 && valid)
            amax_partials[h * T + i] = fmaxf(fmaxf(sm.red[4 * g], sm.red[4 * g + 1]),
                                             fmaxf(sm.red[4 * g + 2], sm.red[4 * g + 3]));
    }
}

// bf16 V [L][H][128] -> fp16 V^T [H][128][T*128] (zeros past L), each (tile, head) scaled by
// 2^-e with e = vt_tile_exponent of its max|V|, written to tile_exp[h][j].  One workgroup per (token
// tile, head): the tile goes through registers and LDS so both the reads and the writes are 16-byte
// coalesced.
__global__ void __launch_bounds__(256) k_vt_from_bf16(const uint16_t* __restrict__ v, int L, int H,
                                                      uint16_t* __restrict__ vt, int32_t* __restrict__ tile_exp) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[128][136];   // [dim][token], fp16
    __shared__ float red[4];
    const int j = blockIdx.x, h = blockIdx.y, T = gridDim.x;
    const int tid = threadIdx.x;
    u32x4 w[8];
    u32 amb = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = tid + 256 * u;               // 2048 chunks of 8 dims
        const int tok = c >> 4, d0 = (c & 15) * 8;
        const int row = j * 128 + tok;
        w[u] = (u32x4){0, 0, 0, 0};
        if (row < L) w[u] = *reinterpret_cast<const u32x4*>(v + ((int64_t)row * H + h) * 128 + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) amb = max(amb, max(w[u][e] & 0x7FFFu, (w[u][e] >> 16) & 0x7FFFu));
    }
    // the largest |v| as a bf16 magnitude pattern (finite magnitudes order as their patterns)
    const float amax = block_max_nonneg<4>(bf16_to_f32((uint16_t)amb), red);
    const int ve = vt_tile_exponent(amax);
    if (tid == 0) tile_exp[h * T + j] = ve;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = tid + 256 * u;
        const int tok = c >> 4, d0 = (c & 15) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[d0 + 2 * e][tok] = f16_scaled(bf16lo(w[u][e]), ve);
            tile[d0 + 2 * e + 1][tok] = f16_scaled(bf16hi(w[u][e]), ve);
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

// One V scale per head: head_exp[h] = E = the largest of the head's tile exponents, and every tile
// stored with a smaller exponent e is rescaled in place by 2^(e - E) (exact wherever the result is an
// fp16 normal; a value more than 2^28 below the head's max|V| may round to the fp16 subnormal grid).
// One workgroup per (token tile, head); a tile already at E is not touched, so with V in the usual
// range (every exponent 0) the pass reads only the exponents.
__global__ void __launch_bounds__(256) k_vt_unify(uint16_t* __restrict__ vt, int T,
                                                  const int32_t* __restrict__ tile_exp,
                                                  int32_t* __restrict__ head_exp) {
    __shared__ int red[4];
    const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int e = INT_MIN;
    for (int t = tid; t < T; t += 256) e = max(e, tile_exp[h * T + t]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e = max(e, __shfl_xor(e, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = e;
    __syncthreads();
    const int E = max(max(red[0], red[1]), max(red[2], red[3]));
    if (j == 0 && tid == 0) head_exp[h] = E;
    const int sh = tile_exp[h * T + j] - E;
    if (sh == 0) return;
    const int64_t Lp = (int64_t)T * 128;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = tid + 256 * u;               // 2048 chunks of 8 keys: rows (h, d), d < 128
        const int d = c >> 4, t0 = (c & 15) * 8;
        u32x4* p = reinterpret_cast<u32x4*>(vt + ((int64_t)h * 128 + d) * Lp + j * 128 + t0);
        u32x4 w = *p;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const v2h x = as_v2h(w[k]);
            w[k] = pack_f16x2(ldexpf((float)x.x, sh), ldexpf((float)x.y, sh));
        }
        *p = w;
    }
}

// The INT32 accumulators of one (query tile, key tile) pair through the same tile routines.
__global__ void __launch_bounds__(256) k_qk_tile(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                 int L, int H, int h, int i, int j,
                                                 int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) int8_t ktile[128 * 128];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const int q0 = i * 128 + 32 * wv;
    v4i qf[2][2];
    load_q_frags(q, L, H, h, q0, fr, fg, qf);
    stage_k(ktile, k, L, H, h, j, wv, lane);
    dma_barrier();
    v4i s[2][8];
    qk_scores(ktile, qf, fr, fg, s, SCORE_BIAS_BITS);      // as the attention kernel, bias removed below
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 32 * wv + 16 * qb + fr, cc = key_of_row(16 * kb + 4 * fg + r);
                const bool ok = (i * 128 + rr) < L && (j * 128 + cc) < L;
                out[rr * 128 + cc] = ok ? s[qb][kb][r] - SCORE_BIAS_BITS : 0;
            }
}

namespace {
template <int OUT>
int launch_attn(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                const uint16_t* vt, const int32_t* v_exp, int L, int H, const int32_t* kv_idx,
                const int32_t* kv_cnt, int kmax, float sm_scale, void* out, float* amax_partials,
                const float* out_scale, uint8_t* out_e8m0, hipStream_t st) {
    if (L == 0) return QVD_OK;
    const int T = (L + 127) / 128;
    const unsigned pairs = (unsigned)((T * H + 1) / 2);
    const float c = sm_scale * LOG2E;
    TimingScope ts("sparse_attn", st);
    hipLaunchKernelGGL(k_sparse_attn<OUT>, dim3(pairs), dim3(512), 0, st, q, q_scale, k, k_scale, vt, v_exp,
                       L, H, kv_idx, kv_cnt, kmax, c, out, amax_partials, out_scale, out_e8m0);
    return launch_status("sparse_attn");
}
}  // namespace

int launch_vt_unify(uint16_t* vt, int L, int H, const int32_t* tile_exp, int32_t* head_exp, hipStream_t st) {
    if (L == 0) return QVD_OK;
    const int T = (L + 127) / 128;
    TimingScope ts("vt_unify", st);
    hipLaunchKernelGGL(k_vt_unify, dim3(T, H), dim3(256), 0, st, vt, T, tile_exp, head_exp);
    return launch_status("vt_unify");
}

int launch_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                          const uint16_t* vt, const int32_t* v_exp, int L, int H, const int32_t* kv_idx,
                          const int32_t* kv_cnt, int kmax, float sm_scale, uint16_t* out,
                          float* amax_partials, hipStream_t st) {
    if (amax_partials)
        return launch_attn<OUT_BF16_AMAX>(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax,
                                          sm_scale, out, amax_partials, nullptr, nullptr, st);
    return launch_attn<OUT_BF16>(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale, out,
                                 nullptr, nullptr, nullptr, st);
}

int launch_sparse_attn_vt_e4m3(const int8_t* q, const float* q_scale, const int8_t* k,
                               const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int L, int H,
                               const int32_t* kv_idx, const int32_t* kv_cnt, int kmax, float sm_scale,
                               const float* out_scale, uint8_t* out_q, hipStream_t st) {
    return launch_attn<OUT_E4M3>(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale,
                                 out_q, nullptr, out_scale, nullptr, st);
}

int launch_sparse_attn_vt_mxfp4(const int8_t* q, const float* q_scale, const int8_t* k,
                                const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int L, int H,
                                const int32_t* kv_idx, const int32_t* kv_cnt, int kmax, float sm_scale,
                                uint8_t* out_packed, uint8_t* out_e8m0, hipStream_t st) {
    return launch_attn<OUT_MXFP4>(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale,
                                  out_packed, nullptr, nullptr, out_e8m0, st);
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

// sparse_attn's workspace: fp16 V^T, then the tile exponents [H][T] and the head exponents [H]
size_t attn_ws_tile_exp_off(int L, int H) { return (vt_bytes(L, H) + 255) & ~(size_t)255; }
size_t attn_ws_head_exp_off(int L, int H) {
    const size_t T = (size_t)(L + 127) / 128;
    return (attn_ws_tile_exp_off(L, H) + 4 * (size_t)H * T + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

size_t qvd_sparse_attn_ws_bytes(int32_t L, int32_t H) {
    return (L < 0 || H < 1) ? 0 : attn_ws_head_exp_off(L, H) + 4 * (size_t)H;
}

int qvd_vt_from_bf16(const uint16_t* v, int32_t L, int32_t H, uint16_t* vt, int32_t* tile_exp, void* stream) {
    QVD_REQUIRE(L >= 0 && H >= 1 && H <= 65535, QVD_ESHAPE, "qvd_vt_from_bf16: L = %d, H = %d", L, H);
    QVD_REQUIRE((double)vt_bytes(L, H) < 4294967296.0, QVD_ESHAPE, "qvd_vt_from_bf16: V^T must stay below 4 GiB");
    if (L == 0) return QVD_OK;
    QVD_PTR(v);
    QVD_PTR(vt);
    QVD_PTR(tile_exp);
    QVD_ALIGN(v);
    QVD_ALIGN(vt);
    QVD_DEVICE_OK();
    hipStream_t st = (hipStream_t)stream;
    TimingScope ts("vt_from_bf16", st);
    hipLaunchKernelGGL(k_vt_from_bf16, dim3((L + 127) / 128, H), dim3(256), 0, st, v, L, H, vt, tile_exp);
    return launch_status("qvd_vt_from_bf16");
}

int qvd_vt_unify(uint16_t* vt, int32_t L, int32_t H, const int32_t* tile_exp, int32_t* head_exp,
                 void* stream) {
    QVD_REQUIRE(L >= 0 && H >= 1 && H <= 65535, QVD_ESHAPE, "qvd_vt_unify: L = %d, H = %d", L, H);
    if (L == 0) return QVD_OK;
    QVD_PTR(vt);
    QVD_PTR(tile_exp);
    QVD_PTR(head_exp);
    QVD_ALIGN(vt);
    QVD_DEVICE_OK();
    return launch_vt_unify(vt, L, H, tile_exp, head_exp, (hipStream_t)stream);
}

int qvd_sparse_attn_vt(const int8_t* q, const float* q_scale, const int8_t* k,
                       const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L, int32_t H,
                       const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax, float sm_scale,
                       uint16_t* out, float* out_amax_partials, void* stream) {
    int s = validate_attn("qvd_sparse_attn_vt", q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt, kmax,
                          sm_scale, out);
    if (s || L == 0) return s;
    QVD_PTR(v_exp);
    QVD_DEVICE_OK();
    return launch_sparse_attn_vt(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale, out,
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
    const size_t need = qvd_sparse_attn_ws_bytes(L, H);
    QVD_REQUIRE(ws_bytes >= need, QVD_EWORKSPACE, "sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
    QVD_DEVICE_OK();
    hipStream_t st = (hipStream_t)stream;
    uint16_t* vt = (uint16_t*)ws;
    int32_t* tile_exp = (int32_t*)((char*)ws + attn_ws_tile_exp_off(L, H));
    int32_t* head_exp = (int32_t*)((char*)ws + attn_ws_head_exp_off(L, H));
    {
        TimingScope ts("vt_from_bf16", st);
        hipLaunchKernelGGL(k_vt_from_bf16, dim3((L + 127) / 128, H), dim3(256), 0, st, v, L, H, vt, tile_exp);
        s = launch_status("sparse_attn (V transpose)");
        if (s) return s;
    }
    s = launch_vt_unify(vt, L, H, tile_exp, head_exp, st);
    if (s) return s;
    return launch_sparse_attn_vt(q, q_scale, k, k_scale, vt, head_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale,
                                 out, out_amax_partials, st);
}

int qvd_sparse_attn_vt_e4m3(const int8_t* q, const float* q_scale, const int8_t* k,
                            const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L,
                            int32_t H, const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax,
                            float sm_scale, const float* out_scale, uint8_t* out_q, void* stream) {
    int s = validate_attn("qvd_sparse_attn_vt_e4m3", q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt,
                          kmax, sm_scale, reinterpret_cast<uint16_t*>(out_q));
    if (s || L == 0) return s;
    QVD_PTR(v_exp);
    QVD_PTR(out_scale);
    QVD_DEVICE_OK();
    return launch_sparse_attn_vt_e4m3(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax, sm_scale,
                                      out_scale, out_q, (hipStream_t)stream);
}

int qvd_sparse_attn_vt_mxfp4(const int8_t* q, const float* q_scale, const int8_t* k,
                             const float* k_scale, const uint16_t* vt, const int32_t* v_exp, int32_t L,
                             int32_t H, const int32_t* kv_idx, const int32_t* kv_cnt, int32_t kmax,
                             float sm_scale, uint8_t* out_packed, uint8_t* out_e8m0, void* stream) {
    int s = validate_attn("qvd_sparse_attn_vt_mxfp4", q, q_scale, k, k_scale, vt, L, H, kv_idx, kv_cnt,
                          kmax, sm_scale, reinterpret_cast<uint16_t*>(out_packed));
    if (s || L == 0) return s;
    QVD_PTR(v_exp);
    QVD_PTR(out_e8m0);
    QVD_REQUIRE(((uintptr_t)out_e8m0 & 3u) == 0, QVD_EALIGN,
                "qvd_sparse_attn_vt_mxfp4: out_e8m0 must be 4-byte aligned");
    QVD_DEVICE_OK();
    return launch_sparse_attn_vt_mxfp4(q, q_scale, k, k_scale, vt, v_exp, L, H, kv_idx, kv_cnt, kmax,
                                       sm_scale, out_packed, out_e8m0, (hipStream_t)stream);
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
