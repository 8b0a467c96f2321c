// Sparse-tile selector: which key tiles each (head, query tile) attends to.
//
// comfyui-wiki "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3", section "Trim 改变了什么",
// training bullet: the model attends with 80% sparsity; the pages do not say how the kept tiles are
// chosen.  The rule built here: key tile j is ranked for query tile i by the dot product of the
// mean-pooled query and key tiles, dequantized from their INT8 codes; the diagonal is always kept
// and the kept - 1 best other tiles join it, equal scores going to the lower index; the list is
// sorted by tile index.  The row's own factor sq_i / n_i is positive and cannot change the ranking,
// so the rank key is D(h, i, j) * w(h, j): D = sum_e Qsum_i[e] Ksum_j[e], the exact integer dot of
// the per-tile code sums, and w = double(sk_j) / n_j, each rounded once in float64.
//
//   k_tile_sums   : per (tile, head, Q|K) the int32 sums of the codes over the tile's rows
//   k_tile_scores : D * w for 64 x 64 blocks of (i, j), exact: 24-bit integer products summed four at
//                   a time in int32 (|sum| < 2^30), then in float64 (|D| < 2^36, so every sum is exact)
//   k_select      : per (head, query tile) a radix select of the kept - 1 best keys (one byte per
//                   pass), then the kept tiles written in tile order
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qvd {

namespace {

constexpr int SEL_MAX_T = 1024;          // tiles per sequence the selector handles (L <= 131,072)

// sums[z][h][t][e], z = 0 for Q, 1 for K.  256 threads: thread = (row group rg of 32, 16-byte chunk c)
__global__ void __launch_bounds__(256) k_tile_sums(const int8_t* __restrict__ q8, const int8_t* __restrict__ k8,
                                                   int L, int H, int T, int32_t* __restrict__ sums) {
    __shared__ int part[32][129];
    const int t = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const int8_t* src = z == 0 ? q8 : k8;
    const int tid = threadIdx.x, c = tid & 7, rg = tid >> 3;
    int acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = t * 128 + rg + 32 * m;
        if (r < L) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + ((int64_t)r * H + h) * 128 + 16 * c);
            const u32 w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[4 * q + b] += (int)(int8_t)((w[q] >> (8 * b)) & 0xFFu);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) part[rg][16 * c + e] = acc[e];
    __syncthreads();
    if (tid < 128) {
        int s = 0;
#pragma unroll 8
        for (int g = 0; g < 32; ++g) s += part[g][tid];
        sums[(((int64_t)z * H + h) * T + t) * 128 + tid] = s;
    }
}

// scores[h][i][j] = double(D) * (double(sk[h][j]) / n_j).  Block: 64 i x 64 j of one head; thread
// (ti, tj) = (tid / 16, tid % 16) owns i = i0 + ti + 16a, j = j0 + tj + 16b (a, b < 4).  Rows are
// padded to 132 words so that 16 different rows read at one column fall on distinct bank quads.
constexpr int SC_LD = 132;

__global__ void __launch_bounds__(256) k_tile_scores(const int32_t* __restrict__ sums,
                                                     const float* __restrict__ k_scale, int L, int H, int T,
                                                     double* __restrict__ scores) {
    __shared__ __attribute__((aligned(16))) int qs[64 * SC_LD];
    __shared__ __attribute__((aligned(16))) int ks[64 * SC_LD];
    const int h = blockIdx.z, i0 = 64 * blockIdx.y, j0 = 64 * blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* qsum = sums + (int64_t)h * T * 128;
    const int32_t* ksum = sums + ((int64_t)H + h) * T * 128;
    // 64 rows x 32 chunks of 16 bytes per operand; tiles past T load zeros
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = 256 * it + tid, row = idx >> 5, ch = idx & 31;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (i0 + row < T) a = *reinterpret_cast<const u32x4*>(qsum + (int64_t)(i0 + row) * 128 + 4 * ch);
        if (j0 + row < T) b = *reinterpret_cast<const u32x4*>(ksum + (int64_t)(j0 + row) * 128 + 4 * ch);
        *reinterpret_cast<u32x4*>(qs + row * SC_LD + 4 * ch) = a;
        *reinterpret_cast<u32x4*>(ks + row * SC_LD + 4 * ch) = b;
    }
    __syncthreads();
    const int ti = tid >> 4, tj = tid & 15;
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
    for (int d = 0; d < 128; d += 4) {
        int4 qv[4], kv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qv[a] = *reinterpret_cast<const int4*>(qs + (ti + 16 * a) * SC_LD + d);
#pragma unroll
        for (int b = 0; b < 4; ++b) kv[b] = *reinterpret_cast<const int4*>(ks + (tj + 16 * b) * SC_LD + d);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                // |code sum| <= 128 * 127 < 2^23: each product is exact in the 24-bit multiplier's 32-bit
                // result, and four of them stay below 2^30
                int s4 = __mul24(qv[a].x, kv[b].x);
                s4 += __mul24(qv[a].y, kv[b].y);
                s4 += __mul24(qv[a].z, kv[b].z);
                s4 += __mul24(qv[a].w, kv[b].w);
                acc[a][b] += (double)s4;
            }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int j = j0 + tj + 16 * b;
        if (j >= T) continue;
        const int n = (j + 1) * 128 <= L ? 128 : L - j * 128;
        const double w = (double)k_scale[h * T + j] / (double)n;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int i = i0 + ti + 16 * a;
            if (i < T) scores[((int64_t)h * T + i) * T + j] = acc[a][b] * w;
        }
    }
}

// ascending order of the float64 values as unsigned integers (finite values; -0 never occurs here:
// a zero score is the product of an integer 0 and a positive weight)
QVD_DEV unsigned long long ordered(double x) {
    const unsigned long long u = __double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// One workgroup per (query tile i, head h); thread tid owns tiles j = tid + 256 m.  Rank key of a tile
// other than the diagonal: ~ordered(score), so that a smaller key is a better tile.  The need =
// min(kept, T) - 1 smallest keys are found by a radix select, one byte per pass from the top: each
// pass histograms the byte of the keys that still match the prefix, and the bin where the count
// reaches `need` extends the prefix.  The result is the key K of the need-th best tile: every key
// below K is kept, and of the keys equal to K the ones of lowest tile index until `need` is met.
__global__ void __launch_bounds__(256) k_select(const double* __restrict__ scores, int T, int kept,
                                                int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
    __shared__ int hist[256];
    __shared__ int flag[SEL_MAX_T];
    __shared__ int wcount[4];
    __shared__ int pick[2];
    const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const double* row = scores + ((int64_t)h * T + i) * T;
    constexpr int M = SEL_MAX_T / 256;
    unsigned long long key[M];
    bool live[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int j = tid + 256 * m;
        live[m] = j < T && j != i;
        key[m] = live[m] ? ~ordered(row[j]) : ~0ull;
    }
    for (int j = tid; j < SEL_MAX_T; j += 256) flag[j] = 0;
    __syncthreads();
    const int cnt = kept < T ? kept : T;
    int need = cnt - 1;
    unsigned long long prefix = 0ull, hmask = 0ull;
    if (need > 0) {
        for (int p = 7; p >= 0; --p) {
            hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (live[m] && (key[m] & hmask) == prefix) atomicAdd(&hist[(int)((key[m] >> (8 * p)) & 0xFFull)], 1);
            __syncthreads();
            if (wv == 0) {
                // lane l holds bins 4l .. 4l+3: inclusive scan over the wave, then the bin that reaches `need`
                int c[4], run = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    run += hist[4 * lane + q];
                    c[q] = run;
                }
                int incl = run;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int t = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += t;
                }
                const int before = incl - run;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lo = before + (q == 0 ? 0 : c[q - 1]), hi = before + c[q];
                    if (lo < need && need <= hi) {
                        pick[0] = 4 * lane + q;
                        pick[1] = lo;
                    }
                }
            }
            __syncthreads();
            const int d = pick[0];
            need -= pick[1];
            prefix |= (unsigned long long)d << (8 * p);
            hmask |= 0xFFull << (8 * p);
        }
        // keep every key below the threshold; of the keys equal to it, the first `need` in tile order
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (live[m] && key[m] < prefix) flag[tid + 256 * m] = 1;
        int taken = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const bool eq = live[m] && key[m] == prefix;
            const unsigned long long b = __ballot(eq);
            __syncthreads();
            if (lane == 0) wcount[wv] = __popcll(b);
            __syncthreads();
            int off = taken;
            for (int w = 0; w < wv; ++w) off += wcount[w];
            if (eq && off + __popcll(b & ((1ull << lane) - 1ull)) < need) flag[tid + 256 * m] = 1;
            taken += wcount[0] + wcount[1] + wcount[2] + wcount[3];
        }
    }
    if (tid == 0) flag[i] = 1;
    __syncthreads();
    // the flagged tiles in tile order (ballot prefix sums)
    int32_t* out = kv_idx + ((int64_t)h * T + i) * kept;
    int base = 0;
    for (int j0 = 0; j0 < T; j0 += 256) {
        const int j = j0 + tid;
        const bool on = j < T && flag[j] != 0;
        const unsigned long long m = __ballot(on);
        if (lane == 0) wcount[wv] = __popcll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wv; ++w) off += wcount[w];
        if (on) out[off + __popcll(m & ((1ull << lane) - 1ull))] = j;
        base += wcount[0] + wcount[1] + wcount[2] + wcount[3];
        __syncthreads();
    }
    for (int r = cnt + tid; r < kept; r += 256) out[r] = -1;
    if (tid == 0) kv_cnt[h * T + i] = cnt;
}

}  // namespace

size_t select_ws_bytes(int L, int H) {
    const size_t T = (size_t)(L + 127) / 128;
    return ((2 * (size_t)H * T * 128 * 4 + 255) & ~(size_t)255) + (size_t)H * T * T * 8;
}

int launch_select_tiles(const int8_t* q8, const int8_t* k8, const float* k_scale, int L, int H, int kept,
                        int32_t* kv_idx, int32_t* kv_cnt, void* ws, hipStream_t st) {
    if (L == 0) return QVD_OK;
    const int T = (L + 127) / 128;
    int32_t* sums = (int32_t*)ws;
    double* scores = (double*)((char*)ws + ((2 * (size_t)H * T * 128 * 4 + 255) & ~(size_t)255));
    TimingScope ts("select_tiles", st);
    hipLaunchKernelGGL(k_tile_sums, dim3(T, H, 2), dim3(256), 0, st, q8, k8, L, H, T, sums);
    int s = launch_status("select_tiles (sums)");
    if (s) return s;
    hipLaunchKernelGGL(k_tile_scores, dim3((T + 63) / 64, (T + 63) / 64, H), dim3(256), 0, st, sums, k_scale, L,
                       H, T, scores);
    s = launch_status("select_tiles (scores)");
    if (s) return s;
    hipLaunchKernelGGL(k_select, dim3(T, H), dim3(256), 0, st, scores, T, kept, kv_idx, kv_cnt);
    return launch_status("select_tiles (select)");
}

}  // namespace qvd

using namespace qvd;

extern "C" {

size_t qvd_select_tiles_ws_bytes(int32_t L, int32_t H) {
    return (L < 0 || H < 1) ? 0 : select_ws_bytes(L, H);
}

int qvd_select_tiles(const int8_t* q, const int8_t* k, const float* k_scale, int32_t L, int32_t H,
                     int32_t kept, int32_t* kv_idx, int32_t* kv_cnt, void* ws, size_t ws_bytes, void* stream) {
    QVD_REQUIRE(L >= 0 && L <= 128 * SEL_MAX_T && H >= 1 && H <= 65535, QVD_ESHAPE,
                "qvd_select_tiles: L = %d (at most %d), H = %d", L, 128 * SEL_MAX_T, H);
    QVD_REQUIRE(kept >= 1 && kept <= SEL_MAX_T, QVD_ESHAPE, "qvd_select_tiles: kept = %d (1 .. %d)", kept,
                SEL_MAX_T);
    if (L == 0) return QVD_OK;
    QVD_PTR(q);
    QVD_PTR(k);
    QVD_PTR(k_scale);
    QVD_PTR(kv_idx);
    QVD_PTR(kv_cnt);
    QVD_PTR(ws);
    QVD_ALIGN(q);
    QVD_ALIGN(k);
    QVD_ALIGN(ws);
    QVD_REQUIRE(ws_bytes >= select_ws_bytes(L, H), QVD_EWORKSPACE, "qvd_select_tiles: workspace %zu < %zu bytes",
                ws_bytes, select_ws_bytes(L, H));
    QVD_DEVICE_OK();
    return launch_select_tiles(q, k, k_scale, L, H, kept, kv_idx, kv_cnt, ws, (hipStream_t)stream);
}

}  // extern "C"
