// a1: per-input-channel mean |x| over the calibration tokens, and a2: the scale table.
//
// Statistic: "AWQ (Activation-aware Weight Quantization)", section 重要通道识别的统计依据
// (mean of |X_calib[:, j]| per input channel) and "AWQ 激活感知量化", section 1
// (I_i = E|X_i|, averaged over the calibration samples).  Scale family: the first page,
// section 缩放因子优化的完整流程, step 3 (s_j(alpha) = activation_scale[j]^alpha).
//
// The reduction runs down the token axis of a row-major [T, K] bf16 matrix.  Each lane owns
// 8 consecutive channels and reads them with one 16-byte load per row, so a wavefront reads
// 1 KB of one row and every access is fully coalesced.  Sums are float64; a workgroup reduces
// its 4 wavefronts in a fixed order and writes one partial row; a second kernel adds the
// partial rows in a fixed order.  No atomics: the result does not depend on scheduling.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = 512;   // channels per workgroup (64 lanes x 8)

template <bool VEC>
__global__ __launch_bounds__(kStatsThreads) void k_stats_partial(const uint16_t* __restrict__ X, int64_t T,
                                                                 int64_t K, int64_t rows_per_chunk,
                                                                 double* __restrict__ partial) {
    __shared__ double red[4][kStatsCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c0 = (int64_t)blockIdx.x * kStatsCols + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(T, r0 + rows_per_chunk);
    double acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0;

    if (VEC && c0 + 8 <= K) {
        const uint16_t* base = X + c0;
        int64_t r = r0 + wave;
        // four rows in flight per wavefront
        for (; r + 12 < r1; r += 16) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *(const u32x4*)(base + (r + 4 * u) * K);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    acc[2 * h] += (double)fabsf(bf16_lo(v[u][h]));
                    acc[2 * h + 1] += (double)fabsf(bf16_hi(v[u][h]));
                }
            }
        }
        for (; r < r1; r += 4) {
            u32x4 v = *(const u32x4*)(base + r * K);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                acc[2 * h] += (double)fabsf(bf16_lo(v[h]));
                acc[2 * h + 1] += (double)fabsf(bf16_hi(v[h]));
            }
        }
    } else {
        for (int64_t r = r0 + wave; r < r1; r += 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < K) acc[j] += (double)fabsf(bf16_lo((uint32_t)X[r * K + c0 + j]));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = acc[j];
    __syncthreads();
    for (int c = threadIdx.x; c < kStatsCols; c += kStatsThreads) {
        const int64_t col = (int64_t)blockIdx.x * kStatsCols + c;
        if (col < K) partial[(int64_t)blockIdx.y * K + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
}

__global__ __launch_bounds__(256) void k_stats_final(const double* __restrict__ partial, int64_t chunks, int64_t K,
                                                     double* __restrict__ sum_abs, int accumulate,
                                                     int64_t total_tokens, float* __restrict__ mean_abs) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double s = 0.0;
    for (int64_t c0 = 0; c0 < chunks; c0 += 8) {   // 8 loads in flight, added in the same fixed order
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = c0 + j < chunks ? partial[(c0 + j) * K + k] : 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[j];
    }
    if (accumulate) s = sum_abs[k] + s;
    sum_abs[k] = s;
    if (mean_abs) mean_abs[k] = (float)(s / (double)total_tokens);
}

StatsPlan plan_stats(int64_t T, int64_t K) {
    StatsPlan p;
    p.col_blocks = (K + kStatsCols - 1) / kStatsCols;
    // aim for ~1024 workgroups (4 per CU) with at least 64 rows each
    int64_t want = (1024 + p.col_blocks - 1) / p.col_blocks;
    int64_t max_chunks = (T + 63) / 64;
    p.chunks = want < max_chunks ? want : max_chunks;
    if (p.chunks < 1) p.chunks = 1;
    p.rows_per_chunk = (T + p.chunks - 1) / p.chunks;
    p.rows_per_chunk = (p.rows_per_chunk + 15) / 16 * 16;
    p.chunks = (T + p.rows_per_chunk - 1) / p.rows_per_chunk;
    p.ws_bytes = (size_t)p.chunks * (size_t)K * sizeof(double);
    return p;
}

hipError_t launch_stats(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, int accumulate,
                        int64_t total_tokens, float* mean_abs, double* partials, const StatsPlan& p,
                        hipStream_t st) {
    dim3 grid((unsigned)p.col_blocks, (unsigned)p.chunks);
    if (K % 8 == 0)
        k_stats_partial<true><<<grid, kStatsThreads, 0, st>>>(X, T, K, p.rows_per_chunk, partials);
    else
        k_stats_partial<false><<<grid, kStatsThreads, 0, st>>>(X, T, K, p.rows_per_chunk, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_stats_final<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(partials, p.chunks, K, sum_abs, accumulate,
                                                              total_tokens, mean_abs);
    return hipGetLastError();
}

// s[i, k] = fl32(max(m_k, 1e-8) ^ (i / (n_grid - 1))) in float64; inv[i, k] = fl32(1 / s[i, k]).
__global__ __launch_bounds__(256) void k_scale_table(const float* __restrict__ mean_abs, int64_t K, int n_grid,
                                                     float* __restrict__ s_tab, float* __restrict__ inv_tab) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int i = blockIdx.y;
    if (k >= K) return;
    const double m = fmax((double)mean_abs[k], 1e-8);
    const double a = (double)i / (double)(n_grid - 1);
    const float s = (float)pow(m, a);
    s_tab[(int64_t)i * K + k] = s;
    if (inv_tab) inv_tab[(int64_t)i * K + k] = 1.0f / s;
}

hipError_t launch_scale_table(const float* mean_abs, int64_t K, int n_grid, float* s_tab, float* inv_tab,
                              hipStream_t st) {
    dim3 grid((unsigned)((K + 255) / 256), (unsigned)n_grid);
    k_scale_table<<<grid, 256, 0, st>>>(mean_abs, K, n_grid, s_tab, inv_tab);
    return hipGetLastError();
}

}  // namespace awq
