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
    lds_poison_start(&red[0][0], 4 * kStatsCols);
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

// sum_abs[k] = sum over the chunks of partial[chunk][k] (+ the held value when accumulating);
// mean_abs[k] = float32(sum / total_tokens).  A workgroup takes 32 channels; thread (c, l) adds
// chunks l, l + 8, ... of channel c and the 8 sums of a channel are added in lane order through
// LDS, so many loads are in flight even for a few thousand channels.  The partial sums of |bf16|
// values are exact in float64, so the order does not change the result.
__global__ __launch_bounds__(256) void k_stats_final(const double* __restrict__ partial, int64_t chunks, int64_t K,
                                                     double* __restrict__ sum_abs, int accumulate,
                                                     int64_t total_tokens, float* __restrict__ mean_abs) {
    __shared__ double sm[8][32];
    lds_poison_start(&sm[0][0], 8 * 32);
    const int c = threadIdx.x & 31, l = threadIdx.x >> 5;
    const int64_t k = (int64_t)blockIdx.x * 32 + c;
    const int64_t kk = k < K ? k : K - 1;
    double t = 0.0;
    for (int64_t b0 = l; b0 < chunks; b0 += 8 * 8) {   // 8 loads in flight per thread
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = b0 + 8 * j < chunks ? partial[(b0 + 8 * j) * K + kk] : 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += v[j];
    }
    sm[l][c] = t;
    __syncthreads();
    if (l == 0 && k < K) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += sm[i][c];
        if (accumulate) s = sum_abs[k] + s;
        sum_abs[k] = s;
        if (mean_abs) mean_abs[k] = (float)(s / (double)total_tokens);
    }
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
    k_stats_final<<<(unsigned)((K + 31) / 32), 256, 0, st>>>(partials, p.chunks, K, sum_abs, accumulate,
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

// ---- variants ("AWQ (Activation-aware Weight Quantization)", 重要通道识别的统计依据: the statistic
// may be max |x| instead of the mean; "AWQ 激活感知量化", section 3: s_i = (E|X_i|)^alpha / mean_j |W_ij|,
// and its demo normalizes s by its maximum).

// max_t |x_tk| of a [T, K] bf16 matrix: workgroup partial rows (float32, exact), then the max over
// partial rows (order-independent), optionally with the values already held (accumulate).
__global__ __launch_bounds__(kStatsThreads) void k_max_partial(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                                                              int64_t rows_per_chunk, float* __restrict__ partial) {
    __shared__ float red[4][kStatsCols];
    lds_poison_start(&red[0][0], 4 * kStatsCols);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c0 = (int64_t)blockIdx.x * kStatsCols + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(T, r0 + rows_per_chunk);
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = 0.f;
    for (int64_t r = r0 + wave; r < r1; r += 4) {
        if ((K & 7) == 0 && c0 + 8 <= K) {
            const u32x4 v = *(const u32x4*)(X + r * K + c0);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                m[2 * h] = fmaxf(m[2 * h], fabsf(bf16_lo(v[h])));
                m[2 * h + 1] = fmaxf(m[2 * h + 1], fabsf(bf16_hi(v[h])));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < K) m[j] = fmaxf(m[j], fabsf(bf16_lo((uint32_t)X[r * K + c0 + j])));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = m[j];
    __syncthreads();
    for (int c = threadIdx.x; c < kStatsCols; c += kStatsThreads) {
        const int64_t col = (int64_t)blockIdx.x * kStatsCols + c;
        if (col < K) partial[(int64_t)blockIdx.y * K + col] = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    }
}

__global__ __launch_bounds__(256) void k_max_final(const float* __restrict__ partial, int64_t chunks, int64_t K,
                                                   int accumulate, float* __restrict__ max_abs) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    float m = accumulate ? max_abs[k] : 0.f;
    for (int64_t c = 0; c < chunks; ++c) m = fmaxf(m, partial[c * K + k]);
    max_abs[k] = m;
}

hipError_t launch_act_max(const uint16_t* X, int64_t T, int64_t K, float* max_abs, int accumulate, void* ws,
                          const StatsPlan& p, hipStream_t st) {
    float* partial = (float*)ws;
    dim3 grid((unsigned)p.col_blocks, (unsigned)p.chunks);
    k_max_partial<<<grid, kStatsThreads, 0, st>>>(X, T, K, p.rows_per_chunk, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_max_final<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(partial, p.chunks, K, accumulate, max_abs);
    return hipGetLastError();
}

// mean_j |W_kj| of a [K, N] bf16 matrix: one workgroup per row k, each lane a strided float64 sum
// (exact for bf16 magnitudes whose exponents span less than ~2^30), a fixed-order tree through
// LDS, then one division and the float32 rounding.
__global__ __launch_bounds__(256) void k_weight_mean_abs(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                         float* __restrict__ w_mean) {
    __shared__ double red[256];
    lds_poison_start(&red[0], 256);
    const int64_t k = blockIdx.x;
    double s = 0.0;
    for (int64_t n = threadIdx.x; n < N; n += 256) s += (double)fabsf(bf16_lo((uint32_t)W[k * N + n]));
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) w_mean[k] = (float)(red[0] / (double)N);
}

hipError_t launch_weight_mean_abs(const uint16_t* W, int64_t K, int64_t N, float* w_mean, hipStream_t st) {
    k_weight_mean_abs<<<(unsigned)K, 256, 0, st>>>(W, K, N, w_mean);
    return hipGetLastError();
}

// t[i, k] = max(stat_k, 1e-8)^alpha_i / max(w_mean_k, 1e-8) (without the division when w_mean is
// null), divided by max_k t[i, k] when normalize, in float64; s[i, k] = float32(t[i, k]).  One
// workgroup per alpha: the row maximum is an order-independent reduction of the same values.
__global__ __launch_bounds__(256) void k_scale_table_ex(const float* __restrict__ stat,
                                                        const float* __restrict__ w_mean, int64_t K, int n_grid,
                                                        int normalize, float* __restrict__ s_tab) {
    __shared__ double red[256];
    lds_poison_start(&red[0], 256);
    const int i = blockIdx.x;
    const double a = (double)i / (double)(n_grid - 1);
    auto t_of = [&](int64_t k) {
        double t = pow(fmax((double)stat[k], 1e-8), a);
        if (w_mean) t = t / fmax((double)w_mean[k], 1e-8);
        return t;
    };
    double mx = 1.0;
    if (normalize) {
        double m = 0.0;
        for (int64_t k = threadIdx.x; k < K; k += 256) m = fmax(m, t_of(k));
        red[threadIdx.x] = m;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if ((int)threadIdx.x < o) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + o]);
            __syncthreads();
        }
        mx = red[0];
    }
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const double t = t_of(k);
        s_tab[(int64_t)i * K + k] = (float)(normalize ? t / mx : t);
    }
}

hipError_t launch_scale_table_ex(const float* stat, const float* w_mean, int64_t K, int n_grid, int normalize,
                                 float* s_tab, hipStream_t st) {
    k_scale_table_ex<<<(unsigned)n_grid, 256, 0, st>>>(stat, w_mean, K, n_grid, normalize, s_tab);
    return hipGetLastError();
}

}  // namespace awq
