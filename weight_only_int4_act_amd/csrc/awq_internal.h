// Host-side launchers of the libawq kernels (internal; the public ABI is include/awq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

constexpr int kMaxGrid = 64;   // largest alpha / clip-ratio grid

// ---- a1: statistic
struct StatsPlan {
    int64_t col_blocks;      // workgroups along K (512 channels each)
    int64_t chunks;          // workgroups along T
    int64_t rows_per_chunk;
    size_t ws_bytes;         // float64 partials [chunks, K]
};
StatsPlan plan_stats(int64_t T, int64_t K);
hipError_t launch_stats(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, int accumulate,
                        int64_t total_tokens, float* mean_abs, double* partials, const StatsPlan& p,
                        hipStream_t st);

// max |x| per channel (workspace: the statistic's partials; accumulate: max with the held values)
hipError_t launch_act_max(const uint16_t* X, int64_t T, int64_t K, float* max_abs, int accumulate, void* ws,
                          const StatsPlan& p, hipStream_t st);
// mean_j |W_kj| per input channel
hipError_t launch_weight_mean_abs(const uint16_t* W, int64_t K, int64_t N, float* w_mean, hipStream_t st);

// ---- a2: scale table (and its reciprocal, used inside the search)
hipError_t launch_scale_table(const float* mean_abs, int64_t K, int n_grid, float* s_tab, float* inv_tab,
                              hipStream_t st);
// variants: optional mean |W| denominator and per-row normalization by the maximum
hipError_t launch_scale_table_ex(const float* stat, const float* w_mean, int64_t K, int n_grid, int normalize,
                                 float* s_tab, hipStream_t st);

// ---- a3/a4: search
struct SearchPlan {
    int group_size, n_grid, zero_point;
    int variant;             // row blocks of 16 tokens per wavefront (4 or 5)
    int na;                  // alpha slots per workgroup
    int bm;                  // token rows per workgroup
    int n_asplit;            // alpha slices
    int64_t nb;              // 16-column blocks (N rounded up)
    int64_t tb;              // token blocks
    int64_t tiles, tiles_per_xcd, grid;
    // workspace layout (byte offsets): scale table, reciprocals, W tiles, X tiles, loss partials,
    // clip ratio per grid point
    size_t off_s, off_inv, off_wt, off_xt, off_part, off_clip, ws_bytes;
};
// clip: the quantizer is clipped (awq_clip_search, or awq_search with a clip ratio); the workspace
// layout does not depend on it
SearchPlan plan_search(int64_t T, int64_t K, int64_t N, int group_size, int zero_point, int n_grid, bool clip);
// alpha grid from mean_abs, every point's quantizer clipped by clip_ratio (0 or 1: none)
hipError_t launch_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                         const float* mean_abs, float clip_ratio, const SearchPlan& p, void* ws, double* losses,
                         int32_t* best, float* s_best, hipStream_t st);
// the rows of a caller's scale table (n_grid x K, device) instead of the alpha grid
hipError_t launch_search_table(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                               const float* table, float clip_ratio, const SearchPlan& p, void* ws, double* losses,
                               int32_t* best, float* s_best, hipStream_t st);
// several matrices sharing X (K rows each, N[j] columns, j < n_w), searched as one column-tile
// stream (each padded to a multiple of 16 columns); plan for N = sum_j round_up(N[j], 16)
hipError_t launch_search_multi(const uint16_t* X, int64_t T, int n_w, const uint16_t* const* W, const int64_t* N,
                               int64_t K, const float* mean_abs, float clip_ratio, const SearchPlan& p, void* ws,
                               double* losses, double* losses_each, int32_t* best, float* s_best, hipStream_t st);
// clip-ratio grid 1 .. clip_min at the fixed scales s
hipError_t launch_clip_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                              const float* s, float clip_min, const SearchPlan& p, void* ws, double* losses,
                              int32_t* best, float* clip_best, hipStream_t st);

// ---- a5: pack (clip_ratio 0 or 1: no clipping)
hipError_t launch_pack(const uint16_t* W, int64_t K, int64_t N, const float* s, int group_size,
                       int zero_point, float clip_ratio, uint32_t* codes, float* scales, uint8_t* zeros,
                       hipStream_t st);

// ---- power-of-two greedy over the per-channel scales
struct GreedyPlan {
    int group_size, n_cand;
    int64_t groups, n_slices, part_stride;
    size_t off_idx, off_part, off_rtn, ws_bytes;
};
GreedyPlan plan_greedy(int64_t K, int64_t N, int group_size, int n_cand);
hipError_t launch_greedy(const uint16_t* W, int64_t K, int64_t N, const float* mean_abs, int zero_point,
                         int passes, const GreedyPlan& p, void* ws, float* s_best, double* err_rtn, double* err,
                         hipStream_t st);

// ---- a6: W4A16 product
// Arrival counters of the M <= 16 product: one uint32 per 256 output columns, at the start of
// every W4A16 workspace (N up to 4194304 columns).
constexpr size_t kGemmCounterBytes = 65536;
struct GemmPlan {
    int variant;             // 0: M = 1 GEMV; 1: 2..16 rows; 2: 17..32 rows; 5: LDS-shared x' (M > 32);
                             // -1: size not supported
    int64_t grid_x, grid_y, grid_z;
    int ksplit;              // workgroups along K
    int64_t mpad;            // M rounded up to the workgroup's row tile
    int vgroup;              // M = 1: rows of K a wavefront takes at a time (a slice of a group);
                             // 2..16 rows: quantization groups of K per workgroup
    int gpw;                 // M = 1: slices per wavefront
    int qr;                  // M = 1: lanes per column quadruple (1: 256 columns per workgroup, 4: 64)
    int cstride;             // arrival counter i at word i * cstride of the counter region
    // workspace layout (byte offsets): split-K partials, arrival counters (M <= 16, zero between
    // calls), x' in fragment order and group sums of x' (M > 16)
    size_t off_part, off_cnt, off_xp, off_sg, ws_bytes;
};
GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int group_size);
hipError_t launch_gemm(const uint16_t* X, int64_t M, const float* s, const uint32_t* codes,
                       const float* scales, const uint8_t* zeros, int64_t K, int64_t N, int group_size,
                       uint16_t* Y, void* ws, const GemmPlan& p, hipStream_t st);

}  // namespace awq
