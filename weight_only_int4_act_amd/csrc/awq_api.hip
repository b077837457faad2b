// C ABI of libawq (declared in include/awq.h): argument validation on the host, then launches on
// the caller's stream.  Nothing is allocated, freed or synchronized here.
#include "../../include/awq.h"
#include "awq_internal.h"

#include <mutex>

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return AWQ_OK;
    g_last_hip_error = (int)e;
    return AWQ_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }
constexpr int64_t kIntMax = 0x7fffffff;
constexpr int64_t kGemmRowsMax = (int64_t)65535 * 64;   // M: workgroup rows of the product's grid
// every size is checked against these bounds before any arithmetic on it, so no size query or
// plan can overflow
bool in_range(int64_t v, int64_t hi) { return v > 0 && v <= hi; }

int check_cfg(const awq_qconfig* cfg, int64_t K) {
    if (!cfg) return AWQ_ERR_INVALID_ARG;
    if (cfg->w_bit != 4) return AWQ_ERR_UNSUPPORTED;
    if (!group_ok(cfg->group_size)) return AWQ_ERR_UNSUPPORTED;
    if (cfg->n_grid < 2 || cfg->n_grid > 64) return AWQ_ERR_UNSUPPORTED;
    if (cfg->zero_point != 0 && cfg->zero_point != 1) return AWQ_ERR_INVALID_ARG;
    if (!(cfg->clip_ratio >= 0.f && cfg->clip_ratio <= 1.f)) return AWQ_ERR_UNSUPPORTED;   // NaN fails too
    if (K % cfg->group_size != 0) return AWQ_ERR_INVALID_ARG;
    return AWQ_OK;
}

}  // namespace

extern "C" {

size_t awq_act_stats_workspace_size(int64_t T, int64_t K) {
    if (!in_range(T, kIntMax) || !in_range(K, kIntMax)) return 0;
    return awq::plan_stats(T, K).ws_bytes;
}

int awq_act_stats(const void* X_bf16, int64_t T, int64_t K, double* sum_abs, int accumulate,
                  int64_t total_tokens, float* mean_abs, void* workspace, size_t ws_bytes, void* stream) {
    if (!X_bf16 || !sum_abs || !in_range(T, kIntMax) || !in_range(K, kIntMax) || total_tokens < T)
        return AWQ_ERR_INVALID_ARG;
    if (accumulate != 0 && accumulate != 1) return AWQ_ERR_INVALID_ARG;
    if (!aligned(X_bf16, 16) || !aligned(sum_abs, 8) || (mean_abs && !aligned(mean_abs, 4)))
        return AWQ_ERR_INVALID_ARG;
    const awq::StatsPlan p = awq::plan_stats(T, K);
    if (ws_bytes < p.ws_bytes || (p.ws_bytes && !workspace)) return AWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_stats((const uint16_t*)X_bf16, T, K, sum_abs, accumulate, total_tokens,
                                        mean_abs, (double*)workspace, p, (hipStream_t)stream));
}

int awq_scale_table(const float* mean_abs, int64_t K, int32_t n_grid, float* s_table, void* stream) {
    if (!mean_abs || !s_table || !in_range(K, kIntMax)) return AWQ_ERR_INVALID_ARG;
    if (n_grid < 2 || n_grid > 64) return AWQ_ERR_UNSUPPORTED;
    if (!aligned(mean_abs, 4) || !aligned(s_table, 4)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_scale_table(mean_abs, K, n_grid, s_table, nullptr, (hipStream_t)stream));
}

int awq_act_max(const void* X_bf16, int64_t T, int64_t K, float* max_abs, int accumulate, void* workspace,
                size_t ws_bytes, void* stream) {
    if (!X_bf16 || !max_abs || !in_range(T, kIntMax) || !in_range(K, kIntMax)) return AWQ_ERR_INVALID_ARG;
    if (accumulate != 0 && accumulate != 1) return AWQ_ERR_INVALID_ARG;
    if (!aligned(X_bf16, 16) || !aligned(max_abs, 4)) return AWQ_ERR_INVALID_ARG;
    const awq::StatsPlan p = awq::plan_stats(T, K);
    if (ws_bytes < p.ws_bytes || (p.ws_bytes && !workspace)) return AWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_act_max((const uint16_t*)X_bf16, T, K, max_abs, accumulate, workspace, p,
                                          (hipStream_t)stream));
}

int awq_weight_mean_abs(const void* W_bf16, int64_t K, int64_t N, float* w_mean, void* stream) {
    if (!W_bf16 || !w_mean || !in_range(K, kIntMax) || !in_range(N, kIntMax)) return AWQ_ERR_INVALID_ARG;
    if (!aligned(W_bf16, 2) || !aligned(w_mean, 4)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_weight_mean_abs((const uint16_t*)W_bf16, K, N, w_mean, (hipStream_t)stream));
}

int awq_scale_table_ex(const float* stat, const float* w_mean, int64_t K, int32_t n_grid, int32_t normalize,
                       float* s_table, void* stream) {
    if (!stat || !s_table || !in_range(K, kIntMax)) return AWQ_ERR_INVALID_ARG;
    if (n_grid < 2 || n_grid > 64) return AWQ_ERR_UNSUPPORTED;
    if (normalize != 0 && normalize != 1) return AWQ_ERR_INVALID_ARG;
    if (!aligned(stat, 4) || !aligned(s_table, 4) || (w_mean && !aligned(w_mean, 4))) return AWQ_ERR_INVALID_ARG;
    return hip_status(
        awq::launch_scale_table_ex(stat, w_mean, K, n_grid, normalize, s_table, (hipStream_t)stream));
}

size_t awq_search_workspace_size(int64_t T, int64_t K, int64_t N, const awq_qconfig* cfg) {
    if (!in_range(T, kIntMax) || !in_range(K, kIntMax) || !in_range(N, kIntMax) || T * K > kIntMax ||
        check_cfg(cfg, K) != AWQ_OK)
        return 0;
    return awq::plan_search(T, K, N, cfg->group_size, cfg->zero_point, cfg->n_grid, false).ws_bytes;
}

namespace {

// Checks shared by both searches; 0 when the call may go ahead.
int check_search(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N, const float* vec,
                 const awq_qconfig* cfg, void* workspace, size_t ws_bytes, const double* losses, const int32_t* best,
                 const float* out, bool clip, awq::SearchPlan* p) {
    if (!X_bf16 || !W_bf16 || !vec || !losses || !best || !out) return AWQ_ERR_INVALID_ARG;
    if (!in_range(T, kIntMax) || !in_range(K, kIntMax) || !in_range(N, kIntMax) || T * K > kIntMax)
        return AWQ_ERR_INVALID_ARG;
    int st = check_cfg(cfg, K);
    if (st != AWQ_OK) return st;
    if (!aligned(X_bf16, 16) || !aligned(W_bf16, 2) || !aligned(vec, 4) || !aligned(losses, 8) ||
        !aligned(best, 4) || !aligned(out, 4))
        return AWQ_ERR_INVALID_ARG;
    *p = awq::plan_search(T, K, N, cfg->group_size, cfg->zero_point, cfg->n_grid, clip);
    // tile counts and the 16-byte index into the tiled copy of X are 32-bit in the kernel; the
    // kernel addresses the staged inputs (scale table, reciprocals, W tiles) and one token tile of
    // tiled X through buffer resources with 32-bit byte offsets
    if (p->tiles > kIntMax || p->tb * p->bm * K / 8 > kIntMax ||
        (int64_t)(p->off_xt - p->off_s) > (int64_t)0xffffffff || (int64_t)p->bm * K * 2 > kIntMax)
        return AWQ_ERR_INVALID_ARG;
    if (ws_bytes < p->ws_bytes || !workspace) return AWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return AWQ_ERR_INVALID_ARG;
    return AWQ_OK;
}

}  // namespace

int awq_search(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N, const float* mean_abs,
               const awq_qconfig* cfg, void* workspace, size_t ws_bytes, double* losses, int32_t* best,
               float* s_best, void* stream) {
    awq::SearchPlan p;
    const bool clip = cfg && cfg->clip_ratio > 0.f && cfg->clip_ratio < 1.f;
    const int st =
        check_search(X_bf16, T, W_bf16, K, N, mean_abs, cfg, workspace, ws_bytes, losses, best, s_best, clip, &p);
    if (st != AWQ_OK) return st;
    return hip_status(awq::launch_search((const uint16_t*)X_bf16, T, (const uint16_t*)W_bf16, K, N, mean_abs,
                                         cfg->clip_ratio, p, workspace, losses, best, s_best, (hipStream_t)stream));
}

int awq_search_table(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N, const float* s_table,
                     const awq_qconfig* cfg, void* workspace, size_t ws_bytes, double* losses, int32_t* best,
                     float* s_best, void* stream) {
    awq::SearchPlan p;
    const bool clip = cfg && cfg->clip_ratio > 0.f && cfg->clip_ratio < 1.f;
    const int st =
        check_search(X_bf16, T, W_bf16, K, N, s_table, cfg, workspace, ws_bytes, losses, best, s_best, clip, &p);
    if (st != AWQ_OK) return st;
    return hip_status(awq::launch_search_table((const uint16_t*)X_bf16, T, (const uint16_t*)W_bf16, K, N, s_table,
                                               cfg->clip_ratio, p, workspace, losses, best, s_best,
                                               (hipStream_t)stream));
}

int awq_clip_search(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N, const float* s,
                    const awq_qconfig* cfg, float clip_min, void* workspace, size_t ws_bytes, double* losses,
                    int32_t* best, float* clip_best, void* stream) {
    if (!(clip_min > 0.f && clip_min <= 1.f)) return AWQ_ERR_INVALID_ARG;
    awq::SearchPlan p;
    const int st =
        check_search(X_bf16, T, W_bf16, K, N, s, cfg, workspace, ws_bytes, losses, best, clip_best, true, &p);
    if (st != AWQ_OK) return st;
    return hip_status(awq::launch_clip_search((const uint16_t*)X_bf16, T, (const uint16_t*)W_bf16, K, N, s,
                                              clip_min, p, workspace, losses, best, clip_best, (hipStream_t)stream));
}

size_t awq_search_multi_workspace_size(int64_t T, int64_t K, int32_t n_w, const int64_t* N,
                                      const awq_qconfig* cfg) {
    if (n_w < 1 || n_w > AWQ_MAX_PROJECTIONS || !N) return 0;
    int64_t cols = 0;
    for (int j = 0; j < n_w; ++j) {
        if (N[j] <= 0 || N[j] > kIntMax) return 0;
        cols += (N[j] + 15) / 16 * 16;
    }
    if (!in_range(T, kIntMax) || !in_range(K, kIntMax) || T * K > kIntMax || cols > kIntMax ||
        check_cfg(cfg, K) != AWQ_OK)
        return 0;
    const bool clip = cfg->clip_ratio > 0.f && cfg->clip_ratio < 1.f;
    return awq::plan_search(T, K, cols, cfg->group_size, cfg->zero_point, cfg->n_grid, clip).ws_bytes;
}

int awq_search_multi(const void* X_bf16, int64_t T, int32_t n_w, const void* const* W_bf16, const int64_t* N,
                     int64_t K, const float* mean_abs, const awq_qconfig* cfg, void* workspace, size_t ws_bytes,
                     double* losses, double* losses_each, int32_t* best, float* s_best, void* stream) {
    if (n_w < 1 || n_w > AWQ_MAX_PROJECTIONS || !W_bf16 || !N) return AWQ_ERR_INVALID_ARG;
    int64_t cols = 0;
    for (int j = 0; j < n_w; ++j) {
        if (!W_bf16[j] || !aligned(W_bf16[j], 2) || N[j] <= 0 || N[j] > kIntMax) return AWQ_ERR_INVALID_ARG;
        cols += (N[j] + 15) / 16 * 16;
    }
    if (losses_each && !aligned(losses_each, 8)) return AWQ_ERR_INVALID_ARG;
    awq::SearchPlan p;
    const bool clip = cfg && cfg->clip_ratio > 0.f && cfg->clip_ratio < 1.f;
    const int st =
        check_search(X_bf16, T, W_bf16[0], K, cols, mean_abs, cfg, workspace, ws_bytes, losses, best, s_best, clip, &p);
    if (st != AWQ_OK) return st;
    return hip_status(awq::launch_search_multi((const uint16_t*)X_bf16, T, n_w, (const uint16_t* const*)W_bf16, N,
                                               K, mean_abs, cfg->clip_ratio, p, workspace, losses, losses_each, best,
                                               s_best, (hipStream_t)stream));
}

size_t awq_greedy_workspace_size(int64_t K, int64_t N, const awq_qconfig* cfg, int32_t n_cand) {
    if (!in_range(K, kIntMax) || !in_range(N, kIntMax) || check_cfg(cfg, K) != AWQ_OK || n_cand < 2 ||
        n_cand > AWQ_MAX_POW2_CANDIDATES || K / cfg->group_size > 65535)
        return 0;
    return awq::plan_greedy(K, N, cfg->group_size, n_cand).ws_bytes;
}

int awq_greedy_search(const void* W_bf16, int64_t K, int64_t N, const float* mean_abs, const awq_qconfig* cfg,
                      int32_t n_cand, int32_t passes, void* workspace, size_t ws_bytes, float* s_best,
                      double* err_rtn, double* err, void* stream) {
    if (!W_bf16 || !mean_abs || !s_best || !in_range(K, kIntMax) || !in_range(N, kIntMax)) return AWQ_ERR_INVALID_ARG;
    int st = check_cfg(cfg, K);
    if (st != AWQ_OK) return st;
    if (cfg->clip_ratio > 0.f && cfg->clip_ratio < 1.f) return AWQ_ERR_UNSUPPORTED;
    if (n_cand < 2 || n_cand > AWQ_MAX_POW2_CANDIDATES || passes < 1 || passes > 64) return AWQ_ERR_INVALID_ARG;
    if (K / cfg->group_size > 65535 || N > kIntMax) return AWQ_ERR_INVALID_ARG;
    if (!aligned(W_bf16, 2) || !aligned(mean_abs, 4) || !aligned(s_best, 4) || (err_rtn && !aligned(err_rtn, 8)) ||
        (err && !aligned(err, 8)))
        return AWQ_ERR_INVALID_ARG;
    const awq::GreedyPlan p = awq::plan_greedy(K, N, cfg->group_size, n_cand);
    if (ws_bytes < p.ws_bytes || !workspace) return AWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_greedy((const uint16_t*)W_bf16, K, N, mean_abs, cfg->zero_point, passes, p,
                                         workspace, s_best, err_rtn, err, (hipStream_t)stream));
}

int awq_pack(const void* W_bf16, int64_t K, int64_t N, const float* s, const awq_qconfig* cfg, uint32_t* codes,
             float* scales, uint8_t* zeros, void* stream) {
    if (!W_bf16 || !s || !codes || !scales || !zeros || !in_range(K, kIntMax) || !in_range(N, kIntMax))
        return AWQ_ERR_INVALID_ARG;
    int st = check_cfg(cfg, K);
    if (st != AWQ_OK) return st;
    if (K / cfg->group_size > 65535) return AWQ_ERR_INVALID_ARG;
    if (!aligned(W_bf16, 2) || !aligned(s, 4) || !aligned(codes, 4) || !aligned(scales, 4))
        return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_pack((const uint16_t*)W_bf16, K, N, s, cfg->group_size, cfg->zero_point,
                                       cfg->clip_ratio, codes, scales, zeros, (hipStream_t)stream));
}

size_t awq_w4a16_gemm_workspace_size(int64_t M, int64_t K, int64_t N, int32_t group_size) {
    if (!in_range(M, kGemmRowsMax) || !in_range(K, kIntMax) || !in_range(N, (int64_t)(awq::kGemmCounterBytes / 4) * 256) ||
        !group_ok(group_size) || K % group_size)
        return 0;
    return awq::plan_gemm(M, K, N, group_size).ws_bytes;
}

}  // extern "C"

namespace {

// Checks of awq_w4a16_gemm's arguments other than the workspace; fills the plan.
int check_gemm(const void* X_bf16, int64_t M, const float* s, const uint32_t* codes, const float* scales,
               const uint8_t* zeros, int64_t K, int64_t N, int32_t group_size, const void* Y_bf16,
               awq::GemmPlan* p) {
    if (!X_bf16 || !s || !codes || !scales || !zeros || !Y_bf16) return AWQ_ERR_INVALID_ARG;
    if (!in_range(M, kGemmRowsMax) || !in_range(K, kIntMax) || !in_range(N, (int64_t)(awq::kGemmCounterBytes / 4) * 256) ||
        N % 8 != 0)
        return AWQ_ERR_INVALID_ARG;
    if (!group_ok(group_size)) return AWQ_ERR_UNSUPPORTED;
    if (K % group_size != 0) return AWQ_ERR_INVALID_ARG;
    if (!aligned(X_bf16, 16) || !aligned(s, 16) || !aligned(codes, 16) || !aligned(scales, 16) ||
        !aligned(zeros, 16) || !aligned(Y_bf16, 16))
        return AWQ_ERR_INVALID_ARG;
    *p = awq::plan_gemm(M, K, N, group_size);
    if (p->variant < 0 || p->grid_y > 65535 || (N + 63) / 64 > kIntMax || (M > 1 && (K + 255) / 256 > 65535))
        return AWQ_ERR_INVALID_ARG;
    // M = 1: the split-K partials are addressed with 32-bit byte offsets (a buffer resource)
    if (p->variant == 0 && p->ksplit * N * 4 > (int64_t)0xffffffff) return AWQ_ERR_INVALID_ARG;
    return AWQ_OK;
}

// The allocation-free entry point's scratch: one fixed array per GPU, held until the process
// ends.  Host code never uses the array's name as an address (on the host it is only a stand-in
// for the device symbol); its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr.  It starts zeroed (the arrival counters at its
// front must be zero) and every completed call leaves those counters zero.
constexpr size_t kScratchBytes = awq::kGemmCounterBytes + ((size_t)16 << 20);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void* scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// Device address of this device's scratch (looked up on the device's first call); nullptr on a
// HIP error (recorded for awq_last_hip_error).
void* device_scratch(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int awq_w4a16_gemm(const void* X_bf16, int64_t M, const float* s, const uint32_t* codes, const float* scales,
                   const uint8_t* zeros, int64_t K, int64_t N, int32_t group_size, void* Y_bf16, void* workspace,
                   size_t ws_bytes, void* stream) {
    awq::GemmPlan p;
    const int st = check_gemm(X_bf16, M, s, codes, scales, zeros, K, N, group_size, Y_bf16, &p);
    if (st != AWQ_OK) return st;
    if (ws_bytes < p.ws_bytes || (p.ws_bytes && !workspace)) return AWQ_ERR_WORKSPACE;
    if (p.ws_bytes && !aligned(workspace, 256)) return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_gemm((const uint16_t*)X_bf16, M, s, codes, scales, zeros, K, N, group_size,
                                       (uint16_t*)Y_bf16, workspace, p, (hipStream_t)stream));
}

size_t awq_w4a16_gemm_static_scratch_bytes(void) { return kScratchBytes; }

int awq_w4a16_gemm_noalloc(const void* X_bf16, int64_t M, const float* s, const uint32_t* codes,
                           const float* scales, const uint8_t* zeros, int64_t K, int64_t N, int32_t group_size,
                           void* Y_bf16, void* stream) {
    awq::GemmPlan p;
    const int st = check_gemm(X_bf16, M, s, codes, scales, zeros, K, N, group_size, Y_bf16, &p);
    if (st != AWQ_OK) return st;
    if (p.ws_bytes > kScratchBytes) return AWQ_ERR_SCRATCH;
    hipError_t e = hipSuccess;
    void* ws = p.ws_bytes ? device_scratch(&e) : nullptr;
    if (e != hipSuccess) return hip_status(e);
    return hip_status(awq::launch_gemm((const uint16_t*)X_bf16, M, s, codes, scales, zeros, K, N, group_size,
                                       (uint16_t*)Y_bf16, ws, p, (hipStream_t)stream));
}

const char* awq_status_string(int status) {
    switch (status) {
        case AWQ_OK: return "ok";
        case AWQ_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or shape)";
        case AWQ_ERR_UNSUPPORTED: return "unsupported configuration (w_bit, group_size, n_grid or clip_ratio)";
        case AWQ_ERR_WORKSPACE: return "workspace too small";
        case AWQ_ERR_HIP: return "HIP runtime error (see awq_last_hip_error)";
        case AWQ_ERR_SCRATCH:
            return "the call needs more scratch than the fixed per-GPU buffer of awq_w4a16_gemm_noalloc "
                   "(awq_w4a16_gemm_static_scratch_bytes); use awq_w4a16_gemm with a workspace";
        default: return "unknown status";
    }
}

int awq_last_hip_error(void) { return g_last_hip_error; }

const char* awq_version(void) { return "libawq 0.1 (gfx950)"; }

}  // extern "C"
