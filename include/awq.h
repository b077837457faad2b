/*
 * awq.h -- C ABI of libawq, the MI355X (gfx950) implementation of the AWQ
 * (activation-aware weight quantization) hot path.
 *
 * The library computes, for one linear layer Y = X W with W laid out
 * [K = input channels, N = output channels]:
 *   1. the per-input-channel activation statistic m_k = mean_t |x_tk|;
 *   2. the per-layer scale search over alpha_i = i/(n_grid-1), scoring
 *      L(alpha) = || X (S^-1 Q(S W) - W) ||^2 with S = diag(m^alpha);
 *   3. INT4 packing of the winning S* W (codes, per-group scales and zeros) and
 *      the W4A16 product Y = (X / s*) Dequant(Wq);
 *   4. variants of the search: over a caller's scale table (other statistics and
 *      scale families), over clip ratios, jointly over projections that share X, and
 *      the power-of-two per-group greedy of [P4].
 *
 * Sources (page title -- section), for the definitions cited below:
 *   [P1] "AWQ (Activation-aware Weight Quantization)" (compassingai.com)
 *   [P2] "大模型 AWQ 量化实战：激活感知权重量化（Activation-aware Weight Quantization）部署" (CSDN)
 *   [P3] "AWQ 激活感知量化" (aiqz.cc)
 *   [P4] "009. AWQ Integration" (blog.yoooo.fun)
 *   [P5] "量化推理算法 GPTQ / AWQ" (slowleelab)
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronizes; scratch space is the caller's `workspace`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *     enqueued asynchronously; outputs are valid once the stream has completed it.
 *   - Matrices are row-major and contiguous.  bf16 inputs and all outputs must be
 *     16-byte aligned.
 *   - Argument errors are detected on the host BEFORE anything is enqueued; then the
 *     call returns a negative status and writes nothing.  AWQ_ERR_HIP is returned when
 *     a kernel launch fails (outputs are then unspecified).
 *   - Calls on distinct streams with distinct outputs and workspaces may run
 *     concurrently.  Calls that share a workspace must be ordered by the caller.
 *   - Results are deterministic: no floating-point atomics; every reduction has a
 *     fixed order, so repeated calls on the same inputs give bit-identical outputs.
 */
#ifndef AWQ_H_
#define AWQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AWQ_OK 0
#define AWQ_ERR_INVALID_ARG (-1) /* null/misaligned pointer, non-positive size, K % group_size != 0, ... */
#define AWQ_ERR_UNSUPPORTED (-2) /* w_bit != 4, group_size not in {32, 64, 128}, n_grid outside [2, 64],
                                    clip_ratio outside [0, 1] */
#define AWQ_ERR_WORKSPACE (-3)   /* workspace smaller than the matching *_workspace_size() */
#define AWQ_ERR_HIP (-4)         /* a HIP call failed; awq_last_hip_error() holds its code */
#define AWQ_ERR_SCRATCH (-5)     /* awq_w4a16_gemm_noalloc: the call needs more than its fixed scratch */

/* Quantization settings ([P4] 架构, AWQConfig; [P2] section 2, quant_config).
 *   w_bit       bits per weight; only 4 is supported.
 *   group_size  g: consecutive input channels (rows of W) sharing one step and zero,
 *               per output column.  Supported: 32, 64, 128.
 *   zero_point  1 = asymmetric min-max with a zero point: Delta = (max - min)/15 over the
 *               group range widened to include 0, zero = clamp(rne(-min/Delta), 0, 15),
 *               code = clamp(rne(p/Delta) + zero, 0, 15).
 *               0 = symmetric absmax ([P3] section 4; [P1] 量化数学基础): Delta = max|p|/7,
 *               level = clamp(rne(p/Delta), -7, 7), stored code = level + 8, zero = 8.
 *               In both modes Delta := 1 when the group is all zero, and the dequantized
 *               value is (code - zero) * Delta.
 *   n_grid      number of alpha points, alpha_i = i/(n_grid-1) ([P1] 缩放因子优化的完整流程
 *               step 3 uses 21: {0, 0.05, ..., 1}).  Supported: 2..64.  awq_clip_search
 *               reads it as the number of clip ratios.
 *   clip_ratio  min-max clipping of the group range before quantization ([P4] 架构,
 *               AWQConfig.clip_ratio; 关键设计 5, applied before the search): both ends of the
 *               range (0 included; max|p| in symmetric mode) are multiplied by c before Delta
 *               and the zero are formed, and codes beyond the clipped range clamp to its end
 *               levels.  0 or 1 = no clipping (so a zero-initialised struct needs no value);
 *               values in (0, 1) clip.  awq_search, awq_search_table, awq_search_multi and
 *               awq_pack use it; awq_clip_search ignores it; awq_greedy_search rejects it.
 */
typedef struct awq_qconfig {
    int32_t w_bit;
    int32_t group_size;
    int32_t zero_point;
    int32_t n_grid;
    float clip_ratio;
} awq_qconfig;

/* ---------------------------------------------------------------- a1: statistic
 * Per-input-channel mean absolute activation ([P1] 重要通道识别的统计依据;
 * [P3] section 1, I_i = E|X_i|; [P4] AWQQuantizer.add_batch accumulates it over
 * calibration batches).
 *   X          bf16 [T, K] calibration activations (T tokens).
 *   sum_abs    float64 [K], in/out.  accumulate = 0: overwritten with sum_t |x_tk|;
 *              accumulate = 1: the batch's sums are added to the values it holds.
 *   total_tokens  token count of all batches accumulated so far (>= T); the mean is
 *              sum_abs / total_tokens.
 *   mean_abs   float32 [K] out (may be NULL): the float32 rounding of that mean.
 *   workspace  >= awq_act_stats_workspace_size(T, K) bytes (fixed-order partial sums).
 * The float64 sums are exact whenever each channel's values span less than about
 * 2^30 in magnitude, so the result does not depend on summation order.
 */
size_t awq_act_stats_workspace_size(int64_t T, int64_t K);
int awq_act_stats(const void* X_bf16, int64_t T, int64_t K, double* sum_abs, int accumulate,
                  int64_t total_tokens, float* mean_abs, void* workspace, size_t ws_bytes,
                  void* stream);

/* ---------------------------------------------------------------- statistic and scale variants
 * Per-input-channel max |x_tk| over the calibration tokens, the alternative statistic that
 * [P1] 重要通道识别的统计依据 names next to the mean.  max_abs float32 [K] out (accumulate = 0)
 * or in/out (accumulate = 1: the maximum with the values it holds).  Exact.
 *   workspace >= awq_act_stats_workspace_size(T, K) bytes.
 */
int awq_act_max(const void* X_bf16, int64_t T, int64_t K, float* max_abs, int accumulate,
                void* workspace, size_t ws_bytes, void* stream);
/* mean_j |W_kj| over the output columns of each input channel: the denominator of the closed
 * form s_i = (E|X_i|)^alpha / mean_j |W_ij| of [P3] section 3.  W bf16 [K, N]; w_mean float32
 * [K] out (float64 sum, one division, one float32 rounding).
 */
int awq_weight_mean_abs(const void* W_bf16, int64_t K, int64_t N, float* w_mean, void* stream);
/* Scale-table variants: s[i, k] = float32(t[i, k]) with, in float64,
 *   t[i, k] = max(stat_k, 1e-8)^alpha_i  [ / max(w_mean_k, 1e-8) when w_mean is not NULL ]
 *             [ / max_k t[i, k] when normalize = 1 ([P3] Python 演示: s / max(s)) ],
 * alpha_i = i/(n_grid-1).  stat: mean |x| (awq_act_stats) or max |x| (awq_act_max).  With
 * w_mean = NULL and normalize = 0 this is awq_scale_table.  s_table float32 [n_grid, K] out.
 */
int awq_scale_table_ex(const float* stat, const float* w_mean, int64_t K, int32_t n_grid,
                       int32_t normalize, float* s_table, void* stream);

/* ---------------------------------------------------------------- a2: scale table
 * s[i, k] = float32( max(m_k, 1e-8) ^ alpha_i ), alpha_i = i/(n_grid-1), evaluated in
 * float64 ([P1] 缩放因子优化的完整流程 step 3: s_j(alpha) = activation_scale[j]^alpha).
 *   mean_abs   float32 [K];  s_table  float32 [n_grid, K] out.
 */
int awq_scale_table(const float* mean_abs, int64_t K, int32_t n_grid, float* s_table, void* stream);

/* ---------------------------------------------------------------- a3 + a4: search
 * For every alpha_i: group-quantize diag(s_i) W, dequantize, divide by s_i, and score
 *   L_i = || X (S_i^-1 Q(S_i W) - W) ||^2
 * ([P1] 缩放因子优化的完整流程 steps 4a-4c; [P5] 4.3 search loop), then pick the first
 * minimum ([P1] step 5; [P5] 4.3 keeps a loss only if strictly smaller) and record
 * s* = s_best ([P1] step 6).
 *   X        bf16 [T, K];  W  bf16 [K, N];  mean_abs  float32 [K] (from awq_act_stats).
 *   losses   float64 [n_grid] out;  best  int32 [1] out;  s_best  float32 [K] out.
 *   workspace >= awq_search_workspace_size(T, K, N, cfg) bytes.
 * One fused kernel per (token tile, column tile, alpha slice): the tile of X is loaded
 * once and reused for every alpha of the slice, each E_i tile is quantized and
 * dequantized in registers, X E_i runs on bf16 matrix cores with float32 accumulation,
 * and only sum-of-squares partials leave the kernel.  Losses are exact sums of those
 * float32 products; they agree with a float64 evaluation to about 1e-3 relative.
 * Size limits (AWQ_ERR_INVALID_ARG beyond them): T * K < 2^31; the scale table, its
 * reciprocals and the float32 copy of W (about 4 K N bytes) within 4 GiB, i.e. K N up to
 * about 1.07e9 (K = 8192: N up to ~131000); a 640-row tile of X (1280 K bytes) below 2^31.
 */
size_t awq_search_workspace_size(int64_t T, int64_t K, int64_t N, const awq_qconfig* cfg);
int awq_search(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N,
               const float* mean_abs, const awq_qconfig* cfg, void* workspace, size_t ws_bytes,
               double* losses, int32_t* best, float* s_best, void* stream);

/* ---------------------------------------------------------------- a5: pack
 * Offline quantization W_q = Quantize(diag(s) W) ([P1] 推理时的等效实现, 预处理), with
 * the quantizer of awq_qconfig evaluated in float64 (p = s*w is exact there), stored as
 *   codes   uint32 [K/8, N]: bits 4j..4j+3 of word (i, n) hold the code of row 8i+j
 *           (two 4-bit weights per byte, [P4] Consequences; [P3] section 6, M = N*b/8);
 *   scales  float32 [K/g, N]: Delta per (group, column);
 *   zeros   uint8   [K/g, N]: zero per (group, column) (8 in symmetric mode).
 *   W  bf16 [K, N];  s  float32 [K] (normally s_best from awq_search).
 */
int awq_pack(const void* W_bf16, int64_t K, int64_t N, const float* s, const awq_qconfig* cfg,
             uint32_t* codes, float* scales, uint8_t* zeros, void* stream);

/* ---------------------------------------------------------------- search over a given table
 * awq_search with the alpha grid's scale table replaced by the caller's: every row s_i of
 * s_table (float32 [cfg->n_grid, K], device, positive finite values) is scored with the same
 * loss, the first minimum wins and s_best = its row.  Use it with awq_scale_table_ex for the
 * statistic and scale-family variants.  workspace >= awq_search_workspace_size(T, K, N, cfg).
 */
int awq_search_table(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N,
                     const float* s_table, const awq_qconfig* cfg, void* workspace, size_t ws_bytes,
                     double* losses, int32_t* best, float* s_best, void* stream);

/* ---------------------------------------------------------------- clip search
 * The search of awq_search with the alpha grid replaced by a grid of clip ratios at fixed
 * scales s (normally s_best): for c_j = float32(1 - (1 - clip_min) * j / (n - 1)),
 * j = 0..n-1 with n = cfg->n_grid (evaluated in float64; c_0 = 1 is the unclipped quantizer),
 *   L_j = || X (S^-1 Q_cj(S W) - W) ||^2,
 * with Q_c the quantizer of awq_qconfig clipped by c ([P4] 关键设计 5 and AWQConfig.clip_ratio;
 * the loss of [P1] 缩放因子优化的完整流程 step 4c); the first minimum wins ([P5] 4.3).
 *   X  bf16 [T, K];  W  bf16 [K, N];  s  float32 [K] (device);  clip_min in (0, 1].
 *   losses  float64 [n] out;  best  int32 [1] out;  clip_best  float32 [1] out (c_best).
 *   workspace >= awq_search_workspace_size(T, K, N, cfg) bytes (the same layout).
 * Pass clip_best as cfg->clip_ratio to awq_pack to store the clipped quantization.
 */
int awq_clip_search(const void* X_bf16, int64_t T, const void* W_bf16, int64_t K, int64_t N,
                    const float* s, const awq_qconfig* cfg, float clip_min, void* workspace,
                    size_t ws_bytes, double* losses, int32_t* best, float* clip_best, void* stream);

/* ---------------------------------------------------------------- projections sharing X
 * Projections that read the same activations (q, k and v; gate and up) share one scale vector
 * once 1/s is applied to X a single time ([P4] 关键设计 4, the fused attn.qkv layer of its
 * usage).  This search scores, for every alpha_i of awq_search's grid,
 *   L_i = sum_j || X (S_i^-1 Q(S_i W_j) - W_j) ||^2,   j < n_w,
 * the first minimum wins and s_best is its row; it equals awq_search on the matrix whose
 * columns are all projections' columns, with each X tile loaded once for all of them.
 *   X  bf16 [T, K] (device);  W_bf16  host array of n_w device pointers, W_j bf16 [K, N[j]];
 *   N  host array of n_w column counts;  1 <= n_w <= AWQ_MAX_PROJECTIONS;
 *   mean_abs float32 [K];  cfg as for awq_search (clip_ratio included).
 *   losses  float64 [n_grid] out (joint);  losses_each  float64 [n_w, n_grid] out or NULL
 *   (each projection's own L_i, reduced separately: they sum to the joint losses up to the
 *   order of the float64 sums);  best  int32 [1] out;  s_best  float32 [K] out.
 *   workspace >= awq_search_multi_workspace_size(T, K, n_w, N, cfg) bytes (0 for bad sizes).
 * Each W_j is padded to a multiple of 16 columns with zeros, which quantize exactly.
 * awq_search's size limits apply with N the sum of the padded column counts.
 */
#define AWQ_MAX_PROJECTIONS 16
size_t awq_search_multi_workspace_size(int64_t T, int64_t K, int32_t n_w, const int64_t* N,
                                       const awq_qconfig* cfg);
int awq_search_multi(const void* X_bf16, int64_t T, int32_t n_w, const void* const* W_bf16, const int64_t* N,
                     int64_t K, const float* mean_abs, const awq_qconfig* cfg, void* workspace, size_t ws_bytes,
                     double* losses, double* losses_each, int32_t* best, float* s_best, void* stream);

/* ---------------------------------------------------------------- power-of-two greedy
 * The search of [P4] 关键设计 1-3: per-channel scales restricted to powers of two around 1,
 * c_j = 2^(j - n_cand/2) for j < n_cand (n_cand = 20: 2^-10 .. 2^9), found by a coordinate
 * greedy inside each group of input channels.  Every channel starts at s = 1; each of `passes`
 * passes visits a group's channels in ascending order and moves s_k to the candidate with the
 * smallest group error (the other channels at their current scales), keeping the current value
 * unless another is strictly smaller (the first such candidate in ascending order on ties).
 * The group error is sum_n sum_{i in group} (m_i (What_in - W_in))^2 with What the packing
 * quantizer of cfg applied to s_i W_in, divided by s_i, and m = mean |x| (awq_act_stats).
 *   W  bf16 [K, N];  mean_abs  float32 [K];  cfg: group size and zero point (clip_ratio must
 *   be 0 or 1, else AWQ_ERR_UNSUPPORTED; n_grid is not used);  2 <= n_cand <=
 *   AWQ_MAX_POW2_CANDIDATES;  1 <= passes <= 64 ([P4] uses 20 and 3).
 *   s_best  float32 [K] out (powers of two);  err_rtn, err  float64 [K/g] out or NULL: each
 *   group's error at s = 1 and at the result.
 *   workspace >= awq_greedy_workspace_size(K, N, cfg, n_cand) bytes.
 * Weights must be finite with |w| < 2^100; the error of each element is exact and only the
 * float64 sums round, so the choices agree with a float64 evaluation except between candidates
 * whose errors differ by about 1e-16 relative.  One launch per decision step (passes * g
 * launches), each over all groups and output columns; no call allocates or synchronizes.
 */
#define AWQ_MAX_POW2_CANDIDATES 32
size_t awq_greedy_workspace_size(int64_t K, int64_t N, const awq_qconfig* cfg, int32_t n_cand);
int awq_greedy_search(const void* W_bf16, int64_t K, int64_t N, const float* mean_abs, const awq_qconfig* cfg,
                      int32_t n_cand, int32_t passes, void* workspace, size_t ws_bytes, float* s_best,
                      double* err_rtn, double* err, void* stream);

/* ---------------------------------------------------------------- a6: W4A16 product
 * Y[m, n] = sum_k (x_mk / s_k) * (code_kn - zero_gn) * Delta_gn,  g = k / group_size
 * ([P1] 推理时的等效实现, 推理: Y = (X diag(1/s*)) Dequant(W_q), with the 1/s* scaling
 * folded into the kernel as the page suggests; [P2] section 3, 4-bit weights unpacked
 * on chip and multiplied with 16-bit activations).
 *   X  bf16 [M, K];  s  float32 [K];  codes/scales/zeros as written by awq_pack;
 *   Y  bf16 [M, N] out.  Accumulation is float32; x/s is rounded to bf16 once.
 *   workspace >= awq_w4a16_gemm_workspace_size(M, K, N, group_size) bytes (the size may be 0),
 *   256-byte aligned.  Its first 64 KiB hold the arrival counters of the split-K products (one
 *   32-bit counter per output tile whose K range is split): they must be ZERO before the first call that uses
 *   the workspace (a zero-filled allocation), this function writes nothing else there and every
 *   completed call leaves them zero, so one workspace serves any sequence of calls of any shape
 *   without clearing (re-zero it after using the memory for anything else).  After them: M = 1
 *   (decode-shaped, one kernel per call) the float32 split-K partials; M > 1 the float32 split-K
 *   partials, x/s as bf16 in matrix-core operand order and its per-group sums (about 2*M*K
 *   bytes).  Calls that share a workspace must be ordered (same stream).
 * Requires N % 8 == 0, K < 2^31, N <= 4194304, at most 65535 * 64 rows, for M > 1
 * K <= 65535 * 256 and, for M > 32, M * K * 2 bytes of x/s below 4 GiB (AWQ_ERR_INVALID_ARG
 * otherwise).
 */
size_t awq_w4a16_gemm_workspace_size(int64_t M, int64_t K, int64_t N, int32_t group_size);
int awq_w4a16_gemm(const void* X_bf16, int64_t M, const float* s, const uint32_t* codes,
                   const float* scales, const uint8_t* zeros, int64_t K, int64_t N,
                   int32_t group_size, void* Y_bf16, void* workspace, size_t ws_bytes,
                   void* stream);

/* ---------------------------------------------------------------- a6 without allocation
 * For callers that cannot allocate: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  awq_w4a16_gemm with the same arguments minus the workspace:
 * the same kernels, the same results (bit for bit), the scratch taken from one fixed buffer per
 * GPU that the library holds for the life of the process
 * (awq_w4a16_gemm_static_scratch_bytes(): 16 MiB plus 64 KiB of arrival counters).  Nothing is
 * allocated, freed or synchronized by the call.  The buffer is shared by every call on that GPU
 * and keeps the last call's contents: calls that can overlap on one GPU (different streams or
 * threads without ordering) race and must not be issued; order them on one stream.  The calling
 * thread's current HIP device must be the device of `stream` (the buffer's device address is
 * looked up once per device, on that device's first call).  A call whose workspace
 * (awq_w4a16_gemm_workspace_size) exceeds the buffer returns AWQ_ERR_SCRATCH before anything is
 * enqueued: M = 1 fits for N up to about 260000 columns; larger M fits when its partials, x/s and
 * group sums do (for example M = 16 with K = N = 8192).
 */
size_t awq_w4a16_gemm_static_scratch_bytes(void);
int awq_w4a16_gemm_noalloc(const void* X_bf16, int64_t M, const float* s, const uint32_t* codes,
                           const float* scales, const uint8_t* zeros, int64_t K, int64_t N,
                           int32_t group_size, void* Y_bf16, void* stream);

/* ---------------------------------------------------------------- status helpers */
const char* awq_status_string(int status);
int awq_last_hip_error(void);   /* hipError_t of the most recent AWQ_ERR_HIP on this thread */
const char* awq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_H_ */
