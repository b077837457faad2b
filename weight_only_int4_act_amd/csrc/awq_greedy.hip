// Power-of-two coordinate greedy over the per-channel scales, one quantization group at a time.
//
// Sources: "009. AWQ Integration", 关键设计 1 (groups of input channels are independent; for each
// channel of a group every power-of-two candidate around 1 is scored with the activation-weighted
// reconstruction error of the whole group; three passes), 关键设计 2 (salient channels move to
// s > 1), 关键设计 3 (the error is measured with the quantizer that packing uses) and Consequences
// (cost O(passes * K * candidates * N * g)).
//
// The walk is sequential inside a group (each decision sees the previous ones) but the error of
// one decision is a sum over all N output columns, and the K/g groups are independent.  One launch
// handles one decision step for every group at once: a thread owns one output column of one group
// and scores every candidate for the step's channel; per-candidate sums leave each workgroup as
// float64 partials.  The next launch's workgroups read those partials in a fixed order and take
// the decision redundantly (every workgroup of a group reaches the same one), so no workgroup ever
// waits on another.
//
// Exactness.  With power-of-two scales p = s*w is exact in float32, and the packing quantizer's
// code, rne(p/Delta) evaluated in float64, equals the exactly rounded quotient: p carries 8
// significant bits and Delta 24, so a quotient that is not exactly a half-integer stays more than
// 2^-25 away from one, far beyond float64's error.  The kernel forms p/Delta with a float32
// reciprocal (error below 3e-6 for the |p/Delta| <= 15 that occur) and settles the rare quotient
// within 2^-17 of a half-integer with an exact float64 residual.  The weighted error of an element,
// m (What - w) = (m/s) (level*Delta - p), is exact as well: level*Delta - p is a multiple of
// Delta's last bit and at most Delta/2 in size, so one fused multiply-add gives it exactly in
// float32, and the product with m/s is exact in float64.  Only the float64 sums of squares round,
// so every decision matches any float64 evaluation of the definition except on differences of
// order 1e-16 between candidates.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

namespace {

constexpr int kThreads = 256;

// Exact round-half-even of p / d for the quantizer's quotients (|p/d| <= 15.0001); r = 1/d with
// at most 1 ulp of error.
__device__ __forceinline__ float rne_quot(float p, float d, float r) {
    const float q = p * r;
    const float fl = floorf(q);
    float n = rintf(q);
    if (fabsf(q - fl - 0.5f) <= 0x1p-17f) {
        const double diff = (double)p - ((double)fl + 0.5) * (double)d;   // exact in float64
        n = diff > 0.0 ? fl + 1.f : diff < 0.0 ? fl : ((((int)fl) & 1) ? fl + 1.f : fl);
    }
    return n;
}

// Quantizer configuration of one (column, group) from the group range.
struct Cfg {
    float d, r, z;   // Delta, 1/Delta, zero point (0 in symmetric mode)
};

template <bool ZP>
__device__ __forceinline__ Cfg make_cfg(float hi, float lo) {
    Cfg c;
    if (ZP) {
        float d = (float)(((double)hi - (double)lo) / 15.0);
        if (d == 0.f) d = 1.f;
        c.d = d;
        c.z = (float)fmin(fmax(rint(-(double)lo / (double)d), 0.0), 15.0);
    } else {
        float d = (float)((double)hi / 7.0);   // hi = max |p|
        if (d == 0.f) d = 1.f;
        c.d = d;
        c.z = 0.f;
    }
    c.r = __builtin_amdgcn_rcpf(c.d);
    return c;
}

// (m/s)^2 (level*Delta - p)^2 for one element; ms = m/s.
template <bool ZP>
__device__ __forceinline__ double elem_err(float p, float ms, const Cfg& c) {
    const float n = rne_quot(p, c.d, c.r);
    const float lv = ZP ? __builtin_amdgcn_fmed3f(n + c.z, 0.f, 15.f) - c.z : __builtin_amdgcn_fmed3f(n, -7.f, 7.f);
    const float es = fmaf(lv, c.d, -p);
    const double t = (double)ms * (double)es;
    return t * t;
}

// The decision of one step for one group, taken from the previous launch's partials:
// part[(slice * n_cand + c)] for slice < n_slices.  Every workgroup of the group computes the
// same sums in the same order.  Returns the chosen candidate index; *cur is the channel's index
// before the step (a value already updated by a concurrent writer gives the same answer, since
// the rule keeps a candidate that is already a minimum).
__device__ int decide(const double* __restrict__ part, int n_slices, int n_cand, int cur, double* sm_chunk,
                      double* sm_sum, double* best_err) {
    const int tid = threadIdx.x;
    const int c = tid & 31, h = tid >> 5;   // candidate, chunk of slices (8 chunks)
    const int per = (n_slices + 7) / 8;
    if (c < n_cand) {
        double s = 0.0;
        const int s0 = h * per, s1 = min(n_slices, s0 + per);
        for (int sl = s0; sl < s1; ++sl) s += part[(int64_t)sl * n_cand + c];
        sm_chunk[h * 32 + c] = s;
    }
    __syncthreads();
    if (tid < n_cand) {
        double s = 0.0;
        for (int hh = 0; hh < 8; ++hh) s += sm_chunk[hh * 32 + tid];
        sm_sum[tid] = s;
    }
    __syncthreads();
    int best = cur;
    for (int k = 0; k < n_cand; ++k)
        if (sm_sum[k] < sm_sum[best]) best = k;
    *best_err = sm_sum[best];
    return best;
}

}  // namespace

__global__ __launch_bounds__(256) void k_greedy_init(int32_t* __restrict__ idx, int64_t K, int one) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < K) idx[k] = one;
}

// One decision step for every group.  Grid (n_slices, K/G), 256 threads, thread = output column.
// step = pass * G + i scores channel i of each group; partials of step t go to part[t & 1].
template <int G, bool ZP>
__global__ __launch_bounds__(256, 2) void k_greedy_step(const uint16_t* __restrict__ W, int64_t N,
                                                     const float* __restrict__ m, int32_t* __restrict__ idx,
                                                     double* __restrict__ part, int64_t part_stride, int n_slices,
                                                     int n_cand, int step, double* __restrict__ err_rtn) {
    __shared__ double sm_chunk[8 * 32];
    __shared__ double sm_sum[32];
    __shared__ double sm_wave[4][32];
    __shared__ float s_scale[G];   // s_j of the group's channels
    __shared__ float s_ms[G];      // m_j / s_j
    const int tid = threadIdx.x;
    const int grp = blockIdx.y, slice = blockIdx.x;
    const int64_t k0 = (int64_t)grp * G;
    const int one = n_cand / 2;
    const int i = step % G;

    __shared__ int s_idx[G];
    for (int j = tid; j < G; j += kThreads) s_idx[j] = idx[k0 + j];
    __syncthreads();
    if (step > 0) {
        const int ip = (step - 1) % G;
        const double* prev = part + ((step - 1) & 1) * part_stride + (int64_t)grp * n_slices * n_cand;
        double e;
        const int best = decide(prev, n_slices, n_cand, s_idx[ip], sm_chunk, sm_sum, &e);
        __syncthreads();
        if (tid == 0) {
            s_idx[ip] = best;
            if (slice == 0) {
                idx[k0 + ip] = best;
                if (step == 1) err_rtn[grp] = sm_sum[one];   // step 0 scored s = 1 everywhere
            }
        }
        __syncthreads();
    }
    for (int j = tid; j < G; j += kThreads) {
        const float s = ldexpf(1.f, s_idx[j] - one);
        s_scale[j] = s;
        s_ms[j] = m[k0 + j] / s;   // exact: division by a power of two
    }
    __syncthreads();

    // this thread's column of the group, scaled: p_j = s_j w_j.  A bf16 times a power of two is
    // again a bf16 value, so the scaled column is kept as packed bf16 pairs (G/2 registers).
    const int64_t n = (int64_t)slice * kThreads + tid;
    uint32_t pk[G / 2];
#pragma unroll
    for (int j = 0; j < G; j += 2) {
        const float a = n < N ? bf16_lo((uint32_t)W[(k0 + j) * N + n]) * s_scale[j] : 0.f;
        const float b = n < N ? bf16_lo((uint32_t)W[(k0 + j + 1) * N + n]) * s_scale[j + 1] : 0.f;
        pk[j / 2] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
    }
    auto pj = [&](int j) { return (j & 1) ? bf16_hi(pk[j >> 1]) : bf16_lo(pk[j >> 1]); };
    const float wi = n < N ? bf16_lo((uint32_t)W[(k0 + i) * N + n]) : 0.f;
    // range of the other channels
    float hiO = 0.f, loO = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (j == i) continue;
        if (ZP) {
            hiO = fmaxf(hiO, pj(j));
            loO = fminf(loO, pj(j));
        } else {
            hiO = fmaxf(hiO, fabsf(pj(j)));
        }
    }
    const Cfg c0 = make_cfg<ZP>(hiO, loO);
    double e0 = 0.0;
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (j != i) e0 += elem_err<ZP>(pj(j), s_ms[j], c0);

    const float mi = m[k0 + i];
    const int wave = tid >> 6, lane = tid & 63;
    for (int c = 0; c < n_cand; ++c) {
        // m_j / s_j are re-read from LDS on every candidate rather than held in G registers
        asm volatile("" ::: "memory");
        const float sc = ldexpf(1.f, c - one);
        const float pc = wi * sc;
        const float msc = mi / sc;
        float hi, lo;
        if (ZP) {
            hi = fmaxf(hiO, pc);
            lo = fminf(loO, pc);
        } else {
            hi = fmaxf(hiO, fabsf(pc));
            lo = 0.f;
        }
        const Cfg cc = make_cfg<ZP>(hi, lo);
        double acc;
        if (cc.d == c0.d && cc.z == c0.z) {
            acc = e0 + elem_err<ZP>(pc, msc, c0);
        } else {
            acc = 0.0;
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (j != i) acc += elem_err<ZP>(pj(j), s_ms[j], cc);
            acc += elem_err<ZP>(pc, msc, cc);
        }
        acc = wave_sum(acc);
        if (lane == 0) sm_wave[wave][c] = acc;
    }
    __syncthreads();
    if (tid < n_cand) {
        const double s = ((sm_wave[0][tid] + sm_wave[1][tid]) + sm_wave[2][tid]) + sm_wave[3][tid];
        part[(step & 1) * part_stride + ((int64_t)grp * n_slices + slice) * n_cand + tid] = s;
    }
}

// Decision of the last step, then the result: s_best = 2^(idx - n_cand/2), final group errors.
template <int G>
__global__ __launch_bounds__(256) void k_greedy_final(int32_t* __restrict__ idx, const double* __restrict__ part,
                                                      int64_t part_stride, int n_slices, int n_cand, int steps,
                                                      float* __restrict__ s_best, double* __restrict__ err_rtn,
                                                      double* __restrict__ err) {
    __shared__ double sm_chunk[8 * 32];
    __shared__ double sm_sum[32];
    const int grp = blockIdx.x;
    const int64_t k0 = (int64_t)grp * G;
    const int one = n_cand / 2;
    const int ip = (steps - 1) % G;
    const double* prev = part + ((steps - 1) & 1) * part_stride + (int64_t)grp * n_slices * n_cand;
    double e;
    const int best = decide(prev, n_slices, n_cand, idx[k0 + ip], sm_chunk, sm_sum, &e);
    __syncthreads();
    if (threadIdx.x == 0) {
        idx[k0 + ip] = best;
        if (err) err[grp] = e;
        if (steps == 1 && err_rtn) err_rtn[grp] = sm_sum[one];
    }
    __syncthreads();
    for (int j = threadIdx.x; j < G; j += blockDim.x) s_best[k0 + j] = ldexpf(1.f, idx[k0 + j] - one);
}

GreedyPlan plan_greedy(int64_t K, int64_t N, int group_size, int n_cand) {
    GreedyPlan p{};
    p.group_size = group_size;
    p.groups = K / group_size;
    p.n_slices = (N + kThreads - 1) / kThreads;
    p.n_cand = n_cand;
    p.part_stride = p.groups * p.n_slices * n_cand;
    size_t off = 0;
    p.off_idx = off;   off = (off + (size_t)K * sizeof(int32_t) + 255) & ~(size_t)255;
    p.off_part = off;  off = (off + 2 * (size_t)p.part_stride * sizeof(double) + 255) & ~(size_t)255;
    p.off_rtn = off;   off = (off + (size_t)p.groups * sizeof(double) + 255) & ~(size_t)255;
    p.ws_bytes = off;
    return p;
}

template <int G, bool ZP>
static hipError_t greedy_steps(const uint16_t* W, int64_t N, const float* m, int32_t* idx, double* part,
                               const GreedyPlan& p, int passes, double* err_rtn, hipStream_t st) {
    const dim3 grid((unsigned)p.n_slices, (unsigned)p.groups);
    const int steps = passes * G;
    for (int t = 0; t < steps; ++t) {
        k_greedy_step<G, ZP><<<grid, kThreads, 0, st>>>(W, N, m, idx, part, p.part_stride, (int)p.n_slices,
                                                         p.n_cand, t, err_rtn);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_greedy(const uint16_t* W, int64_t K, int64_t N, const float* mean_abs, int zero_point,
                         int passes, const GreedyPlan& p, void* ws, float* s_best, double* err_rtn, double* err,
                         hipStream_t st) {
    char* base = (char*)ws;
    int32_t* idx = (int32_t*)(base + p.off_idx);
    double* part = (double*)(base + p.off_part);
    double* rtn = err_rtn ? err_rtn : (double*)(base + p.off_rtn);
    k_greedy_init<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(idx, K, p.n_cand / 2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int g = p.group_size;
    if (g == 32) e = zero_point ? greedy_steps<32, true>(W, N, mean_abs, idx, part, p, passes, rtn, st)
                                : greedy_steps<32, false>(W, N, mean_abs, idx, part, p, passes, rtn, st);
    else if (g == 64) e = zero_point ? greedy_steps<64, true>(W, N, mean_abs, idx, part, p, passes, rtn, st)
                                     : greedy_steps<64, false>(W, N, mean_abs, idx, part, p, passes, rtn, st);
    else e = zero_point ? greedy_steps<128, true>(W, N, mean_abs, idx, part, p, passes, rtn, st)
                        : greedy_steps<128, false>(W, N, mean_abs, idx, part, p, passes, rtn, st);
    if (e != hipSuccess) return e;
    const int steps = passes * g;
    if (g == 32) k_greedy_final<32><<<(unsigned)p.groups, 256, 0, st>>>(idx, part, p.part_stride, (int)p.n_slices,
                                                                       p.n_cand, steps, s_best, rtn, err);
    else if (g == 64) k_greedy_final<64><<<(unsigned)p.groups, 256, 0, st>>>(idx, part, p.part_stride,
                                                                            (int)p.n_slices, p.n_cand, steps,
                                                                            s_best, rtn, err);
    else k_greedy_final<128><<<(unsigned)p.groups, 256, 0, st>>>(idx, part, p.part_stride, (int)p.n_slices,
                                                                p.n_cand, steps, s_best, rtn, err);
    return hipGetLastError();
}

}  // namespace awq
