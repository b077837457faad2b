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
// handles one decision step for every group at once: the g channels of an output column are split
// over g/32 lanes of one wavefront, which score every candidate for the step's channel; the
// per-candidate sums leave each workgroup as float64 partials.  The next launch's workgroups read
// those partials in a fixed order and take the decision redundantly (every workgroup of a group
// reaches the same one), so no workgroup ever waits on another.
//
// Exactness.  With power-of-two scales p = s*w is a bf16 value (8 significant bits) and Delta a
// float32 (24), so p/Delta is either exactly a half-integer or more than 2^-25 away from one.
// The kernel forms the quotient as p * r, r within two ulps of 1/Delta (error below 2^-45), so
// its nearest integer is the packing quantizer's code except at exact half-integers, where either
// neighbour gives the same squared error (the two errors are +-Delta/2, and at the ends of the
// range both clamp to the same level).  The zero point, which does change the codes, settles its
// exact half-integers with an exact residual.  The weighted error of an element,
// m (What - w) = (m/s) (level*Delta - p), is exact: level*Delta - p is a multiple of Delta's last
// bit no larger than Delta/2, and its product with m/s needs at most 48 bits.  Only the float64
// sums of squares round, so every decision matches a float64 evaluation of the definition except
// between candidates whose errors differ by about 1e-16 relative.
//
// Work.  A candidate that keeps the channel's scaled weight inside the range of the other
// channels leaves the group's step and zero unchanged: its error is the others' error at the base
// configuration plus its own element.  Only candidates that stretch the range need the whole
// group again, and those are the largest ones (|c w| grows with c).  Each wavefront therefore
// evaluates the others' error for the base configuration and for the top S candidates, S the most
// any of its columns needs, one configuration per pass over the channels; the rest cost one
// element each.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

namespace {

constexpr int kThreads = 256;

// Quantizer configuration of one (column, group), float64: step, its reciprocal, and the
// clamp bounds of the level (code - zero).
struct Cfg {
    double d, r, lo, hi;
};

// 1/d to within an ulp or two: hardware estimate plus two Newton steps.  That is ample for the
// quotients here, which sit either exactly on a half-integer or more than 2^-25 from one.
__device__ __forceinline__ double recip(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = fma(fma(-d, r, 1.0), r, r);
    return fma(fma(-d, r, 1.0), r, r);
}

template <bool ZP>
__device__ __forceinline__ Cfg make_cfg(float hi, float lo) {
    Cfg c;
    if (ZP) {
        float d = (float)(((double)hi - (double)lo) / 15.0);   // the step exactly as packing forms it
        if (d == 0.f) d = 1.f;
        c.d = d;
        c.r = recip(c.d);
        // zero = rne(-lo/d): the product with r rounds to the right integer except on an exact
        // half-integer, which the exact residual zf*d + lo = (zf - (-lo/d)) d = +-d/2 reveals
        double zf = rint(-(double)lo * c.r);
        const double res = fma(zf, c.d, (double)lo);
        if (fabs(res) == 0.5 * c.d && (((int)zf) & 1)) zf += res > 0.0 ? -1.0 : 1.0;
        const double z = fmin(fmax(zf, 0.0), 15.0);
        c.lo = -z;
        c.hi = 15.0 - z;
    } else {
        float d = (float)((double)hi / 7.0);   // hi = max |p|
        if (d == 0.f) d = 1.f;
        c.d = d;
        c.r = recip(c.d);
        c.lo = -7.0;
        c.hi = 7.0;
    }
    return c;
}

// acc + (ms (level*Delta - p))^2 for one element; ms = m/s.  In symmetric mode |p| <= max|p|
// = 7 Delta (1 + 2^-24) keeps every level inside -7..7, so only the asymmetric form clamps.
template <bool ZP>
__device__ __forceinline__ double elem_acc(double p, double ms, const Cfg& c, double acc) {
    double lv = rint(p * c.r);
    if (ZP) lv = fmin(fmax(lv, c.lo), c.hi);
    const double t = ms * fma(lv, c.d, -p);
    return fma(t, t, acc);
}

// The decision of one step for one group, taken from the previous launch's partials:
// part[(slice * n_cand + c)] for slice < n_slices.  Every workgroup of the group computes the
// same sums in the same order.  Returns the chosen candidate index; cur is the channel's index
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

// One decision step for every group.  Grid (n_slices, K/G), 256 threads.  The G channels of an
// output column are split over P = G/32 lanes of one wavefront (lane = part * 64/P + column), so
// every thread holds 32 scaled weights; a wavefront covers 64/P columns and a workgroup 256/P.
// step = pass * G + i scores channel i of each group; partials of step t go to part[t & 1].
template <int G, bool ZP>
__global__ __launch_bounds__(256) void k_greedy_step(const uint16_t* __restrict__ W, int64_t N,
                                                  const float* __restrict__ m, int32_t* __restrict__ idx,
                                                  double* __restrict__ part, int64_t part_stride, int n_slices,
                                                  int n_cand, int step, double* __restrict__ err_rtn) {
    constexpr int CH = 32, P = G / CH, CPW = kWave / P;   // channels per thread, parts, columns/wave
    // one block so that m_j/s_j sits at LDS offset 0: the per-channel reads then fit the
    // immediate offsets of paired 64-bit LDS reads from a single base register
    __shared__ struct {
        double ms[P * (CH + 1)];   // m_j / s_j (0 for the channel being decided), padded per part
        double chunk[8 * 32];
        double sum[32];
        double wave[4][32];
        float scale[G];            // s_j of the group's channels
        int idx[G];
    } sh;
    lds_poison_start(&sh.ms[0], P * (CH + 1) + 8 * 32 + 32 + 4 * 32);   // ms, chunk, sum, wave
    lds_poison_start(&sh.scale[0], G);
    double* const s_ms = sh.ms;
    double* const sm_chunk = sh.chunk;
    double* const sm_sum = sh.sum;
    double (*const sm_wave)[32] = sh.wave;
    float* const s_scale = sh.scale;
    int* const s_idx = sh.idx;
    const int tid = threadIdx.x;
    const int grp = blockIdx.y, slice = blockIdx.x;
    const int64_t k0 = (int64_t)grp * G;
    const int one = n_cand / 2;
    const int i = step % G;

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
        s_ms[(j / CH) * (CH + 1) + j % CH] = j == i ? 0.0 : (double)(m[k0 + j] / s);   // exact
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int prt = lane / CPW;                          // which CH channels of the column
    const int64_t n = (int64_t)slice * (kThreads / P) + wave * CPW + lane % CPW;
    const int j0 = prt * CH;
    const double* ms_p = s_ms + prt * (CH + 1);
    // This thread's channels of the column, scaled: p_j = s_j w_j (exact), with p_i = 0 (channel i
    // is the one being decided; zero changes no range and, weighted by 0, adds no error).
    uint32_t pk[CH / 2];
#pragma unroll
    for (int j = 0; j < CH; j += 2) {
        float a = n < N ? bf16_lo((uint32_t)W[(k0 + j0 + j) * N + n]) * s_scale[j0 + j] : 0.f;
        float b = n < N ? bf16_lo((uint32_t)W[(k0 + j0 + j + 1) * N + n]) * s_scale[j0 + j + 1] : 0.f;
        a = j0 + j == i ? 0.f : a;
        b = j0 + j + 1 == i ? 0.f : b;
        pk[j / 2] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
    }
    auto pj = [&](int j) { return (j & 1) ? bf16_hi(pk[j >> 1]) : bf16_lo(pk[j >> 1]); };
    const float wi = n < N ? bf16_lo((uint32_t)W[(k0 + i) * N + n]) : 0.f;
    float hiO = 0.f, loO = 0.f;   // range of the other channels (0 included), over all parts
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if (ZP) {
            hiO = fmaxf(hiO, pj(j));
            loO = fminf(loO, pj(j));
        } else {
            hiO = fmaxf(hiO, fabsf(pj(j)));
        }
    }
#pragma unroll
    for (int off = CPW; off < kWave; off <<= 1) {
        hiO = fmaxf(hiO, __shfl_xor(hiO, off, kWave));
        if (ZP) loO = fminf(loO, __shfl_xor(loO, off, kWave));
    }
    const bool owner = prt == i / CH;   // the lane of the column that adds channel i's own error
    const float mi = m[k0 + i];
    // the candidate's own element (weighted only on the lane that owns channel i) and the
    // configuration it implies
    auto own = [&](int c, float& pc, double& msc) {
        const float sc = ldexpf(1.f, c - one);
        pc = wi * sc;
        msc = owner ? (double)(mi / sc) : 0.0;
    };
    auto own_cfg = [&](int c, float& pc, double& msc) {
        own(c, pc, msc);
        return ZP ? make_cfg<ZP>(fmaxf(hiO, pc), fminf(loO, pc)) : make_cfg<ZP>(fmaxf(hiO, fabsf(pc)), 0.f);
    };
    int need = 0;   // candidates (from the top) that stretch this column's range
    for (int c = 0; c < n_cand; ++c) {
        const float pc = wi * ldexpf(1.f, c - one);
        need += ZP ? (pc > hiO || pc < loO) : (fabsf(pc) > hiO);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) need = max(need, __shfl_xor(need, off, kWave));

    const Cfg base = ZP ? make_cfg<ZP>(hiO, loO) : make_cfg<ZP>(hiO, 0.f);
    double e_base = 0.0;
    // slot 0 = base configuration; slot u >= 1 = candidate n_cand - u.  Candidates below the
    // slots stretch no lane's range, so the base configuration is theirs.
    const int slots = min(need, n_cand) + 1;
    for (int u = 0; u < slots; ++u) {
#pragma unroll
        for (int k = 0; k < CH / 2; ++k) asm volatile("" : "+v"(pk[k]));
        const int c = n_cand - u;
        float pc = 0.f;
        double msc = 0.0;
        const Cfg cf = u == 0 ? base : own_cfg(c, pc, msc);
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < CH; ++j) acc = elem_acc<ZP>((double)pj(j), ms_p[j], cf, acc);
        if (u == 0) {
            e_base = acc;
        } else {
            const double e = wave_sum(elem_acc<ZP>((double)pc, msc, cf, acc));
            if (lane == 0) sm_wave[wave][c] = e;
        }
    }
    for (int c = 0; c < n_cand - (slots - 1); ++c) {
        float pc;
        double msc;
        own(c, pc, msc);
        const double e = wave_sum(elem_acc<ZP>((double)pc, msc, base, e_base));
        if (lane == 0) sm_wave[wave][c] = e;
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
    lds_poison_start(&sm_chunk[0], 8 * 32);
    lds_poison_start(&sm_sum[0], 32);
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
    const int cols = kThreads / (group_size / 32);   // output columns per workgroup
    p.n_slices = (N + cols - 1) / cols;
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
