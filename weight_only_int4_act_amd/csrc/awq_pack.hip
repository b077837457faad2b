// a5: offline quantization of the chosen scaling, W_q = Quantize(diag(s*) W), stored as 4-bit
// codes with per-group float32 steps and uint8 zeros.
//
// Sources: "AWQ (Activation-aware Weight Quantization)", section 推理时的等效实现 (precompute the
// quantized scaled weights offline and keep s* as metadata) and section 量化数学基础 (per-group
// step, round, clamp); "AWQ 激活感知量化", section 4 (symmetric step max|w_s|/7) and section 6
// (M = N*b/8 bytes); "009. AWQ Integration", Consequences (4-bit, two weights per byte) and
// 关键设计 3 (the search scores the same quantizer that packing uses).
//
// With a clip ratio c (the configuration's optional min-max clipping, "009. AWQ Integration",
// 关键设计 5) both ends of the range are multiplied by c before the step and the zero are formed.
// The quantizer is evaluated as in float64.  p = s*w is exact there (a float32 times a bf16 has at
// most 32 significant bits), max/min are exact, the step and the zero come from single IEEE
// divisions, and each code is the round-half-even of p/Delta exactly as a float64 division and
// rint give it, so codes, steps and zeros are reproducible bit for bit by any float64 evaluation
// of the same definition.  The codes take a float32 quotient wherever its rounding provably equals
// that one, and the exact float64 rounding (rne_div) near a .5 boundary.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// rne(p / d) for the quantizer's quotients, exactly as a float64 division followed by rint: with r
// within two ulps of 1/d the product p*r rounds to the right integer unless p/d is exactly a
// half-integer (p has at most 32 significant bits and d 24, so any other quotient is more than
// 2^-34 from a half-integer, far beyond the product's error); the exact residual p - n d settles
// that case, and round-half-to-even picks the even neighbour.
__device__ __forceinline__ double rne_div(double p, double d, double r) {
    double n = rint(p * r);
    const double res = fma(-n, d, p);   // exact: n*d and p are within a factor 2 of each other
    const double h = 0.5 * d;
    if (fabs(res) >= h) {               // a half-integer quotient (or a last-bit slip of p*r)
        const double m = res > 0.0 ? n + 1.0 : n - 1.0;   // the other neighbour
        if (fabs(res) > h) n = m;
        else if (((int64_t)n) & 1) n = m;
    }
    return n;
}

// One thread per (group, output column): the group's G weights of the column are loaded first
// (consecutive lanes read consecutive columns of a row: every load is coalesced), then the range,
// the step and zero, and the codes are formed from registers.
template <int G, bool ZP>
__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                              const float* __restrict__ s, double clip,
                                              uint32_t* __restrict__ codes, float* __restrict__ scales,
                                              uint8_t* __restrict__ zeros) {
    __shared__ float sg[G];   // the group's scales, shared by the workgroup's columns
    lds_poison_start(&sg[0], G);
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t jg = blockIdx.y;
    const int64_t k0 = jg * G;
    for (int i = threadIdx.x; i < G; i += blockDim.x) sg[i] = s[k0 + i];
    __syncthreads();
    if (n >= N) return;
    uint32_t wp[G / 2];   // bf16 pairs (rows 2i, 2i+1)
#pragma unroll
    for (int i = 0; i < G; i += 2)
        wp[i / 2] = (uint32_t)W[(k0 + i) * N + n] | ((uint32_t)W[(k0 + i + 1) * N + n] << 16);
    auto pv = [&](int i) {   // p = s*w, exact in float64
        const uint32_t h = wp[i / 2];
        return (double)sg[i] * (double)((i & 1) ? bf16_hi(h) : bf16_lo(h));
    };
    double mx = 0.0, mn = 0.0, am = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const double p = pv(i);
        if (ZP) {
            mx = fmax(mx, p);
            mn = fmin(mn, p);
        } else {
            am = fmax(am, fabs(p));
        }
    }
    // min-max clipping: both ends of the range scaled by the ratio (1: none), codes clamp below
    mx *= clip;
    mn *= clip;
    am *= clip;
    float d;
    double z;
    if (ZP) {
        d = (float)((mx - mn) / 15.0);
        if (d == 0.f) d = 1.f;
        z = fmin(fmax(rint(-mn / (double)d), 0.0), 15.0);
    } else {
        d = (float)(am / 7.0);
        if (d == 0.f) d = 1.f;
        z = 8.0;
    }
    const double dd = (double)d;
    const double r = 1.0 / dd;
    const float rf = 1.0f / d;
    const float zf = (float)z;
    // recompute p in the second pass rather than keep G float64 values live from the first
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < G / 2; ++i) asm volatile("" : "+v"(wp[i]));
#pragma unroll
    for (int i = 0; i < G; i += 8) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // float32 first: q = fl(fl(s w) fl(1/Delta)) is within |q| 1.8e-7 of p/Delta (three
            // roundings of 2^-24 each), so a q farther than |q| 4.8e-7 from a .5 boundary rounds
            // to the same integer as p/Delta (q - rint(q) is exact).  A quotient that close to a
            // boundary, or not finite (1/Delta overflows for a step below ~3e-39), takes the exact
            // float64 rounding (rne_div), which settles ties to even as the definition does
            const uint32_t h = wp[(i + j) / 2];
            const float wv = ((i + j) & 1) ? bf16_hi(h) : bf16_lo(h);
            const float q = (sg[i + j] * wv) * rf;
            float c = rintf(q);
            if (!(fabsf(fabsf(q - c) - 0.5f) > fabsf(q) * 4.8e-7f)) c = (float)rne_div(pv(i + j), dd, r);
            c = ZP ? fminf(fmaxf(c + zf, 0.f), 15.f) : fminf(fmaxf(c, -7.f), 7.f) + 8.f;
            word |= (uint32_t)c << (4 * j);
        }
        codes[((k0 + i) >> 3) * N + n] = word;
    }
    scales[jg * N + n] = d;
    zeros[jg * N + n] = (uint8_t)z;
}

hipError_t launch_pack(const uint16_t* W, int64_t K, int64_t N, const float* s, int group_size,
                       int zero_point, float clip_ratio, uint32_t* codes, float* scales, uint8_t* zeros,
                       hipStream_t st) {
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / group_size));
    const double clip = clip_ratio > 0.f && clip_ratio < 1.f ? (double)clip_ratio : 1.0;
    if (group_size == 32) {
        if (zero_point) k_pack<32, true><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
        else k_pack<32, false><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
    } else if (group_size == 64) {
        if (zero_point) k_pack<64, true><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
        else k_pack<64, false><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
    } else {
        if (zero_point) k_pack<128, true><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
        else k_pack<128, false><<<grid, 256, 0, st>>>(W, K, N, s, clip, codes, scales, zeros);
    }
    return hipGetLastError();
}

}  // namespace awq
