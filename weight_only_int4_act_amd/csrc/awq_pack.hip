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
// The quantizer is evaluated in float64.  p = s*w is exact there (a float32 times a bf16 has at
// most 32 significant bits), max/min are exact, and every division and rounding is a single
// IEEE operation, so codes, steps and zeros are reproducible bit for bit by any float64
// evaluation of the same definition.
//
// One thread per (group, output column): consecutive lanes read consecutive columns of a row,
// so every load and store is coalesced across the wavefront.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

template <bool ZP>
__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                              const float* __restrict__ s, int G, double clip,
                                              uint32_t* __restrict__ codes, float* __restrict__ scales,
                                              uint8_t* __restrict__ zeros) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t jg = blockIdx.y;
    if (n >= N) return;
    const int64_t k0 = jg * G;
    double mx = 0.0, mn = 0.0, am = 0.0;
    for (int i = 0; i < G; ++i) {
        const double pv = (double)s[k0 + i] * (double)bf16_lo((uint32_t)W[(k0 + i) * N + n]);
        if (ZP) {
            mx = fmax(mx, pv);
            mn = fmin(mn, pv);
        } else {
            am = fmax(am, fabs(pv));
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
    for (int i = 0; i < G; i += 8) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t k = k0 + i + j;
            const double pv = (double)s[k] * (double)bf16_lo((uint32_t)W[k * N + n]);
            double c = rint(pv / dd);
            c = ZP ? fmin(fmax(c + z, 0.0), 15.0) : fmin(fmax(c, -7.0), 7.0) + 8.0;
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
    if (zero_point)
        k_pack<true><<<grid, 256, 0, st>>>(W, K, N, s, group_size, clip, codes, scales, zeros);
    else
        k_pack<false><<<grid, 256, 0, st>>>(W, K, N, s, group_size, clip, codes, scales, zeros);
    return hipGetLastError();
}

}  // namespace awq
