// a6: the W4A16 product Y = (X diag(1/s*)) Dequant(W_q) on packed 4-bit weights.
//
// Sources: "AWQ (Activation-aware Weight Quantization)", section 推理时的等效实现 (online step:
// scale the activations by 1/s* per input channel, or fold that into the kernel's dequant step)
// and the ASCII 架构图 (Dequant + MatMul with s* fused); "大模型 AWQ 量化实战", section 3 (4-bit
// weights unpacked on chip and multiplied with 16-bit activations).
//
// Y[m, n] = sum_g Delta_gn * sum_{k in g} (x_mk / s_k) * (code_kn - zero_gn).
// The inner sum runs on bf16 matrix cores: (code - zero) is a small integer and exact in bf16,
// x/s is rounded to bf16 once; each group's float32 partial is scaled by its Delta and added
// to a float32 accumulator.  The 1/s* scaling is applied while the activation fragment is
// formed, so no scaled copy of X is written.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Workgroup: 4 wavefronts, 64 output columns (16 per wavefront) x 16*MB token rows.
template <int G, int MB>
__global__ __launch_bounds__(256) void k_w4a16_mfma(const uint16_t* __restrict__ X, int64_t M,
                                                    const float* __restrict__ s,
                                                    const uint32_t* __restrict__ codes,
                                                    const float* __restrict__ scales,
                                                    const uint8_t* __restrict__ zeros, int64_t K, int64_t N,
                                                    uint16_t* __restrict__ Y) {
    constexpr int C = G / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n = (int64_t)blockIdx.x * 64 + wave * 16 + r16;
    const bool nvalid = n < N;
    const int64_t nc = nvalid ? n : N - 1;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MB;
    const int64_t n_groups = K / G;

    const uint16_t* xr[MB];
    bool mvalid[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t m = m0 + 16 * mb + r16;
        mvalid[mb] = m < M;
        xr[mb] = X + (mvalid[mb] ? m : M - 1) * K + 8 * q;
    }

    floatx4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int64_t jg = 0; jg < n_groups; ++jg) {
        const float d = scales[jg * N + nc];
        const float z = (float)zeros[jg * N + nc];
        floatx4 accg[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) accg[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t k0 = jg * G + 32 * c + 8 * q;
            const uint32_t word = nvalid ? codes[(k0 >> 3) * N + nc] : 0u;
            u32x4 bw;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = nvalid ? (float)((word >> (8 * h)) & 0xF) - z : 0.f;
                const float hi = nvalid ? (float)((word >> (8 * h + 4)) & 0xF) - z : 0.f;
                bw[h] = pack_bf16x2(lo, hi);
            }
            const floatx4 s0 = *(const floatx4*)(s + k0);
            const floatx4 s1 = *(const floatx4*)(s + k0 + 4);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const u32x4 xv = *(const u32x4*)(xr[mb] + jg * G + 32 * c);
                u32x4 av;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float sl = h < 2 ? s0[2 * h] : s1[2 * h - 4];
                    const float sh = h < 2 ? s0[2 * h + 1] : s1[2 * h - 3];
                    av[h] = mvalid[mb] ? pack_bf16x2(bf16_lo(xv[h]) / sl, bf16_hi(xv[h]) / sh) : 0u;
                }
                accg[mb] = mfma16x16x32(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bw), accg[mb]);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][i] = fmaf(d, accg[mb][i], acc[mb][i]);
    }
    if (!nvalid) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + 16 * mb + 4 * q + i;
            if (m < M) {
                const __bf16 v = (__bf16)acc[mb][i];
                Y[m * N + n] = __builtin_bit_cast(uint16_t, v);
            }
        }
}

namespace {
typedef void (*gemm_fn)(const uint16_t*, int64_t, const float*, const uint32_t*, const float*, const uint8_t*,
                        int64_t, int64_t, uint16_t*);
template <int MB>
gemm_fn pick_g(int g) {
    if (g == 32) return k_w4a16_mfma<32, MB>;
    if (g == 64) return k_w4a16_mfma<64, MB>;
    if (g == 128) return k_w4a16_mfma<128, MB>;
    return nullptr;
}
}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int group_size) {
    (void)K;
    (void)group_size;
    GemmPlan p{};
    p.variant = M <= 16 ? 1 : 4;
    p.grid_x = (N + 63) / 64;
    p.grid_y = (M + 16 * p.variant - 1) / (16 * p.variant);
    p.grid_z = 1;
    p.ksplit = 1;
    p.off_part = 0;
    p.off_cnt = 0;
    p.ws_bytes = 0;
    return p;
}

hipError_t launch_gemm(const uint16_t* X, int64_t M, const float* s, const uint32_t* codes,
                       const float* scales, const uint8_t* zeros, int64_t K, int64_t N, int group_size,
                       uint16_t* Y, void* ws, const GemmPlan& p, hipStream_t st) {
    (void)ws;
    gemm_fn fn = p.variant == 1 ? pick_g<1>(group_size) : pick_g<4>(group_size);
    if (!fn) return hipErrorInvalidValue;
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, 1);
    fn<<<grid, 256, 0, st>>>(X, M, s, codes, scales, zeros, K, N, Y);
    return hipGetLastError();
}

}  // namespace awq
