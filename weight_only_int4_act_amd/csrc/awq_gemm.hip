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

// ---------------------------------------------------------------- M = 1: decode-shaped GEMV
// HBM-bound: every byte of packed weights is read once.  A wavefront owns 256 output columns and
// one quantization group (G rows).  Each lane reads 4 adjacent columns x 8 rows of codes with one
// 16-byte load per code row (a wavefront reads 1 KB of one code row: fully coalesced) and issues
// all G/8 loads of its group before consuming them.  Nibbles k and k+4 of a code word become two
// bf16 values 128 + q with one and-or (plus one shift), and v_dot2c_f32_bf16 multiplies them with
// the pair (x'_k, x'_{k+4}) of activations x' = bf16(x/s) staged in LDS in that pair order.  The
// offset and the zero point come out once per group: sum (q - z) x' = sum (128 + q) x' -
// (128 + z) sum x', where sum x' adds the same bf16-rounded values the products used.
// The 4 wavefronts of a workgroup take 4 consecutive groups and reduce through LDS in a fixed
// order; workgroups along K write float32 partials with plain stores and a second small kernel
// adds them in a fixed order and writes the bf16 outputs.  (A last-arriving-workgroup handoff
// inside one kernel would need device-scope release/acquire, which on this multi-die GPU writes
// back and invalidates a whole L2 per workgroup.)  No atomics: results are deterministic.
constexpr int kGemvCols = 256;   // columns per workgroup (64 lanes x 4)
constexpr int kGemvWaves = 4;    // groups per workgroup

template <int G>
__global__ __launch_bounds__(256) void k_w4a16_gemv(const uint16_t* __restrict__ X, const float* __restrict__ s,
                                                    const uint32_t* __restrict__ codes,
                                                    const float* __restrict__ scales,
                                                    const uint8_t* __restrict__ zeros, int K, int N,
                                                    uint16_t* __restrict__ Y, float* __restrict__ part) {
    constexpr int R = G / 8;                     // code rows per group
    __shared__ uint32_t xpair[kGemvWaves][G / 2]; // code row r, pair j: bf16 (x'_{8r+j}, x'_{8r+j+4})
    __shared__ float sxs[kGemvWaves];
    __shared__ float red[kGemvWaves][kGemvCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cb = blockIdx.x, kb = blockIdx.y, nkb = gridDim.y;
    const int n_groups = K / G;
    const int g = kb * kGemvWaves + wave;
    const bool gvalid = g < n_groups;
    const int gg = gvalid ? g : n_groups - 1;
    const int n0 = cb * kGemvCols + lane * 4;
    const bool nvalid = n0 < N;                  // N % 4 == 0
    const int nc = nvalid ? n0 : N - 4;

    // issue every code load of the group first (R x 16 bytes per lane in flight)
    u32x4 cw[R];
    const uint32_t* cbase = codes + (int64_t)gg * R * N + nc;
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = *(const u32x4*)(cbase + (int64_t)r * N);
    const floatx4 dsc = *(const floatx4*)(scales + (int64_t)gg * N + nc);
    const uint32_t zw = *(const uint32_t*)(zeros + (int64_t)gg * N + nc);

    // x' = bf16(x / s) of the group in pair order: lane l < G/2 forms pair l (row l/4, slot l%4)
    float sx = 0.f;
    if (lane < G / 2) {
        const int r = lane >> 2, j = lane & 3;
        const int k1 = gg * G + 8 * r + j, k2 = k1 + 4;
        const __bf16 b1 = (__bf16)(bf16_lo((uint32_t)X[k1]) / s[k1]);
        const __bf16 b2 = (__bf16)(bf16_lo((uint32_t)X[k2]) / s[k2]);
        sx = (float)b1 + (float)b2;
        xpair[wave][lane] = (uint32_t)__builtin_bit_cast(unsigned short, b1) |
                            ((uint32_t)__builtin_bit_cast(unsigned short, b2) << 16);
    }
    sx = wave_sum(sx);
    if (lane == 0) sxs[wave] = sx;
    __syncthreads();

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t xp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xp[j] = xpair[wave][4 * r + j];   // broadcast reads
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = cw[r][c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t h = ((w >> (4 * j)) & 0x000F000Fu) | 0x43004300u;   // bf16 (128+q_j, 128+q_{j+4})
                acc[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h),
                                                         __builtin_bit_cast(bf16x2_t, xp[j]), acc[c], false);
            }
        }
    }
    const float sxw = sxs[wave];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float z = (float)((zw >> (8 * c)) & 0xFFu);
        red[wave][lane * 4 + c] = gvalid ? dsc[c] * fmaf(-(128.f + z), sxw, acc[c]) : 0.f;
    }
    __syncthreads();
    const int col = cb * kGemvCols + (int)threadIdx.x;
    const float ps = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
    if (col >= N) return;
    if (nkb == 1) {
        const __bf16 o = (__bf16)ps;
        Y[col] = __builtin_bit_cast(uint16_t, o);
    } else {
        part[(int64_t)kb * N + col] = ps;
    }
}

// Y[n] = bf16(sum_b part[b][n]) in a fixed order.
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int nkb, int N,
                                                     uint16_t* __restrict__ Y) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float t = 0.f;
    for (int b0 = 0; b0 < nkb; b0 += 8) {   // 8 loads in flight, added in the same fixed order
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = b0 + j < nkb ? part[(int64_t)(b0 + j) * N + n] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += v[j];
    }
    const __bf16 o = (__bf16)t;
    Y[n] = __builtin_bit_cast(uint16_t, o);
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
    GemmPlan p{};
    if (M == 1) {
        p.variant = 0;
        p.grid_x = (N + kGemvCols - 1) / kGemvCols;
        p.grid_y = (K / group_size + kGemvWaves - 1) / kGemvWaves;
        p.grid_z = 1;
        p.ksplit = (int)p.grid_y;
        p.off_part = 0;
        p.off_cnt = 0;
        p.ws_bytes = p.grid_y > 1 ? (size_t)p.grid_y * N * sizeof(float) : 0;
        return p;
    }
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
    if (p.variant == 0) {
        float* part = (float*)((char*)ws + p.off_part);
        dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y);
        if (group_size == 32)
            k_w4a16_gemv<32><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else if (group_size == 64)
            k_w4a16_gemv<64><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else
            k_w4a16_gemv<128><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.grid_y == 1) return e;
        k_gemv_reduce<<<(unsigned)((N + 255) / 256), 256, 0, st>>>(part, (int)p.grid_y, (int)N, Y);
        return hipGetLastError();
    }
    gemm_fn fn = p.variant == 1 ? pick_g<1>(group_size) : pick_g<4>(group_size);
    if (!fn) return hipErrorInvalidValue;
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, 1);
    fn<<<grid, 256, 0, st>>>(X, M, s, codes, scales, zeros, K, N, Y);
    return hipGetLastError();
}

}  // namespace awq
