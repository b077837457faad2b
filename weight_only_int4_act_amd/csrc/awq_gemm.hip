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
// HBM-bound: every byte of packed weights is read once.  A workgroup owns 256 output columns and
// 4*GPW quantization groups (G rows each): wavefront w takes groups 4i + w, i < GPW, of them.  Each
// lane reads 4 adjacent columns x 8 rows of codes with one 16-byte load per code row (a
// wavefront reads 1 KB of one code row: fully coalesced); the loads of the next group are issued
// before the current one is consumed.  Nibbles k and k+4 of a code word become two bf16 values
// 128 + q with one shift and one and-or, and v_dot2c_f32_bf16 multiplies them with the pair
// (x'_k, x'_{k+4}) of activations x' = bf16(x/s) staged in LDS in that pair order.  The offset
// and the zero point come out once per group: sum (q - z) x' = sum (128 + q) x' - (128 + z) sum x',
// where sum x' adds the same bf16-rounded values the products used.  The 4 wavefronts reduce
// through LDS in a fixed order; workgroups along K write float32 partials with plain stores and a
// second small kernel adds them in a fixed order and writes the bf16 outputs.  (A
// last-arriving-workgroup handoff inside one kernel would need device-scope release/acquire,
// which on this multi-die GPU writes back and invalidates a whole L2 per workgroup.)  No atomics:
// results are deterministic.
constexpr int kGemvCols = 256;   // columns per workgroup (64 lanes x 4)
constexpr int kGemvWaves = 4;    // wavefronts per workgroup
constexpr int kGemvGpw = 1;      // groups per wavefront

// (a & b) | c in one instruction (at most one scalar operand: the VOP3 constant-bus limit).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

template <int G>
__global__ __launch_bounds__(256) void k_w4a16_gemv(const uint16_t* __restrict__ X, const float* __restrict__ s,
                                                    const uint32_t* __restrict__ codes,
                                                    const float* __restrict__ scales,
                                                    const uint8_t* __restrict__ zeros, int K, int N,
                                                    uint16_t* __restrict__ Y, float* __restrict__ part) {
    constexpr int R = G / 8;                     // code rows per group
    constexpr int NG = kGemvWaves * kGemvGpw;    // groups per workgroup
    // x' of the workgroup's groups: group slot i, code row r, pair j: bf16 (x'_{8r+j}, x'_{8r+j+4})
    __shared__ uint32_t xpair[NG][G / 2];
    __shared__ float sxs[NG];
    __shared__ float red[kGemvWaves][kGemvCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cb = blockIdx.x, kb = blockIdx.y, nkb = gridDim.y;
    const int n_groups = K / G;
    const int n0 = cb * kGemvCols + lane * 4;
    const bool nvalid = n0 < N;                  // N % 4 == 0
    const int nc = nvalid ? n0 : N - 4;
    auto group_of = [&](int i) { return kb * NG + kGemvWaves * i + wave; };   // i-th group of this wave

    struct Buf {
        u32x4 cw[R];
        floatx4 dsc;
        uint32_t zw;
    };
    Buf b0, b1;
    auto issue = [&](int i, Buf& b) {
        const int gg = min(group_of(i), n_groups - 1);
        const uint32_t* cbase = codes + (int64_t)gg * R * N + nc;
#pragma unroll
        for (int r = 0; r < R; ++r) b.cw[r] = *(const u32x4*)(cbase + (int64_t)r * N);
        b.dsc = *(const floatx4*)(scales + (int64_t)gg * N + nc);
        b.zw = *(const uint32_t*)(zeros + (int64_t)gg * N + nc);
    };
    // x' of the workgroup's NG groups in pair order: thread t forms pair t % (G/2) of group slot
    // t / (G/2); the group sums come from a fixed butterfly over the G/2 lanes of a group.  The
    // activation and scale loads are issued before the code loads (loads complete in order), so
    // x' is formed while the codes are still in flight.
    constexpr int XI = (NG * (G / 2) + 255) / 256;   // pairs per thread
    float xa[XI][2], sa[XI][2];
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int t = 256 * u + (int)threadIdx.x;
        const int slot = t / (G / 2), l = t % (G / 2);
        const int gg = min(kb * NG + min(slot, NG - 1), n_groups - 1);
        const int k1 = gg * G + 8 * (l >> 2) + (l & 3), k2 = k1 + 4;
        xa[u][0] = bf16_lo((uint32_t)X[k1]);
        xa[u][1] = bf16_lo((uint32_t)X[k2]);
        sa[u][0] = s[k1];
        sa[u][1] = s[k2];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the activation loads ahead of the code loads
    issue(0, b0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int t = 256 * u + (int)threadIdx.x;
        const int slot = t / (G / 2), l = t % (G / 2);
        float sx = 0.f;
        if (slot < NG) {
            const __bf16 x1 = (__bf16)(xa[u][0] / sa[u][0]);
            const __bf16 x2 = (__bf16)(xa[u][1] / sa[u][1]);
            sx = (float)x1 + (float)x2;
            xpair[slot][l] = (uint32_t)__builtin_bit_cast(unsigned short, x1) |
                             ((uint32_t)__builtin_bit_cast(unsigned short, x2) << 16);
        }
#pragma unroll
        for (int o = 1; o < G / 2 && o < 64; o <<= 1) sx += __shfl_xor(sx, o, 64);
        if (slot < NG && l == 0) sxs[slot] = sx;
    }
    __syncthreads();

    const uint32_t nib = 0x000F000Fu;
    const uint32_t bf128 = __builtin_amdgcn_readfirstlane(0x43004300u);
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](int i, const Buf& b) {
        const int slot = kGemvWaves * i + wave;
        if (group_of(i) >= n_groups) return;
        float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t xp[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xp[j] = xpair[slot][4 * r + j];   // broadcast reads
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = b.cw[r][c];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t h = and_or(w >> (4 * j), nib, bf128);   // bf16 (128+q_j, 128+q_{j+4})
                    d[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h),
                                                           __builtin_bit_cast(bf16x2_t, xp[j]), d[c], false);
                }
            }
        }
        const float sx = sxs[slot];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float z = (float)((b.zw >> (8 * c)) & 0xFFu);
            acc[c] = fmaf(b.dsc[c], fmaf(-(128.f + z), sx, d[c]), acc[c]);
        }
    };
    // two groups per step, so each buffer keeps a fixed set of registers
#pragma unroll
    for (int i = 0; i < kGemvGpw; i += 2) {
        if (i + 1 < kGemvGpw) issue(i + 1, b1);
        consume(i, b0);
        if (i + 1 < kGemvGpw) {
            if (i + 2 < kGemvGpw) issue(i + 2, b0);
            consume(i + 1, b1);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) red[wave][lane * 4 + c] = acc[c];
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

// Y[n] = bf16(sum_b part[b][n]) in a fixed order.  A workgroup takes 32 columns; thread (c, l)
// adds partials b = l, l + 8, ... of column c (all its loads in flight at once), and the 8 sums of
// a column are added in lane order through LDS.  Wide enough to keep many loads in flight even for
// a few thousand columns.
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int nkb, int N,
                                                     uint16_t* __restrict__ Y) {
    __shared__ float sm[8][32];
    const int c = threadIdx.x & 31, l = threadIdx.x >> 5;
    const int n = blockIdx.x * 32 + c;
    const int nn = n < N ? n : N - 1;
    float t = 0.f;
    for (int b0 = l; b0 < nkb; b0 += 8 * 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = b0 + 8 * j < nkb ? part[(int64_t)(b0 + 8 * j) * N + nn] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += v[j];
    }
    sm[l][c] = t;
    __syncthreads();
    if (l == 0 && n < N) {
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) u += sm[i][c];
        const __bf16 o = (__bf16)u;
        Y[n] = __builtin_bit_cast(uint16_t, o);
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
    GemmPlan p{};
    if (M == 1) {
        p.variant = 0;
        p.grid_x = (N + kGemvCols - 1) / kGemvCols;
        p.grid_y = (K / group_size + kGemvWaves * kGemvGpw - 1) / (kGemvWaves * kGemvGpw);
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
        k_gemv_reduce<<<(unsigned)((N + 31) / 32), 256, 0, st>>>(part, (int)p.grid_y, (int)N, Y);
        return hipGetLastError();
    }
    gemm_fn fn = p.variant == 1 ? pick_g<1>(group_size) : pick_g<4>(group_size);
    if (!fn) return hipErrorInvalidValue;
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, 1);
    fn<<<grid, 256, 0, st>>>(X, M, s, codes, scales, zeros, K, N, Y);
    return hipGetLastError();
}

}  // namespace awq
