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

// (a & b) | c in one instruction (at most one scalar operand: the VOP3 constant-bus limit).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

// ---------------------------------------------------------------- M > 1: matrix-core product
// Code word (i, n) holds rows 8i + j (j < 8) of column n at bits 4j..4j+3.  One and-or turns
// nibbles j and j + 4 of a word (shifted right by 4j) into the bf16 pair (128 + q_j, 128 + q_{j+4}),
// so a word becomes a matrix-core B operand whose 8 k slots are rows (0, 4, 1, 5, 2, 6, 3, 7) of the
// word.  The A operand holds x' = bf16(x / s) in the same slot order, so the product sums
// x'_k (128 + q_k); the offset and the zero point leave once per group and column:
//   sum_k x'_k (q_k - z) = sum_k x'_k (128 + q_k) - (128 + z) sum_k x'_k,
// where sum_k x'_k adds the same bf16-rounded values, and the accumulator of a group starts at
// -(128 + z) sum x' so that the products complete it.

// x' = bf16(x / s) in A-operand order and its group sums.  Workgroup (x, y) takes row block x (16
// rows) and 256 channels y (8 K chunks: 8 KB of fragments that lie next to each other in Xp).  Thread
// (row ml + 8h, kb) reads the 8 channels 8*kb .. 8*kb+7 of its row (a row's 32 threads read 512
// contiguous bytes) and forms the 16 bytes that lane 16*(kb%4) + m%16 of fragment (m/16, kb/4)
// feeds to the matrix core:
//   Xp[((m/16) * (K/32) + kb/4) * 64 + 16*(kb%4) + m%16] = pairs (x'_{8kb+j}, x'_{8kb+j+4}), j < 4;
// the entries meet in LDS and leave as contiguous 16-byte stores.  The G/8 consecutive threads of
// one group add their sums with a fixed butterfly; the first writes Sg[g * mpad + m].  Rows m in
// [M, mpad) are zero.
template <int G>
__global__ __launch_bounds__(256) void k_prep_x(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                const float* __restrict__ s, int64_t mpad, u32x4* __restrict__ Xp,
                                                float* __restrict__ Sg) {
    __shared__ u32x4 tile[512];
    const int kbl = threadIdx.x & 31, ml = threadIdx.x >> 5;
    const int64_t kbs = K / 8, kchunks = K / 32;
    const int64_t kb = (int64_t)blockIdx.y * 32 + kbl;
    const int64_t rb = blockIdx.x;
    const bool kvalid = kb < kbs;
    floatx4 s0 = floatx4{1.f, 1.f, 1.f, 1.f}, s1 = s0;
    if (kvalid) {
        s0 = *(const floatx4*)(s + 8 * kb);
        s1 = *(const floatx4*)(s + 8 * kb + 4);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int mi = ml + 8 * h;
        const int64_t m = rb * 16 + mi;
        float x[8];
        if (kvalid && m < M) {
            const u32x4 xv = *(const u32x4*)(X + m * K + 8 * kb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sl = e < 2 ? s0[2 * e] : s1[2 * e - 4];
                const float sh = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
                x[2 * e] = (float)(__bf16)(bf16_lo(xv[e]) / sl);
                x[2 * e + 1] = (float)(__bf16)(bf16_hi(xv[e]) / sh);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        float sx = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
#pragma unroll
        for (int o = 1; o < G / 8; o <<= 1) sx += __shfl_xor(sx, o, 64);
        tile[(kbl >> 2) * 64 + 16 * (kbl & 3) + mi] =
            u32x4{pack_bf16x2(x[0], x[4]), pack_bf16x2(x[1], x[5]), pack_bf16x2(x[2], x[6]), pack_bf16x2(x[3], x[7])};
        if (kvalid && kb % (G / 8) == 0) Sg[(kb / (G / 8)) * mpad + m] = sx;
    }
    __syncthreads();
    const int64_t base = (rb * kchunks + (int64_t)blockIdx.y * 8) * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = (int)threadIdx.x + 256 * h;
        if ((int64_t)blockIdx.y * 8 + e / 64 < kchunks) Xp[base + e] = tile[e];
    }
}

// Workgroup: 4 wavefronts over the same 16*MB rows x 64 columns, splitting the workgroup's groups
// of K between them (wavefront w takes groups gb + w, gb + w + 4, ...); a fixed-order sum through
// LDS joins them.  Lane (r16, q) owns the 4 adjacent columns n0 = 64*bx + 4*r16 .. n0 + 3 (one
// 16-byte code load per code row) and uses column n0 + j as column r16 of its j-th 16-column
// matrix-core tile; its accumulators hold rows 4q .. 4q+3 of each 16-row block.  With ksplit > 1
// the workgroups along K write float32 partials, added in a fixed order by k_gemv_reduce.
template <int G, int MB>
__global__ __launch_bounds__(256, 2) void k_w4a16_mma(const u32x4* __restrict__ Xp, const float* __restrict__ Sg,
                                                   int64_t mpad, int64_t M, const uint32_t* __restrict__ codes,
                                                   const float* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int64_t K, int64_t N,
                                                   uint16_t* __restrict__ Y, float* __restrict__ part) {
    constexpr int C = G / 32;
    __shared__ floatx4 red[3][MB][4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + 4 * r16;
    const bool nvalid = n0 < N;                  // N % 8 == 0: n0 < N implies n0 + 3 < N
    const int64_t nc = nvalid ? n0 : 0;
    const int64_t R0 = (int64_t)blockIdx.y * MB;  // first 16-row block
    const int64_t n_groups = K / G, kchunks = K / 32;
    const int64_t gpk = (n_groups + gridDim.z - 1) / gridDim.z;
    const int64_t gb = (int64_t)blockIdx.z * gpk;
    const int64_t ge = min(gb + gpk, n_groups);

    // the nibble mask in a vector register and the bf16 bias in a scalar one, so that the compiler
    // can form each operand pair with one v_and_or_b32 (one scalar operand per VOP3)
    uint32_t nib;
    asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(nib));
    const uint32_t bf128 = __builtin_amdgcn_readfirstlane(0x43004300u);
    floatx4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mb][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // For MB <= 2 the code words, steps, zeros and x' sums of this wavefront's next group (and, for
    // MB = 1, its x' fragments) are loaded before the current group's products are issued (two
    // register buffers), so a group's memory reads are in flight during the previous group's
    // matrix work; with 4 row blocks the accumulators leave no room for a second buffer.
    constexpr bool XB = MB == 1;
    struct Buf {
        u32x4 cw[C];
        floatx4 dsc;
        uint32_t zw;
        floatx4 sv[MB];
        u32x4 a[XB ? C : 1][MB];
    };
    auto issue = [&](int64_t g, Buf& b) {
#pragma unroll
        for (int c = 0; c < C; ++c) b.cw[c] = *(const u32x4*)(codes + (g * (G / 8) + 4 * c + q) * N + nc);
        b.dsc = *(const floatx4*)(scales + g * N + nc);
        b.zw = *(const uint32_t*)(zeros + g * N + nc);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) b.sv[mb] = *(const floatx4*)(Sg + g * mpad + (R0 + mb) * 16 + 4 * q);
        if constexpr (XB) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) b.a[c][mb] = Xp[((R0 + mb) * kchunks + g * C + c) * 64 + lane];
        }
    };
    auto consume = [&](int64_t g, const Buf& b) {
        floatx4 accg[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float off = -(128.f + (float)((b.zw >> (8 * j)) & 0xFFu));
#pragma unroll
                for (int i = 0; i < 4; ++i) accg[mb][j][i] = off * b.sv[mb][i];
            }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            u32x4 a[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                a[mb] = XB ? b.a[XB ? c : 0][mb] : Xp[((R0 + mb) * kchunks + g * C + c) * 64 + lane];
            const u32x4 cw = b.cw[c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // plain C (the compiler emits v_and_or_b32): these values feed the matrix core
                // directly, and only code the compiler sees gets its VALU -> MFMA wait states
                const u32x4 bo = u32x4{(cw[j] & nib) | bf128, ((cw[j] >> 4) & nib) | bf128,
                                       ((cw[j] >> 8) & nib) | bf128, ((cw[j] >> 12) & nib) | bf128};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    accg[mb][j] = mfma16x16x32(__builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, bo),
                                               accg[mb][j]);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][j][i] = fmaf(b.dsc[j], accg[mb][j][i], acc[mb][j][i]);
    };
    if constexpr (MB <= 2) {
        // two groups per step, so each buffer keeps a fixed set of registers
        Buf b0, b1;
        if (gb + wave < ge) issue(gb + wave, b0);
        for (int64_t g = gb + wave; g < ge; g += 8) {
            if (g + 4 < ge) issue(g + 4, b1);
            consume(g, b0);
            if (g + 4 < ge) {
                if (g + 8 < ge) issue(g + 8, b0);
                consume(g + 4, b1);
            }
        }
    } else {
        for (int64_t g = gb + wave; g < ge; g += 4) {
            Buf b;
            issue(g, b);
            consume(g, b);
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave - 1][mb][j][lane] = acc[mb][j];
    }
    __syncthreads();
    if (wave > 0 || !nvalid) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        floatx4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = ((acc[mb][j] + red[0][mb][j][lane]) + red[1][mb][j][lane]) + red[2][mb][j][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = (R0 + mb) * 16 + 4 * q + i;
            if (m >= M) continue;
            if (gridDim.z == 1) {
                const uint32_t lo = pack_bf16x2(v[0][i], v[1][i]), hi = pack_bf16x2(v[2][i], v[3][i]);
                *(uint2*)(Y + m * N + n0) = uint2{lo, hi};
            } else {
                *(floatx4*)(part + ((int64_t)blockIdx.z * M + m) * N + n0) = floatx4{v[0][i], v[1][i], v[2][i], v[3][i]};
            }
        }
    }
}

// Buffer resource over a byte range (accesses beyond it read zero) and a 16-byte-per-lane direct
// transfer into LDS (buffer_load_dwordx4 ... lds, M0 = LDS base, saved and restored around it).
namespace {
typedef int gi32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ gi32x4 grsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return gi32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff, (int)bytes, 0x00020000};
}
// 16 bytes per active lane from byte offset voff of the resource to LDS address lds + 16*lane
__device__ __forceinline__ void gdma16(gi32x4 rsrc, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "memory");
}
__device__ __forceinline__ void full_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
}  // namespace

// M > 32: 64 rows (4 row blocks) x 256 columns per workgroup.  The 4 wavefronts walk the same K
// groups, each with its own 64 columns (lane (r16, q) of wavefront w owns columns
// n0 = 256*bx + 64*w + 4*r16 .. n0 + 3, as above), so the x' fragments and x' sums of a group are
// copied once per workgroup straight into LDS by direct buffer-to-LDS transfers and read by all
// four (double buffered: the next group's transfers are in flight while the current group's
// products run).  Each wavefront keeps the code words, steps and zeros of its next group in a
// second register buffer.  Every barrier first waits for all of the wavefront's memory operations,
// so the transfers of the buffer it publishes have landed.
template <int G>
__global__ __launch_bounds__(256, 2) void k_w4a16_mma_lds(const u32x4* __restrict__ Xp, const float* __restrict__ Sg,
                                                       int64_t mpad, int64_t M, const uint32_t* __restrict__ codes,
                                                       const float* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, int64_t K, int64_t N,
                                                       uint16_t* __restrict__ Y, float* __restrict__ part) {
    constexpr int C = G / 32, MB = 4;
    constexpr int NE = MB * C * 64;              // 16-byte x' entries of a group (MB row blocks x C chunks)
    constexpr int PT = NE / 256;                 // entries per thread (C of them)
    __shared__ u32x4 xs[2][NE];
    __shared__ floatx4 ss[2][MB * 4];            // x' sums of the group's 64 rows
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 256 + 64 * wave + 4 * r16;
    const bool nvalid = n0 < N;                  // N % 8 == 0: n0 < N implies n0 + 3 < N
    const int64_t nc = nvalid ? n0 : 0;
    const int64_t R0 = (int64_t)blockIdx.y * MB;  // first 16-row block
    const int64_t n_groups = K / G, kchunks = K / 32;
    const int64_t gpk = (n_groups + gridDim.z - 1) / gridDim.z;
    const int64_t gb = min((int64_t)blockIdx.z * gpk, n_groups);
    const int64_t ge = min(gb + gpk, n_groups);

    uint32_t nib;
    asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(nib));
    const uint32_t bf128 = __builtin_amdgcn_readfirstlane(0x43004300u);
    floatx4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mb][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // workgroup-shared x' of a group: entry e = (mb * C + c) * 64 + l is lane l's fragment of row
    // block R0 + mb, chunk g*C + c; wavefront w's i-th transfer fills entries 256 i + 64 w .. + 63,
    // and lanes 0-15 of wavefront 0 bring the sums of rows 4 lane .. 4 lane + 3
    const gi32x4 xrs = grsrc(Xp, (uint32_t)(mpad / 16 * kchunks * 1024));
    const gi32x4 srs = grsrc(Sg, (uint32_t)(n_groups * mpad * 4));
    const uint32_t xs_lds = (uint32_t)(uintptr_t)&xs[0][0];
    const uint32_t ss_lds = (uint32_t)(uintptr_t)&ss[0][0];
    auto xdma = [&](int64_t g, int buf) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i;
            const int mb = e / (C * 64), c = (e / 64) % C, l = e % 64;
            gdma16(xrs, (uint32_t)((((R0 + mb) * kchunks + g * C + c) * 64 + l) * 16),
                   xs_lds + (uint32_t)((buf * NE + 256 * i + 64 * wave) * 16));
        }
        if (wave == 0 && lane < MB * 4)
            gdma16(srs, (uint32_t)((g * mpad + R0 * 16 + 4 * lane) * 4), ss_lds + (uint32_t)(buf * MB * 4 * 16));
    };
    struct Buf {
        u32x4 cw[C];
        floatx4 dsc;
        uint32_t zw;
    };
    auto issue = [&](int64_t g, Buf& b) {
#pragma unroll
        for (int c = 0; c < C; ++c) b.cw[c] = *(const u32x4*)(codes + (g * (G / 8) + 4 * c + q) * N + nc);
        b.dsc = *(const floatx4*)(scales + g * N + nc);
        b.zw = *(const uint32_t*)(zeros + g * N + nc);
    };
    auto consume = [&](const Buf& b, int buf) {
        floatx4 accg[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const floatx4 sv = ss[buf][mb * 4 + q];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float off = -(128.f + (float)((b.zw >> (8 * j)) & 0xFFu));
#pragma unroll
                for (int i = 0; i < 4; ++i) accg[mb][j][i] = off * sv[i];
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            u32x4 a[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) a[mb] = xs[buf][(mb * C + c) * 64 + lane];
            const u32x4 cw = b.cw[c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 bo = u32x4{(cw[j] & nib) | bf128, ((cw[j] >> 4) & nib) | bf128,
                                       ((cw[j] >> 8) & nib) | bf128, ((cw[j] >> 12) & nib) | bf128};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    accg[mb][j] = mfma16x16x32(__builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, bo),
                                               accg[mb][j]);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][j][i] = fmaf(b.dsc[j], accg[mb][j][i], acc[mb][j][i]);
    };
    // one group per step: while the products of group g run (from xs[g & 1]), the loads of group
    // g + 1 are in flight (x' into the other LDS buffer, codes into the other register buffer)
    Buf b0, b1;
    if (gb < ge) {
        xdma(gb, 0);
        issue(gb, b0);
    }
    full_barrier();
    for (int64_t g = gb; g < ge; g += 2) {
        const bool n1 = g + 1 < ge;
        if (n1) {
            xdma(g + 1, 1);
            issue(g + 1, b1);
        }
        consume(b0, 0);
        full_barrier();                           // xs[1] filled, xs[0] no longer read
        if (!n1) break;
        const bool n2 = g + 2 < ge;
        if (n2) {
            xdma(g + 2, 0);
            issue(g + 2, b0);
        }
        consume(b1, 1);
        full_barrier();                           // xs[0] filled, xs[1] no longer read
    }

    if (!nvalid) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = (R0 + mb) * 16 + 4 * q + i;
            if (m >= M) continue;
            if (gridDim.z == 1) {
                const uint32_t lo = pack_bf16x2(acc[mb][0][i], acc[mb][1][i]);
                const uint32_t hi = pack_bf16x2(acc[mb][2][i], acc[mb][3][i]);
                *(uint2*)(Y + m * N + n0) = uint2{lo, hi};
            } else {
                *(floatx4*)(part + ((int64_t)blockIdx.z * M + m) * N + n0) =
                    floatx4{acc[mb][0][i], acc[mb][1][i], acc[mb][2][i], acc[mb][3][i]};
            }
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

// VG: rows a wavefront takes at a time, a divisor of the quantization group G.  Narrow layers
// split each group into G/VG slices (each with the group's step and zero, and the sum of x' over
// its own rows in the offset/zero correction, which is linear in the rows), so that more
// workgroups share K and fill the GPU.
template <int G, int VG>
__global__ __launch_bounds__(256) void k_w4a16_gemv(const uint16_t* __restrict__ X, const float* __restrict__ s,
                                                    const uint32_t* __restrict__ codes,
                                                    const float* __restrict__ scales,
                                                    const uint8_t* __restrict__ zeros, int K, int N,
                                                    uint16_t* __restrict__ Y, float* __restrict__ part) {
    static_assert(G % VG == 0 && VG >= 32, "slice of a group");
    constexpr int R = VG / 8;                    // code rows per slice
    constexpr int NG = kGemvWaves * kGemvGpw;    // slices per workgroup
    // x' of the workgroup's slices: slot i, code row r, pair j: bf16 (x'_{8r+j}, x'_{8r+j+4})
    __shared__ uint32_t xpair[NG][VG / 2];
    __shared__ float sxs[NG];
    __shared__ float red[kGemvWaves][kGemvCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cb = blockIdx.x, kb = blockIdx.y, nkb = gridDim.y;
    const int n_groups = K / VG;                 // slices, from here on called groups
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
        for (int r = 0; r < R; ++r)   // read once: streaming (non-temporal) loads
            b.cw[r] = __builtin_nontemporal_load((const u32x4*)(cbase + (int64_t)r * N));
        const int qg = gg / (G / VG);            // the quantization group of the slice
        b.dsc = *(const floatx4*)(scales + (int64_t)qg * N + nc);
        b.zw = *(const uint32_t*)(zeros + (int64_t)qg * N + nc);
    };
    // x' of the workgroup's NG slices in pair order: thread t forms pair t % (VG/2) of slot
    // t / (VG/2); the slice sums come from a fixed butterfly over the VG/2 lanes of a slice.  The
    // activation and scale loads are issued before the code loads (loads complete in order), so
    // x' is formed while the codes are still in flight.
    constexpr int XI = (NG * (VG / 2) + 255) / 256;  // pairs per thread
    float xa[XI][2], sa[XI][2];
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int t = 256 * u + (int)threadIdx.x;
        const int slot = t / (VG / 2), l = t % (VG / 2);
        const int gg = min(kb * NG + min(slot, NG - 1), n_groups - 1);
        const int k1 = gg * VG + 8 * (l >> 2) + (l & 3), k2 = k1 + 4;
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
        const int slot = t / (VG / 2), l = t % (VG / 2);
        float sx = 0.f;
        if (slot < NG) {
            const __bf16 x1 = (__bf16)(xa[u][0] / sa[u][0]);
            const __bf16 x2 = (__bf16)(xa[u][1] / sa[u][1]);
            sx = (float)x1 + (float)x2;
            xpair[slot][l] = (uint32_t)__builtin_bit_cast(unsigned short, x1) |
                             ((uint32_t)__builtin_bit_cast(unsigned short, x2) << 16);
        }
#pragma unroll
        for (int o = 1; o < VG / 2 && o < 64; o <<= 1) sx += __shfl_xor(sx, o, 64);
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

// Y = bf16(sum_b part[b]) for the matrix-core path, where there are few partials (ksplit <= 8)
// and many outputs: each thread adds the partials of 4 adjacent outputs in a fixed order (all its
// loads issued before the sum) and writes 4 bf16 values.
__global__ __launch_bounds__(256) void k_part_reduce4(const floatx4* __restrict__ part, int nkb, int64_t n4,
                                                      uint2* __restrict__ Y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    floatx4 v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = b < nkb ? part[b * n4 + i] : floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 t = v[0];
#pragma unroll
    for (int b = 1; b < 8; ++b) t += v[b];
    Y[i] = uint2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int G>
hipError_t launch_mma(const uint16_t* X, int64_t M, const float* s, const uint32_t* codes, const float* scales,
                      const uint8_t* zeros, int64_t K, int64_t N, uint16_t* Y, void* ws, const GemmPlan& p,
                      hipStream_t st) {
    char* base = (char*)ws;
    u32x4* Xp = (u32x4*)(base + p.off_xp);
    float* Sg = (float*)(base + p.off_sg);
    float* part = (float*)(base + p.off_part);
    // row blocks along x (up to 2^31 - 1), 256-channel blocks along y (K <= 16.7M)
    k_prep_x<G><<<dim3((unsigned)(p.mpad / 16), (unsigned)((K + 255) / 256)), 256, 0, st>>>(X, M, K, s, p.mpad, Xp, Sg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, (unsigned)p.grid_z);
    if (p.variant == 1)
        k_w4a16_mma<G, 1><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part);
    else if (p.variant == 2)
        k_w4a16_mma<G, 2><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part);
    else if (p.variant == 4)
        k_w4a16_mma<G, 4><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part);
    else
        k_w4a16_mma_lds<G><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part);
    e = hipGetLastError();
    if (e != hipSuccess || p.ksplit == 1) return e;
    if (p.ksplit <= 8) {
        const int64_t n4 = M * N / 4;   // N % 8 == 0
        k_part_reduce4<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>((const floatx4*)part, p.ksplit, n4, (uint2*)Y);
    } else {
        k_gemv_reduce<<<(unsigned)((M * N + 31) / 32), 256, 0, st>>>(part, p.ksplit, (int)(M * N), Y);
    }
    return hipGetLastError();
}
}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int group_size) {
    GemmPlan p{};
    const int64_t n_groups = K / group_size;
    if (M == 1) {
        p.variant = 0;
        p.grid_x = (N + kGemvCols - 1) / kGemvCols;
        // halve the rows a wavefront takes (down to 32) until there are ~1536 workgroups: about
        // six per CU, enough that the last ones to finish leave little of the GPU idle
        p.vgroup = group_size;
        while (p.vgroup > 32 && p.grid_x * (K / p.vgroup) / (kGemvWaves * kGemvGpw) < 1536) p.vgroup /= 2;
        const int64_t n_slices = K / p.vgroup;
        p.grid_y = (n_slices + kGemvWaves * kGemvGpw - 1) / (kGemvWaves * kGemvGpw);
        p.grid_z = 1;
        p.ksplit = (int)p.grid_y;
        p.mpad = 1;
        p.ws_bytes = p.grid_y > 1 ? (size_t)p.grid_y * N * sizeof(float) : 0;
        return p;
    }
    // 16-row blocks per wavefront: as many as the rows need, up to 4.  Variants 1, 2, 4: 64
    // columns per workgroup, its wavefronts splitting the groups (k_w4a16_mma); variant 5 (M > 32
    // when x' and its sums lie within the 32-bit byte range of a buffer resource): 64 rows x 256
    // columns, x' shared through LDS (k_w4a16_mma_lds)
    const int mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    const int64_t rows = 16 * mb;
    p.mpad = (M + rows - 1) / rows * rows;
    const bool lds_ok = p.mpad * K * (int64_t)sizeof(uint16_t) < ((int64_t)1 << 32) &&
                        n_groups * p.mpad * (int64_t)sizeof(float) < ((int64_t)1 << 32);
    p.variant = mb == 4 && lds_ok ? 5 : mb;
    p.grid_x = p.variant == 5 ? (N + 255) / 256 : (N + 63) / 64;
    p.grid_y = p.mpad / rows;
    // split K across workgroups until ~512 workgroups are in flight (2 per CU), keeping enough
    // groups per workgroup and the partials' index range within int
    const int64_t tiles = p.grid_x * p.grid_y;
    int64_t ks = 1;
    const int64_t min_groups = p.variant == 5 ? 2 : 4;   // two (one prefetched) or one per wavefront
    while (tiles * ks < 512 && 2 * ks * min_groups <= n_groups && 2 * ks * M * N < ((int64_t)1 << 31)) ks *= 2;
    p.grid_z = ks;
    p.ksplit = (int)ks;
    size_t off = 0;
    p.off_part = off; off = align256(off + (ks > 1 ? (size_t)ks * M * N * sizeof(float) : 0));
    p.off_xp = off;   off = align256(off + (size_t)p.mpad * K * sizeof(uint16_t));
    p.off_sg = off;   off = align256(off + (size_t)n_groups * p.mpad * sizeof(float));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_gemm(const uint16_t* X, int64_t M, const float* s, const uint32_t* codes,
                       const float* scales, const uint8_t* zeros, int64_t K, int64_t N, int group_size,
                       uint16_t* Y, void* ws, const GemmPlan& p, hipStream_t st) {
    if (p.variant == 0) {
        float* part = (float*)((char*)ws + p.off_part);
        dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y);
        const int vg = p.vgroup;
        if (group_size == 32)
            k_w4a16_gemv<32, 32><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else if (group_size == 64 && vg == 64)
            k_w4a16_gemv<64, 64><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else if (group_size == 64)
            k_w4a16_gemv<64, 32><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else if (vg == 128)
            k_w4a16_gemv<128, 128><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else if (vg == 64)
            k_w4a16_gemv<128, 64><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        else
            k_w4a16_gemv<128, 32><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.grid_y == 1) return e;
        k_gemv_reduce<<<(unsigned)((N + 31) / 32), 256, 0, st>>>(part, (int)p.grid_y, (int)N, Y);
        return hipGetLastError();
    }
    if (group_size == 32) return launch_mma<32>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    if (group_size == 64) return launch_mma<64>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    if (group_size == 128) return launch_mma<128>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    return hipErrorInvalidValue;
}

}  // namespace awq
