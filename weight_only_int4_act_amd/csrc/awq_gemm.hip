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
#include <algorithm>

#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// (a & b) | c in one instruction (at most one scalar operand: the VOP3 constant-bus limit).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

namespace {
// float32 x4 to / from the device-coherent level: buffer operations with the agent-scope
// cache-policy bit (sc1), so a partial written on one die is read back on another.
constexpr int kCpolAgent = 16;
constexpr int kCpolStream = 2;   // non-temporal: data read once
__device__ __forceinline__ void store4_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolAgent);
}
__device__ __forceinline__ floatx4 load4_agent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolAgent));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
}  // namespace

// Split-K partials: workgroup z of a tile writes its float32 sums to part[z][m][n] with agent-scope
// stores (written through to the device-coherent level, not left in one die's L2), waits for them
// and bumps the tile's arrival counter with one agent-scope atomic; the workgroup that arrives last
// reads every partial of the tile with agent-scope loads, adds them in K-block order (so the
// result does not depend on the arrival order), writes Y and sets the counter back to zero.
// Offsets of rows beyond M and columns beyond N lie outside the partials' buffer resource, where
// stores are dropped and loads read zero.
#ifndef AWQ_GEMV_MAX_KSPLIT
#define AWQ_GEMV_MAX_KSPLIT 16      // most K blocks (arrivals at one counter) of a split-K product
#endif
// 2..32 rows: the K split stops at about this many workgroups (one per CU)
constexpr int64_t kGemmSkinnyWorkgroups = 256;

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
    lds_poison_start(&tile[0], 512);
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

// 2..32 rows.  Workgroup: 4 wavefronts over the same 16*MB rows x 64 columns (MB = 1 for up to 16
// rows, 2 for up to 32), splitting the workgroup's groups of K between them (wavefront w takes groups gb + w, gb + w + 4, ...); a fixed-order sum through
// LDS joins them.  Lane (r16, q) owns the 4 adjacent columns n0 = 64*bx + 4*r16 .. n0 + 3 (one
// 16-byte code load per code row) and uses column n0 + j as column r16 of its j-th 16-column
// matrix-core tile; its accumulators hold rows 4q .. 4q+3 of each 16-row block.  With several
// workgroups along K (gridDim.z), the last of a tile to arrive adds their partials (see above).
template <int G, int MB>
__global__ __launch_bounds__(256, 2) void k_w4a16_mma(const u32x4* __restrict__ Xp, const float* __restrict__ Sg,
                                                   int64_t mpad, int64_t M, const uint32_t* __restrict__ codes,
                                                   const float* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int64_t K, int64_t N,
                                                   uint16_t* __restrict__ Y, float* __restrict__ part,
                                                   uint32_t* __restrict__ cnt, int cstride) {
    constexpr int C = G / 32;
    __shared__ floatx4 red[3][MB][4][64];
    // the wavefront index in a scalar register: the group loop is then uniform per wavefront
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
    if constexpr (kLdsPoison) {   // debug build: the cross-wavefront sums start as NaN
        if (wave > 0) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int j = 0; j < 4; ++j) red[wave - 1][mb][j][lane] = __builtin_bit_cast(floatx4, lds_nan16());
        }
        __syncthreads();
    }
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

    // The code words, steps, zeros and x' sums of the wavefront's next group, and its x' fragments,
    // are loaded before the current group's products are issued (two register buffers of each).  No
    // load is issued under a condition (a load past the wavefront's last group reads that group
    // again: a valid address, still in the cache) and scheduling barriers keep the next group's loads
    // ahead of the current group's products, so the compiler counts the loads in flight exactly and
    // each group waits for its own buffer only, not for the prefetch.
    struct Buf {
        u32x4 cw[C];
        floatx4 dsc;
        uint32_t zw;
        floatx4 sv[MB];
    };
    auto issue = [&](int64_t g, Buf& b, u32x4 (&a)[C][MB]) {
#pragma unroll
        for (int c = 0; c < C; ++c)   // read once: streaming (non-temporal) loads
            b.cw[c] = __builtin_nontemporal_load((const u32x4*)(codes + (g * (G / 8) + 4 * c + q) * N + nc));
        b.dsc = *(const floatx4*)(scales + g * N + nc);
        b.zw = *(const uint32_t*)(zeros + g * N + nc);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) b.sv[mb] = *(const floatx4*)(Sg + g * mpad + (R0 + mb) * 16 + 4 * q);
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) a[c][mb] = Xp[((R0 + mb) * kchunks + g * C + c) * 64 + lane];
    };
    auto consume = [&](const Buf& b, const u32x4 (&a)[C][MB]) {
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
            const u32x4 cw = b.cw[c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // plain C (the compiler emits v_and_or_b32): these values feed the matrix core
                // directly, and only code the compiler sees gets its VALU -> MFMA wait states
                const u32x4 bo = u32x4{(cw[j] & nib) | bf128, ((cw[j] >> 4) & nib) | bf128,
                                       ((cw[j] >> 8) & nib) | bf128, ((cw[j] >> 12) & nib) | bf128};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    accg[mb][j] = mfma16x16x32(__builtin_bit_cast(bf16x8, a[c][mb]), __builtin_bit_cast(bf16x8, bo),
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
    {
        Buf b0, b1;
        u32x4 a0[C][MB], a1[C][MB];
        const int64_t nw = ge - gb > wave ? (ge - gb - wave + 3) / 4 : 0;   // the wavefront's groups
        auto gw = [&](int64_t i) { return gb + wave + 4 * i; };            // its i-th group
        const int64_t gl = nw > 0 ? gw(nw - 1) : n_groups - 1;
        issue(min(gw(0), gl), b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        int64_t i = 0;
        for (; i + 2 <= nw; i += 2) {
            issue(min(gw(i + 1), gl), b1, a1);
            __builtin_amdgcn_sched_barrier(0);
            consume(b0, a0);
            __builtin_amdgcn_sched_barrier(0);
            issue(min(gw(i + 2), gl), b0, a0);
            __builtin_amdgcn_sched_barrier(0);
            consume(b1, a1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i < nw) consume(b0, a0);
    }

    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave - 1][mb][j][lane] = acc[mb][j];
    }
    __syncthreads();
    if (wave > 0) return;
    // wavefront 0: rows (R0 + mb) * 16 + 4q + i, columns n0 .. n0+3, as float32 x4 over the columns
    floatx4 v[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        floatx4 t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = ((acc[mb][j] + red[0][mb][j][lane]) + red[1][mb][j][lane]) + red[2][mb][j][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[mb][i] = floatx4{t[0][i], t[1][i], t[2][i], t[3][i]};
    }
    auto row = [&](int mb, int i) { return (R0 + mb) * 16 + 4 * q + i; };
    auto write_y = [&](const floatx4 (&w)[MB][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (nvalid && row(mb, i) < M)
                    *(uint2*)(Y + row(mb, i) * N + n0) = uint2{pack_bf16x2(w[mb][i][0], w[mb][i][1]),
                                                                pack_bf16x2(w[mb][i][2], w[mb][i][3])};
    };
    const int nz = gridDim.z;
    if (nz == 1) {
        write_y(v);
        return;
    }
    const uint32_t pbytes = (uint32_t)((int64_t)nz * M * N * 4);
    const __amdgpu_buffer_rsrc_t pr = rsrc(part, pbytes);
    auto poff = [&](int64_t z, int mb, int i) {
        return (nvalid && row(mb, i) < M) ? (uint32_t)(((z * M + row(mb, i)) * N + n0) * 4) : pbytes;
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) store4_agent(pr, poff(blockIdx.z, mb, i), v[mb][i]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this workgroup's partial has landed
    const int tile = blockIdx.x + gridDim.x * blockIdx.y;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt + (int64_t)tile * cstride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)(nz - 1)) return;
    constexpr int ZB = 4 / MB;   // K blocks whose loads are in flight together
    floatx4 tot[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[mb][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < nz; z0 += ZB) {
        floatx4 pv[ZB][MB][4];
#pragma unroll
        for (int u = 0; u < ZB; ++u)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[u][mb][i] = load4_agent(pr, z0 + u < nz ? poff(z0 + u, mb, i) : pbytes);
#pragma unroll
        for (int u = 0; u < ZB; ++u)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[mb][i] += pv[u][mb][i];
    }
    write_y(tot);
    if (lane == 0) __hip_atomic_store(cnt + (int64_t)tile * cstride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// wait for every memory operation of the wavefront, then the workgroup barrier; written with the
// builtins, so the compiler knows that no load is in flight after it
__device__ __forceinline__ void full_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}
}  // namespace

// M > 32: 64 rows (4 row blocks) x 256 columns per workgroup.  The 4 wavefronts walk the same K
// groups, each with its own 64 columns (lane (r16, q) of wavefront w owns columns
// n0 = 256*bx + 64*w + 4*r16 .. n0 + 3, as above), so the x' fragments and x' sums of a group are
// copied once per workgroup straight into LDS by direct buffer-to-LDS transfers and read by all
// four (double buffered: the next group's transfers are in flight while the current group's
// products run).  Each wavefront keeps the code words, steps and zeros of its next group in a
// second register buffer.  Every barrier first waits for all of the wavefront's memory operations,
// so the transfers of the buffer it publishes have landed.  With several workgroups along K, every
// wavefront writes its columns' partials and the workgroup arrives once (see above).
template <int G>
__global__ __launch_bounds__(256, 2) void k_w4a16_mma_lds(const u32x4* __restrict__ Xp, const float* __restrict__ Sg,
                                                       int64_t mpad, int64_t M, const uint32_t* __restrict__ codes,
                                                       const float* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, int64_t K, int64_t N,
                                                       uint16_t* __restrict__ Y, float* __restrict__ part,
                                                       uint32_t* __restrict__ cnt, int cstride) {
    constexpr int C = G / 32, MB = 4;
    constexpr int NE = MB * C * 64;              // 16-byte x' entries of a group (MB row blocks x C chunks)
    constexpr int PT = NE / 256;                 // entries per thread (C of them)
    __shared__ u32x4 xs[2][NE];
    __shared__ floatx4 ss[2][MB * 4];            // x' sums of the group's 64 rows
    __shared__ uint32_t arrival;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
        if constexpr (kLdsPoison) {   // debug build: NaN where this buffer's transfers will land
#pragma unroll
            for (int i = 0; i < PT; ++i) xs[buf][256 * i + 64 * wave + lane] = lds_nan16();
            if (wave == 0 && lane < MB * 4) ss[buf][lane] = __builtin_bit_cast(floatx4, lds_nan16());
            lds_write_fence();
        }
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
    // g + 1 are in flight (x' into the other LDS buffer, codes into the other register buffer).
    // The loads are issued unconditionally (past the K block's last group they read that group
    // again, into the buffer no one reads any more) and held ahead of the products by scheduling
    // barriers, so the compiler does not make the products wait for the prefetch.
    Buf b0, b1;
    const int64_t gl = max(ge - 1, (int64_t)0);   // (an empty K block reads its neighbour's last group, unused)
    xdma(min(gb, gl), 0);
    issue(min(gb, gl), b0);
    full_barrier();
    int64_t g = gb;
    for (; g + 2 <= ge; g += 2) {   // two groups per step, no branch between a prefetch and its use
        xdma(min(g + 1, gl), 1);
        issue(min(g + 1, gl), b1);
        __builtin_amdgcn_sched_barrier(0);
        consume(b0, 0);
        full_barrier();                           // xs[1] filled, xs[0] no longer read
        xdma(min(g + 2, gl), 0);
        issue(min(g + 2, gl), b0);
        __builtin_amdgcn_sched_barrier(0);
        consume(b1, 1);
        full_barrier();                           // xs[0] filled, xs[1] no longer read
    }
    if (g < ge) consume(b0, 0);                   // the last of an odd number: already in place

    floatx4 v[MB][4];   // rows (R0 + mb) * 16 + 4q + i, columns n0 .. n0+3
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[mb][i] = floatx4{acc[mb][0][i], acc[mb][1][i], acc[mb][2][i], acc[mb][3][i]};
    auto row = [&](int mb, int i) { return (R0 + mb) * 16 + 4 * q + i; };
    auto write_y = [&](const floatx4 (&w)[MB][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (nvalid && row(mb, i) < M)
                    *(uint2*)(Y + row(mb, i) * N + n0) = uint2{pack_bf16x2(w[mb][i][0], w[mb][i][1]),
                                                                pack_bf16x2(w[mb][i][2], w[mb][i][3])};
    };
    const int nz = gridDim.z;
    if (nz == 1) {
        write_y(v);
        return;
    }
    const uint32_t pbytes = (uint32_t)((int64_t)nz * M * N * 4);
    const __amdgpu_buffer_rsrc_t pr = rsrc(part, pbytes);
    auto poff = [&](int64_t z, int mb, int i) {
        return (nvalid && row(mb, i) < M) ? (uint32_t)(((z * M + row(mb, i)) * N + n0) * 4) : pbytes;
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) store4_agent(pr, poff(blockIdx.z, mb, i), v[mb][i]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's partial has landed
    __syncthreads();
    const int tile = blockIdx.x + gridDim.x * blockIdx.y;
    if (tid == 0) arrival = __hip_atomic_fetch_add(cnt + (int64_t)tile * cstride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrival != (uint32_t)(nz - 1)) return;
    floatx4 tot[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[mb][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < nz; ++z) {
        floatx4 pv[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[mb][i] = load4_agent(pr, poff(z, mb, i));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[mb][i] += pv[mb][i];
    }
    write_y(tot);
    if (tid == 0) __hip_atomic_store(cnt + (int64_t)tile * cstride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- M = 1: decode-shaped GEMV
// HBM-bound: every byte of packed weights is read once.  A workgroup owns 256 output columns (64
// on narrow layers and long K, see QR below) and 4*GPW slices of VG rows of K: wavefront w takes
// slices 4i + w, i < GPW.  Each lane reads 4 adjacent columns x 8 rows of codes with one 16-byte
// streaming load per code row (a wavefront reads 1 KB of code rows: whole 64- or 256-byte row
// segments); the loads of the next slice are issued before the current one is consumed.  Nibbles k and k+4 of a code word become two bf16 values 128 + q with
// one shift and one and-or (the B operand of a 16x16x32 bf16 matrix-core product) and meet the pair
// (x'_k, x'_{k+4}) of activations x' = bf16(x/s) staged in LDS in that pair order (in the A operand,
// see QR below).  The offset and the zero point
// come out once per slice: sum (q - z) x' = sum (128 + q) x' - (128 + z) sum x', where sum x'
// adds the same bf16-rounded values the products used.  Wavefronts 1-3 hand their sums to
// wavefront 0 through LDS and leave; wavefront 0 adds them in a fixed order.  With one K block it
// writes Y.  Otherwise it writes the workgroup's float32 partial with agent-scope stores
// (written through to the device-coherent level, not left in one die's L2), waits for them and
// bumps the column block's arrival counter (on a 128-byte line of its own) with one agent-scope
// atomic; the wavefront that
// arrives last reads every partial of the block with agent-scope loads, adds them in K-block
// order (so the result does not depend on the arrival order), writes Y and sets the counter back
// to zero.  No wavefront waits on another workgroup, and there are no floating-point atomics.

constexpr int kGemvCols = 256;   // columns per workgroup (64 lanes x 4)
constexpr int kGemvWaves = 4;    // wavefronts per workgroup

// VG: rows a wavefront takes at a time, a divisor of the quantization group G.  Narrow layers
// split each group into G/VG slices (each with the group's step and zero, and the sum of x' over
// its own rows in the offset/zero correction, which is linear in the rows), so that more
// workgroups share K and fill the GPU.
// QR: lanes per column quadruple.  QR = 1: lane l owns columns 4l .. 4l+3 of the workgroup's 256
// and reads every code row of a slice.  One product per code row and column of the quadruple: lane
// l = 16g + n supplies k slots 8g .. 8g + 7 of column n, i.e. its own column 4l + c, and row 4g of
// the A operand carries x' of the code row in slot group g (lanes 0, 20, 40, 60; every other entry
// is zero), so element 0 of lane l's result, row 4g and column n, is the dot product for its own
// column: no lane exchange, about 7 VALU instructions per code word against 11 with four
// v_dot2c_f32_bf16.  QR = 4: the workgroup owns 64 columns; lane (r16, rq),
// r16 = l % 16, rq = l / 16, owns columns 4 r16 .. 4 r16 + 3 and reads the code rows rq, rq + 4, ...
// of a slice.  That is the B-operand layout of a 16x16x32 bf16 matrix-core product: lane (r16, rq)
// holds k slots 8 rq .. 8 rq + 7 of column r16, here code row rq (+4r) of column 4 r16 + c for the
// c-th product.  Row 0 of the A operand carries x' of the same code rows (lanes r16 = 0), every
// other row is zero, so row 0 of the result is the dot product over the four code rows for the 16
// columns 4 r16 + c; one product per column of the quadruple replaces four v_dot2c per code word
// and the lane swaps that would add the quadruple's four partial sums (about 7 instead of 11 VALU
// instructions per code word).  Narrow layers and long K get four times as many workgroups without a
// longer K split.
template <int G, int VG, int kGemvGpw, int QR>
__global__ __launch_bounds__(256) void k_w4a16_gemv(const uint16_t* __restrict__ X, const float* __restrict__ s,
                                                    const uint32_t* __restrict__ codes,
                                                    const float* __restrict__ scales,
                                                    const uint8_t* __restrict__ zeros, int K, int N,
                                                    uint16_t* __restrict__ Y, float* __restrict__ part,
                                                    uint32_t* __restrict__ cnt, int cstride) {
    static_assert(G % VG == 0 && VG >= 32, "slice of a group");
    static_assert(QR == 1 || QR == 4, "lanes per column quadruple");
    constexpr int R = VG / 8;                    // code rows per slice
    constexpr int RL = R / QR;                   // code rows per lane and slice
    constexpr int COLS = kGemvCols / QR;         // columns per workgroup
    constexpr int NG = kGemvWaves * kGemvGpw;    // slices per workgroup
    // x' of the workgroup's slices: slot i, code row r, pair j: bf16 (x'_{8r+j}, x'_{8r+j+4})
    __shared__ uint32_t xpair[NG][VG / 2];
    __shared__ float sxs[NG];
    __shared__ floatx4 red[kGemvWaves - 1][64];
    __shared__ u32x4 zpad;   // the zero entries of the matrix-core A operand
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cb = blockIdx.x, kb = blockIdx.y, nkb = gridDim.y;
    if (threadIdx.x == 0) zpad = u32x4{0u, 0u, 0u, 0u};   // read after the barrier below
    if constexpr (kLdsPoison) {   // debug build: x', its sums and the cross-wavefront sums start as NaN
        for (int i = threadIdx.x; i < NG * (VG / 2); i += 256) (&xpair[0][0])[i] = kLdsNan;
        if (threadIdx.x < NG) sxs[threadIdx.x] = __builtin_nanf("");
        if (wave > 0) red[wave - 1][lane] = __builtin_bit_cast(floatx4, lds_nan16());
        __syncthreads();
    }
    const int n_groups = K / VG;                 // slices, from here on called groups
    const int rq = QR == 1 ? 0 : lane / (64 / QR);   // this lane's first code row of a slice
    const int n0 = cb * COLS + 4 * (lane % (64 / QR));
    const bool nvalid = n0 < N;                  // N % 4 == 0
    const int nc = nvalid ? n0 : N - 4;
    auto group_of = [&](int i) { return kb * NG + kGemvWaves * i + wave; };   // i-th group of this wave

    struct Buf {
        u32x4 cw[RL];
        floatx4 dsc;
        uint32_t zw;
    };
    Buf b0, b1;
    auto issue = [&](int i, Buf& b) {
        const int gg = min(group_of(i), n_groups - 1);
        const uint32_t* cbase = codes + ((int64_t)gg * R + rq) * N + nc;
#pragma unroll
        for (int r = 0; r < RL; ++r)   // read once: streaming (non-temporal) loads
            b.cw[r] = __builtin_nontemporal_load((const u32x4*)(cbase + (int64_t)(QR * r) * N));
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
        if constexpr (QR == 4) {
            // one matrix-core product per column of the quadruple and group of four code rows; the
            // operand pairs are formed in C so that the compiler inserts the VALU -> MFMA waits
            floatx4 dm[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) dm[c] = floatx4{0.f, 0.f, 0.f, 0.f};
            const bool row0 = (lane & 15) == 0;
            // the mask in a vector register, so that each pair is one v_and_or_b32 (a VOP3 takes no
            // literal; with the mask as a literal the compiler splits it into an and and an or)
            uint32_t nibv;
            asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(nibv));
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                const u32x4 a = *(row0 ? (const u32x4*)&xpair[slot][4 * (QR * r + rq)] : &zpad);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = b.cw[r][c];
                    const u32x4 bo = u32x4{(w & nibv) | bf128, ((w >> 4) & nibv) | bf128, ((w >> 8) & nibv) | bf128,
                                           ((w >> 12) & nibv) | bf128};
                    dm[c] = mfma16x16x32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bo), dm[c]);
                }
            }
            // row 0 of the result: lanes 0-15 (rq = 0), element 0; the other lanes hold zeros and
            // write nothing
#pragma unroll
            for (int c = 0; c < 4; ++c) d[c] = dm[c][0];
        } else {
            // QR = 1: lane l holds code row r of columns 4l + c; row 4g of A carries x' of that code
            // row in k-slot group g (lanes 0, 20, 40, 60), so element 0 of lane l's result is the
            // dot product for its own column 4l + c
            floatx4 dm[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) dm[c] = floatx4{0.f, 0.f, 0.f, 0.f};
            const bool diag = (lane & 15) == ((lane >> 4) << 2);
            uint32_t nibv;
            asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(nibv));
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                const u32x4 a = *(diag ? (const u32x4*)&xpair[slot][4 * r] : &zpad);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = b.cw[r][c];
                    const u32x4 bo = u32x4{(w & nibv) | bf128, ((w >> 4) & nibv) | bf128, ((w >> 8) & nibv) | bf128,
                                           ((w >> 12) & nibv) | bf128};
                    dm[c] = mfma16x16x32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bo), dm[c]);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) d[c] = dm[c][0];
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
    if (wave > 0) red[wave - 1][lane] = floatx4{acc[0], acc[1], acc[2], acc[3]};
    __syncthreads();
    if (wave > 0) return;
    // wavefront 0, lane l: columns n0 .. n0 + 3 of the block
    const floatx4 v = ((floatx4{acc[0], acc[1], acc[2], acc[3]} + red[0][lane]) + red[1][lane]) + red[2][lane];
    const bool own = nvalid && rq == 0;          // QR = 4: only lanes 0-15 hold the sums
    if (nkb == 1) {
        if (own) *(uint2*)(Y + n0) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        return;
    }
    const uint32_t pbytes = (uint32_t)((int64_t)nkb * N * 4);
    const __amdgpu_buffer_rsrc_t pr = rsrc(part, pbytes);
    if (own) store4_agent(pr, (uint32_t)(((int64_t)kb * N + n0) * 4), v);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's partial has landed
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt + (int64_t)cb * cstride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)(nkb - 1)) return;
    // last arrival: the nkb partials of these columns in K-block order (loads of partials beyond
    // nkb fall outside the resource and read zeros, so every load is issued unconditionally)
    floatx4 t = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < nkb; b0 += 16) {
        floatx4 p[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            p[u] = load4_agent(pr, rq == 0 ? (uint32_t)(((int64_t)(b0 + u) * N + n0) * 4) : pbytes);
#pragma unroll
        for (int u = 0; u < 16; ++u) t += p[u];
    }
    if (own) *(uint2*)(Y + n0) = uint2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
    if (lane == 0) __hip_atomic_store(cnt + (int64_t)cb * cstride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    uint32_t* cnt = (uint32_t*)(base + p.off_cnt);
    // row blocks along x (up to 2^31 - 1), 256-channel blocks along y (K <= 16.7M)
    k_prep_x<G><<<dim3((unsigned)(p.mpad / 16), (unsigned)((K + 255) / 256)), 256, 0, st>>>(X, M, K, s, p.mpad, Xp, Sg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, (unsigned)p.grid_z);
    if (p.variant == 1)
        k_w4a16_mma<G, 1><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part, cnt, p.cstride);
    else if (p.variant == 2)
        k_w4a16_mma<G, 2><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part, cnt, p.cstride);
    else
        k_w4a16_mma_lds<G><<<grid, 256, 0, st>>>(Xp, Sg, p.mpad, M, codes, scales, zeros, K, N, Y, part, cnt, p.cstride);
    return hipGetLastError();
}
}  // namespace

// Arrival counters of different output tiles sit on different 128-byte lines when the counter
// region holds them that way, so that the atomics of different tiles are not serialized on one line.
namespace {
int counter_stride(int64_t n_counters) {
    const int64_t words = (int64_t)(kGemmCounterBytes / sizeof(uint32_t));
    return (int)std::max<int64_t>(1, std::min<int64_t>(32, words / std::max<int64_t>(n_counters, 1)));
}
}  // namespace

// Every layout keeps the first kGemmCounterBytes of the workspace for the arrival counters of the
// split-K products and puts its data after them, so the counters (zero between calls) survive calls
// of any shape that share one workspace.
GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int group_size) {
    GemmPlan p{};
    const int64_t n_groups = K / group_size;
    if (M == 1) {
        // halve the rows a wavefront takes (down to 32) until there are ~1536 workgroups (about
        // six per CU, so the last ones to finish leave little of the GPU idle), as long as the K
        // split stays within AWQ_GEMV_MAX_KSPLIT: the arrivals of one column block's K blocks at
        // its counter are serialized; beyond that, each wavefront takes 4 slices
        p.variant = 0;
        p.grid_x = (N + kGemvCols - 1) / kGemvCols;
        int64_t vg = group_size, gpw = 1;
        while (vg > 32 && p.grid_x * (K / vg) / kGemvWaves < 1536 && K / (vg / 2) / kGemvWaves <= AWQ_GEMV_MAX_KSPLIT)
            vg /= 2;
        if ((K / vg + kGemvWaves - 1) / kGemvWaves > AWQ_GEMV_MAX_KSPLIT) gpw = 4;   // (two slices spill registers)
        p.vgroup = (int)vg;
        p.gpw = (int)gpw;
        p.grid_y = (K / vg + kGemvWaves * gpw - 1) / (kGemvWaves * gpw);
        // several slices per wavefront (long K): 64 columns per workgroup instead of 256, four times
        // as many workgroups with the same K split (measured on K = 28672: 32-33 against 35-36 us),
        // while the column blocks' counters fit their region.  Narrow layers (fewer than ~1536
        // workgroups of 256 columns) also take 64 columns per workgroup, with the first of one slice
        // of G rows, four slices of G/2 or four of G per wavefront that leaves at most 1280
        // workgroups (on K = 8192: N = 1024 5.6 against 7.1 us, N = 8192 10.8 against 11.7 us,
        // N = 10240 12.3 against 13.3 us); wide layers keep 256 columns
        p.qr = 1;
        const int64_t blocks64 = (N + 63) / 64;
        const bool fit64 = blocks64 <= (int64_t)(kGemmCounterBytes / sizeof(uint32_t));
        if (gpw > 1 && fit64) {
            p.qr = 4;
            p.grid_x = blocks64;
        } else if (fit64 && p.grid_x * p.grid_y < 1536) {
            const int64_t opts[3][2] = {{1, group_size}, {4, std::max(group_size / 2, 32)}, {4, group_size}};
            gpw = 4;
            vg = group_size;
            for (const auto& o : opts) {
                const int64_t kb = (K / o[1] + kGemvWaves * o[0] - 1) / (kGemvWaves * o[0]);
                if (kb <= AWQ_GEMV_MAX_KSPLIT && blocks64 * kb <= 1280) {
                    gpw = o[0];
                    vg = o[1];
                    break;
                }
            }
            p.vgroup = (int)vg;
            p.gpw = (int)gpw;
            p.grid_y = (K / vg + kGemvWaves * gpw - 1) / (kGemvWaves * gpw);
            p.qr = 4;
            p.grid_x = blocks64;
        }
        p.grid_z = 1;
        p.ksplit = (int)p.grid_y;
        p.cstride = counter_stride(p.grid_x);
        p.mpad = 1;
        p.off_cnt = 0;
        p.off_part = kGemmCounterBytes;
        p.ws_bytes = p.grid_y > 1 ? kGemmCounterBytes + align256((size_t)p.grid_y * N * sizeof(float)) : 0;
        return p;
    }
    // 2..32 rows: 16 or 32 rows x 64 columns per workgroup, its wavefronts splitting the groups of
    // K (k_w4a16_mma); more rows: 64 rows x 256 columns, x' shared through LDS (k_w4a16_mma_lds),
    // which addresses x' and its sums through buffer resources (32-bit byte offsets)
    const int mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    const int64_t rows = 16 * mb;
    p.mpad = (M + rows - 1) / rows * rows;
    const bool lds_ok = p.mpad * K * (int64_t)sizeof(uint16_t) < ((int64_t)1 << 32) &&
                        n_groups * p.mpad * (int64_t)sizeof(float) < ((int64_t)1 << 32);
    if (mb == 4 && !lds_ok) {
        p.variant = -1;   // unsupported size
        return p;
    }
    p.variant = mb == 4 ? 5 : mb;
    p.grid_x = p.variant == 5 ? (N + 255) / 256 : (N + 63) / 64;
    p.grid_y = p.mpad / rows;
    // split K across workgroups, keeping enough groups per workgroup, at most 8 K blocks per tile
    // (the last arrival reads a partial of the whole row tile per K block; 8 measured 1-2 us faster
    // than 16 on the narrow layers) and the partials within the 32-bit byte range of a buffer
    // resource: 2..32 rows until about one workgroup per CU (fewer, longer workgroups: the partials'
    // traffic and the arrival tail grow with the split; on the 70B-shaped block at M = 16, 256
    // workgroups measured 2-3% faster than 512 or 768), more rows until ~512 workgroups are in
    // flight (2 per CU).  Tiles < 512 whenever K is split, so the arrival counters of the tiles fit
    // their region.
    const int64_t tiles = p.grid_x * p.grid_y;
    int64_t ks = 1;
    const bool skinny = p.variant != 5;
    const int64_t min_groups = skinny ? 4 : 2;   // one per wavefront and one prefetched, or two
    auto wider = [&](int64_t k) { return skinny ? tiles * 2 * k <= kGemmSkinnyWorkgroups : tiles * k < 512; };
    while (wider(ks) && 2 * ks * min_groups <= n_groups && 2 * ks <= 8 && 2 * ks * M * N < ((int64_t)1 << 30))
        ks *= 2;
    p.grid_z = ks;
    p.ksplit = (int)ks;
    p.cstride = counter_stride(tiles);
    p.off_cnt = 0;
    size_t off = kGemmCounterBytes;   // the counter region is never used for data
    p.off_part = off; off = align256(off + (ks > 1 ? (size_t)ks * M * N * sizeof(float) : 0));
    p.off_xp = off;   off = align256(off + (size_t)p.mpad * K * sizeof(uint16_t));
    p.off_sg = off;   off = align256(off + (size_t)n_groups * p.mpad * sizeof(float));
    p.ws_bytes = off;
    return p;
}

namespace {
template <int G, int VG>
void launch_gemv(const uint16_t* X, const float* s, const uint32_t* codes, const float* scales, const uint8_t* zeros,
                 int64_t K, int64_t N, uint16_t* Y, float* part, uint32_t* cnt, const GemmPlan& p, hipStream_t st) {
    dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y);
    if (p.qr == 1 && p.gpw == 1)
        k_w4a16_gemv<G, VG, 1, 1><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part, cnt, p.cstride);
    else if (p.qr == 1)
        k_w4a16_gemv<G, VG, 4, 1><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part, cnt, p.cstride);
    else if (p.gpw == 1)
        k_w4a16_gemv<G, VG, 1, 4><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part, cnt, p.cstride);
    else
        k_w4a16_gemv<G, VG, 4, 4><<<grid, 256, 0, st>>>(X, s, codes, scales, zeros, (int)K, (int)N, Y, part, cnt, p.cstride);
}
}  // namespace

hipError_t launch_gemm(const uint16_t* X, int64_t M, const float* s, const uint32_t* codes,
                       const float* scales, const uint8_t* zeros, int64_t K, int64_t N, int group_size,
                       uint16_t* Y, void* ws, const GemmPlan& p, hipStream_t st) {
    if (p.variant == 0) {
        float* part = p.grid_y > 1 ? (float*)((char*)ws + p.off_part) : nullptr;
        uint32_t* cnt = p.grid_y > 1 ? (uint32_t*)((char*)ws + p.off_cnt) : nullptr;
        const int vg = p.vgroup;
        if (group_size == 32)
            launch_gemv<32, 32>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        else if (group_size == 64 && vg == 64)
            launch_gemv<64, 64>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        else if (group_size == 64)
            launch_gemv<64, 32>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        else if (vg == 128)
            launch_gemv<128, 128>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        else if (vg == 64)
            launch_gemv<128, 64>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        else
            launch_gemv<128, 32>(X, s, codes, scales, zeros, K, N, Y, part, cnt, p, st);
        return hipGetLastError();
    }
    if (group_size == 32) return launch_mma<32>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    if (group_size == 64) return launch_mma<64>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    if (group_size == 128) return launch_mma<128>(X, M, s, codes, scales, zeros, K, N, Y, ws, p, st);
    return hipErrorInvalidValue;
}

}  // namespace awq
