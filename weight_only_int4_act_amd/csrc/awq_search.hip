// a3 + a4: the per-layer scale search.
//
// For every alpha_i of the grid the search forms s_i = m^alpha_i, group-quantizes diag(s_i) W,
// dequantizes, divides by s_i and scores L_i = ||X (S_i^-1 Q(S_i W) - W)||^2, then keeps the
// first minimum.  Sources: "AWQ (Activation-aware Weight Quantization)", section
// 缩放因子优化的完整流程 steps 3-6, and the error analysis of section AWQ 的缩放如何改变量化误差
// (Delta Y = X S^-1 eps_SW); "量化推理算法 GPTQ / AWQ", 4.3 (grid loop keeping a loss only when
// strictly smaller).
//
// Work per layer is n_grid * 2*T*K*N flops of X.E_i products (one calibration GEMM per alpha).
// Design (one fused kernel, no output matrix is ever written):
//   * A workgroup owns BM token rows x 16 output columns x NA consecutive alphas.
//   * K is walked one quantization group (G rows of W) at a time.  For the next group, each of
//     NA wavefronts quantizes and dequantizes the 16-column group tile for one alpha entirely in
//     registers: lane (column n, quad q) holds G/4 of the column's G values; the group max/min
//     (or max|p|) is an in-register max3/min3 reduction plus two cross-lane steps.  The error
//     tile E_i = (q*Delta - s*w)/s is rounded to bf16 and written to LDS directly in the
//     matrix-core operand layout (double buffered, one barrier per group).
//   * Every wavefront keeps the bf16 X fragments of its rows for the current group in registers
//     (read from a tiled copy of X, one group ahead) and reuses them for all NA alphas:
//     acc[alpha][row block] += X_chunk . E_alpha_chunk on v_mfma_f32_16x16x32_bf16.
//   * The inputs of the E computation (bf16 W tile, scale and reciprocal rows) reach LDS by
//     direct global->LDS transfers, three groups in flight.
//   * Epilogue: sum of squares of the float32 accumulators, reduced in a fixed order to one
//     float64 partial per (token tile, column tile, alpha).  A second kernel sums the partials
//     in a fixed order and a third picks the first minimum.
//   * Tile order is XCD-aware: the workgroups that run together on one XCD share a token tile,
//     so that XCD's L2 serves the X panel to all of them.  Successive waves of workgroups on an
//     XCD walk K in opposite directions, so each starts on the part of the panel the previous one
//     left in L2, and the W tile (read by one column block's alpha slices only) streams through
//     L2 with the non-temporal hint.
// The quantizer inside the search is the float32 evaluation of the packing quantizer of
// awq_pack (which evaluates it exactly in float64); the two differ only for elements whose
// pre-round value lies within float32 rounding of a .5 boundary.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Matrix-core operand layout used throughout (v_mfma_f32_16x16x32_bf16):
//   A (16 x 32): lane l holds row l%16 and 8 consecutive k of quad l/16
//   B (32 x 16): lane l holds column l%16 and the same 8 k of quad l/16
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. +3
// A K chunk is 32 input channels; a group of G channels is G/32 chunks.  Which 8 channels quad q
// of chunk c holds is a permutation internal to the kernel (the sum over k does not depend on
// it), chosen so that one X row's channels are read as whole 128-byte lines: for G >= 64, chunks
// pair up and quad q of chunk c holds k = 64*(c/2) + 16*q + 8*(c%2) + e, so the four lanes of a
// row read 2 x 64 contiguous bytes with two back-to-back loads.  For G = 32 (one chunk per group)
// quad q holds k = 8*q + e.  The W tiling, the scale rows and the X loads use the same map.
template <int G>
__device__ __forceinline__ int kmap(int c, int q) {
    if constexpr (G >= 64) return 64 * (c >> 1) + 16 * q + 8 * (c & 1);
    else return 8 * q;
}

// W [K, N] bf16 -> Wt (bf16, matrix-core B order): for column block nb (16 columns), chunk kc (32
// channels) and lane l, the 8 values W[G*(kc/C) + kmap(kc%C, l/16) + e][16*nb + l%16], e < 8, as one
// 16-byte word (value e in the low half of 32-bit word e/2 when e is even, in the high half when
// odd), stored at Wt[(nb*kchunks + kc)*64 + l], so that a lane reads its 8 values of a chunk as one
// linear 16-byte word.  Columns beyond N are zero (a zero column quantizes to zero error).
// A workgroup takes one group of rows (G) and 64 columns (4 column blocks): it reads the tile with
// 16-byte loads along the rows (each row's 64 columns are one 128-byte line; 2-byte loads with
// bounds checks where the tile reaches past N or the rows are not 16-byte aligned), transposes it
// through LDS (column-major, rows padded so that 8 consecutive rows of a column are one aligned
// 16-byte read) and writes each column block's C KB of the group as contiguous 16-byte stores.
template <int G>
__global__ __launch_bounds__(256) void k_tile_w(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                int vec, u32x4* __restrict__ Wt) {
    constexpr int C = G / 32;
    constexpr int LD = G + 8;                    // LDS row pitch of a column, in bf16
    __shared__ __align__(16) uint16_t t[64 * LD];
    lds_poison_start(&t[0], 64 * LD);
    const int64_t n_groups = K / G, kchunks = K / 32, nblocks = (N + 15) / 16;
    const int64_t j = (int64_t)blockIdx.x % n_groups;     // group (fastest: a column block's
    const int64_t c0 = (int64_t)blockIdx.x / n_groups * 64;   // output is written in order)
    const int tid = threadIdx.x;
    const bool full = vec && c0 + 64 <= N;
#pragma unroll
    for (int pass = 0; pass < C; ++pass) {
        const int r = pass * 32 + tid / 8, cs = 8 * (tid % 8);
        const uint16_t* src = W + (j * G + r) * N + c0 + cs;
        uint16_t v[8];
        if (full) {
            const u32x4 w = *(const u32x4*)src;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = (uint16_t)(w[e] & 0xffffu);
                v[2 * e + 1] = (uint16_t)(w[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = c0 + cs + e < N ? src[e] : (uint16_t)0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) t[(cs + e) * LD + r] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int idx = tid + 256 * i;           // (column block cb, chunk c, lane), lane fastest
        const int lane = idx & 63, c = (idx >> 6) % C, cb = (idx >> 6) / C;
        const int64_t nb = c0 / 16 + cb;
        if (nb >= nblocks) continue;
        const int col = cb * 16 + (lane & 15);
        const u32x4 w = *(const u32x4*)&t[col * LD + kmap<G>(c, lane >> 4)];
        Wt[(nb * kchunks + j * C + c) * 64 + lane] = w;
    }
}

// X [T, K] bf16 -> Xt: for 16-row block R, chunk kc and lane l, the 16 bytes lane l feeds to the
// matrix core as A operand: X[16R + l%16][G*(kc/C) + kmap(kc%C, l/16) + e], e < 8, stored at
// Xt[(R*kchunks + kc)*64 + l].  Rows >= T are zero.  In this order every X fragment the search
// loads is one contiguous 1 KB block (8 whole cache lines); read in place, a fragment touches 16
// lines and uses half of each, which halves the rate at which the memory pipeline delivers X.
template <int G>
__global__ __launch_bounds__(256) void k_tile_x(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                                                int64_t total, u32x4* __restrict__ Xt) {
    constexpr int C = G / 32;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // one (R, kc, lane)
    if (e >= total) return;
    const int lane = (int)(e & 63);
    const int64_t rest = e >> 6;
    const int64_t kchunks = K / 32;
    const int64_t kc = rest % kchunks, R = rest / kchunks;
    const int64_t row = R * 16 + (lane & 15);
    const int64_t k0 = (kc / C) * G + kmap<G>((int)(kc % C), lane >> 4);
    Xt[e] = row < T ? *(const u32x4*)(X + row * K + k0) : u32x4{0u, 0u, 0u, 0u};
}

// Three-input max/min (one VALU instruction each; the inputs are never NaN).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float min3f(float a, float b, float c) {
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// max(-a, -b, -c) = -min(a, b, c), with the negations as free source modifiers.
__device__ __forceinline__ float nmax3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, -%1, -%2, -%3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float nmaxf(float a, float b) {
    float r;
    asm("v_max_f32 %0, -%1, -%2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// max of two values that come out of lane swaps as raw bits (fmaxf would first canonicalize both).
__device__ __forceinline__ float maxraw(uint32_t a, uint32_t b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// Reductions over the four lanes l, l^16, l^32, l^48 (the four quads of one column) with the
// gfx950 lane-swap instructions.  v_permlane32_swap exchanges the upper 32 lanes of its first
// operand with the lower 32 lanes of its second; v_permlane16_swap exchanges the odd 16-lane rows
// of its first operand with the even rows of its second.
// quad_max: every lane ends with the maximum of v over its column.
__device__ __forceinline__ float quad_max(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = maxraw(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return maxraw(b[0], b[1]);
}
// quad_max2: both maxima of (x, y) over the column in one network.  The first swap pairs x of
// lanes l, l+32 in the lower half and y of lanes l-32, l in the upper half; after the row swap the
// lower half holds the column maximum of x and the upper half that of y; the last swap hands each
// lane both.
__device__ __forceinline__ void quad_max2(float& x, float& y) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float t = maxraw(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    const float u = maxraw(b[0], b[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(u), false, false);
    x = __uint_as_float(c[0]);
    y = __uint_as_float(c[1]);
}

// LDS-only workgroup barrier.  Every cross-wavefront exchange in the search goes through ds_write
// (E tiles and staged E inputs), so waiting for this wavefront's LDS operations is enough; the
// X fragments that are in flight towards LDS are private to their wavefront and are waited for
// with counted vmcnt waits at their use, so the barrier must not drain them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Buffer resource (V#) of a raw byte range: base address, no stride, num_records bytes (accesses at
// or beyond it return zero), and the gfx9 word 3 for untyped 32-bit data.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 byte_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff, (int)bytes, 0x00020000};
}

// Direct buffer -> LDS transfer of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l's bytes
// (at byte offset voff of the resource) land at LDS address `lds + 16*l`.  Issued from inline asm
// so that the compiler does not track it: every wait for these transfers is an explicit, counted
// s_waitcnt vmcnt(N) (vmcnt counts vector-memory operations that complete in issue order).  M0
// carries the LDS base; it is saved and restored around the transfer, and one wait state
// separates the M0 write from its use.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
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
// The same with the non-temporal hint: the lines it brings into L2 are the first to be replaced.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "memory");
}
// Lane J of each 16-lane row of v, for every lane of that row (DPP row_newbcast, folded by the
// compiler into the consuming VALU instruction as a source modifier).
template <int J>
__device__ __forceinline__ float rowbcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xf, 0xf, true));
}

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// CLIP: the quantizer's group range is clipped by the ratio clip_tab[i] of grid point i (both ends
// scaled, codes clamped to the 16 levels); without it the range is the group's own.
template <int G, int NA, int RBW, int NW, bool ZP, bool CLIP>
__global__ __launch_bounds__(NW * 64, 1) void k_search(
    const u32x4* __restrict__ Xt, int T, int K, const u32x4* __restrict__ Wt, int NB,
    const float* __restrict__ s_tab, const float* __restrict__ inv_tab, const float* __restrict__ clip_tab,
    uint32_t stage_bytes, int n_grid, int n_asplit, int n_tiles, int tiles_per_xcd, double* __restrict__ partials) {
    constexpr int C = G / 32;            // K chunks per group
    constexpr int BM = NW * RBW * 16;    // token rows per workgroup
    constexpr int NWE = C * 64;          // 16-byte W entries of a group tile (bf16)
    constexpr int NSE = NA * G / 4;      // 16-byte entries of NA scale rows of one group
    constexpr int SPAD = 2;              // entries between scale and reciprocal rows (LDS banks)
    constexpr int NSTG = NWE + 2 * NSE + SPAD;   // staged 16-byte entries per group
    constexpr int NT = (NSTG + NW * 64 - 1) / (NW * 64);   // staging transfers per thread and group
    constexpr int NSTGP = NT * NW * 64;  // staging entries incl. padding
    static_assert(NW == 8 && NA < NW && NA >= NW / 2 && NT <= 2, "tile shape");   // waves 0-3 always own a slot

    const int tile = xcd_tile(blockIdx.x, tiles_per_xcd);
    if (tile >= n_tiles) return;
    const int asplit = tile % n_asplit;
    const int rest = tile / n_asplit;
    const int nb = rest % NB;
    const int tb = rest / NB;
    const int a0 = asplit * NA;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane >> 4, r16 = lane & 15;
    const int n_groups = K / G;
    const int kchunks = K / 32;
    // K order: the workgroups of one XCD run in waves of one per CU; every other wave walks the
    // groups from the last to the first, so that it starts on the X panel the previous wave left in
    // that XCD's L2.  The sum over K is the same up to float32 rounding order.
    const bool rev = ((blockIdx.x / kNumXcd) / kCusPerXcd) & 1;

    // E tiles (bf16, B-operand layout), double buffered over groups.
    __shared__ u32x4 Es[2][NA][C][64];
    // Staged inputs of the E computation of one group, four groups deep (group g in Stg[g % 4]): the
    // W tile (bf16, in B-operand order), then NA scale rows, then NA reciprocal rows (16-byte
    // entries).
    __shared__ u32x4 Stg[4][NSTGP];
    __shared__ double red[NW][NA];

    floatx4 acc[NA][RBW];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) acc[a][rb] = floatx4{0.f, 0.f, 0.f, 0.f};

    // X fragments of this wavefront's rows (RBW row blocks) for a few K chunks, held in register
    // slots.  With 4 chunks per group there are 3 slots: chunks 0, 1, 2, 3 use slots 0, 1, 2, 0.
    // The matrix-core half of group jg loads chunk 2 at its start, chunk 3 after chunk 0, chunk 1 of
    // group jg + 1 after chunk 1 and chunk 0 of group jg + 1 after chunk 3, so every load has at
    // least two chunks of matrix-core work (or the E half) to arrive while only two slots are live
    // during the E half.  With 1 or 2 chunks per group the slots form a ring: chunk c's slot receives
    // chunk c + XD once its products have been issued.  Each load is one contiguous 1 KB block of
    // the tiled X.
    // The token tile's fragments form one contiguous range of (BM/16) * kchunks KB; a load takes
    // this lane's byte offset in a vector register and the row block and chunk as a scalar offset.
    const auto xrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Xt + (int64_t)tb * (BM / 16) * kchunks * 64), 0,
                                                         (BM / 16) * kchunks * 1024, 0x00020000);
    const uint32_t xvoff = ((uint32_t)(wave * RBW) * kchunks * 64 + lane) * 16;
    constexpr int XD = C >= 4 ? 3 : C >= 2 ? 2 : 1;
    constexpr bool X3 = C == 4;
    auto xslot = [](int c) { return X3 ? (c == 3 ? 0 : c) : c % XD; };
    u32x4 xr[XD][RBW];
    // chunk c (compile-time, < C) of group g (counted in this workgroup's K order, clamped to the
    // last group) into ring slot `slot`: the group and row block in the scalar offset, the chunk in
    // the instruction's immediate field.
    auto load_X = [&](int g, int c, int slot) {
        g = min(g, n_groups - 1);
        const uint32_t goff = (uint32_t)(rev ? n_groups - 1 - g : g) * (C * 1024);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
            xr[slot][rb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         xrsrc, xvoff + c * 1024, goff + (uint32_t)(rb * kchunks) * 1024, 0));
    };

    // ---- staging of the E inputs of group jg: entry e (thread t copies e = t + 512 r, r < NT
    // transfers) is a 16-byte piece of the W tile, of a scale row or of a reciprocal row.  SPAD
    // entries between the scale and the reciprocal rows shift the latter by 8 LDS banks (they hold
    // a copy of the first scale entry), and the entries past NSTG re-read the last valid entry.
    // The scale table, its reciprocals and the W tiles lie in one range of the workspace that
    // starts at s_tab (stage_bytes long, checked below 4 GB by the host); a transfer's source is a
    // byte offset in it that advances by a fixed step per group.
    const i32x4 srsrc = byte_rsrc(s_tab, stage_bytes);
    uint32_t stg_off[NT], stg_step[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r) {
        const int e = min((int)threadIdx.x + NW * 64 * r, NSTG - 1);
        const int es = e - NWE;
        const int which = es >= NSE + SPAD;              // 0: scale row (or padding), 1: reciprocal row
        const int idx = which ? es - NSE - SPAD : (es < NSE ? es : 0);
        const int a = idx / (G / 4), off = (idx % (G / 4)) * 4;
        const char* src;
        if (e < NWE) {
            src = (const char*)(Wt + (int64_t)nb * kchunks * 64 + e);
            stg_step[r] = (uint32_t)(C * 64 * sizeof(u32x4));
        } else {
            src = (const char*)((which ? inv_tab : s_tab) + (int64_t)min(a0 + a, n_grid - 1) * K + off);
            stg_step[r] = (uint32_t)(G * sizeof(float));
        }
        stg_off[r] = (uint32_t)(src - (const char*)s_tab);
    }
    const uint32_t stg_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&Stg[0][0]) +
                             (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64 * 16;
    // NTW: this wavefront's first transfer is a W tile piece (with G = 128 the W tile is exactly
    // the first transfer of wavefronts 0-3), issued with the non-temporal hint: the W tile is read by
    // the few workgroups of its column block only, so it streams through L2 and leaves it to the X
    // panel, which the other workgroups of the XCD re-read.
    auto stage = [&](auto ntw_tag, int jg, int buf) {   // jg counted in this workgroup's K order
        constexpr bool NTW = decltype(ntw_tag)::value;
        const uint32_t jp = (uint32_t)(rev ? n_groups - 1 - jg : jg);
#pragma unroll
        for (int r = 0; r < NT; ++r) {
            const uint32_t src = stg_off[r] + jp * stg_step[r];
            const uint32_t dst = stg_lds + (uint32_t)(buf * NSTGP + NW * 64 * r) * 16;
            if (NTW && r == 0) dma16_nt(srsrc, src, dst);
            else dma16(srsrc, src, dst);
        }
    };

    // ---- E tile of the group staged in Stg[ibuf], for alpha slot `slot`, into Es[ebuf][slot].
    // Lane (column r16, quad q) owns the G/4 values of its column in the quad's k positions of each
    // chunk: p = s*w, the group max/min (in registers, then across the 4 lanes of the column), the
    // step and zero, then per value: quantize, dequantize, subtract, unscale, round to bf16.
    const int slot = min(wave, NA - 1);
    float crat = 1.f;   // clip ratio of this wavefront's grid point (CLIP only)
    if constexpr (CLIP) crat = clip_tab[min(a0 + slot, n_grid - 1)];
    // E tile of the group staged in Stg[ibuf], for alpha slot `slot`, into Es[ebuf][slot].  The
    // level is rint(p/Delta) without the clamp to the code range: with Delta and the zero taken
    // from the group's own max and min, the level leaves the range only when p/Delta lies at a .5
    // tie at one end of the range, where either neighbour is an equally near rounding (error
    // +-Delta/2).  Like every tie the float32 evaluation meets, it may be taken the other way than
    // the exact quantizer takes it: the sign of that element's error then differs, which moves the
    // loss through its cross terms (percents on a layer of a few outputs, nothing measurable on
    // real ones).  The packing kernel applies the quantizer exactly, clamp included.
    // The staged inputs are read two chunks ahead of their use, so that LDS latency overlaps the
    // arithmetic of the previous chunk.  The scale and reciprocal values of a chunk depend only on
    // the row, and the 16 lanes of a quad (one 16-lane DPP row) need the same 8 rows: lane 16q + j
    // reads the scale (j < 8) or the reciprocal (j >= 8) of row kmap(c, q) + (j & 7) with one 4-byte
    // LDS read, and each multiply takes lane j's value of its row as a row_newbcast:j source.
    const int srow = NWE + (slot * G) / 4;   // this slot's scale row (16-byte entries)
    const int sidx = (r16 < 8 ? srow * 4 : (srow + NSE + SPAD) * 4) + (r16 & 7) + kmap<G>(0, q);
    u32x4 in[2];                             // W values (bf16 pairs) of two chunks
    float sv[C];                             // per chunk: this lane's scale or reciprocal
    auto fetch_in = [&](int ibuf, int c) {
        const u32x4* st = &Stg[ibuf][0];
        in[c & 1] = st[c * 64 + lane];
        sv[c] = ((const float*)st)[sidx + kmap<G>(c, 0)];
    };
    // The first chunk's inputs are issued ahead of compute_E, inside a matrix-core half;
    // compute_E issues the rest, two chunks ahead.
    auto prefetch_E = [&](int ibuf) { fetch_in(ibuf, 0); };
    auto compute_E = [&](int ibuf, int ebuf, bool prefetched) {
        float pk[C * 8];
        // ZP: mx = max(p, 0) and nmn = -min(p, 0) (the group range always includes 0); else
        // mx = max |p|
        float mx = 0.f, nmn = 0.f;
        if (!prefetched) fetch_in(ibuf, 0);
        if constexpr (C > 1) fetch_in(ibuf, 1);
        float cmx[C], cmn[C];       // per-chunk range, combined below as a tree
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const u32x4 w = in[c & 1];
            float* v = &pk[c * 8];
            v[0] = rowbcast<0>(sv[c]) * bf16_lo(w[0]);
            v[1] = rowbcast<1>(sv[c]) * bf16_hi(w[0]);
            v[2] = rowbcast<2>(sv[c]) * bf16_lo(w[1]);
            v[3] = rowbcast<3>(sv[c]) * bf16_hi(w[1]);
            v[4] = rowbcast<4>(sv[c]) * bf16_lo(w[2]);
            v[5] = rowbcast<5>(sv[c]) * bf16_hi(w[2]);
            v[6] = rowbcast<6>(sv[c]) * bf16_lo(w[3]);
            v[7] = rowbcast<7>(sv[c]) * bf16_hi(w[3]);
            if (c + 2 < C) fetch_in(ibuf, c + 2);
            if (ZP) {
                cmx[c] = max3f(max3f(v[0], v[1], v[2]), max3f(v[3], v[4], v[5]), fmaxf(v[6], v[7]));
                cmn[c] = max3f(nmax3f(v[0], v[1], v[2]), nmax3f(v[3], v[4], v[5]), nmaxf(v[6], v[7]));
            } else {
                cmx[c] = max3f(max3f(fabsf(v[0]), fabsf(v[1]), fabsf(v[2])),
                               max3f(fabsf(v[3]), fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7])));
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            mx = fmaxf(mx, cmx[c]);
            if (ZP) nmn = fmaxf(nmn, cmn[c]);
        }
        float d;
        if (ZP) {
            quad_max2(mx, nmn);
            if constexpr (CLIP) {
                mx *= crat;
                nmn *= crat;
            }
            d = (mx + nmn) * (1.0f / 15.0f);
        } else {
            mx = quad_max(mx);
            if constexpr (CLIP) mx *= crat;
            d = mx * (1.0f / 7.0f);
        }
        // an all-zero group has d = 0 and every p = 0, so any finite reciprocal gives e = 0;
        // below FLT_MIN the step only meets values whose squares vanish in the loss
        d = fmaxf(d, 1.17549435e-38f);
        const float rd = __builtin_amdgcn_rcpf(d);
        // clipped range: levels clamp to [-zero, 15 - zero] (zero = rne(-min/Delta)) or [-7, 7]
        float llo = -7.f, lhi = 7.f;
        if constexpr (CLIP && ZP) {
            const float z = fminf(rintf(nmn * rd), 15.f);
            llo = -z;
            lhi = 15.f - z;
        }
        auto level = [&](float t) {
            const float l = rintf(t);
            if constexpr (CLIP) return __builtin_amdgcn_fmed3f(l, llo, lhi);
            else return l;
        };
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const float* v = &pk[c * 8];
            float e[8];   // (level*Delta - s*w) / s
            e[0] = fmaf(level(v[0] * rd), d, -v[0]) * rowbcast<8>(sv[c]);
            e[1] = fmaf(level(v[1] * rd), d, -v[1]) * rowbcast<9>(sv[c]);
            e[2] = fmaf(level(v[2] * rd), d, -v[2]) * rowbcast<10>(sv[c]);
            e[3] = fmaf(level(v[3] * rd), d, -v[3]) * rowbcast<11>(sv[c]);
            e[4] = fmaf(level(v[4] * rd), d, -v[4]) * rowbcast<12>(sv[c]);
            e[5] = fmaf(level(v[5] * rd), d, -v[5]) * rowbcast<13>(sv[c]);
            e[6] = fmaf(level(v[6] * rd), d, -v[6]) * rowbcast<14>(sv[c]);
            e[7] = fmaf(level(v[7] * rd), d, -v[7]) * rowbcast<15>(sv[c]);
            Es[ebuf][slot][c][lane] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                                pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
        }
    };

    // Matrix-core work of one group: for each chunk and alpha, the RBW products with this wavefront's
    // X fragments; the E fragment of an alpha for the next chunk is read from LDS as soon as the
    // current one has been consumed, and the chunk's X registers are reloaded XD chunks ahead as soon
    // as its products have been issued.
    // The staging transfers of a step are issued inside the matrix-core half, after chunk SC, where
    // their issue cost hides behind the matrix work; XS = X loads of the half issued before them.
    constexpr int SC = C >= 4 ? 1 : 0;
    constexpr int XS = (SC + 1 + (X3 ? 1 : 0)) * RBW;
    // PRE: after the products of alpha NA-2 in the last chunk (when the other alphas' E fragments
    // are dead), issue the LDS reads of the first inputs of an E computation (staged in Stg[pbuf]).
    auto mfma_group = [&](auto pre_tag, auto ntw_tag, int jg, int buf, int sjg, int sbuf, int pbuf) {
        constexpr bool PRE = decltype(pre_tag)::value;
        constexpr int PA = NA > 2 ? NA - 2 : 0;
        if constexpr (X3) load_X(jg, 2, 2);
        u32x4 B[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) B[a] = Es[buf][a][0][lane];
        if constexpr (X3) __builtin_amdgcn_sched_group_barrier(0x020, RBW, 0);      // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);                         // DS read
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int a = 0; a < NA; ++a) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
                    acc[a][rb] = mfma16x16x32(__builtin_bit_cast(bf16x8, xr[xslot(c)][rb]),
                                              __builtin_bit_cast(bf16x8, B[a]), acc[a][rb]);
                if (c + 1 < C) B[a] = Es[buf][a][c + 1 < C ? c + 1 : 0][lane];
                if (PRE && c == C - 1 && a == PA) prefetch_E(pbuf);
            }
            if constexpr (X3) {
                if (c == 0) load_X(jg, 3, 0);
                if (c == 1) load_X(jg + 1, 1, 1);
                if (c == 3) load_X(jg + 1, 0, 0);
            } else {
                load_X(jg + (c + XD) / C, (c + XD) % C, c % XD);
            }
            // issue order inside the chunk: per alpha, its RBW products then the next chunk's E
            // fragment read; the X reloads last.  Keeps one E fragment set and one X set live.
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                __builtin_amdgcn_sched_group_barrier(0x008, RBW, 0);   // MFMA
                if (c + 1 < C) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                if (PRE && c == C - 1 && a == PA)
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS read
            }
            if (!X3 || c != 2) __builtin_amdgcn_sched_group_barrier(0x020, RBW, 0);   // VMEM read
            __builtin_amdgcn_sched_barrier(0);
            if (c == SC) stage(ntw_tag, sjg, sbuf);
        }
    };

    // Debug build: NaN into this wavefront's share of a staging buffer (the entries its transfers
    // fill) and into its E tile slot, at the start of the step in which they are refilled
    auto poison_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < NT; ++r) Stg[buf][NW * 64 * r + wave * 64 + lane] = lds_nan16();
    };
    auto poison_E = [&](int ebuf) __attribute__((always_inline)) {
        if (wave < NA) {
#pragma unroll
            for (int c = 0; c < C; ++c) Es[ebuf][slot][c][lane] = lds_nan16();
        }
    };
    if constexpr (kLdsPoison) {
        if (lane == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) red[wave][a] = __builtin_nan("");
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) poison_stage(g);
        lds_write_fence();
    }

    // ---- prologue: the first X chunks in registers, inputs of groups 0-3 staged, E(0) computed.
#pragma unroll
    for (int c = 0; c < (X3 ? 2 : XD); ++c) load_X(c / C, c % C, c);
#pragma unroll
    for (int g = 0; g < 4; ++g) stage(Flag<false>{}, min(g, n_groups - 1), g);
    wait_vmcnt<0>();
    lds_barrier();
    if (wave < NA) compute_E(0, 0, false);   // the spare wavefront has no alpha slot
    lds_barrier();

    // Main loop.  The two wavefronts that share a SIMD (w and w + 4) run the two halves of a
    // group step in opposite order: wavefronts 0-3 issue their X.E(jg) matrix-core work first and
    // then compute their E(jg+1) tile; wavefronts 4-7 compute E(jg+1) first and then issue their
    // matrix-core work.  Both halves only read E(jg) and write E(jg+1), so the order is free, and
    // on every SIMD one wavefront keeps the matrix core busy while the other uses the VALU.
    // Inside its matrix-core half every wavefront also reads the first inputs of the next E tile it
    // computes: wavefronts 0-3 those of E(jg+1) (in Stg[(jg+1) % 4]) for the E half that follows,
    // wavefronts 4-7 those of E(jg+2) (in Stg[(jg+2) % 4]) for the start of the next step, so no
    // E half begins with an LDS wait.
    // Every wavefront issues stage(jg + 4) [NT transfers] inside its matrix-core half, which also
    // issues C*RBW X loads (the last chunk of group jg, then the other chunks of group jg + 1), XS
    // of them before the staging.  A staged buffer is filled by the transfers of all wavefronts, so
    // each wavefront waits for its own share of stage(jg + 3), issued in step jg - 1, right before
    // the barrier that ends step jg; it is read from step jg + 1 on (wavefronts 4-7 read the first
    // inputs of E(jg + 3) at the end of step jg + 1).  Vector-memory operations complete in issue
    // order, and after that staging a wavefront has issued the rest of that half (C*RBW - XS loads)
    // and one more matrix-core half (C*RBW + NT operations).  The compiler's own waits for the X
    // registers, which cannot see the staging transfers, wait at most for a staging issued one E
    // half earlier.  The prologue waited for stages 0-3.
    const bool mfma_first = (wave & 4) == 0;
    if (!mfma_first) prefetch_E(min(1, n_groups - 1) & 3);
    for (int jg = 0; jg < n_groups; ++jg) {
        const int buf = jg & 1;
        const int sb = jg & 3;                  // held group jg (consumed by E(jg)); refilled with jg + 4
        const int sbn = (jg + 1) & 3;           // group jg + 1
        const int sbn2 = (jg + 2) & 3;          // group jg + 2
        const int sjg = min(jg + 4, n_groups - 1);
        const bool next = jg + 1 < n_groups;   // the last step has no E tile to prepare
        if constexpr (kLdsPoison) {
            // Stg[sb] was last read by E(jg) in step jg - 1 and is refilled in this step; Es[buf ^ 1]
            // was last read in step jg - 1 and receives E(jg + 1) in this step
            poison_stage(sb);
            poison_E(buf ^ 1);
            lds_write_fence();
        }
        if (mfma_first) {
            mfma_group(Flag<true>{}, Flag<C == 4>{}, jg, buf, sjg, sb, sbn);
            if (next) compute_E(sbn, buf ^ 1, true);
        } else {
            // the spare wavefront (no alpha slot of its own) skips the E half
            if (wave < NA && next) compute_E(sbn, buf ^ 1, true);
            mfma_group(Flag<true>{}, Flag<false>{}, jg, buf, sjg, sb, sbn2);
        }
        wait_vmcnt<2 * C * RBW - XS + NT>();
        lds_barrier();
    }
    // drain the trailing (redundant) transfers before the LDS is reused or released
    wait_vmcnt<0>();

    // ---- epilogue: sum of squares per alpha over valid rows; fixed-order reductions.
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        float ss = 0.f;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tb * BM + (wave * RBW + rb) * 16 + 4 * q + i;
                const float v = row < T ? acc[a][rb][i] : 0.f;
                ss = fmaf(v, v, ss);
            }
        const double t = wave_sum((double)ss);
        if (lane == 0) red[wave][a] = t;
    }
    __syncthreads();
    if (threadIdx.x < NA && a0 + (int)threadIdx.x < n_grid) {
        double sum = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][threadIdx.x];
        partials[((int64_t)tb * NB + nb) * n_grid + a0 + threadIdx.x] = sum;
    }
}

// L[i] = sum over tiles of partials[tile][i]: one workgroup per alpha, strided fixed-order sums
// and a fixed tree.
__global__ __launch_bounds__(256) void k_reduce_losses(const double* __restrict__ partials, int64_t tiles,
                                                       int n_grid, double* __restrict__ losses) {
    __shared__ double sm[256];
    lds_poison_start(&sm[0], 256);
    const int i = blockIdx.x;
    double s = 0.0;
    for (int64_t t0 = threadIdx.x; t0 < tiles; t0 += 8 * 256) {   // 8 loads in flight, fixed order
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = t0 + 256 * j < tiles ? partials[(t0 + 256 * j) * n_grid + i] : 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[j];
    }
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) losses[i] = sm[0];
}

// L_j[i] = sum over the token tiles and the column tiles [nb0, nb1) of partials[tile][i] (one
// projection of a multi-matrix search): one workgroup per alpha, same fixed order as above.
__global__ __launch_bounds__(256) void k_reduce_losses_range(const double* __restrict__ partials, int64_t tb,
                                                             int64_t nb_total, int64_t nb0, int64_t nb1, int n_grid,
                                                             double* __restrict__ losses) {
    __shared__ double sm[256];
    lds_poison_start(&sm[0], 256);
    const int i = blockIdx.x;
    const int64_t w = nb1 - nb0, tiles = tb * w;
    double s = 0.0;
    for (int64_t t = threadIdx.x; t < tiles; t += 256) {
        const int64_t r = t / w, c = nb0 + t % w;
        s += partials[(r * nb_total + c) * n_grid + i];
    }
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) sm[threadIdx.x] += sm[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) losses[i] = sm[0];
}

// best = first index of the minimum loss; row = table[best] (K values: the scale row s_best of the
// alpha search; 1 value: the clip ratio of the clip search).
__global__ __launch_bounds__(256) void k_select(const double* __restrict__ losses, int n_grid,
                                                const float* __restrict__ table, int64_t K,
                                                int32_t* __restrict__ best, float* __restrict__ row) {
    __shared__ int b;
    if (threadIdx.x == 0) {
        int bi = 0;
        for (int i = 1; i < n_grid; ++i)
            if (losses[i] < losses[bi]) bi = i;
        b = bi;
        if (blockIdx.x == 0) *best = bi;
    }
    __syncthreads();
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < K; k += (int64_t)gridDim.x * 256)
        row[k] = table[(int64_t)b * K + k];
}

// Clip search: every grid row of the scale table is the fixed s (and its float32 reciprocal).
__global__ __launch_bounds__(256) void k_fixed_scale_rows(const float* __restrict__ s, int64_t K,
                                                          float* __restrict__ s_tab, float* __restrict__ inv_tab) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int j = blockIdx.y;
    if (k >= K) return;
    const float v = s[k];
    s_tab[(int64_t)j * K + k] = v;
    inv_tab[(int64_t)j * K + k] = 1.0f / v;
}

// A caller's table of candidate scale rows and their float32 reciprocals, into the workspace.
__global__ __launch_bounds__(256) void k_table_rows(const float* __restrict__ table, int64_t K,
                                                    float* __restrict__ s_tab, float* __restrict__ inv_tab) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int j = blockIdx.y;
    if (k >= K) return;
    const float v = table[(int64_t)j * K + k];
    s_tab[(int64_t)j * K + k] = v;
    inv_tab[(int64_t)j * K + k] = 1.0f / v;
}

struct ClipRatios {
    float c[kMaxGrid];
};
__global__ void k_write_clip(ClipRatios r, int n, float* __restrict__ tab) {
    if ((int)threadIdx.x < n) tab[threadIdx.x] = r.c[threadIdx.x];
}

namespace {

// Instantiations: (group size, zero point, clipping) x two tile shapes.  8 wavefronts (2 per SIMD),
// 7 alphas (or clip ratios) per workgroup (21 = 3 slices of 7), and RBW row blocks of 16 per
// wavefront: RBW = 5 (640 token rows, 140 accumulator VGPRs per lane) cuts the E work per product
// by a fifth against RBW = 4 (512 rows); the plan takes it unless padding the tokens to 640-row
// tiles costs more than that.
constexpr int kNA = 7, kNW = 8;

typedef void (*search_fn)(const u32x4*, int, int, const u32x4*, int, const float*, const float*, const float*,
                          uint32_t, int, int, int, int, double*);

template <int RBW, bool CLIP>
search_fn pick_rbw(int g, int zp) {
    if (zp) {
        if (g == 32) return k_search<32, kNA, RBW, kNW, true, CLIP>;
        if (g == 64) return k_search<64, kNA, RBW, kNW, true, CLIP>;
        if (g == 128) return k_search<128, kNA, RBW, kNW, true, CLIP>;
    } else {
        if (g == 32) return k_search<32, kNA, RBW, kNW, false, CLIP>;
        if (g == 64) return k_search<64, kNA, RBW, kNW, false, CLIP>;
        if (g == 128) return k_search<128, kNA, RBW, kNW, false, CLIP>;
    }
    return nullptr;
}

search_fn pick(int g, int zp, int rbw, bool clip) {
    if (clip) return rbw == 5 ? pick_rbw<5, true>(g, zp) : pick_rbw<4, true>(g, zp);
    return rbw == 5 ? pick_rbw<5, false>(g, zp) : pick_rbw<4, false>(g, zp);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

SearchPlan plan_search(int64_t T, int64_t K, int64_t N, int group_size, int zero_point, int n_grid, bool clip) {
    SearchPlan p{};
    p.group_size = group_size;
    p.n_grid = n_grid;
    p.zero_point = zero_point;
    // rows per workgroup: 640 (RBW = 5) unless its padding of T exceeds 512-row tiles' by more than
    // the ~4.5% it gains per row (measured on the 4096x4096 layer).  The workspace holds either
    // shape.
    const int64_t pad5 = (T + 639) / 640 * 640, pad4 = (T + 511) / 512 * 512;
    p.variant = pad5 * 1000 <= pad4 * 1045 ? 5 : 4;   // row blocks per wavefront
    const int64_t xt_rows = pad5 > pad4 ? pad5 : pad4;
    const int64_t max_tb = (T + 511) / 512;
    p.na = kNA;
    p.bm = p.variant * kNW * 16;
    p.n_asplit = (n_grid + kNA - 1) / kNA;
    p.nb = (N + 15) / 16;
    p.tb = (T + p.bm - 1) / p.bm;
    p.tiles = p.tb * p.nb * p.n_asplit;
    p.tiles_per_xcd = (p.tiles + kNumXcd - 1) / kNumXcd;
    p.grid = p.tiles_per_xcd * kNumXcd;
    size_t off = 0;
    p.off_s = off;    off = align256(off + (size_t)n_grid * K * sizeof(float));
    p.off_inv = off;  off = align256(off + (size_t)n_grid * K * sizeof(float));
    p.off_wt = off;   off = align256(off + (size_t)p.nb * 16 * K * sizeof(uint16_t));
    p.off_xt = off;   off = align256(off + (size_t)xt_rows * K * sizeof(uint16_t));
    p.off_part = off; off = align256(off + (size_t)max_tb * p.nb * n_grid * sizeof(double));
    p.off_clip = off; off = align256(off + (size_t)n_grid * sizeof(float));
    p.ws_bytes = off;
    return p;
}

namespace {

// W [K, N] into the tiled bf16 stream at column block nb0 (its padding columns are zero).
hipError_t tile_w(const uint16_t* W, int64_t K, int64_t N, const SearchPlan& p, void* ws, int64_t nb0,
                  hipStream_t st) {
    u32x4* Wt = (u32x4*)((char*)ws + p.off_wt) + nb0 * (K / 32) * 64;
    const unsigned tgrid = (unsigned)((N + 63) / 64 * (K / p.group_size));
    // 16-byte row loads need 16-byte aligned rows
    const int vec = N % 8 == 0 && ((uintptr_t)W & 15) == 0;
    if (p.group_size == 32) k_tile_w<32><<<tgrid, 256, 0, st>>>(W, K, N, vec, Wt);
    else if (p.group_size == 64) k_tile_w<64><<<tgrid, 256, 0, st>>>(W, K, N, vec, Wt);
    else k_tile_w<128><<<tgrid, 256, 0, st>>>(W, K, N, vec, Wt);
    return hipGetLastError();
}

// The common part of every search once the scale table, its reciprocals, (when clipping) the clip
// ratios of the grid and the W tiles are in the workspace: tile X, run the fused kernel, reduce the
// partials and pick the first minimum.
hipError_t run_search_tiled(const uint16_t* X, int64_t T, int64_t K, const SearchPlan& p, void* ws, bool clip,
                            double* losses, int32_t* best, const float* sel_table, int64_t sel_len, float* sel_row,
                            hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    u32x4* Wt = (u32x4*)(base + p.off_wt);
    u32x4* Xt = (u32x4*)(base + p.off_xt);
    double* part = (double*)(base + p.off_part);
    const float* clip_tab = (const float*)(base + p.off_clip);
    hipError_t e;
    const int64_t xtotal = p.tb * (p.bm / 16) * (K / 32) * 64;
    const unsigned xgrid = (unsigned)((xtotal + 255) / 256);
    if (p.group_size == 32) k_tile_x<32><<<xgrid, 256, 0, st>>>(X, T, K, xtotal, Xt);
    else if (p.group_size == 64) k_tile_x<64><<<xgrid, 256, 0, st>>>(X, T, K, xtotal, Xt);
    else k_tile_x<128><<<xgrid, 256, 0, st>>>(X, T, K, xtotal, Xt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    search_fn fn = pick(p.group_size, p.zero_point, p.variant, clip);
    if (!fn) return hipErrorInvalidValue;
    const uint32_t stage_bytes = (uint32_t)(p.off_xt - p.off_s);   // scale table, reciprocals, W tiles
    fn<<<(unsigned)p.grid, kNW * 64, 0, st>>>(Xt, (int)T, (int)K, Wt, (int)p.nb, s_tab, inv_tab, clip_tab,
                                             stage_bytes, p.n_grid, p.n_asplit, (int)p.tiles, (int)p.tiles_per_xcd,
                                             part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_reduce_losses<<<(unsigned)p.n_grid, 256, 0, st>>>(part, p.tb * p.nb, p.n_grid, losses);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned sgrid = (unsigned)((sel_len + 255) / 256 < 64 ? (sel_len + 255) / 256 : 64);
    k_select<<<sgrid, 256, 0, st>>>(losses, p.n_grid, sel_table, sel_len, best, sel_row);
    return hipGetLastError();
}

hipError_t run_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N, const SearchPlan& p,
                      void* ws, bool clip, double* losses, int32_t* best, const float* sel_table, int64_t sel_len,
                      float* sel_row, hipStream_t st) {
    hipError_t e = tile_w(W, K, N, p, ws, 0, st);
    if (e != hipSuccess) return e;
    return run_search_tiled(X, T, K, p, ws, clip, losses, best, sel_table, sel_len, sel_row, st);
}

hipError_t write_clip_table(const ClipRatios& r, int n, float* tab, hipStream_t st) {
    k_write_clip<<<1, kMaxGrid, 0, st>>>(r, n, tab);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                         const float* mean_abs, float clip_ratio, const SearchPlan& p, void* ws, double* losses,
                         int32_t* best, float* s_best, hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    hipError_t e = launch_scale_table(mean_abs, K, p.n_grid, s_tab, inv_tab, st);
    if (e != hipSuccess) return e;
    const bool clip = clip_ratio > 0.f && clip_ratio < 1.f;
    if (clip) {
        ClipRatios r{};
        for (int j = 0; j < p.n_grid; ++j) r.c[j] = clip_ratio;
        if ((e = write_clip_table(r, p.n_grid, (float*)(base + p.off_clip), st)) != hipSuccess) return e;
    }
    return run_search(X, T, W, K, N, p, ws, clip, losses, best, s_tab, K, s_best, st);
}

hipError_t launch_search_table(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                               const float* table, float clip_ratio, const SearchPlan& p, void* ws, double* losses,
                               int32_t* best, float* s_best, hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    dim3 grid((unsigned)((K + 255) / 256), (unsigned)p.n_grid);
    k_table_rows<<<grid, 256, 0, st>>>(table, K, s_tab, inv_tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool clip = clip_ratio > 0.f && clip_ratio < 1.f;
    if (clip) {
        ClipRatios r{};
        for (int j = 0; j < p.n_grid; ++j) r.c[j] = clip_ratio;
        if ((e = write_clip_table(r, p.n_grid, (float*)(base + p.off_clip), st)) != hipSuccess) return e;
    }
    return run_search(X, T, W, K, N, p, ws, clip, losses, best, s_tab, K, s_best, st);
}

hipError_t launch_search_multi(const uint16_t* X, int64_t T, int n_w, const uint16_t* const* W, const int64_t* N,
                               int64_t K, const float* mean_abs, float clip_ratio, const SearchPlan& p, void* ws,
                               double* losses, double* losses_each, int32_t* best, float* s_best, hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    hipError_t e = launch_scale_table(mean_abs, K, p.n_grid, s_tab, inv_tab, st);
    if (e != hipSuccess) return e;
    const bool clip = clip_ratio > 0.f && clip_ratio < 1.f;
    if (clip) {
        ClipRatios r{};
        for (int j = 0; j < p.n_grid; ++j) r.c[j] = clip_ratio;
        if ((e = write_clip_table(r, p.n_grid, (float*)(base + p.off_clip), st)) != hipSuccess) return e;
    }
    int64_t nb0 = 0;
    for (int j = 0; j < n_w; ++j) {
        if ((e = tile_w(W[j], K, N[j], p, ws, nb0, st)) != hipSuccess) return e;
        nb0 += (N[j] + 15) / 16;
    }
    if ((e = run_search_tiled(X, T, K, p, ws, clip, losses, best, s_tab, K, s_best, st)) != hipSuccess) return e;
    if (!losses_each) return hipSuccess;
    const double* part = (const double*)(base + p.off_part);
    nb0 = 0;
    for (int j = 0; j < n_w; ++j) {
        const int64_t nb1 = nb0 + (N[j] + 15) / 16;
        k_reduce_losses_range<<<(unsigned)p.n_grid, 256, 0, st>>>(part, p.tb, p.nb, nb0, nb1, p.n_grid,
                                                                 losses_each + (int64_t)j * p.n_grid);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        nb0 = nb1;
    }
    return hipSuccess;
}

hipError_t launch_clip_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                              const float* s, float clip_min, const SearchPlan& p, void* ws, double* losses,
                              int32_t* best, float* clip_best, hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    float* clip_tab = (float*)(base + p.off_clip);
    dim3 grid((unsigned)((K + 255) / 256), (unsigned)p.n_grid);
    k_fixed_scale_rows<<<grid, 256, 0, st>>>(s, K, s_tab, inv_tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // c_j = float32(1 - (1 - c_min) j / (n - 1)), evaluated in float64 in this order
    ClipRatios r{};
    const double cm = (double)clip_min;
    for (int j = 0; j < p.n_grid; ++j) r.c[j] = (float)(1.0 - (1.0 - cm) * j / (p.n_grid - 1));
    if ((e = write_clip_table(r, p.n_grid, clip_tab, st)) != hipSuccess) return e;
    return run_search(X, T, W, K, N, p, ws, true, losses, best, clip_tab, 1, clip_best, st);
}

}  // namespace awq
