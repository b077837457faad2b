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
//   * Every wavefront keeps the bf16 X fragments of its rows for the current 32-wide K chunk in
//     registers (loaded once, prefetched one chunk ahead) and reuses them for all NA alphas:
//     acc[alpha][row block] += X_chunk . E_alpha_chunk on v_mfma_f32_16x16x32_bf16.
//   * Epilogue: sum of squares of the float32 accumulators, reduced in a fixed order to one
//     float64 partial per (token tile, column tile, alpha).  A second kernel sums the partials
//     in a fixed order and a third picks the first minimum.
//   * Tile order is XCD-aware: the workgroups that run together on one XCD share a token tile,
//     so that XCD's L2 serves the X panel to all of them.
// The quantizer inside the search is the float32 evaluation of the packing quantizer of
// awq_pack (which evaluates it exactly in float64); the two differ only for elements whose
// pre-round value lies within float32 rounding of a .5 boundary.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Matrix-core operand layout used throughout (v_mfma_f32_16x16x32_bf16):
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) .. +7
//   B (32 x 16): lane l holds column l%16, k = 8*(l/16) .. +7
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. +3
// A K chunk is 32 consecutive input channels; a group of G channels is G/32 chunks.

// W [K, N] bf16 -> Wt: for column block nb (16 columns), chunk kc (32 channels) and lane l, the
// 8 bf16 values W[32*kc + 8*(l/16) + e][16*nb + l%16], e = 0..7, as one 16-byte word.  Columns
// beyond N are zero (a zero column quantizes to zero error).
__global__ __launch_bounds__(256) void k_tile_w(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                int64_t total, u32x4* __restrict__ Wt) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const int lane = (int)(e & 63);
    const int64_t rest = e >> 6;
    const int64_t kchunks = K / 32;
    const int64_t kc = rest % kchunks, nb = rest / kchunks;
    const int64_t k0 = kc * 32 + 8 * (lane >> 4);
    const int64_t n = nb * 16 + (lane & 15);
    uint32_t v[4] = {0, 0, 0, 0};
    if (n < N) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
            v[h] = (uint32_t)W[(k0 + 2 * h) * N + n] | ((uint32_t)W[(k0 + 2 * h + 1) * N + n] << 16);
    }
    Wt[e] = u32x4{v[0], v[1], v[2], v[3]};
}

template <int G, int NA, int RBW, int NW, bool ZP>
__global__ __launch_bounds__(NW * 64, 1) void k_search(
    const uint16_t* __restrict__ X, int T, int K, const u32x4* __restrict__ Wt, int NB,
    const float* __restrict__ s_tab, const float* __restrict__ inv_tab, int n_grid, int n_asplit,
    int n_tiles, int tiles_per_xcd, double* __restrict__ partials) {
    constexpr int C = G / 32;            // K chunks per group
    constexpr int BM = NW * RBW * 16;    // token rows per workgroup
    constexpr int V = G / 4;             // group values per lane (one column, one quad)

    const int tile = xcd_tile(blockIdx.x, tiles_per_xcd);
    if (tile >= n_tiles) return;
    const int asplit = tile % n_asplit;
    const int rest = tile / n_asplit;
    const int nb = rest % NB;
    const int tb = rest / NB;
    const int a0 = asplit * NA;
    const int na = min(NA, n_grid - a0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane >> 4, r16 = lane & 15;
    const int n_groups = K / G;
    const int kchunks = K / 32;

    __shared__ u32x4 Es[2][NA][C][64];
    __shared__ double red[NW][NA];

    floatx4 acc[NA][RBW];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) acc[a][rb] = floatx4{0.f, 0.f, 0.f, 0.f};

    // A-fragment sources: row = tile row of this lane in row block rb; rows >= T read row T-1
    // (valid memory) and are zeroed.
    const uint16_t* xrow[RBW];
    bool rvalid[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        const int row = tb * BM + (wave * RBW + rb) * 16 + r16;
        rvalid[rb] = row < T;
        xrow[rb] = X + (int64_t)min(row, T - 1) * K + 8 * q;
    }
    auto load_A = [&](int kc, u32x4 (&A)[RBW]) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            u32x4 v = *(const u32x4*)(xrow[rb] + kc * 32);
            A[rb] = rvalid[rb] ? v : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // Quantize/dequantize the 16-column tile of group jg for alpha a0 + wave; write E (bf16) into
    // Es[buf][wave] in B-operand layout.
    auto compute_E = [&](int jg, int buf) {
        const int a = a0 + wave;
        const u32x4* wsrc = Wt + ((int64_t)nb * kchunks + (int64_t)jg * C) * 64 + lane;
        u32x4 wv[C];
#pragma unroll
        for (int c = 0; c < C; ++c) wv[c] = wsrc[c * 64];
        const float* srow = s_tab + (int64_t)a * K + jg * G + 8 * q;
        const float* irow = inv_tab + (int64_t)a * K + jg * G + 8 * q;
        float p[V];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const floatx4 s0 = *(const floatx4*)(srow + 32 * c);
            const floatx4 s1 = *(const floatx4*)(srow + 32 * c + 4);
            p[8 * c + 0] = s0[0] * bf16_lo(wv[c][0]);
            p[8 * c + 1] = s0[1] * bf16_hi(wv[c][0]);
            p[8 * c + 2] = s0[2] * bf16_lo(wv[c][1]);
            p[8 * c + 3] = s0[3] * bf16_hi(wv[c][1]);
            p[8 * c + 4] = s1[0] * bf16_lo(wv[c][2]);
            p[8 * c + 5] = s1[1] * bf16_hi(wv[c][2]);
            p[8 * c + 6] = s1[2] * bf16_lo(wv[c][3]);
            p[8 * c + 7] = s1[3] * bf16_hi(wv[c][3]);
        }
        float d, lo, hi;
        if (ZP) {
            float mx = 0.f, mn = 0.f;   // the group range always includes 0
#pragma unroll
            for (int i = 0; i < V; i += 2) {
                mx = fmaxf(mx, fmaxf(p[i], p[i + 1]));
                mn = fminf(mn, fminf(p[i], p[i + 1]));
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mn = fminf(mn, __shfl_xor(mn, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            mn = fminf(mn, __shfl_xor(mn, 32, 64));
            d = (mx - mn) / 15.0f;
            if (d == 0.f) d = 1.f;
            const float z = fminf(fmaxf(rintf(-mn / d), 0.f), 15.f);
            lo = -z;
            hi = 15.f - z;
        } else {
            float am = 0.f;
#pragma unroll
            for (int i = 0; i < V; i += 2) am = fmaxf(am, fmaxf(fabsf(p[i]), fabsf(p[i + 1])));
            am = fmaxf(am, __shfl_xor(am, 16, 64));
            am = fmaxf(am, __shfl_xor(am, 32, 64));
            d = am / 7.0f;
            if (d == 0.f) d = 1.f;
            lo = -7.f;
            hi = 7.f;
        }
        const float rd = 1.0f / d;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const floatx4 i0 = *(const floatx4*)(irow + 32 * c);
            const floatx4 i1 = *(const floatx4*)(irow + 32 * c + 4);
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pv = p[8 * c + j];
                const float lv = fminf(fmaxf(rintf(pv * rd), lo), hi);
                const float es = fmaf(lv, d, -pv);          // quantization error in the scaled domain
                e[j] = es * (j < 4 ? i0[j & 3] : i1[j & 3]);  // back to the original domain
            }
            Es[buf][wave][c][lane] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                           pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
        }
    };

    if (wave < na) compute_E(0, 0);
    __syncthreads();

    u32x4 A[RBW], An[RBW];
    load_A(0, A);
    for (int jg = 0; jg < n_groups; ++jg) {
        const int buf = jg & 1;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int kc_next = jg * C + c + 1;
            if (kc_next < kchunks) load_A(kc_next, An);
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                if (a < na) {
                    const u32x4 bw = Es[buf][a][c][lane];
                    const bf16x8 B = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
                    for (int rb = 0; rb < RBW; ++rb)
                        acc[a][rb] = mfma16x16x32(__builtin_bit_cast(bf16x8, A[rb]), B, acc[a][rb]);
                }
            }
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) A[rb] = An[rb];
        }
        if (jg + 1 < n_groups && wave < na) compute_E(jg + 1, buf ^ 1);
        __syncthreads();
    }

    // Epilogue: sum of squares per alpha; fixed-order reductions (lanes, then wavefronts).
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        float ss = 0.f;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(acc[a][rb][i], acc[a][rb][i], ss);
        const double t = wave_sum((double)ss);
        if (lane == 0) red[wave][a] = t;
    }
    __syncthreads();
    if (threadIdx.x < na) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += red[w][threadIdx.x];
        partials[((int64_t)tb * NB + nb) * n_grid + a0 + threadIdx.x] = s;
    }
}

// L[i] = sum over tiles of partials[tile][i]: one workgroup per alpha, strided fixed-order sums
// and a fixed tree.
__global__ __launch_bounds__(256) void k_reduce_losses(const double* __restrict__ partials, int64_t tiles,
                                                       int n_grid, double* __restrict__ losses) {
    __shared__ double sm[256];
    const int i = blockIdx.x;
    double s = 0.0;
    for (int64_t t = threadIdx.x; t < tiles; t += 256) s += partials[t * n_grid + i];
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) losses[i] = sm[0];
}

// best = first index of the minimum loss; s_best = s_tab[best].
__global__ __launch_bounds__(256) void k_select(const double* __restrict__ losses, int n_grid,
                                                const float* __restrict__ s_tab, int64_t K,
                                                int32_t* __restrict__ best, float* __restrict__ s_best) {
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
        s_best[k] = s_tab[(int64_t)b * K + k];
}

namespace {

// Instantiations: (group size, zero point) x one tile shape.
// 8 wavefronts (2 per SIMD), 4 row blocks of 16 each -> 512 token rows per workgroup, 7 alphas
// per workgroup (21 = 3 slices of 7).  Accumulators: 7 x 4 x 4 = 112 VGPRs per lane.
constexpr int kNA = 7, kRBW = 4, kNW = 8;
constexpr int kBM = kNW * kRBW * 16;

typedef void (*search_fn)(const uint16_t*, int, int, const u32x4*, int, const float*, const float*, int,
                          int, int, int, double*);

search_fn pick(int g, int zp) {
    if (zp) {
        if (g == 32) return k_search<32, kNA, kRBW, kNW, true>;
        if (g == 64) return k_search<64, kNA, kRBW, kNW, true>;
        if (g == 128) return k_search<128, kNA, kRBW, kNW, true>;
    } else {
        if (g == 32) return k_search<32, kNA, kRBW, kNW, false>;
        if (g == 64) return k_search<64, kNA, kRBW, kNW, false>;
        if (g == 128) return k_search<128, kNA, kRBW, kNW, false>;
    }
    return nullptr;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

SearchPlan plan_search(int64_t T, int64_t K, int64_t N, int group_size, int zero_point, int n_grid) {
    SearchPlan p{};
    p.group_size = group_size;
    p.n_grid = n_grid;
    p.zero_point = zero_point;
    p.variant = 0;
    p.na = kNA;
    p.bm = kBM;
    p.n_asplit = (n_grid + kNA - 1) / kNA;
    p.nb = (N + 15) / 16;
    p.tb = (T + kBM - 1) / kBM;
    p.tiles = p.tb * p.nb * p.n_asplit;
    p.tiles_per_xcd = (p.tiles + kNumXcd - 1) / kNumXcd;
    p.grid = p.tiles_per_xcd * kNumXcd;
    size_t off = 0;
    p.off_s = off;    off = align256(off + (size_t)n_grid * K * sizeof(float));
    p.off_inv = off;  off = align256(off + (size_t)n_grid * K * sizeof(float));
    p.off_wt = off;   off = align256(off + (size_t)p.nb * 16 * K * sizeof(uint16_t));
    p.off_part = off; off = align256(off + (size_t)p.tb * p.nb * n_grid * sizeof(double));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_search(const uint16_t* X, int64_t T, const uint16_t* W, int64_t K, int64_t N,
                         const float* mean_abs, const SearchPlan& p, void* ws, double* losses,
                         int32_t* best, float* s_best, hipStream_t st) {
    char* base = (char*)ws;
    float* s_tab = (float*)(base + p.off_s);
    float* inv_tab = (float*)(base + p.off_inv);
    u32x4* Wt = (u32x4*)(base + p.off_wt);
    double* part = (double*)(base + p.off_part);

    hipError_t e = launch_scale_table(mean_abs, K, p.n_grid, s_tab, inv_tab, st);
    if (e != hipSuccess) return e;
    const int64_t total = p.nb * (K / 32) * 64;
    k_tile_w<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(W, K, N, total, Wt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    search_fn fn = pick(p.group_size, p.zero_point);
    if (!fn) return hipErrorInvalidValue;
    fn<<<(unsigned)p.grid, kNW * 64, 0, st>>>(X, (int)T, (int)K, Wt, (int)p.nb, s_tab, inv_tab, p.n_grid,
                                             p.n_asplit, (int)p.tiles, (int)p.tiles_per_xcd, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_reduce_losses<<<(unsigned)p.n_grid, 256, 0, st>>>(part, p.tb * p.nb, p.n_grid, losses);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_select<<<(unsigned)((K + 255) / 256 < 64 ? (K + 255) / 256 : 64), 256, 0, st>>>(losses, p.n_grid, s_tab,
                                                                                     K, best, s_best);
    return hipGetLastError();
}

}  // namespace awq
