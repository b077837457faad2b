// Device-side types and helpers shared by the libawq kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kNumXcd = 8;    // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kCusPerXcd = 32;

// bf16 <-> f32 on raw bit patterns (exact widening; RNE narrowing handled by the compiler).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the XCDs (workgroup i runs on XCD i % 8).
// Remap the launch index so that each XCD walks a contiguous range of the logical tile
// order: tiles that share operands then share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int block, int tiles_per_xcd) {
    return (block % kNumXcd) * tiles_per_xcd + block / kNumXcd;
}

// Debug build (compiled with AWQ_LDS_POISON): every pipelined LDS buffer is filled with NaN
// between its last reader and its next writer, so a read that a missing wait or barrier lets run
// early sees NaN (which reaches the outputs) instead of plausible stale data.  Off in the library
// the product uses.
#ifdef AWQ_LDS_POISON
constexpr bool kLdsPoison = true;
#else
constexpr bool kLdsPoison = false;
#endif
// 0x7ff87ff8: NaN as float32, as both bf16 halves and, in pairs, as float64
constexpr uint32_t kLdsNan = 0x7ff87ff8u;
__device__ __forceinline__ u32x4 lds_nan16() { return u32x4{kLdsNan, kLdsNan, kLdsNan, kLdsNan}; }
// Debug build: fill a workgroup's floating-point LDS array with NaN at kernel start (every thread
// strides over it), then a barrier; a no-op otherwise.  Called by every thread, before any early
// return.
template <typename T>
__device__ __forceinline__ void lds_poison_start(T* p, int count) {
    if constexpr (kLdsPoison) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        const int words = (int)(count * sizeof(T) / 4);
        for (int i = (int)threadIdx.x; i < words; i += (int)blockDim.x) q[i] = kLdsNan;
        __syncthreads();
    }
}
// wait until this wavefront's LDS writes (the poison) have landed, before a direct transfer into
// the same addresses is issued
__device__ __forceinline__ void lds_write_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace awq
