// dsa_common.h -- shared device definitions for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) double f64x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kWave = 64;

// Indexer constants.
constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kScoreThreads = 256;    // 4 waves
constexpr int kKeyTile = 32;          // keys per MFMA tile (32x32x16 output columns)

// Selector constants.
constexpr int kSelectThreads = 512;
constexpr int kMaxTopK = 4096;        // largest top_k (DSA_MAX_TOPK)

// Bound on |fp32 score - canonical fp64 score| in units of
// 2^-24 * max_s ||k_s||_2 * sum_h |w_h| ||q_h||_2 (see the indexer source).
constexpr double kDeltaCoef = 104.0;

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 and +0 map alike.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane i's bytes land at lds + 16 i (4 i).
// Written as inline asm on purpose: the compiler, seeing an LDS DMA in flight, would wait
// for it before every later LDS read it cannot prove disjoint, i.e. before the current
// tile's reads, and serialise the next tile's gather with this tile's compute.  The waits
// for these DMAs are therefore all explicit (vmcnt before the tile barrier); the compiler's
// own vmcnt waits for other loads can only over-wait on them (the counter is in order).
// M0 holds the LDS address; one wait state separates its write from the DMA.
__device__ __forceinline__ void dma_lds16(const void* src, const void* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(const void* src, const void* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(m0) : "memory", "m0");
}

}  // namespace dsa
