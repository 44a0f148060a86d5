// ceiling.hip -- measured ceilings beside the published peaks, for gfx950.
//
// Two measurement kernels (not part of the DSA path; bench.py reports what they reach):
//   - ceiling_mfma_kernel: bf16 32x32x16 MFMA chains and nothing else (operands in registers,
//     eight independent accumulators per wave), one workgroup per CU (its LDS allotment keeps a
//     second one off), 4 or 8 waves, so one or two waves per SIMD like the indexer's scoring
//     kernel.  Operands are either constant (1.0) or hashed bf16 values of random sign,
//     mantissa and exponent in [2^-3, 2^1): the matrix pipe draws more power, and the clock
//     drops, with random operands.
//   - ceiling_copy_kernel: a 16-byte-per-lane stream over one contiguous chunk per block, a copy (what the HBM delivers to a
//     plain read-and-write stream) or a read only (what it delivers to loads alone, the mix of a
//     gather), with ordinary or nontemporal accesses.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kCeilingLdsBytes = 96 * 1024;  // more than half a CU's LDS: one workgroup per CU

__device__ __forceinline__ uint32_t ceiling_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// bf16 operand e of fragment j for thread gid (seed separates the A and B operands).
__device__ __forceinline__ uint16_t ceiling_operand(uint32_t gid, int j, int e, uint32_t seed, bool random) {
    if (!random) return 0x3f80u;  // 1.0
    const uint32_t h = ceiling_hash(gid * 64u + (uint32_t)(j * 8 + e) + seed);
    return (uint16_t)(((h >> 31) << 15) | ((124u + ((h >> 7) & 3u)) << 7) | (h & 0x7fu));
}

__global__ __launch_bounds__(512) void ceiling_mfma_kernel(float* __restrict__ out, int iters, int random) {
    __shared__ float s_hold[kCeilingLdsBytes / 4];
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[j][e] = __builtin_bit_cast(__bf16, ceiling_operand(gid, j, e, 0x1234567u, random != 0));
            b[j][e] = __builtin_bit_cast(__bf16, ceiling_operand(gid, j, e, 0x89abcdeu, random != 0));
        }
    f32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = mfma_32x32x16(a[j & 3], b[(j >> 2) + 2 * (j & 1)], c[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    // The LDS allotment only limits residency; this never-true branch keeps it allocated.
    if (iters < 0) {
        s_hold[threadIdx.x] = s;
        __syncthreads();
        s += s_hold[(threadIdx.x + 1) % blockDim.x];
    }
    out[gid] = s;
}

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane
constexpr int kStreamThreads = 256;

// Block b streams its own contiguous chunk [b*per, min(n, (b+1)*per)) of 16-byte elements,
// kStreamUnroll block-wide rows at a time (per is a multiple of kStreamUnroll * kStreamThreads).
// Contiguous chunks per block reach more of the HBM than a grid-wide stride.
// dst == nullptr: read only (an XOR of everything read goes to sink[thread], so no load is dropped).
template <bool kNontemporal>
__global__ __launch_bounds__(kStreamThreads) void ceiling_copy_kernel(const u32x4* __restrict__ src,
                                                                      u32x4* __restrict__ dst, size_t n, size_t per,
                                                                      uint32_t* __restrict__ sink) {
    constexpr size_t kRow = kStreamThreads;
    const size_t begin = (size_t)blockIdx.x * per;
    const size_t end = begin + per < n ? begin + per : n;
    auto ld = [&](size_t j) -> u32x4 { return kNontemporal ? __builtin_nontemporal_load(&src[j]) : src[j]; };
    auto st = [&](size_t j, u32x4 v) {
        if (kNontemporal) __builtin_nontemporal_store(v, &dst[j]);
        else dst[j] = v;
    };
    uint32_t x = 0u;
    size_t o = begin + threadIdx.x;
    for (; begin < end && o + (kStreamUnroll - 1) * kRow < end; o += kStreamUnroll * kRow) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld(o + u * kRow);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            if (dst) st(o + u * kRow, v[u]);
            else x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    for (; o < end; o += kRow) {
        const u32x4 v = ld(o);
        if (dst) st(o, v);
        else x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (!dst) sink[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = x;
}

hipError_t launch_ceiling_mfma(float* out, int n_cu, int iters, bool random, int waves_per_simd, hipStream_t s) {
    ProfScope ps(s, kProfCeilingMfma);
    ceiling_mfma_kernel<<<n_cu, 256 * waves_per_simd, 0, s>>>(out, iters, random ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_ceiling_copy(const void* src, void* dst, size_t bytes, uint32_t* sink, bool nontemporal,
                               hipStream_t s) {
    ProfScope ps(s, kProfCeilingCopy);
    const u32x4* a = reinterpret_cast<const u32x4*>(src);
    u32x4* b = reinterpret_cast<u32x4*>(dst);
    const size_t n = bytes / 16;
    constexpr size_t kTile = (size_t)kStreamUnroll * kStreamThreads;
    const size_t per = (n + (size_t)kCeilingCopyBlocks * kTile - 1) / ((size_t)kCeilingCopyBlocks * kTile) * kTile;
    if (nontemporal) ceiling_copy_kernel<true><<<kCeilingCopyBlocks, kStreamThreads, 0, s>>>(a, b, n, per, sink);
    else ceiling_copy_kernel<false><<<kCeilingCopyBlocks, kStreamThreads, 0, s>>>(a, b, n, per, sink);
    return hipGetLastError();
}

}  // namespace dsa
