// attention.hip -- sparse absorbed-MLA prefill attention for gfx950.
//
// "GLM prefill now attends only to the keys its indexer picks", How it works: the
// 512-wide latent and 64-wide rope caches form one 576-wide key per position; each
// query gathers only its top-k rows; every head shares that gathered block; the
// latent is also the value, so the output is 512 wide per head.
//
// One workgroup per query, one wave per 16 heads.  Per 32-key tile:
//   gather   the 32 selected rows into LDS twice: row-major (keys x 576) for the
//            logits and transposed (512 x keys) for the value product; the
//            [top_k x 576] block never exists in HBM
//   logits   S^T[key][head] = K . Q^T on 16x16x32 bf16 MFMA (M = keys, N = heads,
//            18 K-steps over 576); Q stays in VGPRs for the whole row
//   softmax  online, fp32, base-2 with log2(e) folded into the scale; invalid keys
//            (-1, > position, padding) contribute nothing
//   values   O^T[d][head] += V^T . P^T on 16x16x32 MFMA: the logits' output layout
//            is already the B operand (lane = head, 8 keys per lane) once the K order
//            of the product is permuted to match, so P never leaves registers
#include <math.h>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kAttnTile = 32;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kKrowStride = kDqk + 8;   // 1168 B: conflict-free 16-lane column reads
constexpr int kVtStride = kAttnTile + 4;  // 72 B

__global__ __launch_bounds__(512) void sparse_attn_kernel(AttentionArgs A) {
    const int t = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int c16 = lane & 15;
    const int nthreads = blockDim.x;
    const int h = wave * 16 + c16;
    const int64_t p = A.pos0 + t;

    __shared__ __attribute__((aligned(16))) uint16_t Krow[kAttnTile][kKrowStride];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kDv][kVtStride];
    __shared__ int s_key[kAttnTile];

    bf16x8 qf[kDqk / 32];
    {
        const uint16_t* qrow = A.q + ((size_t)t * A.H + h) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qrow + ks * 32));
    }
    f32x4 o[kDv / 16];
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) o[dt] = f32x4{};
    // lsum: sum of the bf16 weights actually multiplied into V (normalises the output);
    // lexp: sum of the unrounded fp32 weights (gives the log-sum-exp).
    float m = -INFINITY, lsum = 0.f, lexp = 0.f;
    const float sl2 = A.scale * 1.4426950408889634f;
    const int32_t* irow = A.idx + (size_t)t * A.top_k;
    const int n_tiles = (A.top_k + kAttnTile - 1) / kAttnTile;

    for (int tile = 0; tile < n_tiles; ++tile) {
        __syncthreads();
        if (threadIdx.x < kAttnTile) {
            const int j = tile * kAttnTile + threadIdx.x;
            const int key = j < A.top_k ? irow[j] : -1;
            s_key[threadIdx.x] = (key >= 0 && key <= p && key < A.N) ? key : -1;
        }
        __syncthreads();
        // Latent columns: 4 keys x 8 columns per item -> row-major and transposed copies.
        for (int it = threadIdx.x; it < (kAttnTile / 4) * (kDv / 8); it += nthreads) {
            const int kq = it >> 6, c = it & 63;
            u16x8 v[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                int key = s_key[kq * 4 + x];
                key = key < 0 ? 0 : key;
                v[x] = *reinterpret_cast<const u16x8*>(A.kv + (size_t)key * A.kv_stride + c * 8);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) *reinterpret_cast<u16x8*>(&Krow[kq * 4 + x][c * 8]) = v[x];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u16x4 pk = {v[0][e], v[1][e], v[2][e], v[3][e]};
                *reinterpret_cast<u16x4*>(&Vt[c * 8 + e][kq * 4]) = pk;
            }
        }
        // Rope columns: row-major only.
        for (int it = threadIdx.x; it < kAttnTile * ((kDqk - kDv) / 8); it += nthreads) {
            const int j = it >> 3, c = kDv / 8 + (it & 7);
            int key = s_key[j];
            key = key < 0 ? 0 : key;
            *reinterpret_cast<u16x8*>(&Krow[j][c * 8]) =
                *reinterpret_cast<const u16x8*>(A.kv + (size_t)key * A.kv_stride + c * 8);
        }
        __syncthreads();

        f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) {
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Krow[c16][ks * 32 + 8 * g]));
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Krow[16 + c16][ks * 32 + 8 * g]));
            s0 = mfma_16x16x32(a0, qf[ks], s0);
            s1 = mfma_16x16x32(a1, qf[ks], s1);
        }
        float lg[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lg[r] = s_key[4 * g + r] >= 0 ? s0[r] * sl2 : -INFINITY;
            lg[4 + r] = s_key[16 + 4 * g + r] >= 0 ? s1[r] * sl2 : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) tmax = fmaxf(tmax, lg[r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m, tmax);
        float alpha = 1.f;
        u16x8 pb;
        float ps = 0.f, pe = 0.f;
        if (mnew == -INFINITY) {
#pragma unroll
            for (int r = 0; r < 8; ++r) pb[r] = 0;
        } else {
            alpha = exp2f(m - mnew);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float e = exp2f(lg[r] - mnew);
                const uint16_t b = float_to_bf16_rne(e);
                pb[r] = b;
                ps += bf16_bits_to_float(b);
                pe += e;
            }
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        pe += __shfl_xor(pe, 16);
        pe += __shfl_xor(pe, 32);
        lsum = lsum * alpha + ps;
        lexp = lexp * alpha + pe;
        m = mnew;
        const bf16x8 pbf = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
            const uint16_t* vp = &Vt[dt * 16 + c16][0];
            const u16x4 lo = *reinterpret_cast<const u16x4*>(vp + 4 * g);
            const u16x4 hi = *reinterpret_cast<const u16x4*>(vp + 16 + 4 * g);
            const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[dt] *= alpha;
            o[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, av), pbf, o[dt]);
        }
    }

    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    uint16_t* orow = A.out + ((size_t)t * A.H + h) * kDv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) {
        u16x4 pk;
#pragma unroll
        for (int r = 0; r < 4; ++r) pk[r] = float_to_bf16_rne(o[dt][r] * inv);
        *reinterpret_cast<u16x4*>(orow + dt * 16) = pk;
    }
    if (A.lse && g == 0)
        A.lse[(size_t)t * A.H + h] = lexp > 0.f ? (m + log2f(lexp)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_sparse_attention(const AttentionArgs& a, hipStream_t s) {
    const int threads = 64 * (a.H / 16);
    ProfScope ps(s, kProfAttention);
    sparse_attn_kernel<<<a.Lb, threads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
