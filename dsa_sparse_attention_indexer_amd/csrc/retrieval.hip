// retrieval.hip -- inner-product top-k over a corpus (vector retrieval) for gfx950.
//
// What is computed (LiteTopK abstract: the Indexer-TopK operation also serves
// vector retrieval in recommendation systems and vector databases):
//   score(t, j) = q[t,:] . x[j,:]  over every corpus row j (one head, no ReLU,
//   no weights, no causality), keep the top_k rows by (score desc, row asc),
//   emit them ascending, -1 pad.
//
// The selection is the indexer's, unchanged.  Since ReLU(s) - ReLU(-s) = s, the
// indexer score of the two-head query (q, -q) with weights (1, -1) (other heads
// zero) is the inner product, also in the canonical fp64 order (the two head
// sums are exact negatives, and one of the two terms is zero).  This file
// therefore only supplies:
//   - retrieval_prep_kernel: that two-head form of each query row and the row
//     table (every row sees all N corpus rows), read by row_prep (error bound,
//     threshold), select (fp64 band re-score) and the fold;
//   - retrieval_score_kernel: the fp32 scores themselves, on bf16 MFMA with the
//     corpus as the A operand (32 rows) and 32 queries as the B operand, for the
//     strided sample (threshold estimate) and the candidate filter.
// The filter's fp32 dot products are the same 8-step MFMA chain the indexer's
// per-head products use, so the indexer's bound (which also pays for the head
// sum) covers them.
#include <float.h>
#include <limits.h>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kRetSets = 4;                  // 32-query sets per workgroup
constexpr int kRetQueries = 32 * kRetSets;   // queries per workgroup; each of its 4 waves holds all of them
constexpr int kRetStage = 16;                // staged candidates per query per wave

__global__ __launch_bounds__(256) void retrieval_prep_kernel(const uint16_t* __restrict__ q, int Lb, int64_t N,
                                                             uint16_t* __restrict__ q_emb, float* __restrict__ w_emb,
                                                             RowInfo* rows, int n_rows) {
    const int r = blockIdx.x;
    if (r == 0)
        for (int i = threadIdx.x; i < n_rows; i += blockDim.x) rows[i] = RowInfo{i, N - 1, 0, 0, N};
    if (r >= Lb) return;
    const u16x8* src = reinterpret_cast<const u16x8*>(q + (size_t)r * kIdxDim);
    u16x8* dst = reinterpret_cast<u16x8*>(q_emb + (size_t)r * kIdxHeads * kIdxDim);
    for (int v = threadIdx.x; v < kIdxHeads * kIdxDim / 8; v += blockDim.x) {
        const int h = v / (kIdxDim / 8), c = v % (kIdxDim / 8);
        u16x8 o = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (h == 0) o = src[c];
        if (h == 1) o = src[c] ^ (unsigned short)0x8000;  // bf16 negation
        dst[v] = o;
    }
    if (threadIdx.x < kIdxHeads)
        w_emb[(size_t)r * kIdxHeads + threadIdx.x] = threadIdx.x == 0 ? 1.0f : (threadIdx.x == 1 ? -1.0f : 0.0f);
}

struct RetrievalScore {
    const RetrievalArgs& A;
    int wave, lane, hf, c;
    const u16x8* xt;  // filter: the tiled corpus

    // A operand of tile t: lane (hf, c) supplies corpus row c of the tile, dims 64 hf + 8 kk ..
    template <bool kSample>
    __device__ __forceinline__ void load(u16x8 (&a)[8], int64_t t) const {
        if (kSample) {
            int64_t j = t * kKeyTile + c;
            j = j < A.sample_n ? j : A.sample_n - 1;
            const int64_t row = j * A.N / A.sample_n;
            const u16x8* p = reinterpret_cast<const u16x8*>(A.x + (size_t)row * kIdxDim + 64 * hf);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) a[kk] = p[kk];
        } else {
            const u16x8* p = xt + (size_t)t * (kKeyTileBytes / 16) + lane;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) a[kk] = p[kk * 64];
        }
    }
};

// Stages n entries of this lane's set-s query (both lane halves take part; hf 0's
// entries first) and flushes to the row's appended list when the stage is full.
__device__ __forceinline__ void ret_flush(const RetrievalArgs& A, const uint2* st, int n, int row, int hf, int lane,
                                          bool go) {
    int base = 0;
    if (go && hf == 0) base = atomicAdd(&A.count[(size_t)row * kCandSegs], n);
    base = __shfl(base, lane & 31);
    if (go) {
        const int half = (n + 1) >> 1;
        const int j0 = hf ? half : 0, j1 = hf ? n : half;
        uint2* dst = A.cand + (size_t)row * A.cap;
        for (int j = j0; j < j1; ++j)
            if (base + j < A.cap) dst[base + j] = st[j];
    }
}

template <bool kSample>
__global__ __launch_bounds__(256) void retrieval_score_kernel(RetrievalArgs A) {
    // Workgroup -> (query group g, corpus part).  With a multiple of 8 parts, the groups of one
    // part share an XCD (and its L2), which streams that part once for all of them.
    int part, g;
    if ((A.parts & 7) == 0) {
        const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, p8 = A.parts >> 3;
        part = (j % p8) * 8 + xcd;
        g = j / p8;
    } else {
        part = blockIdx.x % A.parts;
        g = blockIdx.x / A.parts;
    }
    if (g >= A.n_groups) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
    __shared__ uint2 s_stage[kScoreThreads / kWave][kRetQueries][kRetStage];

    // This wave's tiles: segment (part, wave) of the corpus (or of the sample).
    const int64_t n_keys = kSample ? A.sample_n : A.N;
    const int64_t n_tiles = (n_keys + kKeyTile - 1) / kKeyTile;
    const int64_t segs = (int64_t)A.parts * (kScoreThreads / kWave);
    const int64_t tps = (n_tiles + segs - 1) / segs;
    const int64_t t0 = (int64_t)(part * (kScoreThreads / kWave) + wave) * tps;
    const int64_t t1 = t0 + tps < n_tiles ? t0 + tps : n_tiles;
    if (t0 >= t1) return;

    // B operand: lane (hf, c) of set s holds query 32 s + c of the group, dims 64 hf + 8 kk ..
    bf16x8 b[kRetSets][8];
    float tau[kRetSets];
    bool live[kRetSets];
    int row[kRetSets], scnt[kRetSets];
#pragma unroll
    for (int s = 0; s < kRetSets; ++s) {
        const int r = g * kRetQueries + 32 * s + c;
        const bool valid = r < A.Lb;
        row[s] = valid ? r : 0;
        scnt[s] = 0;
        const u16x8* qp = reinterpret_cast<const u16x8*>(A.q + (size_t)row[s] * kIdxDim + 64 * hf);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            b[s][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
            asm volatile("" : "+a"(b[s][kk]));  // keep the query fragments in AGPRs
        }
        if (kSample) {
            live[s] = valid;
            tau[s] = 0.f;
        } else {
            live[s] = valid && A.mode[row[s]] == kModeNormal;
            tau[s] = live[s] ? A.tau[row[s]] : INFINITY;
        }
    }
    const RetrievalScore R{A, wave, lane, hf, c, reinterpret_cast<const u16x8*>(A.x_tile)};

    auto tile = [&](const u16x8 (&a)[8], int64_t t) {
        f32x16 acc[kRetSets];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int s = 0; s < kRetSets; ++s)
                acc[s] = mfma_32x32x16(__builtin_bit_cast(bf16x8, a[kk]), b[s][kk], kk == 0 ? f32x16{} : acc[s]);
        // Lane (hf, c) holds query c's scores of tile rows 8 (i / 4) + 4 hf + i % 4.
        const int64_t key0 = t * kKeyTile + 4 * hf;
        const bool tail = (t + 1) * kKeyTile > n_keys;
#pragma unroll
        for (int s = 0; s < kRetSets; ++s) {
            if (kSample) {
                if (live[s]) {
                    float* dst = A.sample + (size_t)row[s] * A.sample_stride;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int64_t j = key0 + 8 * (i >> 2) + (i & 3);
                        if (!tail || j < n_keys) dst[j] = acc[s][i] + 0.0f;
                    }
                }
                continue;
            }
            bool any = false;
#pragma unroll
            for (int i = 0; i < 16; ++i) any = any || acc[s][i] >= tau[s];
            if (__ballot(any) == 0) continue;
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t j = key0 + 8 * (i >> 2) + (i & 3);
                if (acc[s][i] >= tau[s] && (!tail || j < n_keys)) m |= 1u << i;
            }
            const int n = __builtin_popcount(m);
            const int n_other = __shfl_xor(n, 32);
            const int before = hf ? n_other : 0, total = n + n_other;
            uint2* st = &s_stage[wave][32 * s + c][0];
            const bool full = scnt[s] + total > kRetStage;
            ret_flush(A, st, scnt[s], row[s], hf, lane, full && scnt[s] > 0);
            if (full) scnt[s] = 0;
            __builtin_amdgcn_wave_barrier();
            if (total > kRetStage) {  // more than a stage: straight to the list
                int base = 0;
                if (hf == 0) base = atomicAdd(&A.count[(size_t)row[s] * kCandSegs], total);
                base = __shfl(base, lane & 31) + before;
                uint2* dst = A.cand + (size_t)row[s] * A.cap;
                int o = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((m >> i) & 1u) {
                        const uint32_t key = (uint32_t)(key0 + 8 * (i >> 2) + (i & 3));
                        if (base + o < A.cap) dst[base + o] = make_uint2(__float_as_uint(acc[s][i] + 0.0f), key);
                        ++o;
                    }
            } else {
                int o = scnt[s] + before;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((m >> i) & 1u) {
                        const uint32_t key = (uint32_t)(key0 + 8 * (i >> 2) + (i & 3));
                        st[o++] = make_uint2(__float_as_uint(acc[s][i] + 0.0f), key);
                    }
                scnt[s] += total;
            }
            __builtin_amdgcn_wave_barrier();
        }
    };

    // Tile t sits in buffer (t - t0) % 3; loads run three tiles ahead (clamped to the last).
    u16x8 a0[8], a1[8], a2[8];
    auto tl = [&](int64_t t) { return t < t1 ? t : t1 - 1; };
    R.template load<kSample>(a0, t0);
    R.template load<kSample>(a1, tl(t0 + 1));
    R.template load<kSample>(a2, tl(t0 + 2));
    for (int64_t t = t0; t < t1; t += 3) {
        tile(a0, t);
        R.template load<kSample>(a0, tl(t + 3));
        if (t + 1 < t1) tile(a1, t + 1);
        R.template load<kSample>(a1, tl(t + 4));
        if (t + 2 < t1) tile(a2, t + 2);
        R.template load<kSample>(a2, tl(t + 5));
    }
    if (!kSample) {
#pragma unroll
        for (int s = 0; s < kRetSets; ++s) {
            __builtin_amdgcn_wave_barrier();
            ret_flush(A, &s_stage[wave][32 * s + c][0], scnt[s], row[s], hf, lane, scnt[s] > 0);
        }
    }
}

// Key parts per query group: enough workgroups for 256 compute units, each wave keeping
// at least 8 tiles; a multiple of 8 when there are 8 or more (XCD-local parts).
static int retrieval_parts(int n_groups, int64_t n_tiles) {
    int64_t p = (256 + n_groups - 1) / n_groups;
    const int64_t by_tiles = n_tiles / (8 * (kScoreThreads / kWave));
    if (p > by_tiles) p = by_tiles;
    if (p > 256) p = 256;
    if (p < 1) p = 1;
    if (p >= 8) p &= ~(int64_t)7;
    return (int)p;
}

hipError_t launch_retrieval_block(RetrievalArgs r, const IndexerArgs& a, bool need_sample, int n_table_rows,
                                  hipStream_t s) {
    {
        ProfScope ps(s, kProfRetrievalPrep);
        const int grid = a.Lb > 1 ? a.Lb : 1;
        retrieval_prep_kernel<<<grid, 256, 0, s>>>(r.q, a.Lb, r.N, const_cast<uint16_t*>(a.q_idx),
                                                   const_cast<float*>(a.w), const_cast<RowInfo*>(a.rows),
                                                   n_table_rows);
    }
    r.n_groups = (r.Lb + kRetQueries - 1) / kRetQueries;
    if (need_sample) {
        ProfScope ps(s, kProfRetrievalSample);
        r.parts = retrieval_parts(r.n_groups, (r.sample_n + kKeyTile - 1) / kKeyTile);
        retrieval_score_kernel<true><<<r.n_groups * r.parts, kScoreThreads, 0, s>>>(r);
    }
    hipError_t e = launch_row_prep(a, s);
    if (e != hipSuccess) return e;
    {
        ProfScope ps(s, kProfRetrievalFilter);
        r.parts = retrieval_parts(r.n_groups, (r.N + kKeyTile - 1) / kKeyTile);
        retrieval_score_kernel<false><<<r.n_groups * r.parts, kScoreThreads, 0, s>>>(r);
    }
    return launch_select_fold(a, s);
}

}  // namespace dsa
