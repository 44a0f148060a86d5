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

constexpr int kRetRing = 4;  // tiles of each wave's LDS ring (DMA runs kRetRing - 1 tiles ahead)

// DMA of the A operand of tile t (32 corpus rows, 256 bytes each) into an LDS slot, row-major
// with the 16-byte chunks of row rho stored at chunk position (chunk ^ (rho & 15)): the MFMA
// reads of one k-step (32 rows, the same chunk) then hit distinct banks, and each DMA
// instruction reads 4 whole rows (1 KB) of the corpus.  Instruction kk fills LDS bytes
// kk * 1024 + 16 l, i.e. row 4 kk + l / 16, position l % 16.  Rows past N (the last tile)
// repeat row N - 1; the sample's tile rows are the sampled rows.
template <bool kSample>
__device__ __forceinline__ void ret_dma(const RetrievalArgs& A, const char* slot, int64_t t, int lane) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int rho = 4 * kk + (lane >> 4);
        const int chunk = (lane & 15) ^ (rho & 15);
        int64_t row;
        if (kSample) {
            int64_t j = t * kKeyTile + rho;
            j = j < A.sample_n ? j : A.sample_n - 1;
            row = j * A.N / A.sample_n;
        } else {
            row = t * kKeyTile + rho;
            row = row < A.N ? row : A.N - 1;
        }
        dma_lds16(reinterpret_cast<const char*>(A.x + (size_t)row * kIdxDim) + 16 * chunk, slot + 1024 * kk);
    }
}

// Each wave streams its tiles through a ring of LDS slots filled by DMA three tiles ahead,
// with two accumulator sets: the 32 MFMAs of tile t+1 are issued one by one between the 64
// per-entry checks of tile t's scores, so the checks (and the rare candidate stores, into
// the lane's private list) run in the matrix cores' shadow.
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
    const int n_segs = A.parts * 8;
    const int sid = (part * (kScoreThreads / kWave) + wave) * 2 + hf;
    __shared__ __attribute__((aligned(16))) char s_ring[kScoreThreads / kWave][kRetRing][kKeyTileBytes];

    // This wave's tiles: segment (part, wave) of the corpus (or of the sample).
    const int64_t n_keys = kSample ? A.sample_n : A.N;
    const int64_t n_tiles = (n_keys + kKeyTile - 1) / kKeyTile;
    const int64_t segs = (int64_t)A.parts * (kScoreThreads / kWave);
    const int64_t tps = (n_tiles + segs - 1) / segs;
    const int64_t t0 = (int64_t)(part * (kScoreThreads / kWave) + wave) * tps;
    const int64_t t1 = t0 + tps < n_tiles ? t0 + tps : n_tiles;

    // B operand: lane (hf, c) of set s holds query 32 s + c of the group, dims 64 hf + 8 kk ..
    bf16x8 b[kRetSets][8];
    float tau[kRetSets];
    bool live[kRetSets];
    int row[kRetSets], o[kRetSets];
    float4* runs[kRetSets];
    uint32_t* ids[kRetSets];
    float* smp[kRetSets];
#pragma unroll
    for (int s = 0; s < kRetSets; ++s) {
        const int r = g * kRetQueries + 32 * s + c;
        const bool valid = r < A.Lb;
        row[s] = valid ? r : 0;
        o[s] = 0;
        if (kSample) {
            live[s] = valid;
            tau[s] = 0.f;
            smp[s] = A.sample + (size_t)row[s] * A.sample_stride;
        } else {
            live[s] = valid && A.mode[row[s]] == kModeNormal;
            tau[s] = live[s] ? A.tau[row[s]] : INFINITY;
            const size_t base = ((size_t)row[s] * n_segs + sid) * A.seg_cap;
            runs[s] = A.seg_runs + base;
            ids[s] = A.seg_ids + base;
        }
    }
    if (t0 < t1) {
        auto tl = [&](int64_t t) { return t < t1 ? t : t1 - 1; };
        const char* ring = &s_ring[wave][0][0];
        auto slot = [&](int64_t t) { return ring + (size_t)((t - t0) & (kRetRing - 1)) * kKeyTileBytes; };
        // DMA of the first three tiles, then the query fragments (all loads in flight together).
        ret_dma<kSample>(A, slot(t0), t0, lane);
        ret_dma<kSample>(A, slot(t0 + 1), tl(t0 + 1), lane);
        ret_dma<kSample>(A, slot(t0 + 2), tl(t0 + 2), lane);
        u16x8 qraw[kRetSets][8];
#pragma unroll
        for (int s = 0; s < kRetSets; ++s) {
            const u16x8* qp = reinterpret_cast<const u16x8*>(A.q + (size_t)row[s] * kIdxDim + 64 * hf);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) qraw[s][kk] = qp[kk];
        }
#pragma unroll
        for (int s = 0; s < kRetSets; ++s)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                b[s][kk] = __builtin_bit_cast(bf16x8, qraw[s][kk]);
                asm volatile("" : "+a"(b[s][kk]));  // keep the query fragments in AGPRs
            }

        // Run r of set s in a tile's scores: query 32 s + c, tile rows 8 r + 4 hf + 0..3 (entries
        // 4 r .. 4 r + 3).  Filter: a run whose largest score passes the threshold is stored
        // whole (the gather picks its entries; rows past N in the last tile are zero padding
        // that the gather drops).  Sample: every run is stored.
        auto run_check = [&](const f32x16 (&cu)[kRetSets], int j, int64_t t, const float (&te)[kRetSets], bool tail) {
            const int s = j >> 2, r = j & 3;
            // (select canonicalises -0 when it reads candidates; the sample does it here)
            const float z = kSample ? 0.0f : -0.0f;  // x + -0 is x, also for x = -0
            const float4 v = make_float4(cu[s][4 * r] + z, cu[s][4 * r + 1] + z, cu[s][4 * r + 2] + z,
                                         cu[s][4 * r + 3] + z);
            const int64_t key = t * kKeyTile + 8 * r + 4 * hf;
            if (kSample) {
                if (te[s] == 0.f) {
                    if (!tail) {
                        *reinterpret_cast<float4*>(smp[s] + key) = v;
                    } else {
                        if (key < n_keys) smp[s][key] = v.x;
                        if (key + 1 < n_keys) smp[s][key + 1] = v.y;
                        if (key + 2 < n_keys) smp[s][key + 2] = v.z;
                        if (key + 3 < n_keys) smp[s][key + 3] = v.w;
                    }
                }
            } else if (fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)) >= te[s]) {
                const int slot = o[s] < A.seg_cap ? o[s] : A.seg_cap - 1;
                runs[s][slot] = v;
                ids[s][slot] = (uint32_t)(key >> 2);
                ++o[s];
            }
        };
        // MFMAs of tile u (A operand from its LDS slot) into nx, interleaved with the run checks
        // of tile t = u - 1 (scores in cu), one per two MFMAs.  Its DMA was issued three tiles
        // ago; the DMAs of the two tiles after it (16) and any stores may still be in flight.
        auto step = [&](f32x16 (&nx)[kRetSets], int64_t u, const f32x16 (&cu)[kRetSets], int64_t t) {
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            const bool ok = t >= t0 && t < t1;
            const bool tail = (t + 1) * kKeyTile > n_keys;
            float te[kRetSets];  // the check threshold: +inf when tile t is not this wave's
#pragma unroll
            for (int s = 0; s < kRetSets; ++s) te[s] = kSample ? (ok && live[s] ? 0.f : 1.f) : (ok ? tau[s] : INFINITY);
            // lane (hf, c) reads row c, chunk 8 hf + kk (dims 64 hf + 8 kk ..) of the slot
            const u16x8* sp = reinterpret_cast<const u16x8*>(slot(u)) + 16 * c;
            auto rd = [&](int kk) { return sp[(8 * hf + kk) ^ (c & 15)]; };
            u16x8 a_cur = rd(0);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const u16x8 a_nxt = rd(kk < 7 ? kk + 1 : 7);
#pragma unroll
                for (int s = 0; s < kRetSets; ++s) {
                    nx[s] = mfma_32x32x16(__builtin_bit_cast(bf16x8, a_cur), b[s][kk], kk == 0 ? f32x16{} : nx[s]);
                    if ((kk * kRetSets + s) & 1) run_check(cu, (kk * kRetSets + s) >> 1, t, te, tail);
                }
                a_cur = a_nxt;
            }
            // the slot of tile u - 1 is free again: refill it with tile u + 3
            __builtin_amdgcn_wave_barrier();
            ret_dma<kSample>(A, slot(u + 3), tl(u + 3), lane);
        };
        f32x16 acc0[kRetSets], acc1[kRetSets];
#pragma unroll
        for (int s = 0; s < kRetSets; ++s) acc1[s] = f32x16{};
        step(acc0, t0, acc1, t0 - 1);  // no checks: tile t0 - 1 is not this wave's
        for (int64_t u = t0 + 1; u < t1 + 1; u += 2) {
            step(acc1, u, acc0, u - 1);
            step(acc0, u + 1, acc1, u);
        }
        // The last steps requested (clamped) tiles past t1: let those DMAs land before the
        // wave ends, so no write reaches this workgroup's LDS after it is released.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (!kSample) {
#pragma unroll
        for (int s = 0; s < kRetSets; ++s)
            if (g * kRetQueries + 32 * s + c < A.Lb) A.seg_count[(size_t)row[s] * n_segs + sid] = o[s];
    }
}

// Concatenates the entries of a row's stored runs that pass its threshold (and are corpus
// rows, not the last tile's zero padding) into its candidate list.  The runs of all the row's
// segments are numbered 0 .. R-1 through a prefix sum of the segment counts; each chunk of
// runs is read once, counted, scanned and written.  count = cap + 1 when a segment or the
// list overflowed, which sends the row to the fold.
constexpr int kGatherThreads = 256;
constexpr int kGatherMaxSegs = 2048;  // 8 segments per part, at most 256 parts
constexpr int kGatherPer = 8;        // runs per thread per chunk
__global__ __launch_bounds__(kGatherThreads) void retrieval_gather_kernel(RetrievalArgs A, int n_segs) {
    const int r = blockIdx.x;
    if (r >= A.Lb || A.mode[r] != kModeNormal) return;
    __shared__ int s_pre[kGatherMaxSegs + 1];  // runs before segment j
    __shared__ int s_sum[kGatherThreads];
    __shared__ int s_bad;
    const float tau = A.tau[r];
    const int* cnt = A.seg_count + (size_t)r * n_segs;
    const size_t base = (size_t)r * n_segs * A.seg_cap;
    const int tid = threadIdx.x;
    // Segment counts -> exclusive prefix in s_pre (each thread scans a contiguous chunk).
    const int per = (n_segs + kGatherThreads - 1) / kGatherThreads;
    const int j0 = tid * per, j1 = min(n_segs, j0 + per);
    int mine = 0;
    bool bad = false;
    for (int j = j0; j < j1; ++j) {
        const int n = cnt[j];
        bad = bad || n > A.seg_cap;
        s_pre[j] = min(n, A.seg_cap);
        mine += min(n, A.seg_cap);
    }
    if (tid == 0) s_bad = 0;
    s_sum[tid] = mine;
    __syncthreads();
    if (bad) s_bad = 1;
    for (int d = 1; d < kGatherThreads; d <<= 1) {
        const int v = tid >= d ? s_sum[tid - d] : 0;
        __syncthreads();
        s_sum[tid] += v;
        __syncthreads();
    }
    {
        int run = s_sum[tid] - mine;
        for (int j = j0; j < j1; ++j) {
            const int n = s_pre[j];
            s_pre[j] = run;
            run += n;
        }
    }
    const int R = s_sum[kGatherThreads - 1];
    if (tid == 0) s_pre[n_segs] = R;
    __syncthreads();
    if (s_bad) {
        if (tid == 0) A.count[(size_t)r * kCandSegs] = A.cap + 1;
        return;
    }
    // Run q lives in segment j with s_pre[j] <= q < s_pre[j + 1].
    auto locate = [&](int q) {
        int lo = 0, hi = n_segs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= q) lo = mid;
            else hi = mid - 1;
        }
        return base + (size_t)lo * A.seg_cap + (size_t)(q - s_pre[lo]);
    };
    auto passes = [&](float v, int64_t key) { return v >= tau && key < A.N; };
    // One pass over the runs, in chunks of kGatherThreads * kGatherPer: thread t loads runs
    // q0 + j * kGatherThreads + t (all loads in flight together), counts their passing
    // entries, and after a block scan of the counts writes them from the running offset.
    uint32_t* dst = A.cand + (size_t)r * 2 * A.cap;
    int written = 0;  // entries of earlier chunks (block-uniform)
    for (int q0 = 0; q0 < R; q0 += kGatherThreads * kGatherPer) {
        float4 v[kGatherPer];
        uint32_t id[kGatherPer];
#pragma unroll
        for (int j = 0; j < kGatherPer; ++j) {
            const int q = q0 + j * kGatherThreads + tid;
            const size_t at = locate(q < R ? q : R - 1);
            v[j] = A.seg_runs[at];
            id[j] = A.seg_ids[at];
        }
        int n_mine = 0;
#pragma unroll
        for (int j = 0; j < kGatherPer; ++j) {
            if (q0 + j * kGatherThreads + tid >= R) id[j] = UINT32_MAX;  // past the runs: keys beyond N
            const int64_t key = (int64_t)id[j] * 4;
            n_mine += passes(v[j].x, key) + passes(v[j].y, key + 1) + passes(v[j].z, key + 2) + passes(v[j].w, key + 3);
        }
        __syncthreads();
        s_sum[tid] = n_mine;
        __syncthreads();
        for (int d = 1; d < kGatherThreads; d <<= 1) {
            const int x = tid >= d ? s_sum[tid - d] : 0;
            __syncthreads();
            s_sum[tid] += x;
            __syncthreads();
        }
        int off = written + s_sum[tid] - n_mine;
#pragma unroll
        for (int j = 0; j < kGatherPer; ++j) {
            const int64_t key = (int64_t)id[j] * 4;
            const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (passes(f[e], key + e)) {
                    if (off < A.cap) {
                        dst[off] = __float_as_uint(f[e]);
                        dst[A.cap + off] = (uint32_t)(key + e);
                    }
                    ++off;
                }
        }
        written += s_sum[kGatherThreads - 1];
    }
    if (tid == 0) A.count[(size_t)r * kCandSegs] = written > A.cap ? A.cap + 1 : written;
}

int retrieval_groups(int Lb) { return (Lb + kRetQueries - 1) / kRetQueries; }

// Key parts per query group: enough workgroups for 256 compute units, each wave keeping
// at least 8 tiles; a multiple of 8 when there are 8 or more (XCD-local parts).
int retrieval_parts(int n_groups, int64_t n_tiles) {
    int64_t p = (256 + n_groups - 1) / n_groups;
    const int64_t by_tiles = n_tiles / (8 * (kScoreThreads / kWave));
    if (p > by_tiles) p = by_tiles;
    if (p > 256) p = 256;
    if (p < 1) p = 1;
    if (p >= 8) p &= ~(int64_t)7;
    return (int)p;
}

// Runs per segment list: a segment's lane sees 4 runs per tile, each stored with probability
// about 4 p (p = 2.5 top_k / N, the candidate rate); mean plus six standard deviations and 8,
// or every run of the segment when the row keeps all keys.
int retrieval_seg_cap(int parts, int64_t n_tiles, int top_k, bool keep_all) {
    const int64_t tps = (n_tiles + parts * 4 - 1) / (parts * 4);
    const int64_t most = tps * 4;  // a segment never stores more runs than that
    if (keep_all) return (int)most;
    const double n = (double)n_tiles * kKeyTile;
    double p = 4.0 * 2.5 * top_k / n;
    if (p > 1.0) p = 1.0;
    const double mean = (double)most * p;
    int64_t cap = (int64_t)(mean + 6.0 * sqrt(mean) + 8.0);
    cap = (cap + 7) & ~(int64_t)7;
    return (int)(cap < most ? cap : most);
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
    r.n_groups = retrieval_groups(r.Lb);
    if (need_sample) {
        ProfScope ps(s, kProfRetrievalSample);
        r.parts = retrieval_parts(r.n_groups, (r.sample_n + kKeyTile - 1) / kKeyTile);
        retrieval_score_kernel<true><<<r.n_groups * r.parts, kScoreThreads, 0, s>>>(r);
    }
    hipError_t e = launch_row_prep(a, s);
    if (e != hipSuccess) return e;
    {
        ProfScope ps(s, kProfRetrievalFilter);
        const int64_t n_tiles = (r.N + kKeyTile - 1) / kKeyTile;
        r.parts = retrieval_parts(r.n_groups, n_tiles);
        r.seg_cap = retrieval_seg_cap(r.parts, n_tiles, a.top_k, !need_sample);
        retrieval_score_kernel<false><<<r.n_groups * r.parts, kScoreThreads, 0, s>>>(r);
    }
    {
        ProfScope ps(s, kProfRetrievalGather);
        retrieval_gather_kernel<<<r.Lb, kGatherThreads, 0, s>>>(r, r.parts * 8);
    }
    return launch_select_fold(a, s);
}

}  // namespace dsa
