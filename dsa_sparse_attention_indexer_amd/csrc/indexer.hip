// indexer.hip -- DSA lightning-indexer scoring and exact top-k selection for gfx950.
//
// What is computed ("GLM prefill now attends only to the keys its indexer
// picks", How it works; LiteTopK abstract):
//   score(t,s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]),  s <= p_t = pos0 + t,
//   keep the top_k keys by (score desc, key asc), emit them ascending, -1 pad.
//
// Pipeline per query block (all on one stream, no host synchronisation):
//   1. key_stats        max ||k||_2, max |k| and the lowest set-bit exponent over the
//                       causal key range (for the error bound and the exactness test)
//   2. score<sample>    bf16 MFMA scores of a strided key sample per 4-row group
//                       (LiteTopK: a small sample estimates the score range)
//   3. row_prep         per row: error bound delta_t (0 when fp32 is provably exact),
//                       threshold tau_t = (sample rank-r score) - 2 delta_t
//   4. score<filter>    bf16 MFMA scores of every causal key; keys with score >= tau_t
//                       are written back as (score, key) candidates (only promising
//                       candidates leave the chip)
//   5. select           exact top-k of the candidates: value-binned selection of the fp32
//                       k-th score, fp64 re-score of the keys within 2 delta of it, rank
//                       count with the lower-index tie rule, ascending output
//   6. fold (fallback)  rows whose candidate set could be incomplete or overflowed run
//                       the pages' blocked fold: 4,096-key blocks merged into a running
//                       exact top-k list
//
// fp32 vs the canonical fp64 order.  The fp64 order that defines ties is
//   d_h = sum_i q*k (i ascending), r_h = max(d_h, +0), s = sum_h fl(w_h r_h) (h ascending).
// |s32 - s64| <= delta_t with delta_t = 104 * 2^-24 * max_s||k_s|| * sum_h |w_h| ||q_h||:
// each 32x32x16 MFMA step is modelled as a depth-5 tree of fp32 additions with
// directed rounding (<= 10 u per step of the running magnitude, 8 steps -> 80 u of
// ||q_h|| ||k||), the 16-term per-lane head sum plus the cross-lane add adds <= 18 u,
// and the rest covers the fp64 evaluation and rounding of the bound itself.  Keys
// with s32 > kth + 2 delta are surely selected, keys below kth - 2 delta surely not;
// only the band in between is re-scored in fp64.
#include <float.h>
#include <limits.h>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kSegs = kCandSegs;  // candidate segments per row: (key half, scoring wave)

// Where block row r's query, weights, output and keys live.
struct RowRef {
    const uint16_t* q;     // [32][128]
    const float* w;        // [32]
    int32_t* out;          // [top_k]
    const uint16_t* keys;  // the sequence's k_idx rows
    int64_t pos;           // position in the sequence
    int64_t nkeys;         // keys of the sequence any of its queries may see
    int64_t tbase;         // the sequence's first tile in the tiled key copy
    int64_t ntiles;        // ... and its tile count there
    bool valid;            // a query row (not a padding or past-the-end row)
};
__device__ __forceinline__ RowRef row_ref(const IndexerArgs& P, int r) {
    if (!P.rows) {
        const int rr = r < P.Lb ? r : 0;
        return RowRef{P.q_idx + (size_t)rr * kIdxHeads * kIdxDim, P.w + (size_t)rr * kIdxHeads,
                      P.out + (size_t)rr * P.top_k, P.k_idx, P.pos0 + rr, P.N, 0, P.n_ktiles, r < P.Lb};
    }
    const RowInfo ri = P.rows[r < P.Lb ? r : 0];
    const bool v = r < P.Lb && ri.qrow >= 0;
    const int64_t q = ri.qrow >= 0 ? ri.qrow : 0;
    return RowRef{P.q_idx + (size_t)q * kIdxHeads * kIdxDim, P.w + (size_t)q * kIdxHeads,
                  P.out + (size_t)q * P.top_k, P.k_idx + (size_t)ri.kbase * kIdxDim, ri.pos, ri.nkeys,
                  ri.tbase, (ri.nkeys + kKeyTileKeys - 1) / kKeyTileKeys, v};
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int bf16_lsb_exp(uint16_t b) {
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    if (e == 0) return -133 + __builtin_ctz((unsigned)m);
    return (e - 134) + __builtin_ctz((unsigned)(m | 0x80));
}

__device__ __forceinline__ int f32_lsb_exp(float f) {
    uint32_t u = __float_as_uint(f) & 0x7fffffffu;
    int e = (int)(u >> 23);
    uint32_t m = u & 0x7fffffu;
    if (e == 0) return -149 + __builtin_ctz(m);
    return (e - 150) + __builtin_ctz(m | 0x800000u);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Wave-aggregated append: lanes with pred get consecutive slots from *counter (one LDS
// atomic per wave).  Returns the lane's slot, or -1.  Call with every lane of the wave
// that reached this point.
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return -1;
    const int leader = __builtin_ctzll(m);
    int base = 0;
    if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(counter, __builtin_popcountll(m));
    base = __shfl(base, leader);
    return pred ? base + mbcnt64(m) : -1;
}

// Canonical fp64 term fl(w_h * max(0, sum_i q_h[i] k[i])) with i ascending.  A product of
// two bf16 values is exact in fp64, so fma(q, k, d) rounds exactly as d + fl(q*k) does.
__device__ double canonical_head_term(const uint16_t* __restrict__ q_h,
                                      const uint16_t* __restrict__ k_row, float w_h) {
#pragma clang fp contract(off)
    double d = 0.0;
    const u16x8* qa = reinterpret_cast<const u16x8*>(q_h);
    const u16x8* ka = reinterpret_cast<const u16x8*>(k_row);
    for (int c = 0; c < kIdxDim / 8; ++c) {
        const u16x8 qv = qa[c], kv = ka[c];
        for (int j = 0; j < 8; ++j)
            d = __builtin_fma((double)bf16_bits_to_float(qv[j]), (double)bf16_bits_to_float(kv[j]), d);
    }
    const double r = d > 0.0 ? d : 0.0;
    return (double)w_h * r;
}

// ------------------------------------------------------------------ 1. key stats

static_assert(kKeyTileKeys == kKeyTile, "scoring tiles and the tiled key copy disagree");

// One wave per 32-key tile (tile = global wave index, then strided): eight 1-KB row-major
// loads (16 lanes per key row), the statistics, then the tile is re-ordered through LDS
// and written as eight 1-KB stores in the scoring order.  Keys past the end are zero.
constexpr int kStatsThreads = 256;
constexpr int kStatsRowPad = 17;  // LDS row stride in 16-byte chunks (16 + 1 against bank conflicts)
// seqs == null: one sequence of n_keys keys.  Otherwise tile t belongs to the sequence whose
// tile range holds it, and its keys are that sequence's.
__global__ __launch_bounds__(kStatsThreads) void key_stats_kernel(const uint16_t* __restrict__ k_idx,
                                                                  int64_t n_keys, const SeqKeys* seqs,
                                                                  int n_seqs, int64_t n_tiles,
                                                                  KeyStats* slots,
                                                                  uint16_t* __restrict__ k_tile) {
    __shared__ u16x8 s_t[kStatsThreads / kWave][kKeyTileKeys * kStatsRowPad];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u16x8* st = s_t[wave];
    float nmax = 0.f, amax = 0.f;
    int emin = INT_MAX;
    const int64_t n_waves = (int64_t)gridDim.x * (kStatsThreads / kWave);
    for (int64_t t = (int64_t)blockIdx.x * (kStatsThreads / kWave) + wave; t < n_tiles; t += n_waves) {
        const uint16_t* src = k_idx;
        int64_t kn = n_keys, tl = t;
        if (seqs) {  // first sequence whose tiles end after t (wave-uniform search)
            int lo = 0, hi = n_seqs - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (t < seqs[mid].tend) hi = mid;
                else lo = mid + 1;
            }
            const SeqKeys sk = seqs[lo];
            src = k_idx + (size_t)sk.kbase * kIdxDim;
            kn = sk.nkeys;
            tl = t - sk.tbase;
        }
        u16x8 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // chunk q = 64 i + lane: key q / 16 of the tile, dims 8 (q % 16) ..
            const int q = i * 64 + lane;
            const int64_t key = tl * kKeyTileKeys + (q >> 4);
            v[i] = key < kn ? reinterpret_cast<const u16x8*>(src + key * kIdxDim)[q & 15] : u16x8{};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t b = v[i][j];
                const float x = bf16_bits_to_float((uint16_t)b);
                ss = fmaf(x, x, ss);
                amax = fmaxf(amax, fabsf(x));
                // exponent of the lowest set bit (branch-free form of bf16_lsb_exp)
                const uint32_t mag = b & 0x7fffu, e = mag >> 7, m = mag & 0x7fu;
                const int l = (int)(e ? e : 1u) - 134 + __builtin_ctz((e ? 0x80u : 0u) | m | (mag ? 0u : 1u));
                emin = mag ? min(emin, l) : emin;
            }
            for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
            nmax = fmaxf(nmax, sqrtf(ss));
            const int q = i * 64 + lane;
            if (k_tile) st[(q >> 4) * kStatsRowPad + (q & 15)] = v[i];
        }
        // Store i: lane l = 32 hf + c writes key c, dims 64 hf + 8 i .. (the scoring order).
        // (LDS accesses of one wave complete in order, so the reads see this tile's writes
        // and the next tile's writes come after them.)  No copy wanted: statistics only.
        if (k_tile) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u16x8 w = st[(lane & 31) * kStatsRowPad + (lane >> 5) * 8 + i];
                reinterpret_cast<u16x8*>(k_tile)[t * (int64_t)(kKeyTileBytes / 16) + i * 64 + lane] = w;
            }
        }
    }
    nmax = wave_max(nmax);
    amax = wave_max(amax);
    emin = wave_min_i(emin);
    __shared__ float s_n[4], s_a[4];
    __shared__ int s_e[4];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_n[w] = nmax;
        s_a[w] = amax;
        s_e[w] = emin;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) {
            nmax = fmaxf(nmax, s_n[i]);
            amax = fmaxf(amax, s_a[i]);
            emin = min(emin, s_e[i]);
        }
        // 128 fp32 squares+adds and the sqrt: relative error < 2^-16; pad by 2^-14.
        const float up = nmax * (1.0f + 1.0f / 16384.0f);
        slots[blockIdx.x] = KeyStats{__float_as_uint(up), __float_as_uint(amax), emin, 0};
    }
}

// ------------------------------------------------------------------ 2/4. MFMA scoring

// One workgroup = 8 consecutive query rows over one half of their causal keys (two
// workgroups per row group; the half follows the XCD the workgroup lands on, so each
// XCD's L2 streams only its half of the key cache).  Each of the 4 waves scores all 8
// rows over its own contiguous quarter of that half: candidate segment 4*half + wave, so
// a row's 8 segments cover ascending key ranges.  Eight rows per wave means every key
// byte brought into the CU feeds 8 x 32 heads of MFMA work, which halves the per-CU key
// stream that the vector L1 has to sustain compared with four rows.
//
// Lane l owns head (l & 31) of the A operand and key (l & 31) of the B operand; its half
// (l >> 5) holds dimensions [64*half, 64*half+64) of both, eight MFMA K-steps of 8.  Key
// tiles are loaded straight into the B layout, three tiles ahead.  The 8 rows' query
// fragments fill the AGPRs (the MFMAs read A operands from there directly), leaving the
// VGPRs to the accumulators and the key tiles; the head weights are read from LDS.
//
// The rows run as four pairs: the MFMA chains of one pair execute under the epilogue
// (ReLU, weighted head sum, filter) of the previous pair.  After the cross-half add both
// lane halves hold the scores of both rows of a pair, so the low half files survivors
// of the first row and the high half those of the second.  Survivors are staged in LDS
// per (wave, row) and flushed to the row's segment as coalesced (score, key) runs, with
// wave-uniform counters (no atomics).
constexpr int kRowsPerWave = kRowsPerGroup;   // 8
constexpr int kPairs = kRowsPerWave / 2;
constexpr int kKeyHalves = 2;
constexpr int kStageSlots = 64;  // LDS staging entries per (wave, row) for filter survivors
static_assert(kKeyHalves * (kScoreThreads / kWave) == kSegs, "one candidate segment per (half, wave)");

// sum_e w_e * r[e] with e ascending (fused multiply-adds), where lane 16g + e of W holds w_e
// for the lanes of its 16-lane row g: DPP row_newbcast:e hands that lane's value to every
// lane of the row, so the weights take one register per query row instead of 16.  A DPP
// source needs two wait states after a VALU write of it; W is written once, before the
// scoring loop, and the build checks the generated code for any closer write.
__device__ __forceinline__ float weighted_head_sum(float W, const float (&r)[16]) {
    float p;
    asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf"
        : "=&v"(p)
        : "v"(W), "v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]), "v"(r[4]), "v"(r[5]), "v"(r[6]), "v"(r[7]));
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %7 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %8 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(p)
        : "v"(W), "v"(r[8]), "v"(r[9]), "v"(r[10]), "v"(r[11]), "v"(r[12]), "v"(r[13]), "v"(r[14]), "v"(r[15]));
    return p;
}

// Scheduling pattern for the region ending here (the next pair's 16 MFMAs and this
// pair's epilogue): one MFMA, then two VALU instructions, repeated.  Spreading the
// epilogue thinly keeps the matrix pipe fed (the default schedule bunches the VALU work
// and leaves the last MFMAs back to back).
__device__ __forceinline__ void interleave_with_mfma() {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x2, 2, 0);  // VALU
    }
}

// kSkip: a row pair with no live row (padding, or rows that keep all keys) skips its MFMAs
// and epilogue (wave-uniform branches); for groups holding few live rows (decode, batches of
// single queries).  Without it the schedule is branch-free.
template <bool kSample, bool kSkip>
struct ScoreTile {
    const IndexerArgs& P;
    const uint16_t* keys;       // the group's sequence: k_idx rows (sample)
    const u16x8* ktile;         // ... and its tiled copy (filter)
    uint32_t n_kt;              // ... tiles of that copy
    const bf16x8 (&a)[kRowsPerWave][8];
    const float (&wl)[kRowsPerWave];  // per row: lane 16g + e holds the weight of its half's head e
    // Per lane half: parameters of row 2q + hf of row pair q.
    float tau_m[kPairs];     // candidate threshold (+inf for rows the filter skips)
    bool live_m[kPairs];
    float* sample0;     // sample: row 0's sample list (rows are sample_stride apart)
    uint2* cand0;       // filter: row 0's segment (rows are cap apart)
    uint32_t n0;        // sample: keys of the group's first row
    uint32_t S;         // sample: sample size
    float s_ratio;      // sample: key stride n0 / S (any in-range keys would do)
    int lane, hf, col;
    int colm;           // col - hf
    int first_pos;      // position of the group's first row
    int first_row;      // the group's first row in the block
    int seg;
    int (&cnt)[kRowsPerWave];   // survivors so far per row (including any past seg)
    uint2* lbuf;                // filter: this wave's LDS staging lists, kStageSlots per row
    int lcnt[kRowsPerWave];     // entries staged per row (wave-uniform)
    int gcnt[kRowsPerWave];     // entries already flushed to the segment per row
    uint32_t tile0;     // first tile of this wave's contiguous range (wave-uniform)
    bool pl[kPairs];    // kSkip: row pair q has a live row (wave-uniform)

    __device__ __forceinline__ uint32_t pos_of(int it) const { return (tile0 + (uint32_t)it) * kKeyTile + col; }

    // Tile indices past the wave's range still address valid keys (clamped), so callers
    // need no guard.  The filter reads the tiled key copy (1 KB per load instruction); the
    // sample's strided keys come from the row-major keys.
    __device__ __forceinline__ void load(bf16x8 (&b)[8], int it) const {
        if (kSample) {
            const uint32_t key = min((uint32_t)((float)pos_of(it) * s_ratio), n0 - 1u);
            const u16x8* kp = reinterpret_cast<const u16x8*>(keys + (size_t)key * kIdxDim + hf * 64);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) b[kk] = __builtin_bit_cast(bf16x8, kp[kk]);
        } else {
            const uint32_t t = min(tile0 + (uint32_t)it, n_kt - 1u);
            const u16x8* kp = ktile + (size_t)t * (kKeyTileBytes / 16) + lane;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) b[kk] = __builtin_bit_cast(bf16x8, kp[kk * 64]);
        }
    }

    // MFMA chains of rows J0 and J0+1 over one key tile, interleaved.
    template <int J0>
    __device__ __forceinline__ void mfma2(f32x16 (&acc)[kRowsPerWave], const bf16x8 (&b)[8]) const {
        f32x16 c0 = {}, c1 = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            c0 = mfma_32x32x16(a[J0][kk], b[kk], c0);
            c1 = mfma_32x32x16(a[J0 + 1][kk], b[kk], c1);
        }
        acc[J0] = c0;
        acc[J0 + 1] = c1;
    }

    // Scores of rows J0, J0+1 for tile it: ReLU, weighted head sum, then the sample store
    // or the threshold filter.
    template <int J0>
    __device__ __forceinline__ void epilogue2(const f32x16 (&acc)[kRowsPerWave], int it) {
        const uint32_t pos = pos_of(it);
        float part[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            float r[16];
#pragma unroll
            for (int e = 0; e < 16; ++e)  // ReLU on the bit pattern: negatives and -0 -> +0
                r[e] = __int_as_float(max(__float_as_int(acc[J0 + jj][e]), 0));
            part[jj] = weighted_head_sum(wl[J0 + jj], r);
        }
        // Each lane half holds its 16 heads' partial sum of both rows.  One swap of the
        // upper half of row J0 with the lower half of row J0+1 leaves lane half hf with
        // both partial sums of row J0 + hf, which handles that row from here on.
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                         false, false);
        const float s_mine = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) + 0.0f;
        const uint32_t j_mine = J0 + hf;
        constexpr int q = J0 / 2;
        interleave_with_mfma();
        if (kSample) {
            if (pos < S && live_m[q]) sample0[j_mine * (uint32_t)P.sample_stride + pos] = s_mine;
        } else {
            // Rows not scored here have an infinite threshold.  Causality, pos <= p_row
            // with p_row = first_pos + J0 + hf, is tested as col - hf <= first_pos + J0 -
            // 32 * tile: one compare against a wave-uniform bound.
            const int lim = first_pos + J0 - (int)((tile0 + (uint32_t)it) * kKeyTile);
            // (Two ballots of single compares: each is the compare's own lane mask.)
            const bool above = s_mine >= tau_m[q], causal = colm <= lim;
            const uint64_t m = __builtin_amdgcn_ballot_w64(above) & __builtin_amdgcn_ballot_w64(causal);
            const bool keep = above && causal;
            if (m) {
                const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
                // Slot within the row's staging list: entries already staged plus the
                // survivors among the lower lanes of this half.
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(m1, __builtin_amdgcn_mbcnt_lo(hf ? 0u : m0, 0u));
                const uint32_t o = (uint32_t)(hf ? lcnt[J0 + 1] : lcnt[J0]) + below;  // < kStageSlots
                if (keep) lbuf[j_mine * kStageSlots + o] = uint2{__float_as_uint(s_mine), pos};
                const int c0 = __builtin_popcount(m0), c1 = __builtin_popcount(m1);
                lcnt[J0] += c0;
                lcnt[J0 + 1] += c1;
                cnt[J0] += c0;
                cnt[J0 + 1] += c1;
            }
        }
    }

    // Staged survivors of row j -> its global segment: one coalesced 8-byte store per lane.
    // Entries past the segment's capacity are dropped (the row is then re-done by the
    // fold, which the count past seg signals).
    __device__ __forceinline__ void flush_row(int j) {
        uint32_t base = (uint32_t)gcnt[j];
        if (P.parts > 2) {  // shared list: reserve the slots (one atomic per flush)
            uint32_t b = 0u;
            if (lane == 0) b = atomicAdd(reinterpret_cast<unsigned*>(&P.count[(size_t)(first_row + j) * kSegs]),
                                         (unsigned)lcnt[j]);
            base = __builtin_amdgcn_readfirstlane(b);
        }
        if (lane < lcnt[j]) {
            const uint2 e = lbuf[j * kStageSlots + lane];
            const uint32_t o = base + (uint32_t)lane;
            if (o < (uint32_t)seg) cand0[(uint32_t)j * (uint32_t)P.cap + o] = e;
        }
        gcnt[j] += lcnt[j];
        lcnt[j] = 0;
    }
    // A tile adds at most 32 survivors per row, so rows holding kStageSlots/2 or more are
    // flushed before each tile: a staging list never overflows, and global stores (which
    // the in-order memory counter would make the key-tile loads wait for) stay rare.
    __device__ __forceinline__ void flush_full() {
        if (kSample) return;
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
            if (lcnt[j] >= kStageSlots / 2) flush_row(j);
    }
    __device__ __forceinline__ void flush_all() {
        if (kSample) return;
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
            if (lcnt[j] > 0) flush_row(j);
    }

    // One tile: each pair's MFMA chains run under the epilogue of the pair before (pair 3
    // of tile it-1 for pair 0).  The two compiler memory barriers keep each half-step's
    // staging-list accesses in their half-step (measured slightly faster than without).
    __device__ __forceinline__ void step(f32x16 (&acc)[kRowsPerWave], const bf16x8 (&b)[8], int it) {
        flush_full();
        asm volatile("" ::: "memory");
        if (kSkip) {
            if (pl[0]) mfma2<0>(acc, b);
            if (pl[3]) epilogue2<6>(acc, it - 1);
            if (pl[1]) mfma2<2>(acc, b);
            if (pl[0]) epilogue2<0>(acc, it);
            asm volatile("" ::: "memory");
            if (pl[2]) mfma2<4>(acc, b);
            if (pl[1]) epilogue2<2>(acc, it);
            if (pl[3]) mfma2<6>(acc, b);
            if (pl[2]) epilogue2<4>(acc, it);
            return;
        }
        mfma2<0>(acc, b);
        epilogue2<6>(acc, it - 1);
        mfma2<2>(acc, b);
        epilogue2<0>(acc, it);
        asm volatile("" ::: "memory");
        mfma2<4>(acc, b);
        epilogue2<2>(acc, it);
        mfma2<6>(acc, b);
        epilogue2<4>(acc, it);
    }
};

template <bool kSample, bool kSkip>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(IndexerArgs P, int n_groups) {
    // Workgroups go round-robin over the 8 XCDs: XCDs 0-3 take key half 0, 4-7 half 1.
    // Two parts: XCDs 0-3 take key half 0 and 4-7 half 1.  More parts: consecutive
    // workgroups take consecutive parts of one group.
    const bool appended = P.parts > 2;
    int part, g;
    if (!appended) {
        const int xcd = blockIdx.x & 7;
        part = xcd >> 2;
        g = (int)(blockIdx.x >> 3) * 4 + (xcd & 3);
    } else {
        part = (int)blockIdx.x % P.parts;
        g = (int)blockIdx.x / P.parts;
    }
    if (g >= n_groups) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;
    const int col = lane & 31;
    const int segment = part * (kScoreThreads / kWave) + wave;
    const int n_segs = P.parts * (kScoreThreads / kWave);
    __shared__ __attribute__((aligned(16))) float s_w[kRowsPerWave][2][16];
    __shared__ uint2 s_stage[kScoreThreads / kWave][kRowsPerWave * kStageSlots];

    const int seg = appended ? P.cap : P.cap / kSegs;  // capacity of this wave's list per row
    float tau_r[kRowsPerWave];
    bool live[kRowsPerWave];
    int64_t n_keys = 0;
    const int r0 = g * kRowsPerWave;
    const RowRef gref = row_ref(P, r0);  // a group's rows share one sequence
    const uint16_t* qrow[kRowsPerWave];
    const float* wrow[kRowsPerWave];
    uint32_t S = 0, n0 = 0;
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
        const int r = r0 + j;
        const RowRef ref = row_ref(P, r);
        const bool valid = ref.valid;
        qrow[j] = valid ? ref.q : gref.q;
        wrow[j] = valid ? ref.w : gref.w;
        const int64_t p = ref.pos;  // <= nkeys - 1
        if (kSample) {
            live[j] = valid;
            tau_r[j] = 0.f;
        } else {
            const bool use = valid && P.mode[r] == kModeNormal;
            live[j] = use;
            tau_r[j] = use ? P.tau[r] : INFINITY;
            if (use && p + 1 > n_keys) n_keys = p + 1;
        }
    }
    if (kSample) {
        const int64_t p = gref.pos;
        n0 = (uint32_t)(p + 1);
        S = (uint32_t)sample_size(n0, P.top_k, P.cap);
        n_keys = S;
    }
    // Weights in the order each lane half reads them: head 8*(i/4) + 4*half + i%4.
    {
        const int j = threadIdx.x >> 5, h2 = (threadIdx.x >> 4) & 1, i = threadIdx.x & 15;
        s_w[j][h2][i] = wrow[j][8 * (i >> 2) + 4 * h2 + (i & 3)];
    }
    __syncthreads();
    float wl[kRowsPerWave];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) wl[j] = s_w[j][hf][lane & 15];

    int cnt[kRowsPerWave] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n_keys > 0) {
        bf16x8 a[kRowsPerWave][8];
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
            const u16x8* qp = reinterpret_cast<const u16x8*>(qrow[j] + (size_t)col * kIdxDim + hf * 64);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                a[j][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
                asm volatile("" : "+a"(a[j][kk]));  // keep the query fragments in AGPRs
            }
        }
        // Segment s covers the contiguous tile range [s*tps, (s+1)*tps).
        const int n_tiles = (int)((n_keys + kKeyTile - 1) / kKeyTile);
        const int tps = (n_tiles + n_segs - 1) / n_segs;
        const int t0 = segment * tps;
        const int n_my = n_tiles > t0 ? min(n_tiles - t0, tps) : 0;
        // Rows of a group are consecutive (invalid rows never store), so every row's
        // list is addressed from row 0's.
        ScoreTile<kSample, kSkip> T{P, gref.keys,
                             reinterpret_cast<const u16x8*>(P.k_tile) + (size_t)gref.tbase * (kKeyTileBytes / 16),
                             (uint32_t)gref.ntiles, a, wl,
                             {hf ? tau_r[1] : tau_r[0], hf ? tau_r[3] : tau_r[2], hf ? tau_r[5] : tau_r[4],
                              hf ? tau_r[7] : tau_r[6]},
                             {hf ? live[1] : live[0], hf ? live[3] : live[2], hf ? live[5] : live[4],
                              hf ? live[7] : live[6]},
                             kSample ? P.sample + (size_t)r0 * P.sample_stride : nullptr,
                             kSample ? nullptr : P.cand + (size_t)r0 * P.cap + (appended ? 0 : (size_t)segment * seg),
                             n0, S, kSample && S > 0 ? (float)n0 / (float)S : 0.f, lane, hf, col, col - hf,
                             (int)gref.pos, r0, seg, cnt,
                             s_stage[wave], {0, 0, 0, 0, 0, 0, 0, 0}, {0, 0, 0, 0, 0, 0, 0, 0}, (uint32_t)t0,
                             {kSkip && (live[0] || live[1]), kSkip && (live[2] || live[3]),
                              kSkip && (live[4] || live[5]), kSkip && (live[6] || live[7])}};
        // Tile it sits in buffer it % 3; tile it+3 is loaded once tile it's MFMAs are issued.
        bf16x8 b0[8], b1[8], b2[8];
        f32x16 acc[kRowsPerWave];
        if (n_my > 0) {
            T.load(b0, 0);
            T.load(b1, 1);
            T.load(b2, 2);
            if (!kSkip || T.pl[0]) T.template mfma2<0>(acc, b0);
            if (!kSkip || T.pl[1]) T.template mfma2<2>(acc, b0);
            if (!kSkip || T.pl[0]) T.template epilogue2<0>(acc, 0);
            if (!kSkip || T.pl[2]) T.template mfma2<4>(acc, b0);
            if (!kSkip || T.pl[1]) T.template epilogue2<2>(acc, 0);
            if (!kSkip || T.pl[3]) T.template mfma2<6>(acc, b0);
            T.load(b0, 3);
            if (!kSkip || T.pl[2]) T.template epilogue2<4>(acc, 0);
            int it = 1;
            for (; it + 2 < n_my; it += 3) {
                T.step(acc, b1, it);
                T.load(b1, it + 3);
                T.step(acc, b2, it + 1);
                T.load(b2, it + 4);
                T.step(acc, b0, it + 2);
                T.load(b0, it + 5);
            }
            if (it < n_my) T.step(acc, b1, it);
            if (it + 1 < n_my) T.step(acc, b2, it + 1);
            T.flush_full();  // the last epilogue adds up to 32 more entries to rows 6, 7
            if (!kSkip || T.pl[3]) T.template epilogue2<6>(acc, n_my - 1);
            T.flush_all();
        }
    }
    if (!kSample && lane == 0) {
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
            if (r0 + j < P.Lb && !appended) P.count[(size_t)(r0 + j) * kSegs + segment] = cnt[j];  // pad rows too (0)
    }
}

// ------------------------------------------------------------------ block-wide selection

// Up to kSegs (score, key) lists, read as one.
struct CandList {
    const float* s[kSegs];
    const int* i[kSegs];
    int n[kSegs];
    int nseg;
};

constexpr int kBins = 2048;
constexpr int kDirect = 512;
constexpr int kRescoreKeys = 16;   // band keys per fp64 MFMA block
constexpr int kRescoreRound = 128;  // band keys re-scored per round (8 blocks x 2 head halves)

// One row's selection scratch.  The phases use the union in turn: binned k-th search
// (sel), fp64 re-score staging (rs), then the selected keys (out, fold path only).
struct SelectScratch {
    union {
        struct {
            int hist[kBins];
            float direct[kDirect];
        } sel;
        int out[kMaxTopK];
        double term[kRescoreRound][kIdxHeads];  // head terms of one re-score round
    };
    int bad[kRescoreRound];  // band keys of the round whose dot products need the sequential order
    float red_f[32];
    int red_i[32];
    int sh[16];
};

__device__ __forceinline__ void block_minmax(float& mn, float& mx, SelectScratch& S) {
    mn = wave_min(mn);
    mx = wave_max(mx);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        S.red_f[w] = mn;
        S.red_f[16 + w] = mx;
    }
    __syncthreads();
    mn = S.red_f[0];
    mx = S.red_f[16];
    for (int i = 1; i < nw; ++i) {
        mn = fminf(mn, S.red_f[i]);
        mx = fmaxf(mx, S.red_f[16 + i]);
    }
    __syncthreads();
}

// Inclusive scan of one int per thread in thread order (block of at most 16 waves).
__device__ __forceinline__ int block_incl_scan(int v, SelectScratch& S) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    __syncthreads();
    if (lane == 63) S.red_i[w] = x;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += S.red_i[i];
    __syncthreads();
    return x + base;
}

__device__ __forceinline__ int bin_of(float s, float vmin, double scale) {
    const double d = ((double)s - (double)vmin) * scale;
    const int b = (int)d;
    return b < kBins - 1 ? b : kBins - 1;
}

// Values owned by this thread: a block-strided walk over a CandList ...
struct ListSrc {
    const CandList& L;
    template <class F>
    __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
        for (int g = 0; g < kSegs; ++g)
            if (g < L.nseg)
                for (int i = threadIdx.x; i < L.n[g]; i += blockDim.x) f(L.s[g][i] + 0.0f);
    }
};
// ... or this thread's register-resident chunk.
template <int CH>
struct RegSrc {
    const float (&v)[CH];
    int nv;
    template <class F>
    __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
        for (int e = 0; e < CH; ++e)
            if (e < nv) f(v[e]);
    }
};

// k-th largest value (1-based) under the float order (-0 == +0), by value-linear binning
// (LiteTopK's bins: cheap even when every score shares an exponent) refined up to three
// times, then a rank count over the crossing bin.  Requires 1 <= k <= total.  Returns
// false (uniformly) if a bin still holds more than kDirect distinct values after that.
template <class Src>
__device__ bool block_kth_binned(const Src& src, int k, float* out, SelectScratch& S) {
    constexpr int kLevels = 3;
    float vmin = INFINITY, vmax = -INFINITY;
    src.for_each([&](float v) {
        vmin = fminf(vmin, v);
        vmax = fmaxf(vmax, v);
    });
    block_minmax(vmin, vmax, S);
    float lv_min[kLevels];
    double lv_scale[kLevels];
    int lv_bin[kLevels];
    int nlv = 0, above = 0;
    auto active = [&](float v) {
        bool in = true;
#pragma unroll
        for (int l = 0; l < kLevels; ++l)
            if (l < nlv) in = in && bin_of(v, lv_min[l], lv_scale[l]) == lv_bin[l];
        return in;
    };
    for (;;) {
        if (vmin == vmax) {
            *out = vmin;
            return true;
        }
        const double scale = (double)kBins / ((double)vmax - (double)vmin);
        for (int i = threadIdx.x; i < kBins; i += blockDim.x) S.sel.hist[i] = 0;
        __syncthreads();
        src.for_each([&](float v) {
            if (active(v)) atomicAdd(&S.sel.hist[bin_of(v, vmin, scale)], 1);
        });
        __syncthreads();
        // Descending bin order: thread t owns bins kBins-1-t*per down to kBins-per-t*per.
        const int per = kBins / blockDim.x;
        int c = 0;
        for (int j = 0; j < per; ++j) c += S.sel.hist[kBins - 1 - threadIdx.x * per - j];
        const int incl = block_incl_scan(c, S) + above;
        const int excl = incl - c;
        if (threadIdx.x == 0) S.sh[0] = -1;
        __syncthreads();
        if (excl < k && k <= incl) {
            int acc = excl;
            for (int j = 0; j < per; ++j) {
                const int b = kBins - 1 - threadIdx.x * per - j;
                if (acc + S.sel.hist[b] >= k) {
                    S.sh[0] = b;
                    S.sh[1] = acc;
                    S.sh[2] = S.sel.hist[b];
                    break;
                }
                acc += S.sel.hist[b];
            }
        }
        __syncthreads();
        const int b = S.sh[0];
        above = S.sh[1];
        const int nb = S.sh[2];
        __syncthreads();
        if (b < 0) return false;  // unreachable for 1 <= k <= total
#pragma unroll
        for (int l = 0; l < kLevels; ++l)
            if (l == nlv) {
                lv_min[l] = vmin;
                lv_scale[l] = scale;
                lv_bin[l] = b;
            }
        ++nlv;
        if (nb <= kDirect) {
            if (threadIdx.x == 0) S.sh[3] = 0;
            __syncthreads();
            src.for_each([&](float v) {
                const int o = wave_append(active(v), &S.sh[3]);
                if (o >= 0 && o < kDirect) S.sel.direct[o] = v;
            });
            __syncthreads();
            const int n = S.sh[3] < kDirect ? S.sh[3] : kDirect;
            const int r = k - above;  // rank inside the bin, 1-based
            for (int x = threadIdx.x; x < n; x += blockDim.x) {
                const float vx = S.sel.direct[x];
                int gt = 0, ge = 0;
                for (int y = 0; y < n; ++y) {
                    const float vy = S.sel.direct[y];
                    gt += vy > vx;
                    ge += vy >= vx;
                }
                if (gt < r && r <= ge) S.red_f[31] = vx;  // every writer holds the same value
            }
            __syncthreads();
            *out = S.red_f[31];
            __syncthreads();
            return true;
        }
        if (nlv == kLevels) return false;
        vmin = INFINITY;
        vmax = -INFINITY;
        src.for_each([&](float v) {
            if (active(v)) {
                vmin = fminf(vmin, v);
                vmax = fmaxf(vmax, v);
            }
        });
        block_minmax(vmin, vmax, S);
    }
}

// Bitonic sort (ascending) of n = power of two ints in LDS.  Wave w owns the pairs
// [w*pw, (w+1)*pw); stages whose stride is at most pw stay inside that wave's chunk and
// need no block barrier (LDS accesses of one wave complete in order).
__device__ void block_bitonic_sort(int* a, int n) {
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pairs = n >> 1;
    int pw = 1;
    while (pw * nw < pairs) pw <<= 1;
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int j = lane; j < pw; j += 64) {
                const int i = w * pw + j;
                if (i < pairs) {
                    const int lo = 2 * i - (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool asc = (lo & size) == 0;
                    const int x = a[lo], y = a[hi];
                    if ((x > y) == asc) {
                        a[lo] = y;
                        a[hi] = x;
                    }
                }
            }
            const int next = stride > 1 ? stride >> 1 : size;  // stride of the following stage
            if (stride > pw || (next > pw && size < n) || (stride == 1 && size == n)) __syncthreads();
            else __builtin_amdgcn_wave_barrier();
        }
    }
}

// fp64 canonical scores of band entries [0, nb) (keys in band_key), in place into band_s.
//
// The canonical head dot product d_h = sum_i q_i k_i is a sequential fp64 sum of exact
// bf16 x bf16 products.  When every product is a multiple of 2^e (e = lowest set-bit
// exponent of q_h plus that of k) and sum_i |q_i k_i| <= |q_h|_1 |k|_inf < 2^(53+e),
// every partial sum in any order is exactly representable, so the sequential sum equals
// the exact one and any summation order gives it.  Those dot products run on fp64 MFMA
// (16 band keys x 16 heads x 4 dims per instruction); keys failing the test take the
// sequential path.  The head terms fl(w_h max(d_h, +0)) and their ascending-h sum are
// always evaluated in the canonical order.
__device__ __forceinline__ void band_rescore(int nb, const int* band_key, double* band_s, const uint16_t* __restrict__ q_row,
                             const float* __restrict__ w_row, const QHeadStat* __restrict__ qs_row,
                             const uint16_t* __restrict__ k_idx, SelectScratch& S) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    for (int m0 = 0; m0 < nb; m0 += kRescoreRound) {
        if (threadIdx.x < kRescoreRound) S.bad[threadIdx.x] = 0;
        __syncthreads();
        // Wave w: block w/2 of the round (band keys m0 + 16*(w/2) ..), heads 16*(w%2) ..
        // Lane (g, c) feeds key 16*(w/2) + c (A) and head 16*(w%2) + c (B), dimensions
        // 32g .. 32g+31, one per K-step.
        for (int wb = wave; wb < 2 * (kRescoreRound / kRescoreKeys); wb += nwaves) {
            const int mb = m0 + kRescoreKeys * (wb >> 1);
            if (mb >= nb) continue;
            const int head = 16 * (wb & 1) + c;
            const int key = band_key[mb + c < nb ? mb + c : mb];
            const u16x8* kp = reinterpret_cast<const u16x8*>(k_idx + (size_t)key * kIdxDim + 32 * g);
            const u16x8* qp = reinterpret_cast<const u16x8*>(q_row + head * kIdxDim + 32 * g);
            u16x8 kv[4], qv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kv[j] = kp[j];
                qv[j] = qp[j];
            }
            // Exactness statistics of key mb + c over all 128 dimensions.
            float kinf = 0.f;
            int ke = INT_MAX;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kinf = fmaxf(kinf, fabsf(bf16_bits_to_float(kv[j][e])));
                    if ((kv[j][e] & 0x7fff) != 0) ke = min(ke, bf16_lsb_exp(kv[j][e]));
                }
            kinf = fmaxf(kinf, __shfl_xor(kinf, 16));
            kinf = fmaxf(kinf, __shfl_xor(kinf, 32));
            ke = min(ke, __shfl_xor(ke, 16));
            ke = min(ke, __shfl_xor(ke, 32));
            f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int ks = 0; ks < 32; ks += 2) {
                const double a0 = (double)bf16_bits_to_float(kv[ks >> 3][ks & 7]);
                const double b0 = (double)bf16_bits_to_float(qv[ks >> 3][ks & 7]);
                const double a1 = (double)bf16_bits_to_float(kv[(ks + 1) >> 3][(ks + 1) & 7]);
                const double b1 = (double)bf16_bits_to_float(qv[(ks + 1) >> 3][(ks + 1) & 7]);
                acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc1, 0, 0, 0);
            }
            // Lane (g, c) holds d for keys mb + g + 4i (i = 0..3) and its head.
            const double wh = (double)w_row[head];
            const double qh1 = qs_row[head].l1;
            const int qhe = qs_row[head].e;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = g + 4 * i;
                const float kinf_m = __shfl(kinf, m);
                const int ke_m = __shfl(ke, m);
                if (mb + m < nb) {
                    const double d = acc0[i] + acc1[i];
                    const bool exact = kinf_m == 0.f || qhe == INT_MAX ||
                                       qh1 * (double)kinf_m < ldexp(1.0, 53 + qhe + ke_m);
                    const int slot = mb - m0 + m;
                    if (!exact) S.bad[slot] = 1;
                    const double r = d > 0.0 ? d : 0.0;
                    S.term[slot][head] = wh * r;  // a lone product: nothing to contract
                }
            }
        }
        __syncthreads();
        // Keys whose dot products could round: the canonical sequential evaluation.
        for (int it = threadIdx.x; it < kRescoreRound * kIdxHeads; it += blockDim.x) {
            const int bl = it >> 5, h = it & 31;
            if (m0 + bl < nb && S.bad[bl])
                S.term[bl][h] = canonical_head_term(q_row + h * kIdxDim,
                                                    k_idx + (size_t)band_key[m0 + bl] * kIdxDim, w_row[h]);
        }
        __syncthreads();
        if (threadIdx.x < kRescoreRound && m0 + (int)threadIdx.x < nb) {
#pragma clang fp contract(off)
            double sum = 0.0;
            for (int h = 0; h < kIdxHeads; ++h) sum = sum + S.term[threadIdx.x][h];
            if (sum == 0.0) sum = 0.0;
            band_s[m0 + threadIdx.x] = sum;
        }
        __syncthreads();
    }
}

// Is band entry x among the `need` best of the band under (score desc, key asc)?
__device__ __forceinline__ bool band_wins(int x, int nb, int need, const int* band_key, const double* band_s) {
    const double sx = band_s[x];
    const int ix = band_key[x];
    int beat = 0;
#pragma unroll 4
    for (int y = 0; y < nb; ++y) {
        const double sy = band_s[y];
        beat += (sy > sx) || (sy == sx && band_key[y] < ix);
    }
    return beat < need;
}

// Sets bit band_pos[x] of win for each band entry x among the `need` best of the band under
// (score desc, key asc).  One wave per entry: its lanes compare the band against it in
// 64-entry slices and count what beats it with a ballot.
__device__ __forceinline__ void band_mark_winners(int nb, int need, const int* band_key, const double* band_s,
                                                  const int* band_pos, uint32_t* win) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
    for (int x = wave; x < nb; x += nwaves) {
        const double sx = band_s[x];
        const int ix = band_key[x];
        int beat = 0;
        for (int y0 = 0; y0 < nb; y0 += 64) {
            const int y = y0 + lane;
            bool b = false;
            if (y < nb) {
                const double sy = band_s[y];
                b = (sy > sx) || (sy == sx && band_key[y] < ix);
            }
            beat += __builtin_popcountll(__ballot(b));
        }
        if (lane == 0 && beat < need) atomicOr(&win[band_pos[x] >> 5], 1u << (band_pos[x] & 31));
    }
}

// Exact top-k of an unordered candidate list under (canonical score desc, key asc), used
// by the blocked fold.  Writes the k selected keys (unordered) to sel_i and their fp32
// scores to sel_s.  band_i / band_s / band_f: storage for up to band_cap near-threshold
// entries.  Returns false (uniformly) if a buffer would overflow.
__device__ bool select_core(const CandList& L, int k, float delta, const uint16_t* __restrict__ q_row,
                            const float* __restrict__ w_row, const QHeadStat* __restrict__ qs_row,
                            const uint16_t* __restrict__ k_idx, int* band_i,
                            double* band_s, float* band_f, int band_cap, int* sel_i, float* sel_s,
                            SelectScratch& S) {
    float kth;
    if (!block_kth_binned(ListSrc{L}, k, &kth, S)) return false;
    const double lo = (double)kth - 2.0 * (double)delta;
    const double hi = (double)kth + 2.0 * (double)delta;
    if (threadIdx.x == 0) {
        S.sh[4] = 0;  // keys above the band
        S.sh[5] = 0;  // band size
        S.sh[6] = 0;  // selected keys written
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kSegs; ++g)
        if (g < L.nseg)
            for (int i = threadIdx.x; i < L.n[g]; i += blockDim.x) {
                const float sv = L.s[g][i] + 0.0f;
                const double sd = (double)sv;
                const int o = wave_append(sd > hi, &S.sh[4]);
                if (o >= 0 && o < k) {
                    sel_i[o] = L.i[g][i];
                    sel_s[o] = sv;
                }
                const int b = wave_append(sd <= hi && sd >= lo, &S.sh[5]);
                if (b >= 0 && b < band_cap) {
                    band_i[b] = L.i[g][i];
                    band_s[b] = sd;
                    band_f[b] = sv;
                }
            }
    __syncthreads();
    const int n_in = S.sh[4];
    const int nb = S.sh[5];
    __syncthreads();
    if (nb > band_cap || n_in >= k || n_in + nb < k) return false;
    if (delta > 0.f && nb > 0) band_rescore(nb, band_i, band_s, q_row, w_row, qs_row, k_idx, S);
    if (threadIdx.x == 0) S.sh[6] = n_in;
    __syncthreads();
    for (int x0 = 0; x0 < nb; x0 += blockDim.x) {
        const int x = x0 + threadIdx.x;
        const bool win = x < nb && band_wins(x, nb, k - n_in, band_i, band_s);
        const int o = wave_append(win, &S.sh[6]);
        if (o >= 0 && o < k) {
            sel_i[o] = band_i[x];
            sel_s[o] = band_f[x];
        }
    }
    __syncthreads();
    const bool ok = S.sh[6] == k;  // always true; guards the writes above
    __syncthreads();
    return ok;
}

// ------------------------------------------------------------------ 3. row prep

// Order-preserving unsigned key of a float (larger float, larger key) and its inverse.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// A value no larger than the rk-th largest of vals[0..n) (1 <= rk <= n <= 64 * 256), for
// a block of 256 threads.  The values become order-preserving keys; the bits above the
// highest bit in which the smallest and largest key differ are common to all of them, and
// up to two 11-bit radix passes over the bits below find the bucket holding the rk-th
// largest key.  Its lowest key is returned (the candidate threshold only has to be a safe
// estimate; the bucket spans at most 2^-22 of the key range).
__device__ float rank_floor_256(const float* __restrict__ vals, int n, int rk, SelectScratch& S) {
    constexpr int kPer = 64;
    uint32_t key[kPer];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = (int)threadIdx.x + i * 256;
        key[i] = j < n ? order_key(vals[j]) : 0u;
        if (j < n) {
            kmin = min(kmin, key[i]);
            kmax = max(kmax, key[i]);
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        S.red_i[w] = (int)kmin;
        S.red_i[4 + w] = (int)kmax;
    }
    __syncthreads();
    kmin = (uint32_t)S.red_i[0];
    kmax = (uint32_t)S.red_i[4];
    for (int i = 1; i < 4; ++i) {
        kmin = min(kmin, (uint32_t)S.red_i[i]);
        kmax = max(kmax, (uint32_t)S.red_i[4 + i]);
    }
    __syncthreads();
    if (kmin == kmax) return order_key_value(kmin);
    // Keys = common high bits | d, with d < 2^(top+1).  Pass p takes the 11 bits of d ending
    // at bit top - 11p (bits under 0 read as zero); the passes stop once bit 0 is reached.
    constexpr int kDigit = 11, kDigitBins = 1 << kDigit, kOwn = kDigitBins / 256;
    static_assert(kDigitBins <= kBins, "the digit histogram lives in the selection bins");
    const int top = 31 - __builtin_clz(kmin ^ kmax);
    const uint32_t common = top == 31 ? 0u : (kmax >> (top + 1)) << (top + 1);
    uint32_t prefix = 0u;  // digits found so far, as a number
    int remaining = rk;
    int sh = top - (kDigit - 1);  // d >> sh (or d << -sh) puts the current digit in bits 0..10
    int* hist = S.sel.hist;
    for (int pass = 0;; ++pass, sh -= kDigit) {
#pragma unroll
        for (int b = 0; b < kOwn; ++b) hist[(int)threadIdx.x + 256 * b] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (i * 256 >= n) break;  // uniform
            const int j = (int)threadIdx.x + i * 256;
            const uint32_t d = key[i] - common;
            const bool in = j < n && (pass == 0 || (d >> (sh + kDigit)) == prefix);
            const uint32_t digit = (sh >= 0 ? d >> sh : d << -sh) & (uint32_t)(kDigitBins - 1);
            if (in) atomicAdd(&hist[digit], 1);
        }
        __syncthreads();
        // Thread t owns bins kDigitBins-1-kOwn*t down to kDigitBins-kOwn*(t+1), so the scan
        // counts keys from the largest bin down.
        const int hi_bin = kDigitBins - 1 - kOwn * (int)threadIdx.x;
        int c = 0;
#pragma unroll
        for (int b = 0; b < kOwn; ++b) c += hist[hi_bin - b];
        const int incl = block_incl_scan(c, S);
        if (incl - c < remaining && remaining <= incl) {
            int acc = incl - c;
            for (int b = 0; b < kOwn; ++b) {
                const int h = hist[hi_bin - b];
                if (acc + h >= remaining) {
                    S.sh[0] = hi_bin - b;
                    S.sh[1] = acc;
                    break;
                }
                acc += h;
            }
        }
        __syncthreads();
        prefix = (prefix << kDigit) | (uint32_t)S.sh[0];
        remaining -= S.sh[1];
        __syncthreads();
        if (sh <= 0 || pass == 1) break;  // every bit of d is decided, or 22 of them are
    }
    const uint32_t floor_d = sh >= 0 ? prefix << sh : prefix >> -sh;
    return order_key_value(common + floor_d);
}

constexpr int kRowPrepThreads = 256;  // 8 threads per head; one radix bin per thread

__global__ __launch_bounds__(kRowPrepThreads) void row_prep_kernel(IndexerArgs P) {
    const int r = blockIdx.x;
    const RowRef ref = row_ref(P, r);
    const int64_t p = ref.pos;
    const int64_t nt = (p < ref.nkeys - 1 ? p : ref.nkeys - 1) + 1;
    __shared__ double s_l1[kIdxHeads], s_l2[kIdxHeads];
    __shared__ int s_eq[kIdxHeads];
    __shared__ float s_delta;
    __shared__ SelectScratch S;
    if (r == 0 && threadIdx.x == 0) {
        P.fb_ctrl[0] = 0;
        P.fb_ctrl[1] = 0;
    }
    if (P.parts > 2 && threadIdx.x == 0) P.count[(size_t)r * kSegs] = 0;  // appended list counter
    if (!ref.valid) {  // padding row of a batched block: nothing to select
        if (threadIdx.x == 0) {
            P.mode[r] = kModePad;
            P.tau[r] = INFINITY;
            P.delta[r] = 0.f;
        }
        return;
    }
    if (nt <= P.top_k) {
        if (threadIdx.x == 0) {
            P.mode[r] = kModeAll;
            P.tau[r] = INFINITY;
            P.delta[r] = 0.f;
        }
        return;
    }
    // Per-head |q|_1, |q|_2^2 and lowest set-bit exponent (8 threads per head).
    {
        const int h = threadIdx.x >> 3, part = threadIdx.x & 7;
        const u16x8* qp = reinterpret_cast<const u16x8*>(ref.q + (size_t)h * kIdxDim + part * 16);
        double l1 = 0.0, l2 = 0.0;
        int em = INT_MAX;
        for (int c = 0; c < 2; ++c) {
            const u16x8 v = qp[c];
            for (int j = 0; j < 8; ++j) {
                const double x = (double)bf16_bits_to_float(v[j]);
                l1 += fabs(x);
                l2 += x * x;
                if ((v[j] & 0x7fff) != 0) em = min(em, bf16_lsb_exp(v[j]));
            }
        }
        for (int o = 1; o < 8; o <<= 1) {
            l1 += __shfl_xor(l1, o);
            l2 += __shfl_xor(l2, o);
            em = min(em, __shfl_xor(em, o));
        }
        if (part == 0) {
            s_l1[h] = l1;
            s_l2[h] = l2;
            s_eq[h] = em;
            // for the exact re-score: the bound covers the rounding of the sums above
            P.qstat[(size_t)r * kIdxHeads + h] = QHeadStat{l1 * (1.0 + 1.0 / 1048576.0), em, 0};
        }
    }
    // Key statistics: wave 0 reduces the partial slots.
    KeyStats ks{};
    if (threadIdx.x < 64) {
        unsigned kn = 0u, ki = 0u;
        int ke = INT_MAX;
#pragma unroll
        for (int u = 0; u < kStatSlots / 64; ++u) {  // loads issued together
            const int i = (int)threadIdx.x + 64 * u;
            const KeyStats e = i < P.n_kstats ? P.kstats[i] : KeyStats{0u, 0u, INT_MAX, 0};
            kn = max(kn, e.knorm_bits);
            ki = max(ki, e.kinf_bits);
            ke = min(ke, e.kexp_min);
        }
        for (int o = 32; o > 0; o >>= 1) {
            kn = max(kn, (unsigned)__shfl_xor((int)kn, o));
            ki = max(ki, (unsigned)__shfl_xor((int)ki, o));
            ke = min(ke, __shfl_xor(ke, o));
        }
        ks.knorm_bits = kn;
        ks.kinf_bits = ki;
        ks.kexp_min = ke;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        // Lane h < 32 takes head h; the per-head terms are then reduced across the wave
        // (the fp64 sums feed bounds that carry their own rounding margins).
        const double knorm = (double)__uint_as_float(ks.knorm_bits);
        const double kinf = (double)__uint_as_float(ks.kinf_bits);
        const int h = threadIdx.x;
        double dsum = 0.0, lhs = 0.0;
        int emin = INT_MAX;
        bool used = false, subnormal = false;
        if (h < kIdxHeads) {
            const float wh = ref.w[h];
            dsum = fabs((double)wh) * sqrt(s_l2[h]);
            if (wh != 0.f && s_l1[h] > 0.0) {
                used = true;
                lhs = fabs((double)wh) * s_l1[h] * kinf;
                emin = f32_lsb_exp(wh) + s_eq[h];
            }
            // each head's dot product must also stay above the fp32 subnormal range
            subnormal = s_l1[h] > 0.0 && s_eq[h] + ks.kexp_min < -100;
        }
        for (int o = 32; o > 0; o >>= 1) {
            dsum += __shfl_xor(dsum, o);
            lhs += __shfl_xor(lhs, o);
            emin = min(emin, __shfl_xor(emin, o));
        }
        const bool any = __ballot(used) != 0, any_subnormal = __ballot(subnormal) != 0;
        if (threadIdx.x == 0) {
            // Exactness: every product and partial sum of the fp32 evaluation is a multiple
            // of 2^e and below 2^(24+e) in magnitude -> fp32 scores are exact.
            bool exact;
            if (!any || ks.kexp_min == INT_MAX) {
                exact = true;  // every score is exactly zero
            } else {
                const int e = emin + ks.kexp_min;
                exact = (e >= -100) && (lhs * (1.0 + 1e-12) < ldexp(1.0, 24 + e)) && !any_subnormal;
            }
            float d = 0.f;
            if (!exact) {
                const double dd = kDeltaCoef * ldexp(1.0, -24) * knorm * dsum;
                d = (float)(dd * (1.0 + 1.0 / 1048576.0));
                if (!(d > 0.f)) d = FLT_MIN;
            }
            s_delta = d;
            P.delta[r] = d;
            P.mode[r] = kModeNormal;
        }
    }
    __syncthreads();
    const int g0 = r & ~(kRowsPerGroup - 1);
    const int64_t pg = row_ref(P, g0).pos;  // the group's first row (same sequence)
    const int64_t n0 = (pg < ref.nkeys - 1 ? pg : ref.nkeys - 1) + 1;
    const int Sn = sample_size(n0, P.top_k, P.cap);
    if (Sn == 0) {  // the whole group keeps every causal key (at most cap per row)
        if (threadIdx.x == 0) P.tau[r] = -INFINITY;
        return;
    }
    const int rk = sample_rank(n0, Sn, P.top_k);
    const float that = rank_floor_256(P.sample + (size_t)r * P.sample_stride, Sn, rk, S);
    if (threadIdx.x == 0) {
        const double t = (double)that - 2.0 * (double)s_delta;
        float tf = (float)t;
        if ((double)tf > t) tf = nextafterf(tf, -INFINITY);
        P.tau[r] = tf;
    }
}

// ------------------------------------------------------------------ 5. select

__device__ void write_sorted_output(int* sel, int k, int32_t* out_row) {
    int n2 = 1;
    while (n2 < k) n2 <<= 1;
    for (int i = k + threadIdx.x; i < n2; i += blockDim.x) sel[i] = INT_MAX;
    __syncthreads();
    block_bitonic_sort(sel, n2);
    for (int i = threadIdx.x; i < k; i += blockDim.x) out_row[i] = sel[i];
}

constexpr int kSelBand = 1024;
// Appended candidate lists are put back in key order through a bitmap of the causal keys
// held in the re-score's term array, when the keys fit it.
constexpr int kSelBitmapKeys = kRescoreRound * kIdxHeads * 64;  // 32 KB of bits
constexpr int kSelChunk = 16;  // candidates per thread: the block has cap / 16 threads

// Exact top-k of one row's candidates.  The eight segments written by the scoring waves
// are each in ascending key order and cover ascending key ranges, so their concatenation
// is sorted by key.  Thread t holds positions e * blockDim + t (e < 16) of it in registers,
// so each load instruction reads consecutive entries, and the ascending output is a stable
// compaction of the selected positions (per-element wave ballots and one block scan).
__global__ __launch_bounds__(1024) void select_kernel(IndexerArgs P) {
    const int r = blockIdx.x;
    const int mode = P.mode[r];
    if (mode == kModePad) return;
    const RowRef ref = row_ref(P, r);
    const int64_t p = ref.pos;
    const int64_t nt = (p < ref.nkeys - 1 ? p : ref.nkeys - 1) + 1;
    const int k = P.top_k;
    int32_t* out_row = ref.out;
    if (mode == kModeAll) {
        for (int j = threadIdx.x; j < k; j += blockDim.x) out_row[j] = j < nt ? j : -1;
        return;
    }
    __shared__ SelectScratch S;
    __shared__ int s_band_key[kSelBand];
    __shared__ int s_band_pos[kSelBand];
    __shared__ double s_band_s[kSelBand];
    __shared__ uint32_t s_win[kSelChunk * 1024 / 32];
    // Eight key-ordered segments, or (more key parts) one appended list in no key order.
    const bool appended = P.parts > 2;
    const int seg = appended ? P.cap : P.cap / kSegs;
    int cnt[kSegs], start[kSegs];
    int total = 0;
    bool ok = !P.force_fallback;
#pragma unroll
    for (int w = 0; w < kSegs; ++w) {
        cnt[w] = appended && w > 0 ? 0 : P.count[(size_t)r * kSegs + w];
        ok = ok && cnt[w] <= seg;
        start[w] = total;
        total += cnt[w];
    }
    ok = ok && total >= k;
    const float tau_f = P.tau[r];
    const float delta = P.delta[r];
    float v[kSelChunk];
    int key[kSelChunk];
    int nv = 0;
    const int nthr = (int)blockDim.x, tid = (int)threadIdx.x;
    if (ok) {
#pragma unroll
        for (int e = 0; e < kSelChunk; ++e) {
            const int j = e * nthr + tid;
            v[e] = -INFINITY;
            key[e] = 0;
            if (j < total) {
                int w = 0, s0 = 0;
#pragma unroll
                for (int x = 1; x < kSegs; ++x)
                    if (j >= start[x]) {
                        w = x;
                        s0 = start[x];
                    }
                const uint2 c = P.cand[(size_t)r * P.cap + (size_t)w * seg + (j - s0)];
                v[e] = __uint_as_float(c.x) + 0.0f;
                key[e] = (int)c.y;
            }
        }
        nv = total > tid ? min((total - tid + nthr - 1) / nthr, kSelChunk) : 0;
    }
    float kth = 0.f;
    if (ok) ok = block_kth_binned(RegSrc<kSelChunk>{v, nv}, k, &kth, S);
    const double lo = (double)kth - 2.0 * (double)delta;
    const double hi = (double)kth + 2.0 * (double)delta;
    if (ok && tau_f != -INFINITY && lo < (double)tau_f) ok = false;  // candidate set not provably complete
    if (ok) {
        if (threadIdx.x == 0) {
            S.sh[4] = 0;
            S.sh[5] = 0;
        }
        for (int i = threadIdx.x; i < kSelChunk * 1024 / 32; i += blockDim.x) s_win[i] = 0u;
        __syncthreads();
        int n_above = 0;
#pragma unroll
        for (int e = 0; e < kSelChunk; ++e) {
            const double sd = (double)v[e];
            n_above += e < nv && sd > hi;
            const bool in_band = e < nv && sd <= hi && sd >= lo;
            const int b = wave_append(in_band, &S.sh[5]);
            if (b >= 0 && b < kSelBand) {
                s_band_key[b] = key[e];
                s_band_pos[b] = e * nthr + tid;
                s_band_s[b] = sd;
            }
        }
        for (int o = 32; o > 0; o >>= 1) n_above += __shfl_xor(n_above, o);
        if ((threadIdx.x & 63) == 0) atomicAdd(&S.sh[4], n_above);
        __syncthreads();
        const int n_in = S.sh[4];
        const int nb = S.sh[5];
        __syncthreads();
        ok = nb <= kSelBand && n_in < k && n_in + nb >= k;
        if (ok) {
            if (delta > 0.f && nb > 0)
                band_rescore(nb, s_band_key, s_band_s, ref.q, ref.w, P.qstat + (size_t)r * kIdxHeads, ref.keys, S);
            band_mark_winners(nb, k - n_in, s_band_key, s_band_s, s_band_pos, s_win);
            __syncthreads();
            // Selected = above the band, or a band winner.
            if (!appended) {
                // Stable compaction: the candidate list is in key order, position e * blockDim + t
                // for element e of thread t, so the output offset of (e, t) counts the selected
                // positions of the earlier elements and of the earlier threads in element e.
                const int nw = nthr >> 6, wv = tid >> 6;
                uint64_t m[kSelChunk];
#pragma unroll
                for (int e = 0; e < kSelChunk; ++e) {
                    const int j = e * nthr + tid;
                    m[e] = __ballot(e < nv && ((double)v[e] > hi || ((s_win[j >> 5] >> (j & 31)) & 1u)));
                    if ((tid & 63) == 0) S.out[e * nw + wv] = __builtin_popcountll(m[e]);
                }
                __syncthreads();
                const int ce = tid < kSelChunk * nw ? S.out[tid] : 0;
                const int pre = block_incl_scan(ce, S) - ce;
                if (tid < kSelChunk * nw) S.out[kSelChunk * 16 + tid] = pre;
                __syncthreads();
#pragma unroll
                for (int e = 0; e < kSelChunk; ++e) {
                    if ((m[e] >> (tid & 63)) & 1u) {
                        const int o = S.out[kSelChunk * 16 + e * nw + wv] + mbcnt64(m[e]);
                        if (o < k) out_row[o] = key[e];
                    }
                }
            } else if (nt <= kSelBitmapKeys) {
                // Appended list (no key order), causal keys within the bitmap: mark the
                // selected keys, then each thread emits its words' keys at its scanned offset.
                uint32_t* bm = reinterpret_cast<uint32_t*>(&S.term[0][0]);
                const int nw = (int)((nt + 31) >> 5);
                for (int i = threadIdx.x; i < nw; i += blockDim.x) bm[i] = 0u;
                __syncthreads();
#pragma unroll
                for (int e = 0; e < kSelChunk; ++e) {
                    const int j = e * nthr + tid;
                    if (e < nv && ((double)v[e] > hi || ((s_win[j >> 5] >> (j & 31)) & 1u)))
                        atomicOr(&bm[key[e] >> 5], 1u << (key[e] & 31));
                }
                __syncthreads();
                const int per = (nw + (int)blockDim.x - 1) / (int)blockDim.x;
                const int w0 = (int)threadIdx.x * per, w1 = min(nw, w0 + per);
                int c = 0;
                for (int i = w0; i < w1; ++i) c += __builtin_popcount(bm[i]);
                int o = block_incl_scan(c, S) - c;
                for (int i = w0; i < w1; ++i) {
                    uint32_t b = bm[i];
                    while (b) {
                        const int bit = __builtin_ctz(b);
                        b &= b - 1u;
                        if (o < k) out_row[o] = i * 32 + bit;
                        ++o;
                    }
                }
            } else {
                // Appended list over a larger key range: gather the selection, then sort it.
                int c = 0;
#pragma unroll
                for (int e = 0; e < kSelChunk; ++e) {
                    const int j = e * nthr + tid;
                    c += e < nv && ((double)v[e] > hi || ((s_win[j >> 5] >> (j & 31)) & 1u));
                }
                int o = block_incl_scan(c, S) - c;
#pragma unroll
                for (int e = 0; e < kSelChunk; ++e) {
                    const int j = e * nthr + tid;
                    if (e < nv && ((double)v[e] > hi || ((s_win[j >> 5] >> (j & 31)) & 1u))) {
                        if (o < k) S.out[o] = key[e];
                        ++o;
                    }
                }
                __syncthreads();
                write_sorted_output(S.out, k, out_row);
            }
        }
    }
    if (!ok && threadIdx.x == 0) {
        const int slot = atomicAdd(&P.fb_ctrl[0], 1);
        P.fb_list[slot] = r;
    }
}

// ------------------------------------------------------------------ 6. fallback fold

// Scores keys [k0, k1) of one row with MFMA (one 32-key tile per wave per step) and
// appends those with score > lo to (dst_s, dst_i) at *cnt (LDS counter).
__device__ void fold_score_block(const RowRef& R, int64_t k0, int64_t k1, float lo,
                                 float* dst_s, int* dst_i, int* cnt, int cap) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hf = lane >> 5, col = lane & 31;
    const int n_waves = blockDim.x >> 6;
    const u16x8* qp = reinterpret_cast<const u16x8*>(R.q + (size_t)col * kIdxDim + hf * 8);
    bf16x8 a[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) a[kk] = __builtin_bit_cast(bf16x8, qp[2 * kk]);
    float wf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wf[i] = R.w[8 * (i >> 2) + 4 * hf + (i & 3)];
    const int64_t n_tiles = (k1 - k0 + kKeyTile - 1) / kKeyTile;
    for (int64_t ti = wave; ti < n_tiles; ti += n_waves) {
        const int64_t pos = k0 + ti * kKeyTile + col;
        const int64_t key = pos < k1 ? pos : k1 - 1;
        const u16x8* kp = reinterpret_cast<const u16x8*>(R.keys + key * kIdxDim + hf * 8);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc = mfma_32x32x16(a[kk], __builtin_bit_cast(bf16x8, kp[2 * kk]), acc);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part += wf[i] * fmaxf(acc[i], 0.f);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        s = s + 0.0f;
        // Later keys lose ties, so only a score strictly above kth - 2 delta can enter.
        const bool keep = hf == 0 && pos < k1 && s > lo;
        const uint64_t m = __ballot(keep);
        if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(cnt, __builtin_popcountll(m));
            base = __shfl(base, 0);
            if (keep) {
                const int o = base + mbcnt64(m);
                if (o < cap) {
                    dst_s[o] = s;
                    dst_i[o] = (int)pos;
                }
            }
        }
    }
}

// Persistent: each workgroup takes flagged rows one at a time and runs the exact
// blocked fold over 4,096-key blocks (running list = exact top-k after each block,
// new keys admitted only if score > kth(list) - 2 delta).
__global__ __launch_bounds__(kSelectThreads) void fold_kernel(IndexerArgs P) {
    __shared__ SelectScratch S;
    __shared__ int s_row, s_cnt;
    const int slot = blockIdx.x;
    float* Rs[2] = {P.fold_s + (size_t)slot * 2 * P.fold_cap, P.fold_s + (size_t)slot * 2 * P.fold_cap + P.fold_cap};
    int* Ri[2] = {P.fold_i + (size_t)slot * 2 * P.fold_cap, P.fold_i + (size_t)slot * 2 * P.fold_cap + P.fold_cap};
    int* band_i = P.fold_bi + (size_t)slot * P.fold_cap;
    double* band_s = P.fold_bs + (size_t)slot * P.fold_cap;
    float* band_f = P.fold_bf + (size_t)slot * P.fold_cap;
    const int k = P.top_k;
    if (P.fb_ctrl[0] == 0) return;  // final here (select has finished): nothing to fold
    for (;;) {
        if (threadIdx.x == 0) {
            const int i = atomicAdd(&P.fb_ctrl[1], 1);
            s_row = i < P.fb_ctrl[0] ? P.fb_list[i] : -1;
        }
        __syncthreads();
        const int r = s_row;
        __syncthreads();
        if (r < 0) return;
        const RowRef ref = row_ref(P, r);
        const int64_t p = ref.pos;
        const int64_t nt = (p < ref.nkeys - 1 ? p : ref.nkeys - 1) + 1;
        const float delta = P.delta[r];
        const uint16_t* q_row = ref.q;
        const float* w_row = ref.w;
        int cur = 0, n = 0;
        float lo = -INFINITY;
        for (int64_t b0 = 0; b0 < nt; b0 += kFoldKeys) {
            const int64_t b1 = b0 + kFoldKeys < nt ? b0 + kFoldKeys : nt;
            if (threadIdx.x == 0) s_cnt = n;
            __syncthreads();
            fold_score_block(ref, b0, b1, lo, Rs[cur], Ri[cur], &s_cnt, P.fold_cap);
            __syncthreads();
            n = s_cnt < P.fold_cap ? s_cnt : P.fold_cap;
            __syncthreads();
            if (n > k) {
                // Keep exactly the top-k of the list; their fp32 scores go to the other buffer.
                const int nxt = cur ^ 1;
                CandList L{};
                L.s[0] = Rs[cur];
                L.i[0] = Ri[cur];
                L.n[0] = n;
                L.nseg = 1;
                const bool ok = select_core(L, k, delta, q_row, w_row, P.qstat + (size_t)r * kIdxHeads, ref.keys,
                                            band_i, band_s, band_f,
                                            P.fold_cap, Ri[nxt], Rs[nxt], S);
                (void)ok;  // band capacity == list capacity
                __syncthreads();
                cur = nxt;
                n = k;
                CandList R{};
                R.s[0] = Rs[cur];
                R.i[0] = Ri[cur];
                R.n[0] = n;
                R.nseg = 1;
                float kth = -INFINITY;
                block_kth_binned(ListSrc{R}, k, &kth, S);
                const double l = (double)kth - 2.0 * (double)delta;
                float lf = (float)l;
                if ((double)lf > l) lf = nextafterf(lf, -INFINITY);
                lo = lf;
            }
        }
        int32_t* out_row = ref.out;
        // n == k here (nt > k for every scored row): the list is the exact top-k.
        for (int j = threadIdx.x; j < k; j += blockDim.x) S.out[j] = j < n ? Ri[cur][j] : -1;
        __syncthreads();
        write_sorted_output(S.out, k, out_row);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ causal mask op

__global__ void causal_mask_kernel(int32_t* idx, int64_t L, int top_k, int64_t q_pos0) {
    const int64_t total = L * (int64_t)top_k;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = e / top_k;
        if ((int64_t)idx[e] > q_pos0 + t) idx[e] = -1;
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_key_stats(const uint16_t* k_idx, int64_t n_keys, KeyStats* ks, uint16_t* k_tile,
                             hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    static_assert(kStatsThreads / kWave == 4 && kKeyTileKeys == 32, "key_stats_blocks assumes 4 waves of 32-key tiles");
    const int blocks = key_stats_blocks(n_keys);
    key_stats_kernel<<<blocks, kStatsThreads, 0, s>>>(k_idx, n_keys, nullptr, 0,
                                                     (n_keys + kKeyTileKeys - 1) / kKeyTileKeys, ks, k_tile);
    return hipGetLastError();
}

hipError_t launch_key_stats_batch(const uint16_t* k_idx, const SeqKeys* seqs, int n_seqs, int64_t n_tiles,
                                  KeyStats* ks, uint16_t* k_tile, hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    const int blocks = key_stats_blocks(n_tiles * kKeyTileKeys);
    key_stats_kernel<<<blocks, kStatsThreads, 0, s>>>(k_idx, 0, seqs, n_seqs, n_tiles, ks, k_tile);
    return hipGetLastError();
}

// ------------------------------------------------------------------ batch tables

__global__ void varlen_tables_kernel(VarlenChunk c, int64_t seq0, RowInfo* rows, SeqKeys* seqs,
                                     QueryInfo* qinfo) {
    const int b = blockIdx.y;
    const int64_t L = c.L[b];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (rows) {
        const int64_t padded = (L + kRowsPerGroup - 1) / kRowsPerGroup * kRowsPerGroup;
        for (int64_t i = i0; i < padded; i += stride)
            rows[c.row0[b] + i] = RowInfo{i < L ? c.qrow0[b] + i : -1, c.pos0[b] + i, c.kbase[b], c.tbase[b],
                                          c.nvis[b]};
    }
    if (qinfo)
        for (int64_t i = i0; i < L; i += stride) qinfo[c.qrow0[b] + i] = QueryInfo{c.kbase[b], c.pos0[b] + i};
    if (seqs && i0 == 0)
        seqs[seq0 + b] = SeqKeys{c.kbase[b], c.nvis[b], c.tbase[b],
                                 c.tbase[b] + (c.nvis[b] + kKeyTileKeys - 1) / kKeyTileKeys};
}

hipError_t launch_varlen_tables(const VarlenChunk& c, int64_t seq0, RowInfo* rows, SeqKeys* seqs,
                                QueryInfo* qinfo, hipStream_t s) {
    if (c.n <= 0) return hipSuccess;
    varlen_tables_kernel<<<dim3(4, c.n), 256, 0, s>>>(c, seq0, rows, seqs, qinfo);
    return hipGetLastError();
}

hipError_t launch_indexer_block(const IndexerArgs& a, bool need_sample, hipStream_t s, bool sparse_rows) {
    const int groups = (a.Lb + kRowsPerGroup - 1) / kRowsPerGroup;
    // Two key halves per group (XCD-mapped) while that fills the GPU, else more key parts.
    const int score_wgs = a.parts == 2 ? 8 * ((groups + 3) / 4) : groups * a.parts;
    if (need_sample) {
        ProfScope ps(s, kProfScoreSample);
        if (sparse_rows) score_kernel<true, true><<<score_wgs, kScoreThreads, 0, s>>>(a, groups);
        else score_kernel<true, false><<<score_wgs, kScoreThreads, 0, s>>>(a, groups);
    }
    hipError_t e = launch_row_prep(a, s);
    if (e != hipSuccess) return e;
    {
        ProfScope ps(s, kProfScoreFilter);
        if (sparse_rows) score_kernel<false, true><<<score_wgs, kScoreThreads, 0, s>>>(a, groups);
        else score_kernel<false, false><<<score_wgs, kScoreThreads, 0, s>>>(a, groups);
    }
    return launch_select_fold(a, s);
}

hipError_t launch_row_prep(const IndexerArgs& a, hipStream_t s) {
    ProfScope ps(s, kProfRowPrep);
    row_prep_kernel<<<a.Lb, kRowPrepThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_select_fold(const IndexerArgs& a, hipStream_t s) {
    {
        ProfScope ps(s, kProfSelect);
        select_kernel<<<a.Lb, a.cap / kSelChunk, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfFold);
        fold_kernel<<<kFallbackSlots, kSelectThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_causal_mask(int32_t* idx, int64_t L, int top_k, int64_t q_pos0, hipStream_t s) {
    const int64_t total = L * (int64_t)top_k;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    ProfScope ps(s, kProfCausalMask);
    causal_mask_kernel<<<blocks, 256, 0, s>>>(idx, L, top_k, q_pos0);
    return hipGetLastError();
}

}  // namespace dsa
