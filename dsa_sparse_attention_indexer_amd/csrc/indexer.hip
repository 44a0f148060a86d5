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

constexpr int kSegs = kCandSegs;  // count words per row; key ranges per row group (key half, scoring wave)

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

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum over each row of 16 lanes, left in every lane of the row: DPP quad swaps, then the
// half-row and row mirrors (each step adds the value of a lane in the other group, so all
// lanes of a row end with the same bits).
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    return x;
}

// One wave per 32-key tile (tile = global wave index, then strided): eight 1-KB row-major
// loads (16 lanes per key row; the next tile's loads are issued before this tile's
// arithmetic), the statistics, then the tile is re-ordered through LDS and written as eight
// 1-KB stores in the scoring order.  Keys past the end are zero.
//
// Per element: its square (fp32 FMA; the 16 lanes of a key row are summed by DPP and the
// largest sum is kept, so one square root at the end gives max ||k||), its magnitude, and
// the exponent of its lowest set bit, max(e, 1) - 134 + min(ctz(m), 7) for a bf16 with
// biased exponent e and mantissa m (7 when m = 0), over nonzero elements.  The last runs on
// both halves of a 32-bit word at once: 16-bit lanes hold max(e, 1) + min(ctz, 7), plus 512
// for a zero half so that it never wins the minimum.
constexpr int kStatsThreads = 256;
constexpr int kStatsRowPad = 17;  // LDS row stride in 16-byte chunks (16 + 1 against bank conflicts)
constexpr unsigned short kStatsZeroBias = 512;
// seqs == null: one sequence of n_keys keys.  Otherwise tile t belongs to the sequence whose
// tile range holds it, and its keys are that sequence's.  Tiles [t_begin, n_tiles) are done.
// merge: the statistics are folded into slots[0] with atomics (an append-only key cache)
// instead of one slot per block.
__global__ __launch_bounds__(kStatsThreads) void key_stats_kernel(const uint16_t* __restrict__ k_idx,
                                                                  int64_t n_keys, const SeqKeys* seqs,
                                                                  int n_seqs, int64_t t_begin, int64_t n_tiles,
                                                                  KeyStats* slots,
                                                                  uint16_t* __restrict__ k_tile,
                                                                  unsigned long long* diag, bool merge) {
    if (diag && blockIdx.x == 0 && threadIdx.x < kDiagSlots) diag[threadIdx.x] = 0ull;
    __shared__ u16x8 s_t[kStatsThreads / kWave][kKeyTileKeys * kStatsRowPad];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u16x8* st = s_t[wave];
    float ssmax = 0.f, amax = 0.f;
    u16x2 emin2 = {0xffff, 0xffff};
    const int64_t n_waves = (int64_t)gridDim.x * (kStatsThreads / kWave);

    // Loads of tile t (wave-uniform): lane chunk q = 64 i + lane is key q / 16 of the tile,
    // dims 8 (q % 16) ..; rows past the tile's last key re-read that key (zeroed later).
    auto issue = [&](int64_t t, u16x8 (&v)[8]) -> int {
        const uint16_t* src = k_idx;
        int64_t kn = n_keys, tl = t;
        if (seqs) {  // first sequence whose tiles end after t
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
        const int64_t left = kn - tl * kKeyTileKeys;
        const int nv = left < kKeyTileKeys ? (int)left : kKeyTileKeys;
        const u16x8* row = reinterpret_cast<const u16x8*>(src + tl * kKeyTileKeys * kIdxDim);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = 4 * i + (lane >> 4);
            v[i] = row[(key < nv ? key : nv - 1) * (kIdxDim / 8) + (lane & 15)];
        }
        return nv;
    };

    int64_t t = t_begin + (int64_t)blockIdx.x * (kStatsThreads / kWave) + wave;
    u16x8 cur[8];
    int nv_cur = t < n_tiles ? issue(t, cur) : 0;
    for (; t < n_tiles; t += n_waves) {
        u16x8 nxt[8];
        const int64_t tn = t + n_waves;
        const int nv_nxt = issue(tn < n_tiles ? tn : t, nxt);
        if (nv_cur < kKeyTileKeys) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (4 * i + (lane >> 4) >= nv_cur) cur[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 wv = __builtin_bit_cast(uint4, cur[i]);
            const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = words[j];
                const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
                amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
                const uint32_t c = w & 0x7fff7fffu;
                const u16x2 c2 = __builtin_bit_cast(u16x2, c);
                const u16x2 e1 = __builtin_elementwise_max(c2 >> (unsigned short)7, (u16x2){1, 1});
                const u16x2 zero = (c2 - (unsigned short)1) >> (unsigned short)15;  // 1 for a zero half
                const uint32_t c80 = c | 0x00800080u;
                const uint32_t tz = (uint32_t)__builtin_ctz(c80) | ((uint32_t)__builtin_ctz(c80 >> 16) << 16);
                const u16x2 sv = zero * kStatsZeroBias + e1 + __builtin_bit_cast(u16x2, tz);
                emin2 = __builtin_elementwise_min(emin2, sv);
            }
            ssmax = fmaxf(ssmax, row16_sum(ss));
            const int q = i * 64 + lane;
            if (k_tile) st[(q >> 4) * kStatsRowPad + (q & 15)] = cur[i];
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
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
        nv_cur = nv_nxt;
    }
    float nmax = sqrtf(ssmax);
    int emin;
    {
        const unsigned short m = emin2.x < emin2.y ? emin2.x : emin2.y;
        emin = m >= kStatsZeroBias ? INT_MAX : (int)m - 134;
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
        if (merge) {  // non-negative floats order as their bit patterns
            atomicMax(&slots[0].knorm_bits, __float_as_uint(up));
            atomicMax(&slots[0].kinf_bits, __float_as_uint(amax));
            atomicMin(&slots[0].kexp_min, emin);
        } else {
            slots[blockIdx.x] = KeyStats{__float_as_uint(up), __float_as_uint(amax), emin, 0};
        }
    }
}

// ------------------------------------------------------------------ 2/4. MFMA scoring

// One workgroup = 8 consecutive query rows over one half of their causal keys (two
// workgroups per row group; the half follows the XCD the workgroup lands on, so each
// XCD's L2 streams only its half of the key cache).  Each of the 4 waves scores all 8
// rows over its own contiguous quarter of that half.  Eight rows per wave means every key
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
// per (wave, row) and flushed to the row's list as coalesced (score, key) runs.  A row's
// list of cap slots is shared by its two key halves: half 0 fills it from slot 0 upward
// and half 1 from slot cap - 1 downward, each half's four waves reserving their runs
// through one LDS counter per row.  However a row's survivors spread over its keys (a
// recency bias puts most of them in the newest keys), the list overflows only when their
// total exceeds cap; the two halves' regions can then overlap, and the row, flagged by
// its counts, goes to the fold.
constexpr int kRowsPerWave = kRowsPerGroup;   // 8
constexpr int kPairs = kRowsPerWave / 2;
constexpr int kKeyHalves = 2;
constexpr int kStageSlots = 64;  // LDS staging entries per (wave, row) for filter survivors
static_assert(kKeyHalves * (kScoreThreads / kWave) == kSegs, "key parts and scoring waves per row group");

// sum_e w_e * r[e] with e ascending (fused multiply-adds), where lane 16g + e of W holds w_e
// for the lanes of its 16-lane row g: DPP row_newbcast:e hands that lane's value to every
// lane of the row, so the weights take one register per query row instead of 16.  A DPP
// source needs two wait states after a VALU write of it; W is written once, before the
// scoring loop, and the build checks the generated code for any closer write.  The chain is
// four asm statements of four instructions: the scheduler places each statement as one unit,
// and pieces of four spread under the MFMAs better than two of eight (3% on the filter) or
// sixteen single ones.
__device__ __forceinline__ float weighted_head_sum(float W, const float (&r)[16]) {
    float p;
    asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf"
        : "=&v"(p)
        : "v"(W), "v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]));
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:7 row_mask:0xf bank_mask:0xf"
        : "+v"(p)
        : "v"(W), "v"(r[4]), "v"(r[5]), "v"(r[6]), "v"(r[7]));
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:11 row_mask:0xf bank_mask:0xf"
        : "+v"(p)
        : "v"(W), "v"(r[8]), "v"(r[9]), "v"(r[10]), "v"(r[11]));
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(p)
        : "v"(W), "v"(r[12]), "v"(r[13]), "v"(r[14]), "v"(r[15]));
    return p;
}

// Scheduling pattern for the region ending here (the next pair's 16 MFMAs, this pair's
// head sums and an earlier pair's tail): one MFMA, then three VALU instructions, repeated.
// Spreading the VALU work thinly keeps the matrix pipe fed (the default schedule bunches it
// and leaves the last MFMAs back to back); three per MFMA measured better than two or four.
__device__ __forceinline__ void interleave_with_mfma() {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x2, 3, 0);  // VALU
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
    uint32_t* cand0;    // filter: row 0's list (rows 2 cap words apart: cap scores, then cap keys)
    uint32_t n0;        // sample: keys of the group's first row
    uint32_t S;         // sample: sample size
    float s_ratio;      // sample: key stride n0 / S (any in-range keys would do)
    int lane, hf, col;
    int colm;           // col - hf
    int first_pos;      // position of the group's first row
    int first_row;      // the group's first row in the block
    int down;           // key half 1 of two: the half fills the row's list from its top down
    int* rcnt;          // two key parts: the workgroup's LDS counters of list entries per row
    uint2* lbuf;                // filter: this wave's LDS staging lists, kStageSlots per row, then
                                // one spare slot per lane for stores that keep nothing
    int lcnt[kRowsPerWave];     // entries staged per row (wave-uniform)
    uint32_t tile0;     // first tile of this wave's contiguous range (wave-uniform)
    bool pl[kPairs];    // kSkip: row pair q has a live row (wave-uniform)
    float s4;           // pair 2's scores (rows 4, 5) of the last tile, their tail not yet done

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

    // Scores of rows J0, J0+1 (the ReLU and the weighted head sum): lane half hf gets row
    // J0 + hf's score of its key.
    template <int J0>
    __device__ __forceinline__ float hsum2(const f32x16 (&acc)[kRowsPerWave]) const {
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
        interleave_with_mfma();
        return s_mine;
    }

    // The sample store, or the threshold filter, of rows J0, J0+1's scores for tile it.
    // Branch-free (every lane stores: a survivor at its slot, any other lane at its own
    // spare slot), so that it can issue under the MFMAs of the region it sits in.
    template <int J0>
    __device__ __forceinline__ void tail2(float s_mine, int it) {
        const uint32_t pos = pos_of(it);
        const uint32_t j_mine = J0 + hf;
        constexpr int q = J0 / 2;
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
            const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
            // Slot within the row's staging list: entries already staged plus the survivors
            // among the lower lanes of this half.
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(m1, __builtin_amdgcn_mbcnt_lo(hf ? 0u : m0, 0u));
            const uint32_t o = (uint32_t)(hf ? lcnt[J0 + 1] : lcnt[J0]) + below;  // < kStageSlots
            const uint32_t slot = keep ? j_mine * kStageSlots + o : (uint32_t)(kRowsPerWave * kStageSlots + lane);
            lbuf[slot] = uint2{__float_as_uint(s_mine), pos};
            const int c0 = __builtin_popcount(m0), c1 = __builtin_popcount(m1);
            lcnt[J0] += c0;
            lcnt[J0 + 1] += c1;
        }
    }

    template <int J0>
    __device__ __forceinline__ void epilogue2(const f32x16 (&acc)[kRowsPerWave], int it) {
        tail2<J0>(hsum2<J0>(acc), it);
    }

    // Staged survivors of row j -> the row's list: one coalesced 8-byte store per lane.
    // The run's slots are reserved on the row's counter: the workgroup's LDS counter (two
    // key parts; key half 1 counts its slots down from the list's top) or the row's global
    // counter (more parts).  Entries past the list's capacity are dropped (the row is then
    // re-done by the fold, which its counts signal).
    __device__ __forceinline__ void flush_row(int j) {
        uint32_t b = 0u;
        if (lane == 0)
            b = P.parts > 2 ? atomicAdd(reinterpret_cast<unsigned*>(&P.count[(size_t)(first_row + j) * kSegs]),
                                        (unsigned)lcnt[j])
                            : atomicAdd(reinterpret_cast<unsigned*>(&rcnt[j]), (unsigned)lcnt[j]);
        const uint32_t base = __builtin_amdgcn_readfirstlane(b);
        if (lane < lcnt[j]) {
            const uint2 e = lbuf[j * kStageSlots + lane];
            const uint32_t o = base + (uint32_t)lane;
            if (o < (uint32_t)P.cap) {
                uint32_t* dst = cand0 + (uint32_t)j * 2u * (uint32_t)P.cap + (down ? (uint32_t)P.cap - 1u - o : o);
                dst[0] = e.x;
                dst[P.cap] = e.y;
            }
        }
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

    // One tile: each pair's MFMA chains run under the head sums of the pair before (pair 3
    // of tile it-1 for pair 0) and the tail (filter, staging) of the pair before that, so
    // no tail waits after a region's last head sum with the matrix pipe idle.  Pair 2's tail
    // (rows 4, 5) moves to the next tile's first region; every row still gets one tail
    // between two flush checks.  The two compiler memory barriers keep each half-step's
    // staging-list accesses in their half-step.
    __device__ __forceinline__ void step(f32x16 (&acc)[kRowsPerWave], const bf16x8 (&b)[8], int it) {
        flush_full();
        asm volatile("" ::: "memory");
        float s6 = 0.f, s0 = 0.f, s2 = 0.f;
        if (kSkip) {
            if (pl[0]) mfma2<0>(acc, b);
            if (pl[3]) s6 = hsum2<6>(acc);
            if (pl[2]) tail2<4>(s4, it - 1);
            if (pl[1]) mfma2<2>(acc, b);
            if (pl[0]) s0 = hsum2<0>(acc);
            if (pl[3]) tail2<6>(s6, it - 1);
            asm volatile("" ::: "memory");
            if (pl[2]) mfma2<4>(acc, b);
            if (pl[1]) s2 = hsum2<2>(acc);
            if (pl[0]) tail2<0>(s0, it);
            if (pl[3]) mfma2<6>(acc, b);
            if (pl[2]) s4 = hsum2<4>(acc);
            if (pl[1]) tail2<2>(s2, it);
            return;
        }
        mfma2<0>(acc, b);
        s6 = hsum2<6>(acc);
        tail2<4>(s4, it - 1);
        mfma2<2>(acc, b);
        s0 = hsum2<0>(acc);
        tail2<6>(s6, it - 1);
        asm volatile("" ::: "memory");
        mfma2<4>(acc, b);
        s2 = hsum2<2>(acc);
        tail2<0>(s0, it);
        mfma2<6>(acc, b);
        s4 = hsum2<4>(acc);
        tail2<2>(s2, it);
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
    __shared__ uint2 s_stage[kScoreThreads / kWave][kRowsPerWave * kStageSlots + kWave];
    __shared__ int s_rcnt[kRowsPerWave];  // two key parts: list entries per row from this half

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
    if (threadIdx.x < kRowsPerWave) s_rcnt[threadIdx.x] = 0;
    __syncthreads();
    float wl[kRowsPerWave];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) wl[j] = s_w[j][hf][lane & 15];

    if (n_keys > 0) {
        bf16x8 a[kRowsPerWave][8];
        // All 64 loads are issued before the first is pinned to its AGPRs (pinning each right
        // after its load made every load wait for the previous one).
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
            const u16x8* qp = reinterpret_cast<const u16x8*>(qrow[j] + (size_t)col * kIdxDim + hf * 64);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) a[j][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
        }
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(a[j][kk]));  // keep the query fragments in AGPRs
        // Key range s (part * 4 + wave) covers the contiguous tiles [s*tps, (s+1)*tps).
        const int n_tiles = (int)((n_keys + kKeyTile - 1) / kKeyTile);
        const int tps = (n_tiles + n_segs - 1) / n_segs;
        const int t0 = segment * tps;
        const int n_my = n_tiles > t0 ? min(n_tiles - t0, tps) : 0;
        // Rows of a group are consecutive (invalid rows never store), so every row's
        // list is addressed from row 0's.  With two key parts, half 1 fills the lists
        // from their tops down.
        ScoreTile<kSample, kSkip> T{P, gref.keys,
                             reinterpret_cast<const u16x8*>(P.k_tile) + (size_t)gref.tbase * (kKeyTileBytes / 16),
                             (uint32_t)gref.ntiles, a, wl,
                             {hf ? tau_r[1] : tau_r[0], hf ? tau_r[3] : tau_r[2], hf ? tau_r[5] : tau_r[4],
                              hf ? tau_r[7] : tau_r[6]},
                             {hf ? live[1] : live[0], hf ? live[3] : live[2], hf ? live[5] : live[4],
                              hf ? live[7] : live[6]},
                             kSample ? P.sample + (size_t)r0 * P.sample_stride : nullptr,
                             kSample ? nullptr : P.cand + (size_t)r0 * 2 * P.cap,
                             n0, S, kSample && S > 0 ? (float)n0 / (float)S : 0.f, lane, hf, col, col - hf,
                             (int)gref.pos, r0, !appended && part == 1, s_rcnt,
                             s_stage[wave], {0, 0, 0, 0, 0, 0, 0, 0},
                             (uint32_t)t0,
                             {kSkip && (live[0] || live[1]), kSkip && (live[2] || live[3]),
                              kSkip && (live[4] || live[5]), kSkip && (live[6] || live[7])},
                             0.f};
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
            if (!kSkip || T.pl[2]) T.s4 = T.template hsum2<4>(acc);
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
            T.flush_full();  // the last tails add up to 32 more entries to rows 4-7
            if (!kSkip || T.pl[2]) T.template tail2<4>(T.s4, n_my - 1);
            if (!kSkip || T.pl[3]) T.template epilogue2<6>(acc, n_my - 1);
            T.flush_all();
        }
    }
    // Two key parts: this half's entry count per row, once every wave has reserved its runs
    // (pad rows too: 0).
    if (!kSample && !appended) {
        __syncthreads();
        if (threadIdx.x < kRowsPerWave && r0 + (int)threadIdx.x < P.Lb)
            P.count[(size_t)(r0 + threadIdx.x) * kSegs + part] = s_rcnt[threadIdx.x];
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

template <class Sc>
__device__ __forceinline__ void block_minmax(float& mn, float& mx, Sc& S) {
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
template <class Sc>
__device__ __forceinline__ int block_incl_scan(int v, Sc& S) {
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

// Histogram hist[0..nbins) is complete; `above` values lie above every bin.  Finds, from
// the top bin down, the bin b holding the k-th largest value (1 <= k <= above + total) and
// leaves b in S.sh[0] (-1 if none), the values above b (including `above`) in S.sh[1] and
// hist[b] in S.sh[2].  Thread t sums bins nbins-1-t*per down to nbins-(t+1)*per with
// per = ceil(nbins / blockDim), so every bin is counted whatever the block size.
template <class Sc>
__device__ __forceinline__ void block_find_crossing(const int* hist, int nbins, int k, int above, Sc& S) {
    const int per = (nbins + (int)blockDim.x - 1) / (int)blockDim.x;
    const int top = nbins - 1 - (int)threadIdx.x * per;
    int c = 0;
    for (int j = 0; j < per; ++j) {  // branch-free: the reads of a thread are in flight together
        const int h = hist[max(top - j, 0)];
        c += top - j >= 0 ? h : 0;
    }
    const int incl = block_incl_scan(c, S) + above;
    const int excl = incl - c;
    if (threadIdx.x == 0) S.sh[0] = -1;
    __syncthreads();
    if (excl < k && k <= incl) {
        int acc = excl;
        for (int j = 0; j < per && top - j >= 0; ++j) {
            const int b = top - j;
            if (acc + hist[b] >= k) {
                S.sh[0] = b;
                S.sh[1] = acc;
                S.sh[2] = hist[b];
                break;
            }
            acc += hist[b];
        }
    }
    __syncthreads();
}

// k-th largest value (1-based, 1 <= k <= total) under the float order (-0 == +0) by an
// exact radix select over the order-preserving keys: three passes of 11, 11 and 10 bits
// from the top, each over the values whose higher bits match the digits found so far.
// Cannot fail; the selection's last resort when value binning does not converge.
template <class Src, class Sc>
__device__ float block_kth_radix(const Src& src, int k, Sc& S) {
    uint32_t prefix = 0u;  // the digits found so far
    int remaining = k;
    for (int pass = 0; pass < 3; ++pass) {
        const int hi = 32 - 11 * pass;             // this pass decides bits [lo, hi)
        const int lo = hi > 11 ? hi - 11 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        for (int i = threadIdx.x; i < kBins; i += blockDim.x) S.sel.hist[i] = 0;
        __syncthreads();
        src.for_each([&](float v) {
            const uint32_t key = float_order_key(v);
            if (pass == 0 || (key >> hi) == prefix) atomicAdd(&S.sel.hist[(key >> lo) & dmask], 1);
        });
        __syncthreads();
        block_find_crossing(S.sel.hist, (int)dmask + 1, remaining, 0, S);
        const int b = S.sh[0];
        remaining -= S.sh[1];
        __syncthreads();
        prefix = (prefix << (hi - lo)) | (uint32_t)b;
    }
    return order_key_float(prefix);
}

// k-th largest value (1-based, 1 <= k <= total) under the float order (-0 == +0), by
// value-linear binning (LiteTopK's bins: cheap even when every score shares an exponent)
// refined up to three times, then a rank count over the crossing bin.  A bin may still
// hold more than kDirect values after three levels (scores spread over many scales); then
// *stuck is set and, with kRadix, the exact radix select above finishes the search (its
// result is returned); without it the return value is meaningless.  (select leaves the
// radix out: inlined over its register-resident candidates it costs spills on every row;
// such rows go to the fold, which has it.)
template <bool kRadix, class Src, class Sc>
__device__ float block_kth_binned(const Src& src, int k, Sc& S, bool* stuck) {
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
        if (vmin == vmax) return vmin;
        const double scale = (double)kBins / ((double)vmax - (double)vmin);
        for (int i = threadIdx.x; i < kBins; i += blockDim.x) S.sel.hist[i] = 0;
        __syncthreads();
        src.for_each([&](float v) {
            if (active(v)) atomicAdd(&S.sel.hist[bin_of(v, vmin, scale)], 1);
        });
        __syncthreads();
        block_find_crossing(S.sel.hist, kBins, k, above, S);
        const int b = S.sh[0];
        above = S.sh[1];
        const int nb = S.sh[2];
        __syncthreads();
        if (b < 0 || (nb > kDirect && nlv + 1 == kLevels)) {  // (b < 0 only if k > total)
            *stuck = true;
            if (kRadix) return block_kth_radix(src, k, S);
            return 0.f;
        }
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
            const float kth = S.red_f[31];
            __syncthreads();
            return kth;
        }
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

// Register form of the same network for n = E * blockDim.x: thread t holds elements
// t*E .. t*E+E-1.  A compare-exchange whose partner is in the same thread is a register
// swap, one with a partner in another lane of the wave a shuffle, and only strides that
// cross waves go through LDS (two block barriers each).
template <int E, int S>
__device__ __forceinline__ void bitonic_in_thread(int (&x)[E], int size, int t) {
    if constexpr (S < E) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((e & S) == 0) {
                const bool asc = ((t * E + e) & size) == 0;  // the same for e and e | S (S < size)
                const int lo = min(x[e], x[e | S]), hi = max(x[e], x[e | S]);
                x[e] = asc ? lo : hi;
                x[e | S] = asc ? hi : lo;
            }
    }
}

template <int E>
__device__ void block_bitonic_sort_regs(int* a, int n) {
    const int t = threadIdx.x;
    int x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = a[t * E + e];
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= E) {
                const int ts = stride / E;  // partner thread t ^ ts, same element
                int y[E];
                if (ts < kWave) {
#pragma unroll
                    for (int e = 0; e < E; ++e) y[e] = __shfl_xor(x[e], ts);
                } else {
                    __syncthreads();  // earlier reads of a[] are done
#pragma unroll
                    for (int e = 0; e < E; ++e) a[t * E + e] = x[e];
                    __syncthreads();
#pragma unroll
                    for (int e = 0; e < E; ++e) y[e] = a[(t ^ ts) * E + e];
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = t * E + e;
                    const bool lower = (i & stride) == 0, asc = (i & size) == 0;
                    x[e] = lower == asc ? min(x[e], y[e]) : max(x[e], y[e]);
                }
            } else if (stride == 1) {
                bitonic_in_thread<E, 1>(x, size, t);
            } else if (stride == 2) {
                bitonic_in_thread<E, 2>(x, size, t);
            } else if (stride == 4) {
                bitonic_in_thread<E, 4>(x, size, t);
            } else {
                bitonic_in_thread<E, 8>(x, size, t);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) a[t * E + e] = x[e];
    __syncthreads();
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
                            SelectScratch& S, bool* used_radix) {
    const float kth = block_kth_binned<true>(ListSrc{L}, k, S, used_radix);
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
    // Chunks of 16 values per thread, each chunk's loads branch-free (clamped index) so that
    // they are in flight together; chunks past n are skipped (a uniform test).
#pragma unroll
    for (int c0 = 0; c0 < kPer; c0 += 16) {
        if (c0 * 256 < n) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = vals[min((int)threadIdx.x + (c0 + i) * 256, n - 1)];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool in = (int)threadIdx.x + (c0 + i) * 256 < n;
                key[c0 + i] = in ? order_key(x[i]) : 0u;
                if (in) {
                    kmin = min(kmin, key[c0 + i]);
                    kmax = max(kmax, key[c0 + i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) key[c0 + i] = 0u;
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
    if (r == 0 && threadIdx.x < kFbCtrlWords) P.fb_ctrl[threadIdx.x] = 0;
    if (P.clear_diag && r == 0 && threadIdx.x < kDiagSlots) P.diag[threadIdx.x] = 0ull;
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
        const u16x8 q2[2] = {qp[0], qp[1]};
        for (int c = 0; c < 2; ++c) {
            const u16x8 v = q2[c];
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
        KeyStats e[kStatSlots / 64];
#pragma unroll
        for (int u = 0; u < kStatSlots / 64; ++u)  // branch-free: the loads are in flight together
            e[u] = P.kstats[min((int)threadIdx.x + 64 * u, P.n_kstats - 1)];
#pragma unroll
        for (int u = 0; u < kStatSlots / 64; ++u) {
            kn = max(kn, e[u].knorm_bits);
            ki = max(ki, e[u].kinf_bits);
            ke = min(ke, e[u].kexp_min);
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
    const int per = n2 / (int)blockDim.x;  // elements per thread in the register form
    if (n2 < (int)blockDim.x) block_bitonic_sort(sel, n2);
    else if (per == 1) block_bitonic_sort_regs<1>(sel, n2);
    else if (per == 2) block_bitonic_sort_regs<2>(sel, n2);
    else if (per == 4) block_bitonic_sort_regs<4>(sel, n2);
    else if (per == 8) block_bitonic_sort_regs<8>(sel, n2);
    else if (per == 16) block_bitonic_sort_regs<16>(sel, n2);
    else block_bitonic_sort(sel, n2);
    for (int i = threadIdx.x; i < k; i += blockDim.x) out_row[i] = sel[i];
}

constexpr int kSelBand = 1024;     // band entries select re-scores (more: the row goes to the fold)
constexpr int kSelPer = 32;        // candidates per thread (blocks of many rows): cap / 32 threads
constexpr int kSelPerFew = 16;     // ... blocks of few rows: cap / 16 threads, shorter rows
constexpr int kSelMaxThreads = 4 * kMaxTopK / kSelPer;  // cap <= 4 * kMaxTopK
constexpr int kOneLevel = 256;     // a crossing bin this small ends the k-th search
// Candidate lists hold no key order; the selected keys are put in order through a bitmap of
// the causal keys when there are at most kSelBitmapKeys of them, else by a sort.
constexpr int kSelBitmapWords = 8192;
constexpr int kSelBitmapKeys = kSelBitmapWords * 32;  // 262,144 keys

// select's shared memory.  The phases use the union in turn: the k-th search (sel), the
// band (band), then the output bitmap (or out, to sort).  Small enough (~34 KB) for four
// rows per compute unit.
// Per workgroup, 16 entries x (32 / waves) heads of re-score terms per wave; 512 doubles for
// any wave count up to 16 (they sit in the union's room beside the bitmap).
constexpr int kSelTermSlots = 512;

struct SelectLds {
    union {
        struct {
            int hist[kBins];
            float direct[kDirect];
        } sel;
        struct {
            int key[kSelBand];
            int pos[kSelBand];    // candidate position of the entry
            double s[kSelBand];   // fp32 score, then its canonical fp64 score
            u16x8 q[kIdxHeads * kIdxDim / 8];  // the row's query (re-score operands)
            float w[kIdxHeads];
            QHeadStat qs[kIdxHeads];
            double tb[kSelTermSlots];  // head terms on their way to the entries' lanes
        } band;
        uint32_t bitmap[kSelBitmapWords];
        int out[kMaxTopK];
    };
    uint32_t win[kSelMaxThreads * kSelPer / 32];  // bit j: candidate position j is selected
    float red_f[32];
    int red_i[32];
    int sh[16];
};

// sum_i q_h[i] k[i] in fp64 with i ascending (bf16 x bf16 products are exact in fp64, so
// each fma rounds as the canonical add does).
__device__ double canonical_dot(const uint16_t* __restrict__ q_h, const uint16_t* __restrict__ k_row) {
    double d = 0.0;
    const u16x8* qa = reinterpret_cast<const u16x8*>(q_h);
    const u16x8* ka = reinterpret_cast<const u16x8*>(k_row);
    for (int c = 0; c < kIdxDim / 8; ++c) {
        const u16x8 qv = qa[c], kv = ka[c];
        for (int j = 0; j < 8; ++j)
            d = __builtin_fma((double)bf16_bits_to_float(qv[j]), (double)bf16_bits_to_float(kv[j]), d);
    }
    return d;
}

// Canonical fp64 scores of band entries [0, nb), in place into band_s (keys in band_key).
// One wave per block of 16 entries, all 32 heads, as two halves of 16 heads: an fp64 MFMA
// chain (16 keys x 16 heads x 4 dims per instruction) gives the head dot products when they
// are provably exact in any order (the test of band_rescore); a (key, head) that fails it
// takes the sequential evaluation in its lane.  The head terms fl(w_h max(d_h, +0)) are then
// added in ascending h exactly as the canonical order does: after the MFMAs lane (g, c) holds
// head c of the half for entries g, g+4, g+8, g+12; the terms are transposed through LDS so
// that lane m < 16 holds entry m's, and that lane adds them one head at a time, continuing
// from the first half's sum into the second.  No block barrier.
__device__ __forceinline__ void band_rescore_waves(int nb, const int* band_key, double* band_s,
                                                   const u16x8* q_lds, const float* w_lds,
                                                   const QHeadStat* qs_lds, double* tb_lds,
                                                   const uint16_t* __restrict__ q_row,
                                                   const uint16_t* __restrict__ k_idx) {
#pragma clang fp contract(off)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    if (16 * wave >= nb) return;
    // The head terms reach the lane that sums them through this wave's slice of tb_lds, hp
    // heads at a time (16 x hp doubles; hp a power of two with nwaves * 16 * hp <= 512).
    const int hp = nwaves <= 4 ? 8 : (nwaves <= 8 ? 4 : 2);
    double* tb = tb_lds + wave * 16 * hp;
    // A operand of block mb: lane (g, c) supplies key mb + c, dimensions 32g .. 32g+31.
    auto load_keys = [&](int mb, u16x8 (&kv)[4]) {
        const int key = band_key[mb + c < nb ? mb + c : mb];
        const u16x8* kp = reinterpret_cast<const u16x8*>(k_idx + (size_t)key * kIdxDim + 32 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[j] = kp[j];
    };
    for (int mb = 16 * wave; mb < nb; mb += 16 * nwaves) {
        u16x8 kv[4];
        load_keys(mb, kv);
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
        double acc = 0.0;  // lanes 0-15: the ascending-h sum of entry mb + lane so far
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int head = 16 * half + c;
            // B operand: head c of the half, dimensions 32g .. 32g+31, from the row's query in
            // LDS (read per block: held across the block loop, both halves' fragments and
            // their conversions would take 64 more registers).
            u16x8 qv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) qv[j] = q_lds[(head * kIdxDim + 32 * g) / 8 + j];
            // Two chains (even and odd K-steps) halve the dependent MFMA latency; their sum is
            // exact whenever the result is used (the exactness test below).
            f64x4 d = {0.0, 0.0, 0.0, 0.0}, d1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int ks = 0; ks < 32; ks += 2) {
                d = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_bits_to_float(kv[ks >> 3][ks & 7]),
                                                         (double)bf16_bits_to_float(qv[ks >> 3][ks & 7]), d,
                                                         0, 0, 0);
                d1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_bits_to_float(kv[(ks + 1) >> 3][(ks + 1) & 7]),
                                                          (double)bf16_bits_to_float(qv[(ks + 1) >> 3][(ks + 1) & 7]),
                                                          d1, 0, 0, 0);
            }
            d += d1;
            // Lane (g, c): the dot products of entries mb + g + 4i (i < 4) with this head.
            const double wh = (double)w_lds[head];
            const double l1 = qs_lds[head].l1;
            const int eh = qs_lds[head].e;
            double t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = g + 4 * i;
                const float kinf_m = __shfl(kinf, m);
                const int ke_m = __shfl(ke, m);
                double dh = d[i];
                const bool exact = kinf_m == 0.f || eh == INT_MAX || l1 * (double)kinf_m < ldexp(1.0, 53 + eh + ke_m);
                if (!exact && mb + m < nb)
                    dh = canonical_dot(q_row + head * kIdxDim, k_idx + (size_t)band_key[mb + m] * kIdxDim);
                t[i] = wh * (dh > 0.0 ? dh : 0.0);
            }
            // Lane m < 16 adds the terms of entry m in ascending head order: heads p0 .. p0+hp-1
            // pass through LDS (entry-major, columns XOR-swizzled by the entry against bank
            // conflicts), then the next hp.  A wave's LDS accesses complete in issue order, so
            // the reads see the writes before them; the wave barriers keep the compiler from
            // moving them across each other.
            for (int p0 = 0; p0 < 16; p0 += hp) {
                if (c >= p0 && c < p0 + hp) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = g + 4 * i;
                        tb[m * hp + ((c - p0) ^ (m & (hp - 1)))] = t[i];
                    }
                }
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                if (lane < 16) {
                    for (int j = 0; j < hp; ++j) {
                        const double x = tb[lane * hp + (j ^ (lane & (hp - 1)))];
                        acc = half == 0 && p0 == 0 && j == 0 ? x : acc + x;
                    }
                }
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
            }
        }
        if (lane < 16 && mb + lane < nb) {
            double x = acc;
            if (x == 0.0) x = 0.0;  // -0 -> +0
            band_s[mb + lane] = x;
        }
    }
}

// Exact top-k of one row's candidates.  The row's list holds key half 0's entries in slots
// [0, c0) and key half 1's in [cap - c1, cap) (more key parts: one list in [0, c0)), in no
// key order.  Thread t holds the scores of slots e * blockDim + t (e < kPer; a "position"
// below) in registers (each load instruction reads consecutive slots); keys are read from
// the list only for band entries and for the output, so a row takes 4 waves and ~35 KB of
// LDS and every row of a 1,024-row block is resident at once.
//
//   1. k-th search: a value-linear histogram over [min, max] of the row's scores, then the
//      exact range of the bin holding the k-th score; a second or third level narrows it
//      while that bin holds many scores.  The range widened by 2 delta (and a rounding
//      margin) is the band: scores above it are selected, scores below it are not.  Scores
//      over many scales can leave a band too wide for select; the row then goes to the fold.
//   2. band: the entries between are re-scored in the canonical fp64 order (one wave per
//      16 entries) and ranked by (score desc, key asc) for the remaining slots.
//   3. output: the selected keys mark a bitmap of the causal keys in LDS, and a block scan
//      of the words' bit counts places each key at its rank: ascending key order whatever
//      the list order.  Past kSelBitmapKeys causal keys they are sorted instead.
template <int kPer>
__global__ __launch_bounds__(4 * kMaxTopK / kPer, 4) void select_kernel(IndexerArgs P) {
    static_assert(kPer == 16 || kPer == 32, "per-thread candidates");
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
        if (threadIdx.x == 0) atomicAdd(&P.diag[kDiagRowsAll], 1ull);
        return;
    }
    __shared__ SelectLds S;
    const int nthr = (int)blockDim.x, tid = (int)threadIdx.x;
    // Two key parts: half 0's entries fill the list from slot 0 up, half 1's from slot cap - 1
    // down.  More key parts: one appended list from slot 0.
    const bool appended = P.parts > 2;
    const int cap = P.cap;
    // The row's list: scores in words [0, cap), keys in [cap, 2 cap), read through 32-bit byte
    // offsets from a uniform base (one address register per load instead of two).  Thread t's
    // element e is slot e * blockDim + t of the list, so the slots in use are a mask.
    const char* crow = reinterpret_cast<const char*>(P.cand + (size_t)r * 2 * cap);
    const char* ckey = crow + (size_t)4 * cap;
    auto word = [](const char* base, uint32_t i) { return *reinterpret_cast<const uint32_t*>(base + 4u * i); };
    // Loads of the slots likely in use first, branch-free (unused slots hold stale words,
    // masked below) and guarded only by a kernel argument: they are in flight before the
    // count loads are issued, so waiting for the counts does not wait for them.  The middle
    // quarter of a two-part list (slots 3/8 cap to 5/8 cap: each half holds about 0.32 cap
    // on average) is loaded only when a count reaches it (after the counts arrive; a
    // wave-uniform test), which skips a quarter of the bytes.
    auto late = [&](int e) { return !appended && (e + 1) * 8 > 3 * kPer && e * 8 < 5 * kPer; };
    float v[kPer];
    if (!P.force_fallback) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) v[e] = late(e) ? 0.f : __uint_as_float(word(crow, (uint32_t)(e * nthr + tid)));
    }
    const int c0 = P.count[(size_t)r * kSegs];
    const int c1 = appended ? 0 : P.count[(size_t)r * kSegs + 1];
    const int total = c0 + c1;
    bool ok = !P.force_fallback && total <= cap;    int why = ok ? kDiagFbIncomplete : kDiagFbOverflow;  // the reason if the row falls back
    ok = ok && total >= k;
    const float tau_f = P.tau[r];
    const float delta = P.delta[r];
    // Slot j is in use iff it lies in half 0's run or in half 1's.
    auto slot_used = [&](int j) { return j < c0 || j >= cap - c1; };
    if (ok) {
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (late(e) && (e * nthr < c0 || (e + 1) * nthr > cap - c1))
                v[e] = __uint_as_float(word(crow, (uint32_t)(e * nthr + tid)));
    }
    uint32_t used = 0u;                     // bit e: element e holds a candidate (set below)
    auto in_use = [&](int e) { return ((used >> e) & 1u) != 0u; };
    if (tid == 0) {
        S.sh[4] = 0;
        S.sh[5] = 0;
    }
    float vmin = INFINITY, vmax = -INFINITY;
    if (ok) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) used |= (uint32_t)slot_used(e * nthr + tid) << e;
        asm volatile("" : "+v"(used));  // one register holds the mask (not 32 partial ones)
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const bool in = in_use(e);
            v[e] = in ? v[e] + 0.0f : -INFINITY;
            if (in) {
                vmin = fminf(vmin, v[e]);
                vmax = fmaxf(vmax, v[e]);
            }
        }
    }
    // 1. The band [lo, hi] around the k-th score.  [blo, bhi] holds the k-th score and
    // `above` scores lie above bhi.  A level bins the scores in [blo, bhi]; if the bin b
    // holding the k-th score is small (or three levels are done), the k-th score lies
    // within b's edges, up to the rounding of the bin arithmetic (margin), else the next
    // level narrows [blo, bhi] to the exact range of bin b (bins are monotonic in the score,
    // so that range holds exactly bin b's scores).
    double lo = 0.0, hi = 0.0;
    if (ok) {
        block_minmax(vmin, vmax, S);
        float blo = vmin, bhi = vmax;
        double elo = vmin, ehi = vmax;  // the k-th score lies in [elo, ehi] (up to margin)
        int above = 0;
        for (int level = 0; level < 3 && blo != bhi; ++level) {
            const double scale = (double)kBins / ((double)bhi - (double)blo);
            for (int i = tid; i < kBins; i += nthr) S.sel.hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (in_use(e) && v[e] >= blo && v[e] <= bhi) atomicAdd(&S.sel.hist[bin_of(v[e], blo, scale)], 1);
            __syncthreads();
            block_find_crossing(S.sel.hist, kBins, k, above, S);
            const int b = S.sh[0];  // >= 0: the k-th score lies in [blo, bhi]
            above = S.sh[1];
            const int nbin = S.sh[2];
            if (nbin <= kOneLevel || level == 2) {
                elo = (double)blo + (double)b / scale;
                ehi = (double)blo + (double)(b + 1) / scale;
                break;
            }
            float mn = INFINITY, mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (in_use(e) && v[e] >= blo && v[e] <= bhi && bin_of(v[e], blo, scale) == b) {
                    mn = fminf(mn, v[e]);
                    mx = fmaxf(mx, v[e]);
                }
            block_minmax(mn, mx, S);
            blo = mn;
            bhi = mx;
            elo = mn;
            ehi = mx;
        }
        const double d2 = 2.0 * (double)delta;
        const double margin = (fabs(elo) + fabs(ehi) + 2.0 * d2) * 0x1p-40;
        lo = elo - d2 - margin;
        hi = ehi + d2 + margin;
    }
    if (ok && tau_f != -INFINITY && lo < (double)tau_f) ok = false;  // candidate set not provably complete
    // 2. The band: collect, re-score, rank.
    int nb_row = 0, n_in = 0;
    if (ok) {
        // Positions above the band get their bit of S.win now (one wave owns the 64 bits of an
        // element's ballot); band winners are added after the re-score.  The scores are not
        // needed after this pass.
        int n_above = 0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const double sd = (double)v[e];
            const uint64_t am = __ballot(in_use(e) && sd > hi);
            if ((tid & 63) == 0) {
                const int w0 = (e * nthr + (tid & ~63)) >> 5;
                S.win[w0] = (uint32_t)am;
                S.win[w0 + 1] = (uint32_t)(am >> 32);
                n_above += __builtin_popcountll(am);
            }
            const int b = wave_append(in_use(e) && sd <= hi && sd >= lo, &S.sh[5]);
            if (b >= 0 && b < kSelBand) {
                S.band.pos[b] = e * nthr + tid;
                S.band.s[b] = sd;
            }
        }
        // The row's query, weights and head statistics for the re-score.
        if (delta > 0.f) {
            const u16x8* qg = reinterpret_cast<const u16x8*>(ref.q);
            for (int i = tid; i < kIdxHeads * kIdxDim / 8; i += nthr) S.band.q[i] = qg[i];
            if (tid < kIdxHeads) {
                S.band.w[tid] = ref.w[tid];
                S.band.qs[tid] = P.qstat[(size_t)r * kIdxHeads + tid];
            }
        }
        if ((tid & 63) == 0) atomicAdd(&S.sh[4], n_above);
        __syncthreads();
        n_in = S.sh[4];
        const int nb = S.sh[5];
        ok = nb <= kSelBand && n_in < k && n_in + nb >= k;
        why = kDiagFbBand;
        nb_row = nb;
        if (ok) {
            // The band entries' keys, all loads in flight at once.
            for (int x = tid; x < nb; x += nthr) S.band.key[x] = (int)word(ckey, (uint32_t)S.band.pos[x]);
            __syncthreads();
            if (delta > 0.f && nb > 0)
                band_rescore_waves(nb, S.band.key, S.band.s, S.band.q, S.band.w, S.band.qs, S.band.tb, ref.q,
                                   ref.keys);
            __syncthreads();
            // Entry x wins if fewer than k - n_in band entries beat it (branch-free compares
            // over batches of 8 entries, so the LDS reads of a batch are in flight together).
            const int need = k - n_in;
            for (int x = tid; x < nb; x += nthr) {
                const double sx = S.band.s[x];
                const int ix = S.band.key[x];
                int beat = 0;
                for (int y0 = 0; y0 < nb; y0 += 8) {
                    double sy[8];
                    int ky[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int y = min(y0 + u, nb - 1);
                        sy[u] = S.band.s[y];
                        ky[u] = S.band.key[y];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        beat += (int)((y0 + u < nb) & ((sy[u] > sx) | ((sy[u] == sx) & (ky[u] < ix))));
                }
                if (beat < need) atomicOr(&S.win[S.band.pos[x] >> 5], 1u << (S.band.pos[x] & 31));
            }
            __syncthreads();
        }
    }
    // 3. Output: selected = above the band, or a band winner.
    if (ok) {
        // Bit e: position e * blockDim + tid is selected (all 32 words read at once).
        uint32_t selmask = 0u;
        {
            uint32_t wd[kPer];
#pragma unroll
            for (int e = 0; e < kPer; ++e) wd[e] = S.win[(e * nthr + tid) >> 5];
#pragma unroll
            for (int e = 0; e < kPer; ++e) selmask |= ((wd[e] >> ((e * nthr + tid) & 31)) & 1u) << e;
        }
        auto selected = [&](int e) { return ((selmask >> e) & 1u) != 0u; };
        // Branch-free key loads, as for the scores; a slot that is not selected re-reads the
        // wave's first slot (a line the wave touches anyway), so only selected slots cost traffic.
        int key[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) key[e] = (int)word(ckey, (uint32_t)(selected(e) ? e * nthr + tid : tid));
        if (nt <= kSelBitmapKeys) {
            // Causal keys within the bitmap: mark the selected keys, then each thread writes
            // the keys of its bitmap words [t per, (t + 1) per) from its scanned offset on, so
            // the output ascends.
            const int nw = (int)((nt + 31) >> 5);
            for (int i = tid; i < nw; i += nthr) S.bitmap[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (selected(e)) atomicOr(&S.bitmap[key[e] >> 5], 1u << (key[e] & 31));
            __syncthreads();
            const int per = (nw + nthr - 1) / nthr;
            const int w0 = tid * per, w1 = min(nw, w0 + per);
            int c = 0;
            for (int i = w0; i < w1; ++i) c += __builtin_popcount(S.bitmap[i]);
            int o = block_incl_scan(c, S) - c;
            for (int i = w0; i < w1; ++i) {
                uint32_t bits = S.bitmap[i];
                while (bits) {
                    const int bit = __builtin_ctz(bits);
                    bits &= bits - 1u;
                    if (o < k) out_row[o] = i * 32 + bit;
                    ++o;
                }
            }
        } else {
            // A larger key range: gather the selection, then sort it (a register bitonic
            // network costs less than several bitmap passes past 262,144 keys).
            int c = 0;
#pragma unroll
            for (int e = 0; e < kPer; ++e) c += selected(e);
            int o = block_incl_scan(c, S) - c;
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (selected(e)) {
                    if (o < k) S.out[o] = key[e];
                    ++o;
                }
            __syncthreads();
            write_sorted_output(S.out, k, out_row);
        }
    }
    if (!ok && tid == 0) {
        const int slot = atomicAdd(&P.fb_ctrl[0], 1);
        P.fb_list[slot] = r;
        atomicAdd(&P.diag[kDiagFallback], 1ull);
        atomicAdd(&P.diag[why], 1ull);
    }
    if (ok && tid == 0) {
        atomicAdd(&P.diag[kDiagRows], 1ull);
        atomicAdd(&P.diag[kDiagCandSum], (unsigned long long)total);
        atomicMax(&P.diag[kDiagCandMax], (unsigned long long)total);
        atomicAdd(&P.diag[kDiagBandSum], (unsigned long long)nb_row);
        atomicMax(&P.diag[kDiagBandMax], (unsigned long long)nb_row);
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
    // The next tile's key loads are issued before this tile's MFMAs (tile indices clamped).
    auto load = [&](int64_t ti, bf16x8 (&b)[8]) {
        const int64_t pos = k0 + ti * kKeyTile + col;
        const int64_t key = pos < k1 ? pos : k1 - 1;
        const u16x8* kp = reinterpret_cast<const u16x8*>(R.keys + key * kIdxDim + hf * 8);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) b[kk] = __builtin_bit_cast(bf16x8, kp[2 * kk]);
    };
    bf16x8 b[8];
    if (wave < n_tiles) load(wave, b);
    for (int64_t ti = wave; ti < n_tiles; ti += n_waves) {
        const int64_t pos = k0 + ti * kKeyTile + col;
        bf16x8 bn[8];
        load(ti + n_waves < n_tiles ? ti + n_waves : ti, bn);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc = mfma_32x32x16(a[kk], b[kk], acc);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) b[kk] = bn[kk];
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

// The exact blocked fold of one row's keys [k_lo, k_hi) (at least k of them) over 4,096-key
// blocks: the running list is cut back to its exact top-k whenever the next block could
// overflow it, and after the last block; new keys are admitted only if score > kth(list at
// the last cut) - 2 delta.  Leaves the list's top-k in (Rs[cur], Ri[cur]) (n entries) and
// returns false if a cut failed (never expected).  Every thread of the block calls it.
struct FoldBufs {
    float* Rs[2];
    int* Ri[2];
    int* band_i;
    double* band_s;
    float* band_f;
};
__device__ bool fold_range(const IndexerArgs& P, int r, const RowRef& ref, int64_t k_lo, int64_t k_hi,
                           const FoldBufs& B, SelectScratch& S, int* s_cnt, int& cur, int& n, bool& radix) {
    const int k = P.top_k;
    const float delta = P.delta[r];
    cur = 0;
    n = 0;
    float lo = -INFINITY;
    for (int64_t b0 = k_lo; b0 < k_hi; b0 += kFoldKeys) {
        const int64_t b1 = b0 + kFoldKeys < k_hi ? b0 + kFoldKeys : k_hi;
        if (threadIdx.x == 0) *s_cnt = n;
        __syncthreads();
        fold_score_block(ref, b0, b1, lo, B.Rs[cur], B.Ri[cur], s_cnt, P.fold_cap);
        __syncthreads();
        n = *s_cnt < P.fold_cap ? *s_cnt : P.fold_cap;
        __syncthreads();
        // The list is cut back to its exact top-k only when the next block could overflow
        // it, and after the last block: admitted keys accumulate over many blocks in
        // between (the admission threshold from the last cut stays a valid lower bound, as
        // the list's k-th score only rises), so the cut runs a few times per row, not once
        // per 4,096 keys.
        if (n > k && (n > P.fold_cap - kFoldKeys || b1 >= k_hi)) {
            // Keep exactly the top-k of the list; their fp32 scores go to the other buffer.
            const int nxt = cur ^ 1;
            CandList L{};
            L.s[0] = B.Rs[cur];
            L.i[0] = B.Ri[cur];
            L.n[0] = n;
            L.nseg = 1;
            // The k-th search cannot fail and the band fits (its capacity is the list's), so
            // select_core succeeds; should it not, the row is emitted as -1 and counted.
            const bool ok = select_core(L, k, delta, ref.q, ref.w, P.qstat + (size_t)r * kIdxHeads, ref.keys,
                                        B.band_i, B.band_s, B.band_f, P.fold_cap, B.Ri[nxt], B.Rs[nxt], S,
                                        &radix);
            __syncthreads();
            if (!ok) return false;  // uniform over the block
            cur = nxt;
            n = k;
            CandList R{};
            R.s[0] = B.Rs[cur];
            R.i[0] = B.Ri[cur];
            R.n[0] = n;
            R.nseg = 1;
            const float kth = block_kth_binned<true>(ListSrc{R}, k, S, &radix);
            const double l = (double)kth - 2.0 * (double)delta;
            float lf = (float)l;
            if ((double)lf > l) lf = nextafterf(lf, -INFINITY);
            lo = lf;
        }
    }
    return true;
}

// Key ranges a split row's fold takes: each holds at least top_k keys (so each range's
// top-k list is full), at most kFoldParts of them, and the merge's ranges x top_k entries
// fit the fold's band buffer (fold_cap entries): when every score ties, the whole union is
// the merge's band.
__device__ __forceinline__ int fold_parts(int64_t nt, int k, int fold_cap) {
    int64_t p = nt / k;
    const int64_t fit = fold_cap / k;
    if (p > fit) p = fit;
    return (int)(p < 1 ? 1 : (p > kFoldParts ? kFoldParts : p));
}

// Persistent: each workgroup takes work items one at a time.  Items [0, n_split *
// kFoldParts) are (row j, range p) of the first n_split flagged rows: range p of row j's
// fold_parts() key ranges is folded to its exact top-k, which goes to the row's merge
// area; the workgroup that finishes the row's last range (a device-scope counter) merges
// the ranges' lists with one more exact selection (the top-k of the union of the ranges'
// top-k lists is the row's top-k).  Items past those are the remaining flagged rows, each
// folded whole.  No workgroup waits for another.
__global__ __launch_bounds__(kSelectThreads) void fold_kernel(IndexerArgs P) {
    __shared__ SelectScratch S;
    __shared__ int s_item, s_cnt, s_last;
    const int slot = blockIdx.x;
    const FoldBufs B{{P.fold_s + (size_t)slot * 2 * P.fold_cap, P.fold_s + (size_t)slot * 2 * P.fold_cap + P.fold_cap},
                     {P.fold_i + (size_t)slot * 2 * P.fold_cap, P.fold_i + (size_t)slot * 2 * P.fold_cap + P.fold_cap},
                     P.fold_bi + (size_t)slot * P.fold_cap, P.fold_bs + (size_t)slot * P.fold_cap,
                     P.fold_bf + (size_t)slot * P.fold_cap};
    const int k = P.top_k;
    const int n_fb = P.fb_ctrl[0];  // final here (select has finished)
    if (n_fb == 0) return;          // nothing to fold
    const int n_split = n_fb < kFoldSplitRows ? n_fb : kFoldSplitRows;
    const int n_items = n_split * kFoldParts + (n_fb - n_split);
    int* parts_done = P.fb_ctrl + 4;
    int* part_flags = P.fb_ctrl + 4 + kFoldSplitRows;  // bit 0: a range failed; bit 1: one needed the radix select
    for (;;) {
        if (threadIdx.x == 0) s_item = atomicAdd(&P.fb_ctrl[1], 1);
        __syncthreads();
        const int item = s_item;
        __syncthreads();
        if (item >= n_items) return;
        const bool split = item < n_split * kFoldParts;
        const int j = split ? item / kFoldParts : n_split + (item - n_split * kFoldParts);
        const int part = split ? item % kFoldParts : 0;
        const int r = P.fb_list[j];
        const RowRef ref = row_ref(P, r);
        const int64_t p = ref.pos;
        const int64_t nt = (p < ref.nkeys - 1 ? p : ref.nkeys - 1) + 1;
        const int np = split ? fold_parts(nt, k, P.fold_cap) : 1;
        if (part >= np) continue;  // an unused range slot of a shorter row
        bool radix = false;
        int32_t* out_row = ref.out;
        if (np == 1) {  // the row whole
            int cur, n;
            const bool ok = fold_range(P, r, ref, 0, nt, B, S, &s_cnt, cur, n, radix);
            if (radix && threadIdx.x == 0) atomicAdd(&P.diag[kDiagRadix], 1ull);
            if (!ok) {
                for (int x = threadIdx.x; x < k; x += blockDim.x) out_row[x] = -1;
                if (threadIdx.x == 0) atomicAdd(&P.diag[kDiagFailed], 1ull);
                __syncthreads();
                continue;
            }
            // n == k here (nt > k for every scored row): the list is the exact top-k.
            for (int x = threadIdx.x; x < k; x += blockDim.x) S.out[x] = x < n ? B.Ri[cur][x] : -1;
            __syncthreads();
            write_sorted_output(S.out, k, out_row);
            __syncthreads();
            continue;
        }
        // Range `part` of np: [part nt / np, (part + 1) nt / np), at least k keys.
        const int64_t k_lo = nt * part / np, k_hi = nt * (part + 1) / np;
        int cur, n;
        const bool ok = fold_range(P, r, ref, k_lo, k_hi, B, S, &s_cnt, cur, n, radix);
        float* ms = P.fold_ms + ((size_t)j * kFoldParts) * k;
        int* mi = P.fold_mi + ((size_t)j * kFoldParts) * k;
        // The range's top-k (exactly k entries: the range holds at least k keys) to its slice.
        for (int x = threadIdx.x; x < k; x += blockDim.x) {
            const bool have = ok && x < n;
            ms[(size_t)part * k + x] = have ? B.Rs[cur][x] : -INFINITY;
            mi[(size_t)part * k + x] = have ? B.Ri[cur][x] : -1;
        }
        // Publish the slice (device-scope release), then count the range; the workgroup that
        // counts the last range reads every slice after an acquire fence.
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            if (!ok || radix) atomicOr(&part_flags[j], (ok ? 0 : 1) | (radix ? 2 : 0));
            s_last = atomicAdd(&parts_done[j], 1) == np - 1;
        }
        __syncthreads();
        if (!s_last) continue;
        __threadfence();
        const int flags = atomicOr(&part_flags[j], 0);
        radix = (flags & 2) != 0;
        bool merged = false;
        if ((flags & 1) == 0) {
            CandList L{};
            L.s[0] = ms;
            L.i[0] = mi;
            L.n[0] = np * k;
            L.nseg = 1;
            merged = select_core(L, k, P.delta[r], ref.q, ref.w, P.qstat + (size_t)r * kIdxHeads, ref.keys,
                                 B.band_i, B.band_s, B.band_f, P.fold_cap, B.Ri[0], B.Rs[0], S, &radix);
            __syncthreads();
        }
        if (radix && threadIdx.x == 0) atomicAdd(&P.diag[kDiagRadix], 1ull);  // once per row
        if (!merged) {
            for (int x = threadIdx.x; x < k; x += blockDim.x) out_row[x] = -1;
            if (threadIdx.x == 0) atomicAdd(&P.diag[kDiagFailed], 1ull);
            __syncthreads();
            continue;
        }
        for (int x = threadIdx.x; x < k; x += blockDim.x) S.out[x] = B.Ri[0][x];
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
                             unsigned long long* diag, hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    static_assert(kStatsThreads / kWave == 4 && kKeyTileKeys == 32, "key_stats_blocks assumes 4 waves of 32-key tiles");
    const int blocks = key_stats_blocks(n_keys);
    key_stats_kernel<<<blocks, kStatsThreads, 0, s>>>(k_idx, n_keys, nullptr, 0, 0,
                                                     (n_keys + kKeyTileKeys - 1) / kKeyTileKeys, ks, k_tile, diag,
                                                     false);
    return hipGetLastError();
}

hipError_t launch_key_stats_batch(const uint16_t* k_idx, const SeqKeys* seqs, int n_seqs, int64_t n_tiles,
                                  KeyStats* ks, uint16_t* k_tile, unsigned long long* diag, hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    const int blocks = key_stats_blocks(n_tiles * kKeyTileKeys);
    key_stats_kernel<<<blocks, kStatsThreads, 0, s>>>(k_idx, 0, seqs, n_seqs, 0, n_tiles, ks, k_tile, diag, false);
    return hipGetLastError();
}

__global__ void key_cache_reset_kernel(KeyStats* stats) {
    if (threadIdx.x == 0) *stats = KeyStats{0u, 0u, INT_MAX, 0};
}

hipError_t launch_key_cache_append(const uint16_t* k_idx, int64_t n_old, int64_t n_new, KeyStats* stats,
                                   uint16_t* k_tile, hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    if (n_old == 0) {
        key_cache_reset_kernel<<<1, 64, 0, s>>>(stats);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // The tile holding key n_old is laid out again whole (its keys below n_old included).
    const int64_t t0 = n_old / kKeyTileKeys, t1 = (n_new + kKeyTileKeys - 1) / kKeyTileKeys;
    if (t1 <= t0) return hipSuccess;
    const int blocks = key_stats_blocks((t1 - t0) * kKeyTileKeys);
    key_stats_kernel<<<blocks, kStatsThreads, 0, s>>>(k_idx, n_new, nullptr, 0, t0, t1, stats, k_tile, nullptr, true);
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
        // Blocks of few rows (decode, short chunks) give each row twice the threads: with all
        // rows resident anyway, a row's latency is the launch time.
        if (a.Lb >= 512) select_kernel<kSelPer><<<a.Lb, a.cap / kSelPer, 0, s>>>(a);
        else select_kernel<kSelPerFew><<<a.Lb, a.cap / kSelPerFew, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfFold);
        fold_kernel<<<kFallbackSlots, kSelectThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ score dump (diagnostic)

// One workgroup per block row: the row of `scores` is set to NaN, then every (score, key)
// entry the filter stored for the row (key half 0's in slots [0, c0), half 1's in
// [cap - c1, cap)) is written to its key's column.  With tau = -inf the filter stores every
// causal key.
__global__ __launch_bounds__(256) void score_dump_kernel(IndexerArgs P, float* scores, int64_t n_cols,
                                                         float* delta_out) {
    const int r = blockIdx.x;
    float* row = scores + (size_t)r * n_cols;
    for (int64_t c = threadIdx.x; c < n_cols; c += blockDim.x) row[c] = __uint_as_float(0x7fc00000u);
    __syncthreads();
    const int c0 = P.count[(size_t)r * kSegs], c1 = P.count[(size_t)r * kSegs + 1];
    const uint32_t* e = P.cand + (size_t)r * 2 * P.cap;
    if (c0 + c1 <= P.cap)
        for (int i = threadIdx.x; i < P.cap; i += blockDim.x)
            if (i < c0 || i >= P.cap - c1) {
                const uint32_t key = e[P.cap + i];
                if ((int64_t)key < n_cols) row[key] = __uint_as_float(e[i]);
            }
    if (threadIdx.x == 0 && delta_out) delta_out[r] = P.delta[r];
}

hipError_t launch_score_dump(const IndexerArgs& a, float* scores, int64_t n_cols, float* delta_out, hipStream_t s) {
    const int groups = (a.Lb + kRowsPerGroup - 1) / kRowsPerGroup;
    hipError_t e = launch_row_prep(a, s);
    if (e != hipSuccess) return e;
    score_kernel<false, false><<<8 * ((groups + 3) / 4), kScoreThreads, 0, s>>>(a, groups);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    score_dump_kernel<<<a.Lb, 256, 0, s>>>(a, scores, n_cols, delta_out);
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
