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
//   5. select           exact top-k of the candidates: radix select of the fp32 k-th
//                       score, fp64 re-score of the keys within 2 delta of it, rank
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
__device__ __forceinline__ int wave_min_i(int v) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Canonical fp64 term fl(w_h * max(0, sum_i q_h[i] k[i])) with i ascending.
__device__ double canonical_head_term(const uint16_t* __restrict__ q_h,
                                      const uint16_t* __restrict__ k_row, float w_h) {
#pragma clang fp contract(off)
    double d = 0.0;
    const u16x8* qa = reinterpret_cast<const u16x8*>(q_h);
    const u16x8* ka = reinterpret_cast<const u16x8*>(k_row);
    for (int c = 0; c < kIdxDim / 8; ++c) {
        u16x8 qv = qa[c], kv = ka[c];
        for (int j = 0; j < 8; ++j) {
            double prod = (double)bf16_bits_to_float(qv[j]) * (double)bf16_bits_to_float(kv[j]);
            d = d + prod;
        }
    }
    double r = d > 0.0 ? d : 0.0;
    return (double)w_h * r;
}

// ------------------------------------------------------------------ 1. key stats

__global__ void init_stats_kernel(KeyStats* ks) {
    if (threadIdx.x == 0) {
        ks->knorm_bits = 0u;
        ks->kinf_bits = 0u;
        ks->kexp_min = INT_MAX;
        ks->pad = 0;
    }
}

__global__ __launch_bounds__(256) void key_stats_kernel(const uint16_t* __restrict__ k_idx,
                                                        int64_t n_keys, KeyStats* ks) {
    float nmax = 0.f, amax = 0.f;
    int emin = INT_MAX;
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n_keys;
         s += (int64_t)gridDim.x * blockDim.x) {
        const u16x8* kr = reinterpret_cast<const u16x8*>(k_idx + s * kIdxDim);
        float ss = 0.f;
        for (int c = 0; c < kIdxDim / 8; ++c) {
            u16x8 v = kr[c];
            for (int j = 0; j < 8; ++j) {
                float x = bf16_bits_to_float(v[j]);
                ss = fmaf(x, x, ss);
                amax = fmaxf(amax, fabsf(x));
                if ((v[j] & 0x7fff) != 0) emin = min(emin, bf16_lsb_exp(v[j]));
            }
        }
        nmax = fmaxf(nmax, sqrtf(ss));
    }
    nmax = wave_max(nmax);
    amax = wave_max(amax);
    emin = wave_min_i(emin);
    if ((threadIdx.x & 63) == 0) {
        // 128 fp32 squares+adds and the sqrt: relative error < 2^-16; pad by 2^-14.
        float up = nmax * (1.0f + 1.0f / 16384.0f);
        atomicMax(&ks->knorm_bits, __float_as_uint(up));
        atomicMax(&ks->kinf_bits, __float_as_uint(amax));
        atomicMin(&ks->kexp_min, emin);
    }
}

// ------------------------------------------------------------------ 2/4. MFMA scoring

// One workgroup = 4 consecutive query rows; each of its 4 waves takes every 4th
// 32-key tile.  Lane l owns head (l & 31) of the A operand and key (l & 31) of the B
// operand; its half (l >> 5) holds dimensions [64*half, 64*half+64) split into eight
// MFMA K-steps of 8, the same permutation on both operands.
template <bool kSample>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(IndexerArgs P) {
    const int g = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;
    const int col = lane & 31;
    __shared__ int s_count[kRowsPerGroup];

    int64_t pr[kRowsPerGroup];
    float tau_r[kRowsPerGroup];
    int row_of[kRowsPerGroup];
    bool live[kRowsPerGroup];
    int64_t n_keys = 0;
    const int r0 = g * kRowsPerGroup;
    int S = 0;
    int64_t n0 = 0;
#pragma unroll
    for (int j = 0; j < kRowsPerGroup; ++j) {
        int r = r0 + j;
        bool valid = r < P.Lb;
        row_of[j] = valid ? r : r0;
        int64_t p = P.pos0 + r;
        pr[j] = valid ? p : -1;
        int64_t nt = valid ? (p < P.N - 1 ? p : P.N - 1) + 1 : 0;
        if (kSample) {
            live[j] = valid;
            tau_r[j] = 0.f;
        } else {
            bool use = valid && P.mode[r] == kModeNormal;
            live[j] = use;
            tau_r[j] = use ? P.tau[r] : INFINITY;
            if (use && nt > n_keys) n_keys = nt;
        }
    }
    if (kSample) {
        int64_t p = P.pos0 + r0;
        n0 = (p < P.N - 1 ? p : P.N - 1) + 1;
        S = sample_size(n0, P.top_k, P.cap);
        n_keys = S;
    }
    if (threadIdx.x < kRowsPerGroup) s_count[threadIdx.x] = 0;
    __syncthreads();

    if (n_keys > 0) {
        bf16x8 a[kRowsPerGroup][8];
        float wf[kRowsPerGroup][16];
#pragma unroll
        for (int j = 0; j < kRowsPerGroup; ++j) {
            const u16x8* qp = reinterpret_cast<const u16x8*>(
                P.q_idx + ((size_t)row_of[j] * kIdxHeads + col) * kIdxDim + hf * 64);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) a[j][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int h = 8 * (i >> 2) + 4 * hf + (i & 3);
                wf[j][i] = P.w[(size_t)row_of[j] * kIdxHeads + h];
            }
        }
        const int64_t n_tiles = (n_keys + kKeyTile - 1) / kKeyTile;
        for (int64_t ti = wave; ti < n_tiles; ti += kScoreThreads / kWave) {
            const int64_t pos = ti * kKeyTile + col;
            int64_t key;
            if (kSample) key = pos < S ? (pos * n0) / S : 0;
            else key = pos < P.N ? pos : P.N - 1;
            const u16x8* kp = reinterpret_cast<const u16x8*>(P.k_idx + key * kIdxDim + hf * 64);
            bf16x8 b[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) b[kk] = __builtin_bit_cast(bf16x8, kp[kk]);
            f32x16 acc[kRowsPerGroup];
#pragma unroll
            for (int j = 0; j < kRowsPerGroup; ++j) acc[j] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int j = 0; j < kRowsPerGroup; ++j) acc[j] = mfma_32x32x16(a[j][kk], b[kk], acc[j]);
#pragma unroll
            for (int j = 0; j < kRowsPerGroup; ++j) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) part += wf[j][i] * fmaxf(acc[j][i], 0.f);
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                           false, false);
                float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                s = s + 0.0f;
                if (kSample) {
                    if (hf == 0 && pos < S && live[j]) P.sample[(size_t)row_of[j] * P.sample_stride + pos] = s;
                } else {
                    bool keep = live[j] && hf == 0 && pos <= pr[j] && s >= tau_r[j];
                    uint64_t m = __ballot(keep);
                    if (m) {
                        int base = 0;
                        if (lane == 0) base = atomicAdd(&s_count[j], __builtin_popcountll(m));
                        base = __shfl(base, 0);
                        if (keep) {
                            int o = base + mbcnt64(m);
                            if (o < P.cap) {
                                size_t off = (size_t)row_of[j] * P.cap + o;
                                P.cand_s[off] = s;
                                P.cand_i[off] = (int)pos;
                            }
                        }
                    }
                }
            }
        }
    }
    if (!kSample) {
        __syncthreads();
        if (threadIdx.x < kRowsPerGroup && r0 + (int)threadIdx.x < P.Lb)
            P.count[r0 + threadIdx.x] = s_count[threadIdx.x];
    }
}

// ------------------------------------------------------------------ block-wide radix select

// k-th largest (1-based) of v[0..n) under the float order (-0 == +0); 1 <= k <= n.
// All threads of the block must call it.  hist: 256 ints of LDS, sh: 4 ints of LDS.
__device__ float block_kth_largest(const float* v, int n, int k, int* hist, int* sh) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            uint32_t key = float_order_key(v[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int l = threadIdx.x;
            int c[4], lsum = 0;
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * l - j];
                lsum += c[j];
            }
            int incl = lsum;
            for (int o = 1; o < 64; o <<= 1) {
                int t = __shfl_up(incl, o);
                if (l >= o) incl += t;
            }
            int excl = incl - lsum;
            if (excl < remaining && remaining <= incl) {
                int acc = excl;
                for (int j = 0; j < 4; ++j) {
                    if (acc + c[j] >= remaining) {
                        sh[0] = 255 - 4 * l - j;
                        sh[1] = acc;
                        break;
                    }
                    acc += c[j];
                }
            }
        }
        __syncthreads();
        const int d = sh[0];
        remaining -= sh[1];
        prefix |= (uint32_t)d << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    return order_key_float(prefix);
}

// Bitonic sort (ascending) of n = power of two ints in LDS.
__device__ void block_bitonic_sort(int* a, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool asc = (lo & size) == 0;
                int x = a[lo], y = a[hi];
                if ((x > y) == asc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

struct SelectScratch {
    int hist[256];
    int sh[8];
    double term[32][kIdxHeads];  // fp64 re-score staging: 32 keys x 32 heads
};

// Exact top-k of a candidate list (cs, ci, c) under (canonical score desc, key asc).
// Writes the k selected keys (unordered) to sel_i and, if sel_s is not null, their
// fp32 scores to sel_s.  band_i / band_s / band_f: caller storage for up to band_cap
// near-threshold entries (key, canonical score, fp32 score).
// Returns false (uniformly) when the candidate set cannot be proven complete
// (k-th fp32 score within 2 delta of the filter threshold) or the band overflows.
__device__ bool select_core(const float* cs, const int* ci, int c, int k, float delta,
                            float tau_f, const uint16_t* __restrict__ q_row,
                            const float* __restrict__ w_row, const uint16_t* __restrict__ k_idx,
                            int* band_i, double* band_s, float* band_f, int band_cap, int* sel_i,
                            float* sel_s, SelectScratch& S) {
    const float kth = block_kth_largest(cs, c, k, S.hist, S.sh);
    const double lo = (double)kth - 2.0 * (double)delta;
    const double hi = (double)kth + 2.0 * (double)delta;
    if (tau_f != -INFINITY && lo < (double)tau_f) return false;
    if (threadIdx.x == 0) {
        S.sh[2] = 0;  // selected count
        S.sh[3] = 0;  // band count
    }
    __syncthreads();
    for (int i = threadIdx.x; i < c; i += blockDim.x) {
        const float s = cs[i];
        const double sd = (double)s;
        if (sd > hi) {
            int o = atomicAdd(&S.sh[2], 1);
            if (o < k) {  // at most k - 1 keys lie above kth + 2 delta
                sel_i[o] = ci[i];
                if (sel_s) sel_s[o] = s;
            }
        } else if (sd >= lo) {
            int b = atomicAdd(&S.sh[3], 1);
            if (b < band_cap) {
                band_i[b] = ci[i];
                band_s[b] = sd;
                band_f[b] = s;
            }
        }
    }
    __syncthreads();
    const int n_in = S.sh[2];
    const int nb = S.sh[3];
    if (nb > band_cap) return false;
    const int need = k - n_in;
    if (delta > 0.f) {
        // Re-score the band in the canonical fp64 order: 32 keys x 32 heads per pass.
        for (int b0 = 0; b0 < nb; b0 += 32) {
            for (int it = threadIdx.x; it < 32 * kIdxHeads; it += blockDim.x) {
                const int bl = it >> 5, h = it & 31;
                if (b0 + bl < nb) {
                    const int key = band_i[b0 + bl];
                    S.term[bl][h] = canonical_head_term(q_row + h * kIdxDim,
                                                        k_idx + (size_t)key * kIdxDim, w_row[h]);
                }
            }
            __syncthreads();
            if (threadIdx.x < 32 && b0 + (int)threadIdx.x < nb) {
#pragma clang fp contract(off)
                double s = 0.0;
                for (int h = 0; h < kIdxHeads; ++h) s = s + S.term[threadIdx.x][h];
                if (s == 0.0) s = 0.0;
                band_s[b0 + threadIdx.x] = s;
            }
            __syncthreads();
        }
    }
    // Rank count: a band key is selected iff fewer than `need` band keys beat it.
    for (int x = threadIdx.x; x < nb; x += blockDim.x) {
        const double sx = band_s[x];
        const int ix = band_i[x];
        int beat = 0;
        for (int y = 0; y < nb && beat < need; ++y) {
            const double sy = band_s[y];
            beat += (sy > sx) || (sy == sx && band_i[y] < ix);
        }
        if (beat < need) {
            int o = atomicAdd(&S.sh[2], 1);
            if (o < k) {
                sel_i[o] = ix;
                if (sel_s) sel_s[o] = band_f[x];
            }
        }
    }
    __syncthreads();
    return S.sh[2] == k;  // always true; guards the LDS writes above
}

// ------------------------------------------------------------------ 3. row prep

__global__ __launch_bounds__(256) void row_prep_kernel(IndexerArgs P) {
    const int r = blockIdx.x;
    const int64_t p = P.pos0 + r;
    const int64_t nt = (p < P.N - 1 ? p : P.N - 1) + 1;
    __shared__ double s_l1[kIdxHeads], s_l2[kIdxHeads];
    __shared__ int s_eq[kIdxHeads];
    __shared__ float s_delta;
    __shared__ int s_hist[256];
    __shared__ int s_sh[8];
    if (r == 0 && threadIdx.x == 0) {
        P.fb_ctrl[0] = 0;
        P.fb_ctrl[1] = 0;
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
        const u16x8* qp = reinterpret_cast<const u16x8*>(P.q_idx + ((size_t)r * kIdxHeads + h) * kIdxDim + part * 16);
        double l1 = 0.0, l2 = 0.0;
        int em = INT_MAX;
        for (int c = 0; c < 2; ++c) {
            u16x8 v = qp[c];
            for (int j = 0; j < 8; ++j) {
                double x = (double)bf16_bits_to_float(v[j]);
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
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const KeyStats ks = *P.kstats;
        const double knorm = (double)__uint_as_float(ks.knorm_bits);
        const double kinf = (double)__uint_as_float(ks.kinf_bits);
        const float* wr = P.w + (size_t)r * kIdxHeads;
        // Exactness: every product and partial sum of the fp32 evaluation is a multiple
        // of 2^emin and below 2^(24+emin) in magnitude -> fp32 scores are exact.
        double lhs = 0.0, dsum = 0.0;
        int emin = INT_MAX;
        bool any = false;
        for (int h = 0; h < kIdxHeads; ++h) {
            const float wh = wr[h];
            dsum += fabs((double)wh) * sqrt(s_l2[h]);
            if (wh != 0.f && s_l1[h] > 0.0) {
                any = true;
                lhs += fabs((double)wh) * s_l1[h] * kinf;
                emin = min(emin, f32_lsb_exp(wh) + s_eq[h]);
            }
        }
        bool exact;
        if (!any || ks.kexp_min == INT_MAX) {
            exact = true;  // every score is exactly zero
        } else {
            const int e = emin + ks.kexp_min;
            exact = (e >= -100) && (lhs * (1.0 + 1e-12) < ldexp(1.0, 24 + e));
            // each head's dot product must also stay above the fp32 subnormal range
            for (int h = 0; h < kIdxHeads && exact; ++h)
                if (s_l1[h] > 0.0 && s_eq[h] + ks.kexp_min < -100) exact = false;
        }
        float d = 0.f;
        if (!exact) {
            double dd = kDeltaCoef * ldexp(1.0, -24) * knorm * dsum;
            d = (float)(dd * (1.0 + 1.0 / 1048576.0));
            if (!(d > 0.f)) d = FLT_MIN;
        }
        s_delta = d;
        P.delta[r] = d;
        P.mode[r] = kModeNormal;
    }
    __syncthreads();
    const int g0 = r & ~(kRowsPerGroup - 1);
    const int64_t pg = P.pos0 + g0;
    const int64_t n0 = (pg < P.N - 1 ? pg : P.N - 1) + 1;
    const int S = sample_size(n0, P.top_k, P.cap);
    if (S == 0) {  // the whole group keeps every causal key (at most cap per row)
        if (threadIdx.x == 0) P.tau[r] = -INFINITY;
        return;
    }
    const int rk = sample_rank(n0, S, P.top_k);
    const float that = block_kth_largest(P.sample + (size_t)r * P.sample_stride, S, rk, s_hist, s_sh);
    if (threadIdx.x == 0) {
        double t = (double)that - 2.0 * (double)s_delta;
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

constexpr int kSelBand = 2048;

__global__ __launch_bounds__(kSelectThreads) void select_kernel(IndexerArgs P) {
    const int r = blockIdx.x;
    const int64_t p = P.pos0 + r;
    const int64_t nt = (p < P.N - 1 ? p : P.N - 1) + 1;
    int32_t* out_row = P.out + (size_t)r * P.top_k;
    if (P.mode[r] == kModeAll) {
        for (int j = threadIdx.x; j < P.top_k; j += blockDim.x) out_row[j] = j < nt ? j : -1;
        return;
    }
    __shared__ SelectScratch S;
    __shared__ int s_band_i[kSelBand];
    __shared__ double s_band_s[kSelBand];
    __shared__ float s_band_f[kSelBand];
    __shared__ int s_sel[4096];
    const int c = P.count[r];
    bool ok = !P.force_fallback && c <= P.cap && c >= P.top_k;
    if (ok) {
        ok = select_core(P.cand_s + (size_t)r * P.cap, P.cand_i + (size_t)r * P.cap, c, P.top_k,
                         P.delta[r], P.tau[r], P.q_idx + (size_t)r * kIdxHeads * kIdxDim,
                         P.w + (size_t)r * kIdxHeads, P.k_idx, s_band_i, s_band_s, s_band_f,
                         kSelBand, s_sel, nullptr, S);
    }
    if (!ok) {
        if (threadIdx.x == 0) {
            int slot = atomicAdd(&P.fb_ctrl[0], 1);
            P.fb_list[slot] = r;
        }
        return;
    }
    write_sorted_output(s_sel, P.top_k, out_row);
}

// ------------------------------------------------------------------ 6. fallback fold

// Scores keys [k0, k1) of one row with MFMA (8 waves, one 32-key tile per wave per step)
// and appends those with score > lo to (dst_s, dst_i) at *cnt (LDS counter).
__device__ void fold_score_block(const IndexerArgs& P, int r, int64_t k0, int64_t k1, float lo,
                                 float* dst_s, int* dst_i, int* cnt, int cap) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hf = lane >> 5, col = lane & 31;
    const int n_waves = blockDim.x >> 6;
    const u16x8* qp = reinterpret_cast<const u16x8*>(P.q_idx + ((size_t)r * kIdxHeads + col) * kIdxDim + hf * 64);
    bf16x8 a[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) a[kk] = __builtin_bit_cast(bf16x8, qp[kk]);
    float wf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wf[i] = P.w[(size_t)r * kIdxHeads + 8 * (i >> 2) + 4 * hf + (i & 3)];
    const int64_t n_tiles = (k1 - k0 + kKeyTile - 1) / kKeyTile;
    for (int64_t ti = wave; ti < n_tiles; ti += n_waves) {
        const int64_t pos = k0 + ti * kKeyTile + col;
        const int64_t key = pos < k1 ? pos : k1 - 1;
        const u16x8* kp = reinterpret_cast<const u16x8*>(P.k_idx + key * kIdxDim + hf * 64);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc = mfma_32x32x16(a[kk], __builtin_bit_cast(bf16x8, kp[kk]), acc);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part += wf[i] * fmaxf(acc[i], 0.f);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        s = s + 0.0f;
        // Later keys lose ties, so only a score strictly above kth - 2 delta can enter.
        bool keep = hf == 0 && pos < k1 && s > lo;
        uint64_t m = __ballot(keep);
        if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(cnt, __builtin_popcountll(m));
            base = __shfl(base, 0);
            if (keep) {
                int o = base + mbcnt64(m);
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
    __shared__ int s_sel[4096];
    const int slot = blockIdx.x;
    float* Rs[2] = {P.fold_s + (size_t)slot * 2 * P.fold_cap, P.fold_s + (size_t)slot * 2 * P.fold_cap + P.fold_cap};
    int* Ri[2] = {P.fold_i + (size_t)slot * 2 * P.fold_cap, P.fold_i + (size_t)slot * 2 * P.fold_cap + P.fold_cap};
    int* band_i = P.fold_bi + (size_t)slot * P.fold_cap;
    double* band_s = P.fold_bs + (size_t)slot * P.fold_cap;
    float* band_f = P.fold_bf + (size_t)slot * P.fold_cap;
    const int k = P.top_k;
    for (;;) {
        if (threadIdx.x == 0) {
            int i = atomicAdd(&P.fb_ctrl[1], 1);
            s_row = i < P.fb_ctrl[0] ? P.fb_list[i] : -1;
        }
        __syncthreads();
        const int r = s_row;
        __syncthreads();
        if (r < 0) return;
        const int64_t p = P.pos0 + r;
        const int64_t nt = (p < P.N - 1 ? p : P.N - 1) + 1;
        const float delta = P.delta[r];
        const uint16_t* q_row = P.q_idx + (size_t)r * kIdxHeads * kIdxDim;
        const float* w_row = P.w + (size_t)r * kIdxHeads;
        int cur = 0, n = 0;
        float lo = -INFINITY;
        for (int64_t b0 = 0; b0 < nt; b0 += kFoldKeys) {
            const int64_t b1 = b0 + kFoldKeys < nt ? b0 + kFoldKeys : nt;
            if (threadIdx.x == 0) s_cnt = n;
            __syncthreads();
            fold_score_block(P, r, b0, b1, lo, Rs[cur], Ri[cur], &s_cnt, P.fold_cap);
            __syncthreads();
            n = s_cnt;
            __syncthreads();
            if (n > k) {
                // Keep exactly the top-k of the list; their fp32 scores go to the other buffer.
                const int nxt = cur ^ 1;
                bool ok = select_core(Rs[cur], Ri[cur], n, k, delta, -INFINITY, q_row, w_row, P.k_idx,
                                      band_i, band_s, band_f, P.fold_cap, Ri[nxt], Rs[nxt], S);
                (void)ok;  // band capacity == list capacity: cannot overflow
                __syncthreads();
                cur = nxt;
                n = k;
                const float kth = block_kth_largest(Rs[cur], n, k, S.hist, S.sh);
                double l = (double)kth - 2.0 * (double)delta;
                float lf = (float)l;
                if ((double)lf > l) lf = nextafterf(lf, -INFINITY);
                lo = lf;
            }
        }
        int32_t* out_row = P.out + (size_t)r * k;
        // n == k here (nt > k for every scored row): the list is the exact top-k.
        for (int j = threadIdx.x; j < k; j += blockDim.x) s_sel[j] = j < n ? Ri[cur][j] : -1;
        __syncthreads();
        write_sorted_output(s_sel, k, out_row);
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

hipError_t launch_key_stats(const uint16_t* k_idx, int64_t n_keys, KeyStats* ks, hipStream_t s) {
    ProfScope ps(s, kProfKeyStats);
    init_stats_kernel<<<1, 64, 0, s>>>(ks);
    int blocks = (int)((n_keys + 255) / 256);
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    key_stats_kernel<<<blocks, 256, 0, s>>>(k_idx, n_keys, ks);
    return hipGetLastError();
}

hipError_t launch_indexer_block(const IndexerArgs& a, bool need_sample, hipStream_t s) {
    const int groups = (a.Lb + kRowsPerGroup - 1) / kRowsPerGroup;
    if (need_sample) {
        ProfScope ps(s, kProfScoreSample);
        score_kernel<true><<<groups, kScoreThreads, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfRowPrep);
        row_prep_kernel<<<a.Lb, 256, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfScoreFilter);
        score_kernel<false><<<groups, kScoreThreads, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfSelect);
        select_kernel<<<a.Lb, kSelectThreads, 0, s>>>(a);
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
