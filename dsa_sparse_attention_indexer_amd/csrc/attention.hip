// attention.hip -- sparse absorbed-MLA prefill attention for gfx950.
//
// "GLM prefill now attends only to the keys its indexer picks", How it works: the
// 512-wide latent and 64-wide rope caches form one 576-wide key per position; each
// query gathers only its top-k rows; every head shares that gathered block; the
// latent is also the value, so the output is 512 wide per head.
//
// One workgroup per query, one wave per 16 heads (at least 4 waves: the extra waves of
// a small head count only gather).  Per 32-key tile:
//   gather   the 32 selected rows (row-major, 1152 bytes each) into one of two LDS
//            buffers by DMA (global_load_lds, 16 bytes per lane, consecutive lanes on
//            consecutive pieces of a row).  The next tile's rows and the keys of the
//            tile after it are requested before the current tile is computed, so the
//            gather latency hides behind the MFMAs without staging registers; the
//            [top_k x 576] block never exists in HBM.  The compiler does not track LDS
//            DMA, so each wave waits on vmcnt itself before the tile barrier
//   logits   S^T[key][head] = K . Q^T on 16x16x32 bf16 MFMA (M = keys, N = heads,
//            18 K-steps over 576); Q stays in registers for the whole row
//   softmax  online, fp32, base-2 with log2(e) folded into the scale; invalid keys
//            (-1, > position, padding) contribute nothing
//   values   O^T[d][head] += V^T . P^T on 16x16x32 MFMA.  V^T comes straight from the
//            row-major tile through the LDS transpose read (ds_read_b64_tr_b16), and the
//            logits' output layout is already the B operand (lane = head, 8 keys per
//            lane) once the K order of the product is permuted to match, so P never
//            leaves registers
#include <math.h>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kAttnTile = 32;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowChunks = kDqk * 2 / 16;             // 72 16-byte pieces per key row
constexpr int kTileChunks = kAttnTile * kRowChunks;   // 2304
constexpr int kKrowStride = kDqk + 8;   // 1168 B: conflict-free 16-lane column reads
constexpr int kAttnMinThreads = 256;

typedef __attribute__((ext_vector_type(4))) short s16x4;

// Four bf16 of column block [d0, d0+4) from four consecutive tile rows, transposed
// across each 16-lane group (lane i receives column d0 + i of rows r..r+3 when source
// lane s addresses row r + s/4, columns 4*(s%4)..+4).
__device__ __forceinline__ u16x4 lds_read_tr(const uint16_t* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u16x4, v);
}

// Neighbour packing (LiteDSA page, Fig. 3 and abstract: neighbouring tokens' candidate sets
// overlap, so they are gathered once and attended jointly, each query masking the keys it did
// not select): workgroup b takes queries 2b and 2b + 1.  Its prologue builds the union of the
// two index rows in LDS with a 2-bit mask per key (query q may use the key iff bit q is set);
// each union tile is gathered once and the first H/16 waves attend for query 2b, the next
// H/16 for query 2b + 1.  Rows that are ascending with a -1 tail (what the indexer writes)
// are merged with duplicates removed; other rows are simply concatenated.
constexpr int kPackMaxK = 2048;  // top_k limit of the packed kernel (LDS for the union)

// Union of the pair's rows into s_ukey / s_umask (returns the entry count).  Every thread of
// the workgroup takes part; the result is published by a barrier.
__device__ int pack_union(const AttentionArgs& A, int t0, int* s_ra, int* s_rb, int* s_d, int* s_ukey,
                          uint8_t* s_umask, int* s_cnt, int* s_scan) {
    const int tid = threadIdx.x, nthreads = blockDim.x, K = A.top_k;
    const bool has1 = t0 + 1 < A.Lb;
    const int64_t p0 = A.pos0 + t0, p1 = p0 + 1;
    if (tid < 4) s_cnt[tid] = 0;
    for (int i = tid; i < K; i += nthreads) {
        s_ra[i] = A.idx[(size_t)t0 * K + i];
        s_rb[i] = has1 ? A.idx[(size_t)(t0 + 1) * K + i] : -1;
    }
    __syncthreads();
    // Mergeable: the entries >= 0 form a strictly ascending prefix, then only -1.
    int ca = 0, cb = 0, bad = 0;
    for (int i = tid; i < K; i += nthreads) {
        const int x = s_ra[i], xn = i + 1 < K ? s_ra[i + 1] : -1;
        const int y = s_rb[i], yn = i + 1 < K ? s_rb[i + 1] : -1;
        ca += x >= 0;
        cb += y >= 0;
        bad |= (x < 0 && (x != -1 || xn >= 0)) || (x >= 0 && xn >= 0 && xn <= x);
        bad |= (y < 0 && (y != -1 || yn >= 0)) || (y >= 0 && yn >= 0 && yn <= y);
    }
    if (ca) atomicAdd(&s_cnt[0], ca);
    if (cb) atomicAdd(&s_cnt[1], cb);
    if (bad) atomicOr(&s_cnt[2], 1);
    __syncthreads();
    const int a = s_cnt[0], b = s_cnt[1];
    auto bit0 = [&](int key) { return key >= 0 && key <= p0 ? 1 : 0; };
    auto bit1 = [&](int key) { return has1 && key >= 0 && key <= p1 ? 2 : 0; };
    if (s_cnt[2]) {  // concatenation: every entry of row 0, then every entry of row 1
        for (int i = tid; i < K; i += nthreads) {
            s_ukey[i] = s_ra[i];
            s_umask[i] = (uint8_t)bit0(s_ra[i]);
            s_ukey[K + i] = s_rb[i];
            s_umask[K + i] = (uint8_t)bit1(s_rb[i]);
        }
        __syncthreads();
        return has1 ? 2 * K : K;
    }
    // Sorted: number of entries of row 0 below x (and whether x occurs in it), by bisection.
    auto lower = [&](const int* v, int n, int x) {
        int lo = 0, hi = n;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (v[mid] < x) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    // Inclusive scan of one int per thread, in thread order (Hillis-Steele in s_scan).
    auto block_scan = [&](int v) {
        s_scan[tid] = v;
        __syncthreads();
        for (int d = 1; d < nthreads; d <<= 1) {
            const int u = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += u;
            __syncthreads();
        }
        const int r = s_scan[tid];
        __syncthreads();
        return r;
    };
    // s_d[j] = entries of row 1 before j that also occur in row 0 (each thread a chunk of j).
    const int per = (b + nthreads - 1) / nthreads;
    const int j0 = tid * per, j1 = min(b, j0 + per);
    int dups = 0;
    for (int j = j0; j < j1; ++j) dups += lower(s_ra, a, s_rb[j]) < a && s_ra[lower(s_ra, a, s_rb[j])] == s_rb[j];
    int before = block_scan(dups) - dups;
    for (int j = j0; j < j1; ++j) {
        const int l = lower(s_ra, a, s_rb[j]);
        s_d[j] = before;
        before += l < a && s_ra[l] == s_rb[j];
    }
    if (tid == nthreads - 1) s_d[b] = before;  // the last chunk ends at b (or is empty): all duplicates
    __syncthreads();
    // Union position of a row-0 entry: i + (row-1 entries below it) - (duplicates among those);
    // of a row-1 entry that is not in row 0: j - (duplicates before it) + (row-0 entries below it).
    for (int i = tid; i < a; i += nthreads) {
        const int x = s_ra[i];
        const int l = lower(s_rb, b, x);
        const bool dup = l < b && s_rb[l] == x;
        const int pos = i + l - s_d[l];
        s_ukey[pos] = x;
        s_umask[pos] = (uint8_t)(bit0(x) | (dup ? bit1(x) : 0));
    }
    for (int j = tid; j < b; j += nthreads) {
        const int y = s_rb[j];
        const int l = lower(s_ra, a, y);
        if (l < a && s_ra[l] == y) continue;
        const int pos = j - s_d[j] + l;
        s_ukey[pos] = y;
        s_umask[pos] = (uint8_t)bit1(y);
    }
    __syncthreads();
    return a + b - s_d[b];
}

// Reductions over the four 16-lane groups of a wave (lanes c16, c16+16, c16+32, c16+48 hold
// one head): a row swap (lanes l and l^16) then a half swap (l and l^32), each one VALU
// instruction instead of an LDS permute and its wait.  Both lanes of a swapped pair combine
// the same two values (max, and + are commutative), so every lane of a head gets the same
// result: ((x0 + x16) + (x32 + x48)) for the sum.
__device__ __forceinline__ float max_lane_groups(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_lane_groups(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// kSplit: workgroup (t, s) takes the tiles [s*tps, (s+1)*tps) of query t (tps = tiles per
// split) and writes an unnormalised partial instead of the output.  kPack: workgroup b takes
// the pair (2b, 2b + 1) over the union of their rows (see pack_union).
template <bool kSplit, bool kPack>
__global__ __launch_bounds__(512) void sparse_attn_kernel(AttentionArgs A) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int c16 = lane & 15;
    const int nthreads = blockDim.x;
    const int hq = A.H / 16;                 // waves per query
    const int qsel = kPack ? wave / hq : 0;  // the query of the pair this wave attends for
    const int t = kPack ? 2 * (int)blockIdx.x + qsel : (int)blockIdx.x;
    int64_t p = A.pos0 + t;
    const uint16_t* kv = A.kv;
    if (A.qinfo) {  // a batch: the query's own sequence
        const QueryInfo qi = A.qinfo[t];
        p = qi.pos;
        kv = A.kv + (size_t)qi.kbase * A.kv_stride;
    }
    const bool compute = kPack ? (qsel < 2 && t < A.Lb) : wave < hq;
    const int h = (kPack ? wave - qsel * hq : wave) * 16 + c16;
    // The K order of the value product (and, to match, the row order of the logits):
    // lane group g takes tile rows slot_row(g, 0..3) and 16 + those.  Groups 0, 1 get the
    // even rows 0..14 and groups 2, 3 the odd ones, so the transpose reads of each lane
    // pair of groups land on disjoint LDS banks with the 1168-byte row stride.
    auto slot_row = [](int grp, int j) { return 8 * (grp & 1) + 2 * j + (grp >> 1); };
    const int pi_c = slot_row(c16 >> 2, c16 & 3);  // A-operand row of lane c16 in the logits

    __shared__ __attribute__((aligned(16))) uint16_t Kbuf[2][kAttnTile][kKrowStride];
    __shared__ int s_idx[3][kAttnTile];  // raw top-k entries of three consecutive tiles
    // packed pair: the two rows, duplicate counts, the union and its masks
    constexpr int kPk = kPack ? kPackMaxK : 1;
    __shared__ int s_ra[kPk], s_rb[kPk], s_d[kPk + 1], s_ukey[2 * kPk], s_cnt[4], s_scan[kPack ? 512 : 1];
    __shared__ uint8_t s_umask[2 * kPk];

    const int32_t* irow = A.idx + (size_t)t * A.top_k;
    int n_union = 0;
    if (kPack) n_union = pack_union(A, 2 * (int)blockIdx.x, s_ra, s_rb, s_d, s_ukey, s_umask, s_cnt, s_scan);
    const int n_all = ((kPack ? n_union : A.top_k) + kAttnTile - 1) / kAttnTile;
    const int tps = kSplit ? (n_all + A.splits - 1) / A.splits : n_all;
    const int t_lo = kSplit ? (int)blockIdx.y * tps : 0;
    const int n_tiles = t_lo + tps < n_all ? t_lo + tps : n_all;  // one past this workgroup's last tile
    const int nwaves = nthreads >> 6;
    // Entry j of the row as a key this query may use, or -1.
    const int p32 = (int)p;  // <= N - 1 <= INT32_MAX - 1
    // (packed: union entry tile_j + r, a key one of the pair may use, or -1)
    auto key_of = [&](int slot, int r, int tile_j) -> int {
        if (kPack) {
            const int e = tile_j + r;
            return e < n_union && s_umask[e] ? s_ukey[e] : -1;
        }
        const int key = s_idx[slot][r];
        return (tile_j + r < A.top_k && key >= 0 && key <= p32) ? key : -1;
    };
    // Entry r of the tile at tile_j usable by this wave's query.
    auto usable = [&](int slot, int r, int tile_j) -> bool {
        if (kPack) {
            const int e = tile_j + r;
            return e < n_union && ((s_umask[e] >> qsel) & 1);
        }
        return key_of(slot, r, tile_j) >= 0;
    };
    // DMA of the raw entries of tile j into slot (lanes past top_k fetch nothing).
    auto fetch_idx = [&](int j, int slot) {
        if (!kPack && wave == 0 && lane < kAttnTile && j * kAttnTile + lane < A.top_k)
            dma_lds4(irow + j * kAttnTile + lane, &s_idx[slot][0]);
    };
    // DMA of the rows of tile j (entries in slot) into buffer buf: wave w takes rows
    // w, w + nwaves, ...; a row is 72 pieces, one 64-lane request and one of 8 lanes.
    // The wave's rows are wave + nwaves * i (i < kAttnTile / nwaves <= 8, nwaves >= 4): lane i
    // looks up row i's key, all in one LDS access, and each row's DMA takes its key from that
    // lane, so the rows' lookups do not wait on the LDS one after another.
    auto fetch_rows = [&](int j, int slot, int buf) {
        const int ri = wave + nwaves * (lane & 7);
        const int kl = ri < kAttnTile ? key_of(slot, ri, j * kAttnTile) : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wave + nwaves * i;
            if (r >= kAttnTile) break;
            int key = __builtin_amdgcn_readlane(kl, i);
            key = key < 0 ? 0 : key;  // masked later; any valid row will do
            const char* src = reinterpret_cast<const char*>(kv + (size_t)key * A.kv_stride);
            char* dst = reinterpret_cast<char*>(&Kbuf[buf][r][0]);
            dma_lds16(src + lane * 16, dst);
            if (lane < kRowChunks - 64)
                dma_lds16(src + 1024 + lane * 16, dst + 1024);
        }
    };
    // This wave's DMAs have landed; the barrier then publishes every wave's.
    auto dma_wait = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    if (t_lo < n_tiles) fetch_idx(t_lo, t_lo % 3);
    if (t_lo + 1 < n_tiles) fetch_idx(t_lo + 1, (t_lo + 1) % 3);
    dma_wait();
    __syncthreads();
    if (t_lo < n_tiles) fetch_rows(t_lo, t_lo % 3, t_lo & 1);
    dma_wait();

    bf16x8 qf[kDqk / 32];
    f32x4 o[kDv / 16];
    if (compute) {
        const uint16_t* qrow = A.q + ((size_t)t * A.H + h) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qrow + ks * 32));
        // Take the query fragments' load waits here, once: left to first use, they would
        // sit inside the tile loop and also wait for that tile's gather DMAs.
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) asm volatile("" :: "v"(qf[ks]));
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) o[dt] = f32x4{};
    }
    // lsum: sum of the bf16 weights actually multiplied into V (normalises the output);
    // lexp: sum of the unrounded fp32 weights (gives the log-sum-exp).
    float m = -INFINITY, lsum = 0.f, lexp = 0.f;
    const float sl2 = A.scale * 1.4426950408889634f;
    __syncthreads();

    for (int tile = t_lo; tile < n_tiles; ++tile) {
        const int cur = tile & 1;
        const int slot = tile % 3;
        // Rows of the next tile and the entries of the tile after it are in flight while
        // this one is computed.
        if (tile + 1 < n_tiles) fetch_rows(tile + 1, (tile + 1) % 3, cur ^ 1);
        if (tile + 2 < n_tiles) fetch_idx(tile + 2, (tile + 2) % 3);

        if (compute) {
            f32x4 s0 = f32x4{}, s1 = f32x4{};
            // The two MFMA loops run at raised wave priority: the other wave on this SIMD is
            // then usually in its softmax, and its VALU work fills the slots the matrix pipe
            // leaves (measured ~1% faster than equal priority).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < kDqk / 32; ++ks) {
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Kbuf[cur][pi_c][ks * 32 + 8 * g]));
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Kbuf[cur][16 + pi_c][ks * 32 + 8 * g]));
                s0 = mfma_16x16x32(a0, qf[ks], s0);
                s1 = mfma_16x16x32(a1, qf[ks], s1);
            }
            __builtin_amdgcn_s_setprio(0);
            // Usable entries of the tile as a bit mask (bit r: entry r), one ballot per wave.
            const uint32_t vmask = (uint32_t)__ballot(lane < kAttnTile && usable(slot, lane & 31, tile * kAttnTile));
            // Element r of this lane's logits is tile row slot_row(g, r) (s0) or 16 + that (s1).
            const uint32_t mlo = vmask >> slot_row(g, 0), mhi = vmask >> (16 + slot_row(g, 0));
            float lg[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lg[r] = s0[r] * sl2;
                lg[4 + r] = s1[r] * sl2;
            }
            if (vmask != 0xffffffffu) {  // wave-uniform: most tiles have every entry usable
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lg[r] = (mlo >> (2 * r)) & 1u ? lg[r] : -INFINITY;
                    lg[4 + r] = (mhi >> (2 * r)) & 1u ? lg[4 + r] : -INFINITY;
                }
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) tmax = fmaxf(tmax, lg[r]);
            tmax = max_lane_groups(tmax);
            // The exponentials are taken against a reference m that moves only when a tile's
            // maximum exceeds it by more than 2^8 (weights then stay below 256, well inside
            // bf16 and fp32), so the accumulator rescale is skipped on most tiles.
            const bool bump = tmax > m + 8.0f;
            if (__ballot(bump)) {
                const float alpha = bump ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;
#pragma unroll
                for (int dt = 0; dt < kDv / 16; ++dt) o[dt] *= alpha;
                lsum *= alpha;
                lexp *= alpha;
                m = bump ? tmax : m;
            }
            u16x8 pb;
            float ps = 0.f, pe = 0.f;
            if (m == -INFINITY) {  // nothing usable yet (the same for every head)
#pragma unroll
                for (int r = 0; r < 8; ++r) pb[r] = 0;
            } else {
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    const float e0 = __builtin_amdgcn_exp2f(lg[r] - m);
                    const float e1 = __builtin_amdgcn_exp2f(lg[r + 1] - m);
                    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
                    const uint32_t b2 = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)e0, (__bf16)e1});
                    pb[r] = (uint16_t)b2;
                    pb[r + 1] = (uint16_t)(b2 >> 16);
                    ps += __uint_as_float(b2 << 16) + __uint_as_float(b2 & 0xffff0000u);
                    pe += e0 + e1;
                }
            }
            ps = sum_lane_groups(ps);
            pe = sum_lane_groups(pe);
            lsum += ps;
            lexp += pe;
            const bf16x8 pbf = __builtin_bit_cast(bf16x8, pb);
            // Source lane (g, c16) addresses row slot_row(g, c16/4) (K slots 0-3 of its group)
            // or 16 + that (slots 4-7), columns 4*(c16%4)..+4 of each 16-column block.
            const uint16_t* vlo = &Kbuf[cur][slot_row(g, c16 >> 2)][4 * (c16 & 3)];
            const uint16_t* vhi = vlo + 16 * kKrowStride;
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int dt = 0; dt < kDv / 16; ++dt) {
                const u16x4 lo = lds_read_tr(vlo + dt * 16);
                const u16x4 hi = lds_read_tr(vhi + dt * 16);
                const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, av), pbf, o[dt]);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        dma_wait();
        __syncthreads();
    }

    if (!compute) return;
    if (kSplit) {
        const size_t ph = ((size_t)t * A.splits + blockIdx.y) * A.H + h;
        float* po = A.part_o + ph * kDv + 4 * g;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
        if (g == 0) *reinterpret_cast<f32x4*>(A.part_ml + ph * 4) = f32x4{m, lsum, lexp, 0.f};
        return;
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

// Merge of the split partials of query t, head h (one workgroup of 128 threads, four
// output columns per thread): with M the largest reference max over the splits and
// c_s = 2^(m_s - M), out = sum_s c_s O_s / sum_s c_s l_s and lse = M + log2(sum_s c_s e_s)
// (natural log on output), exactly the normalisation of the unsplit kernel.
__global__ __launch_bounds__(128) void attn_merge_kernel(AttentionArgs A) {
    const int t = blockIdx.x, h = blockIdx.y;
    __shared__ float s_c[kMaxSplits];
    __shared__ float s_norm[2];
    const size_t base = (size_t)t * A.splits * A.H + h;  // partial (t, s, h) = base + s * H
    if (threadIdx.x < 64) {
        float mx = -INFINITY;
        for (int sp = threadIdx.x; sp < A.splits; sp += 64)
            mx = fmaxf(mx, A.part_ml[(base + (size_t)sp * A.H) * 4]);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float den = 0.f, dex = 0.f;
        for (int sp = threadIdx.x; sp < A.splits; sp += 64) {
            const f32x4 ml = *reinterpret_cast<const f32x4*>(A.part_ml + (base + (size_t)sp * A.H) * 4);
            const float c = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - mx);
            s_c[sp] = c;
            den += c * ml[1];
            dex += c * ml[2];
        }
        for (int o = 32; o > 0; o >>= 1) {
            den += __shfl_xor(den, o);
            dex += __shfl_xor(dex, o);
        }
        if (threadIdx.x == 0) {
            s_norm[0] = den > 0.f ? 1.0f / den : 0.f;
            if (A.lse) A.lse[(size_t)t * A.H + h] = dex > 0.f ? (mx + log2f(dex)) * 0.6931471805599453f : -INFINITY;
        }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const float* po = A.part_o + base * kDv + 4 * threadIdx.x;
    const size_t stride = (size_t)A.H * kDv;  // between consecutive splits
    constexpr int kU = 8;                     // loads issued together
    for (int s0 = 0; s0 < A.splits; s0 += kU) {
        f32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = s0 + u < A.splits ? *reinterpret_cast<const f32x4*>(po + (size_t)(s0 + u) * stride) : f32x4{};
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (s0 + u < A.splits) acc += s_c[s0 + u] * v[u];
    }
    const float inv = s_norm[0];
    u16x4 pk;
#pragma unroll
    for (int r = 0; r < 4; ++r) pk[r] = float_to_bf16_rne(acc[r] * inv);
    *reinterpret_cast<u16x4*>(A.out + ((size_t)t * A.H + h) * kDv + 4 * threadIdx.x) = pk;
}

hipError_t launch_sparse_attention(const AttentionArgs& a, hipStream_t s) {
    int threads = 64 * (a.H / 16);
    if (threads < kAttnMinThreads) threads = kAttnMinThreads;
    ProfScope ps(s, kProfAttention);
    sparse_attn_kernel<false, false><<<a.Lb, threads, 0, s>>>(a);
    return hipGetLastError();
}

bool sparse_attention_packable(const AttentionArgs& a) {
    return !a.qinfo && a.H <= 64 && a.top_k <= kPackMaxK;
}

hipError_t launch_sparse_attention_packed(const AttentionArgs& a, hipStream_t s) {
    int threads = 2 * 64 * (a.H / 16);
    if (threads < kAttnMinThreads) threads = kAttnMinThreads;
    ProfScope ps(s, kProfAttention);
    sparse_attn_kernel<false, true><<<(a.Lb + 1) / 2, threads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_sparse_attention_split(const AttentionArgs& a, hipStream_t s) {
    int threads = 64 * (a.H / 16);
    if (threads < kAttnMinThreads) threads = kAttnMinThreads;
    {
        ProfScope ps(s, kProfAttnSplit);
        sparse_attn_kernel<true, false><<<dim3(a.Lb, a.splits), threads, 0, s>>>(a);
    }
    {
        ProfScope ps(s, kProfAttnMerge);
        attn_merge_kernel<<<dim3(a.Lb, a.H), kDv / 4, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace dsa
