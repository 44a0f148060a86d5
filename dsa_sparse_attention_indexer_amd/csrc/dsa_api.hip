// dsa_api.hip -- the C ABI (include/dsa.h): argument checks, workspace carving and
// the query-block loop.  Host code only; every step of the path runs in the kernels
// of indexer.hip and attention.hip.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

// Device scratch of dsa_indexer_topk_noalloc: one copy per GPU the library runs on, held
// until the process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol): it asks each device for the address of its copy once
// (hipGetSymbolAddress, with that device current) and passes that pointer on.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace dsa {
namespace {
std::atomic<uint32_t> g_prof_mask{0};  // kernel classes bracketed by events (bit k: class k)
std::mutex g_prof_mu;
struct ProfRecord {
    int kernel;
    hipEvent_t start, stop;
};
std::vector<ProfRecord> g_prof;
const char* const kProfNames[kProfCount] = {"key_stats", "score_sample", "row_prep", "score_filter",
                                            "select", "fold", "sparse_attention", "causal_mask",
                                            "attn_split", "attn_merge", "retr_prep", "retr_sample",
                                            "retr_filter", "retr_gather", "ceiling_mfma", "ceiling_copy"};
}  // namespace

ProfScope::ProfScope(hipStream_t s, int k) : stream(s), kernel(k), start(nullptr), on(false) {
    if (!((g_prof_mask.load(std::memory_order_relaxed) >> k) & 1u)) return;
    if (hipEventCreate(&start) != hipSuccess) return;
    if (hipEventRecord(start, s) != hipSuccess) {
        (void)hipEventDestroy(start);
        return;
    }
    on = true;
}

ProfScope::~ProfScope() {
    if (!on) return;
    hipEvent_t stop;
    if (hipEventCreate(&stop) != hipSuccess) {
        (void)hipEventDestroy(start);
        return;
    }
    if (hipEventRecord(stop, stream) != hipSuccess) {
        (void)hipEventDestroy(start);
        (void)hipEventDestroy(stop);
        return;
    }
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof.push_back({kernel, start, stop});
}
}  // namespace dsa

namespace {

thread_local char g_last_error[512] = "";

dsa_status_t fail(dsa_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

dsa_status_t hip_fail(hipError_t e, const char* what) {
    return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int resolve_q_block(int32_t q_block) { return q_block <= 0 ? DSA_DEFAULT_Q_BLOCK : q_block; }

bool debug_force_fallback() {
    const char* v = getenv("DSA_DEBUG_FORCE_FALLBACK");
    return v && v[0] == '1';
}

dsa_status_t check_indexer_args(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                                int64_t L, int64_t N, int32_t n_heads, int32_t head_dim,
                                int64_t q_pos0, int32_t top_k, int32_t q_block,
                                const int32_t* out_idx) {
    if (L < 0) return fail(DSA_ERR_INVALID_ARG, "L must be >= 0 (got %lld)", (long long)L);
    if (N <= 0) return fail(DSA_ERR_INVALID_ARG, "N must be > 0 (got %lld)", (long long)N);
    if (N > (int64_t)INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "N above 2^31-1 is not supported");
    if (q_pos0 < 0 || q_pos0 + L > N)
        return fail(DSA_ERR_INVALID_ARG, "need 0 <= q_pos0 and q_pos0 + L <= N (q_pos0=%lld L=%lld N=%lld)",
                    (long long)q_pos0, (long long)L, (long long)N);
    if (top_k < 1 || top_k > DSA_MAX_TOPK)
        return fail(DSA_ERR_INVALID_ARG, "top_k must be in 1..%d (got %d)", DSA_MAX_TOPK, top_k);
    if (q_block < 0) return fail(DSA_ERR_INVALID_ARG, "q_block must be >= 0 (got %d)", q_block);
    if (n_heads != DSA_INDEX_HEADS || head_dim != DSA_INDEX_DIM)
        return fail(DSA_ERR_UNSUPPORTED, "indexer needs %d heads x %d dims (got %d x %d)", DSA_INDEX_HEADS,
                    DSA_INDEX_DIM, n_heads, head_dim);
    if (L > 0 && (!q_idx || !k_idx || !w || !out_idx))
        return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (L > 0 && (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w, 4) || !aligned(out_idx, 4)))
        return fail(DSA_ERR_INVALID_ARG, "q_idx/k_idx must be 16-byte aligned, w/out_idx 4-byte aligned");
    return DSA_OK;
}

// A batch of sequences given by host arrays cu_q, cu_k [B+1] and pos0 [B]: sequence b has
// query rows cu_q[b] .. cu_q[b+1]-1 at positions pos0[b] .., and keys (kv rows)
// cu_k[b] .. cu_k[b+1]-1, indexed 0 .. N_b-1 within it.
struct Batch {
    int64_t B = 0, T = 0, NK = 0;  // sequences, query rows, key rows
    int64_t P = 0;                 // indexer rows: each sequence's run padded to a multiple of 8
    int64_t n_max = 0;             // most keys any query may see
    int64_t tiles = 0;             // 32-key tiles over the keys each sequence's queries may see
};

int64_t round8(int64_t x) { return (x + dsa::kRowsPerGroup - 1) / dsa::kRowsPerGroup * dsa::kRowsPerGroup; }
int64_t visible_keys(const int64_t* cu_q, const int64_t* pos0, int64_t b) {
    const int64_t L = cu_q[b + 1] - cu_q[b];
    return L > 0 ? pos0[b] + L : 0;
}

dsa_status_t check_batch(int64_t B, const int64_t* cu_q, const int64_t* cu_k, const int64_t* pos0, Batch* out) {
    *out = Batch{};
    if (B < 0 || B > DSA_MAX_BATCH)
        return fail(DSA_ERR_INVALID_ARG, "B must be in 0..%d (got %lld)", DSA_MAX_BATCH, (long long)B);
    if (B == 0) return DSA_OK;
    if (!cu_q || !cu_k || !pos0) return fail(DSA_ERR_INVALID_ARG, "null cu_q/cu_k/pos0 host array");
    if (cu_q[0] != 0 || cu_k[0] != 0) return fail(DSA_ERR_INVALID_ARG, "cu_q[0] and cu_k[0] must be 0");
    Batch bt;
    bt.B = B;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = cu_q[b + 1] - cu_q[b], N = cu_k[b + 1] - cu_k[b];
        if (L < 0 || N < 0)
            return fail(DSA_ERR_INVALID_ARG, "cu_q and cu_k must be non-decreasing (sequence %lld)", (long long)b);
        if (N > (int64_t)INT32_MAX)
            return fail(DSA_ERR_UNSUPPORTED, "sequence %lld: more than 2^31-1 keys", (long long)b);
        if (pos0[b] < 0 || pos0[b] + L > N)
            return fail(DSA_ERR_INVALID_ARG, "sequence %lld: need 0 <= pos0 and pos0 + L <= N (pos0=%lld L=%lld N=%lld)",
                        (long long)b, (long long)pos0[b], (long long)L, (long long)N);
        const int64_t nv = visible_keys(cu_q, pos0, b);
        bt.P += round8(L);
        bt.n_max = nv > bt.n_max ? nv : bt.n_max;
        bt.tiles += (nv + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
    }
    bt.T = cu_q[B];
    bt.NK = cu_k[B];
    *out = bt;
    return DSA_OK;
}

// Writes the batch tables, kVarlenChunk sequences per launch.
hipError_t write_batch_tables(int64_t B, const int64_t* cu_q, const int64_t* cu_k, const int64_t* pos0,
                              dsa::RowInfo* rows, dsa::SeqKeys* seqs, dsa::QueryInfo* qinfo, hipStream_t s) {
    int64_t row0 = 0, tbase = 0;
    for (int64_t c0 = 0; c0 < B; c0 += dsa::kVarlenChunk) {
        dsa::VarlenChunk c{};
        c.n = (int)((B - c0) < dsa::kVarlenChunk ? (B - c0) : dsa::kVarlenChunk);
        for (int i = 0; i < c.n; ++i) {
            const int64_t b = c0 + i;
            c.qrow0[i] = cu_q[b];
            c.L[i] = cu_q[b + 1] - cu_q[b];
            c.row0[i] = row0;
            c.pos0[i] = pos0[b];
            c.kbase[i] = cu_k[b];
            c.nvis[i] = visible_keys(cu_q, pos0, b);
            c.tbase[i] = tbase;
            row0 += round8(c.L[i]);
            tbase += (c.nvis[i] + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
        }
        hipError_t e = dsa::launch_varlen_tables(c, c0, rows, seqs, qinfo, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int resolve_q_block8(int32_t q_block) { return (int)round8(resolve_q_block(q_block)); }

dsa::IndexerLayout batch_indexer_layout(const Batch& bt, int32_t top_k, int32_t q_block) {
    const int64_t qb = resolve_q_block8(q_block);
    const int64_t rows = bt.P < qb ? bt.P : qb;
    return dsa::IndexerLayout::make(rows < 1 ? 1 : rows, bt.n_max < 1 ? 1 : bt.n_max, top_k, bt.tiles, bt.P, bt.B);
}

// Checks shared by the attention entry points (everything but positions and workspace).
dsa_status_t check_attention_shape(int32_t H, int32_t d_latent, int32_t d_rope, int32_t top_k, int64_t kv_stride,
                                   float scale) {
    if (top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (d_latent != DSA_D_LATENT || d_rope != DSA_D_ROPE)
        return fail(DSA_ERR_UNSUPPORTED, "need d_latent=%d and d_rope=%d (got %d, %d)", DSA_D_LATENT, DSA_D_ROPE,
                    d_latent, d_rope);
    if (H <= 0 || H % 16 != 0 || H > DSA_MAX_HEADS)
        return fail(DSA_ERR_UNSUPPORTED, "H must be a positive multiple of 16 up to %d (got %d)", DSA_MAX_HEADS, H);
    if (kv_stride < d_latent + d_rope || kv_stride % 8 != 0)
        return fail(DSA_ERR_INVALID_ARG, "kv_stride must be >= %d and a multiple of 8 (got %lld)",
                    d_latent + d_rope, (long long)kv_stride);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DSA_ERR_INVALID_ARG, "scale must be finite");
    return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_version(void) { return "dsa-mi355x 0.1 (gfx950)"; }

dsa_status_t dsa_profile_enable(int on) {
    g_last_error[0] = 0;
    dsa::g_prof_mask.store(on ? (1u << dsa::kProfCount) - 1u : 0u);
    return DSA_OK;
}

dsa_status_t dsa_profile_set(const char* kernels) {
    g_last_error[0] = 0;
    if (!kernels || !kernels[0]) {
        dsa::g_prof_mask.store((1u << dsa::kProfCount) - 1u);
        return DSA_OK;
    }
    uint32_t mask = 0;
    const char* p = kernels;
    while (*p) {
        const char* e = strchr(p, ',');
        const size_t n = e ? (size_t)(e - p) : strlen(p);
        int k = -1;
        for (int i = 0; i < dsa::kProfCount; ++i)
            if (strlen(dsa::kProfNames[i]) == n && strncmp(dsa::kProfNames[i], p, n) == 0) k = i;
        if (k < 0) return fail(DSA_ERR_INVALID_ARG, "unknown kernel class '%.*s'", (int)n, p);
        mask |= 1u << k;
        p = e ? e + 1 : p + n;
    }
    dsa::g_prof_mask.store(mask);
    return DSA_OK;
}

dsa_status_t dsa_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
    g_last_error[0] = 0;
    if (!kernel || !total_ms || !launches) return fail(DSA_ERR_INVALID_ARG, "null argument");
    int k = -1;
    for (int i = 0; i < dsa::kProfCount; ++i)
        if (strcmp(kernel, dsa::kProfNames[i]) == 0) k = i;
    if (k < 0) return fail(DSA_ERR_INVALID_ARG, "unknown kernel class '%s'", kernel);
    std::vector<dsa::ProfRecord> mine;
    {
        std::lock_guard<std::mutex> g(dsa::g_prof_mu);
        std::vector<dsa::ProfRecord> rest;
        for (auto& r : dsa::g_prof) (r.kernel == k ? mine : rest).push_back(r);
        dsa::g_prof.swap(rest);
    }
    double sum = 0.0;
    dsa_status_t st = DSA_OK;
    for (auto& r : mine) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess && st == DSA_OK) st = hip_fail(e, "profile event");
        sum += ms;
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    *total_ms = sum;
    *launches = (int64_t)mine.size();
    return st;
}

const char* dsa_last_error(void) { return g_last_error; }

const char* dsa_status_string(dsa_status_t s) {
    switch (s) {
        case DSA_OK: return "ok";
        case DSA_ERR_INVALID_ARG: return "invalid argument";
        case DSA_ERR_UNSUPPORTED: return "unsupported shape";
        case DSA_ERR_WORKSPACE: return "workspace too small";
        case DSA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int64_t dsa_ceiling_mfma_threads(int32_t waves_per_simd) {
    if (waves_per_simd != 1 && waves_per_simd != 2) return 0;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return (int64_t)n_cu * 256 * waves_per_simd;
}

dsa_status_t dsa_ceiling_mfma_bf16(float* out, int64_t out_len, int32_t iters, int32_t random_operands,
                                   int32_t waves_per_simd, double* flops, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (waves_per_simd != 1 && waves_per_simd != 2)
        return fail(DSA_ERR_INVALID_ARG, "waves_per_simd must be 1 or 2 (got %d)", waves_per_simd);
    if (iters < 1) return fail(DSA_ERR_INVALID_ARG, "iters must be >= 1 (got %d)", iters);
    if (!out || !flops) return fail(DSA_ERR_INVALID_ARG, "out and flops must be non-null");
    const int64_t threads = dsa_ceiling_mfma_threads(waves_per_simd);
    if (threads <= 0) return fail(DSA_ERR_HIP, "could not query the current device's compute units");
    if (out_len < threads)
        return fail(DSA_ERR_INVALID_ARG, "out needs %lld floats (got %lld)", (long long)threads, (long long)out_len);
    const int n_cu = (int)(threads / (256 * waves_per_simd));
    const hipError_t e = dsa::launch_ceiling_mfma(out, n_cu, iters, random_operands != 0, waves_per_simd,
                                                  reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "ceiling_mfma launch");
    *flops = (double)(threads / 64) * (double)iters * 8.0 * 32768.0;
    return DSA_OK;
}

int64_t dsa_ceiling_stream_sink_words(void) { return (int64_t)dsa::kCeilingCopyBlocks * 256; }

dsa_status_t dsa_ceiling_stream(const void* src, void* dst, size_t bytes, uint32_t* sink, int64_t sink_len,
                                int32_t nontemporal, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (!src) return fail(DSA_ERR_INVALID_ARG, "src must be non-null");
    if (!aligned(src, 16) || (dst && !aligned(dst, 16)) || bytes % 16 != 0)
        return fail(DSA_ERR_INVALID_ARG, "src, dst and bytes must be multiples of 16");
    if (!dst && (!sink || sink_len < dsa_ceiling_stream_sink_words()))
        return fail(DSA_ERR_INVALID_ARG, "a read-only stream needs a sink of %lld words",
                    (long long)dsa_ceiling_stream_sink_words());
    if (bytes == 0) return DSA_OK;
    const hipError_t e = dsa::launch_ceiling_copy(src, dst, bytes, sink, nontemporal != 0,
                                                  reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "ceiling_stream launch");
    return DSA_OK;
}

int dsa_sparse_prefill_gate(int64_t B, int64_t L, int64_t N, int64_t min_context) {
    if (min_context <= 0) min_context = 16384;
    return (B == 1 && L > 1 && N >= min_context) ? 1 : 0;
}

size_t dsa_indexer_topk_workspace_bytes(int64_t L, int64_t N, int32_t top_k, int32_t q_block) {
    if (L < 0 || N <= 0 || N > (int64_t)INT32_MAX || top_k < 1 || top_k > DSA_MAX_TOPK || q_block < 0)
        return 0;
    int64_t qb = resolve_q_block(q_block);
    int64_t rows = L < qb ? L : qb;
    if (rows < 1) rows = 1;
    return dsa::IndexerLayout::make(rows, N, top_k).total;
}

}  // extern "C"

namespace {
// dsa_indexer_topk, optionally over a key cache (key_cache != null): the cache's tiled copy
// and statistics replace the call's own key statistics pass.
dsa_status_t indexer_topk_impl(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L, int64_t N,
                               int32_t n_heads, int32_t head_dim, int64_t q_pos0, int32_t top_k, int32_t q_block,
                               int32_t* out_idx, void* workspace, size_t workspace_bytes, dsa_stream_t stream,
                               const void* key_cache, size_t key_cache_bytes, int64_t cached_keys) {
    g_last_error[0] = 0;
    dsa_status_t st = check_indexer_args(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, top_k, q_block, out_idx);
    if (st != DSA_OK) return st;
    if (L == 0) return DSA_OK;
    const bool cached = key_cache != nullptr;
    // Keys any query of the chunk may see.
    const int64_t last = q_pos0 + L - 1;
    const int64_t n_keys = (last < N - 1 ? last : N - 1) + 1;
    if (cached) {
        if (!aligned(key_cache, 256)) return fail(DSA_ERR_INVALID_ARG, "key cache must be 256-byte aligned");
        if (cached_keys < n_keys || cached_keys > N)
            return fail(DSA_ERR_INVALID_ARG, "the key cache must hold the %lld keys the queries see (holds %lld, N=%lld)",
                        (long long)n_keys, (long long)cached_keys, (long long)N);
        if (key_cache_bytes < dsa::key_cache_bytes(n_keys))
            return fail(DSA_ERR_INVALID_ARG, "key cache of %zu bytes is smaller than %zu", key_cache_bytes,
                        dsa::key_cache_bytes(n_keys));
    }
    const int qb = resolve_q_block(q_block);
    const int64_t rows = L < qb ? L : qb;
    const dsa::IndexerLayout lay = dsa::IndexerLayout::make(rows, N, top_k, cached ? 0 : -1);
    if (!workspace || workspace_bytes < lay.total)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", lay.total, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);

    dsa::IndexerArgs a{};
    a.k_idx = k_idx;
    a.N = N;
    a.top_k = top_k;
    a.cap = lay.cap;
    a.sample_stride = lay.sample_stride;
    a.fold_cap = lay.fold_cap;
    a.force_fallback = debug_force_fallback() ? 1 : 0;
    a.diag = reinterpret_cast<unsigned long long*>(ws + lay.off_diag);
    a.qstat = reinterpret_cast<dsa::QHeadStat*>(ws + lay.off_qstat);
    a.tau = reinterpret_cast<float*>(ws + lay.off_tau);
    a.delta = reinterpret_cast<float*>(ws + lay.off_delta);
    a.mode = reinterpret_cast<int*>(ws + lay.off_mode);
    a.count = reinterpret_cast<int*>(ws + lay.off_count);
    a.fb_ctrl = reinterpret_cast<int*>(ws + lay.off_fbctrl);
    a.fb_list = reinterpret_cast<int*>(ws + lay.off_fblist);
    a.sample = reinterpret_cast<float*>(ws + lay.off_sample);
    a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
    a.fold_s = reinterpret_cast<float*>(ws + lay.off_fold_s);
    a.fold_i = reinterpret_cast<int*>(ws + lay.off_fold_i);
    a.fold_bi = reinterpret_cast<int*>(ws + lay.off_fold_bi);
    a.fold_bs = reinterpret_cast<double*>(ws + lay.off_fold_bs);
    a.fold_bf = reinterpret_cast<float*>(ws + lay.off_fold_bf);
    a.fold_ms = reinterpret_cast<float*>(ws + lay.off_fold_ms);
    a.fold_mi = reinterpret_cast<int*>(ws + lay.off_fold_mi);
    a.n_ktiles = (n_keys + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
    if (cached) {
        // The cache's statistics cover every key appended to it (a superset of the keys
        // seen here, which only widens the band the exact re-score covers).
        char* kc = const_cast<char*>(static_cast<const char*>(key_cache));
        a.kstats = reinterpret_cast<dsa::KeyStats*>(kc);
        a.n_kstats = 1;
        a.k_tile = reinterpret_cast<uint16_t*>(kc + dsa::kKeyCacheHeader);
        a.clear_diag = 1;
    } else {
        // Key statistics and the tiled key copy, over every key any query of the chunk may see.
        a.kstats = reinterpret_cast<dsa::KeyStats*>(ws + lay.off_kstats);
        a.n_kstats = dsa::key_stats_blocks(n_keys);
        uint16_t* k_tile = reinterpret_cast<uint16_t*>(ws + lay.off_ktile);
        a.k_tile = k_tile;
        hipError_t e = dsa::launch_key_stats(k_idx, n_keys, a.kstats, k_tile, a.diag, s);
        if (e != hipSuccess) return hip_fail(e, "key statistics launch");
    }

    for (int64_t b0 = 0; b0 < L; b0 += qb) {
        const int64_t Lb = (L - b0) < qb ? (L - b0) : qb;
        a.q_idx = q_idx + (size_t)b0 * DSA_INDEX_HEADS * DSA_INDEX_DIM;
        a.w = w + (size_t)b0 * DSA_INDEX_HEADS;
        a.out = out_idx + (size_t)b0 * top_k;
        a.pos0 = q_pos0 + b0;
        a.Lb = (int)Lb;
        const int64_t last_pos = a.pos0 + Lb - 1;
        const int64_t n_last = (last_pos < N - 1 ? last_pos : N - 1) + 1;
        const bool need_sample = dsa::sample_size(n_last, top_k, lay.cap) > 0;
        a.parts = dsa::key_parts((Lb + dsa::kRowsPerGroup - 1) / dsa::kRowsPerGroup);
        hipError_t e = dsa::launch_indexer_block(a, need_sample, s, Lb <= dsa::kRowsPerGroup / 2);
        if (e != hipSuccess) return hip_fail(e, "indexer launch");
        a.clear_diag = 0;  // later blocks add to the counters
    }
    return DSA_OK;
}
}  // namespace

extern "C" {

dsa_status_t dsa_indexer_topk(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                              int64_t N, int32_t n_heads, int32_t head_dim, int64_t q_pos0, int32_t top_k,
                              int32_t q_block, int32_t* out_idx, void* workspace, size_t workspace_bytes,
                              dsa_stream_t stream) {
    return indexer_topk_impl(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, top_k, q_block, out_idx, workspace,
                             workspace_bytes, stream, nullptr, 0, 0);
}

size_t dsa_indexer_key_cache_bytes(int64_t capacity) {
    if (capacity <= 0 || capacity > (int64_t)INT32_MAX) return 0;
    return dsa::key_cache_bytes(capacity);
}

dsa_status_t dsa_indexer_key_cache_append(const uint16_t* k_idx, int64_t n_old, int64_t n_new, void* key_cache,
                                          size_t key_cache_bytes, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (n_old < 0 || n_new < n_old || n_new > (int64_t)INT32_MAX)
        return fail(DSA_ERR_INVALID_ARG, "need 0 <= n_old <= n_new <= 2^31-1 (n_old=%lld n_new=%lld)",
                    (long long)n_old, (long long)n_new);
    if (!key_cache) return fail(DSA_ERR_INVALID_ARG, "null key cache");
    if (!aligned(key_cache, 256)) return fail(DSA_ERR_INVALID_ARG, "key cache must be 256-byte aligned");
    if (key_cache_bytes < dsa::key_cache_bytes(n_new > 0 ? n_new : 1))
        return fail(DSA_ERR_INVALID_ARG, "key cache of %zu bytes cannot hold %lld keys", key_cache_bytes,
                    (long long)n_new);
    if (n_new > n_old && !k_idx) return fail(DSA_ERR_INVALID_ARG, "null key pointer");
    if (k_idx && !aligned(k_idx, 16)) return fail(DSA_ERR_INVALID_ARG, "k_idx must be 16-byte aligned");
    if (n_new == n_old && n_old > 0) return DSA_OK;
    char* kc = static_cast<char*>(key_cache);
    hipError_t e = dsa::launch_key_cache_append(k_idx, n_old, n_new, reinterpret_cast<dsa::KeyStats*>(kc),
                                                reinterpret_cast<uint16_t*>(kc + dsa::kKeyCacheHeader),
                                                reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "key cache append launch");
    return DSA_OK;
}

size_t dsa_indexer_topk_cached_workspace_bytes(int64_t L, int64_t N, int32_t top_k, int32_t q_block) {
    if (L < 0 || N <= 0 || N > (int64_t)INT32_MAX || top_k < 1 || top_k > DSA_MAX_TOPK || q_block < 0) return 0;
    int64_t qb = resolve_q_block(q_block);
    int64_t rows = L < qb ? L : qb;
    if (rows < 1) rows = 1;
    return dsa::IndexerLayout::make(rows, N, top_k, 0).total;
}

dsa_status_t dsa_indexer_topk_cached(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                                     int64_t N, int32_t n_heads, int32_t head_dim, int64_t q_pos0, int32_t top_k,
                                     int32_t q_block, int32_t* out_idx, const void* key_cache,
                                     size_t key_cache_bytes, int64_t cached_keys, void* workspace,
                                     size_t workspace_bytes, dsa_stream_t stream) {
    if (!key_cache) {
        g_last_error[0] = 0;
        return fail(DSA_ERR_INVALID_ARG, "null key cache");
    }
    return indexer_topk_impl(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, top_k, q_block, out_idx, workspace,
                             workspace_bytes, stream, key_cache, key_cache_bytes, cached_keys);
}

dsa_status_t dsa_indexer_topk_stats(const void* workspace, dsa_indexer_stats_t* out, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (!workspace || !out) return fail(DSA_ERR_INVALID_ARG, "null workspace or output");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    static_assert(dsa::kDiagSlots * sizeof(unsigned long long) <= dsa::kDiagBytes, "counter block");
    unsigned long long c[dsa::kDiagSlots];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(c, workspace, sizeof c, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the selection counters");
    out->rows = (int64_t)c[dsa::kDiagRows];
    out->rows_all_keys = (int64_t)c[dsa::kDiagRowsAll];
    out->rows_fallback = (int64_t)c[dsa::kDiagFallback];
    out->fallback_overflow = (int64_t)c[dsa::kDiagFbOverflow];
    out->fallback_incomplete = (int64_t)c[dsa::kDiagFbIncomplete];
    out->fallback_band = (int64_t)c[dsa::kDiagFbBand];
    out->rows_failed = (int64_t)c[dsa::kDiagFailed];
    out->candidates = (int64_t)c[dsa::kDiagCandSum];
    out->candidates_max = (int64_t)c[dsa::kDiagCandMax];
    out->band = (int64_t)c[dsa::kDiagBandSum];
    out->band_max = (int64_t)c[dsa::kDiagBandMax];
    out->kth_radix = (int64_t)c[dsa::kDiagRadix];
    return DSA_OK;
}

// Workspace of dsa_indexer_scores: the indexer sections it uses, with a candidate capacity
// that holds every key of a row (its 8 scoring key ranges, one extra tile each).
struct ScoreDumpLayout {
    int rows, cap;
    size_t off_diag, off_kstats, off_tau, off_delta, off_mode, off_count, off_fbctrl, off_fblist, off_qstat,
        off_cand, off_ktile, total;
    static ScoreDumpLayout make(int64_t L, int64_t N) {
        ScoreDumpLayout l{};
        auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
        l.rows = (int)round8(L);
        const int64_t n_tiles = (N + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
        const int64_t tps = (n_tiles + dsa::kCandSegs - 1) / dsa::kCandSegs;
        l.cap = (int)(dsa::kCandSegs * (tps + 1) * dsa::kKeyTileKeys);
        size_t o = 0;
        l.off_diag = o; o = al(o + dsa::kDiagBytes);
        l.off_kstats = o; o = al(o + sizeof(dsa::KeyStats) * dsa::kStatSlots);
        l.off_tau = o; o = al(o + 4 * (size_t)l.rows);
        l.off_delta = o; o = al(o + 4 * (size_t)l.rows);
        l.off_mode = o; o = al(o + 4 * (size_t)l.rows);
        l.off_count = o; o = al(o + 4 * (size_t)l.rows * dsa::kCandSegs);
        l.off_fbctrl = o; o = al(o + 4 * (size_t)dsa::kFbCtrlWords);
        l.off_fblist = o; o = al(o + 4 * (size_t)l.rows);
        l.off_qstat = o; o = al(o + sizeof(dsa::QHeadStat) * 32 * (size_t)l.rows);
        l.off_cand = o; o = al(o + 8 * (size_t)l.rows * (size_t)l.cap);
        l.off_ktile = o; o = al(o + dsa::key_tile_bytes(N));
        l.total = o;
        return l;
    }
};

size_t dsa_indexer_scores_workspace_bytes(int64_t L, int64_t N) {
    if (L < 1 || L > DSA_MAX_SCORE_ROWS || N <= 0 || N > (int64_t)INT32_MAX / 2) return 0;
    return ScoreDumpLayout::make(L, N).total;
}

dsa_status_t dsa_indexer_scores(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L, int64_t N,
                                int32_t n_heads, int32_t head_dim, int64_t q_pos0, float* scores, float* delta,
                                void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
    g_last_error[0] = 0;
    dsa_status_t st = check_indexer_args(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, 1, 0, (const int32_t*)scores);
    if (st != DSA_OK) return st;
    if (L > DSA_MAX_SCORE_ROWS)
        return fail(DSA_ERR_INVALID_ARG, "at most %d rows per call (got %lld)", DSA_MAX_SCORE_ROWS, (long long)L);
    if (N > (int64_t)INT32_MAX / 2) return fail(DSA_ERR_UNSUPPORTED, "N above 2^30-1 is not supported here");
    if (L == 0) return DSA_OK;
    if (q_pos0 < 1) return fail(DSA_ERR_INVALID_ARG, "q_pos0 must be >= 1 (a row at position 0 has one key)");
    if (delta && !aligned(delta, 4)) return fail(DSA_ERR_INVALID_ARG, "delta must be 4-byte aligned");
    const ScoreDumpLayout lay = ScoreDumpLayout::make(L, N);
    if (!workspace || workspace_bytes < lay.total)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", lay.total, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    dsa::IndexerArgs a{};
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.w = w;
    a.N = N;
    a.pos0 = q_pos0;
    a.Lb = (int)L;
    a.top_k = 1;  // no row keeps all its keys but the one at position 0 (excluded above)
    a.cap = lay.cap;
    a.sample_stride = 0;
    a.parts = 2;
    a.diag = reinterpret_cast<unsigned long long*>(ws + lay.off_diag);
    a.kstats = reinterpret_cast<dsa::KeyStats*>(ws + lay.off_kstats);
    a.qstat = reinterpret_cast<dsa::QHeadStat*>(ws + lay.off_qstat);
    a.tau = reinterpret_cast<float*>(ws + lay.off_tau);
    a.delta = reinterpret_cast<float*>(ws + lay.off_delta);
    a.mode = reinterpret_cast<int*>(ws + lay.off_mode);
    a.count = reinterpret_cast<int*>(ws + lay.off_count);
    a.fb_ctrl = reinterpret_cast<int*>(ws + lay.off_fbctrl);
    a.fb_list = reinterpret_cast<int*>(ws + lay.off_fblist);
    a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
    const int64_t last = q_pos0 + L - 1;
    const int64_t n_keys = (last < N - 1 ? last : N - 1) + 1;
    uint16_t* k_tile = reinterpret_cast<uint16_t*>(ws + lay.off_ktile);
    a.k_tile = k_tile;
    a.n_ktiles = (n_keys + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
    a.n_kstats = dsa::key_stats_blocks(n_keys);
    hipError_t e = dsa::launch_key_stats(k_idx, n_keys, a.kstats, k_tile, a.diag, s);
    if (e == hipSuccess) e = dsa::launch_score_dump(a, scores, N, delta, s);
    if (e != hipSuccess) return hip_fail(e, "score dump launch");
    return DSA_OK;
}

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on the first call on that device).
dsa_status_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(DSA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kScratchDevices - 1);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
            if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DSA_OK;
}
}  // namespace

dsa_status_t dsa_indexer_topk_noalloc(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                                      int64_t N, int32_t n_heads, int32_t head_dim, int64_t q_pos0, int32_t top_k,
                                      int32_t q_block, int32_t* out_idx, dsa_stream_t stream) {
    g_last_error[0] = 0;
    dsa_status_t st = check_indexer_args(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, top_k, q_block, out_idx);
    if (st != DSA_OK) return st;
    if (L == 0) return DSA_OK;
    const size_t need = dsa_indexer_topk_workspace_bytes(L, N, top_k, q_block);
    if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
        return fail(DSA_ERR_WORKSPACE,
                    "these sizes need %zu bytes of scratch, above the %zu-byte static scratch of the "
                    "no-allocation entry point (a smaller q_block may fit)",
                    need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != DSA_OK) return st;
    return dsa_indexer_topk(q_idx, k_idx, w, L, N, n_heads, head_dim, q_pos0, top_k, q_block, out_idx, ws,
                            (size_t)DSA_NOALLOC_SCRATCH_BYTES, stream);
}

dsa_status_t dsa_causal_mask_topk(int32_t* idx, int64_t L, int32_t top_k, int64_t q_pos0, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (L < 0) return fail(DSA_ERR_INVALID_ARG, "L must be >= 0");
    if (top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1");
    if (q_pos0 < 0) return fail(DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
    if (L == 0) return DSA_OK;
    if (!idx) return fail(DSA_ERR_INVALID_ARG, "null index pointer");
    if (!aligned(idx, 4)) return fail(DSA_ERR_INVALID_ARG, "idx must be 4-byte aligned");
    hipError_t e = dsa::launch_causal_mask(idx, L, top_k, q_pos0, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "causal mask launch");
    return DSA_OK;
}

static dsa_status_t sparse_prefill_impl(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                                       const int32_t* idx, int64_t L, int64_t N, int32_t H, int32_t d_latent,
                                       int32_t d_rope, int32_t top_k, int64_t q_pos0, float scale, int32_t q_block,
                                       uint16_t* out, float* lse, dsa_stream_t stream, bool pack) {
    g_last_error[0] = 0;
    if (L < 0) return fail(DSA_ERR_INVALID_ARG, "L must be >= 0 (got %lld)", (long long)L);
    if (N <= 0) return fail(DSA_ERR_INVALID_ARG, "N must be > 0 (got %lld)", (long long)N);
    if (N > (int64_t)INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "N above 2^31-1 is not supported");
    if (q_pos0 < 0 || q_pos0 + L > N)
        return fail(DSA_ERR_INVALID_ARG, "need 0 <= q_pos0 and q_pos0 + L <= N");
    if (top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (q_block < 0) return fail(DSA_ERR_INVALID_ARG, "q_block must be >= 0");
    if (d_latent != DSA_D_LATENT || d_rope != DSA_D_ROPE)
        return fail(DSA_ERR_UNSUPPORTED, "need d_latent=%d and d_rope=%d (got %d, %d)", DSA_D_LATENT, DSA_D_ROPE,
                    d_latent, d_rope);
    if (H <= 0 || H % 16 != 0 || H > DSA_MAX_HEADS)
        return fail(DSA_ERR_UNSUPPORTED, "H must be a positive multiple of 16 up to %d (got %d)", DSA_MAX_HEADS, H);
    if (kv_stride < d_latent + d_rope || kv_stride % 8 != 0)
        return fail(DSA_ERR_INVALID_ARG, "kv_stride must be >= %d and a multiple of 8 (got %lld)",
                    d_latent + d_rope, (long long)kv_stride);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DSA_ERR_INVALID_ARG, "scale must be finite");
    if (L == 0) return DSA_OK;
    if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(idx, 4) || !aligned(out, 8) || (lse && !aligned(lse, 4)))
        return fail(DSA_ERR_INVALID_ARG, "q/kv must be 16-byte aligned, out 8-byte, idx/lse 4-byte");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int qb = resolve_q_block(q_block);
    for (int64_t b0 = 0; b0 < L; b0 += qb) {
        dsa::AttentionArgs a{};
        const int64_t Lb = (L - b0) < qb ? (L - b0) : qb;
        a.q = q + (size_t)b0 * H * (d_latent + d_rope);
        a.kv = kv;
        a.idx = idx + (size_t)b0 * top_k;
        a.out = out + (size_t)b0 * H * d_latent;
        a.lse = lse ? lse + (size_t)b0 * H : nullptr;
        a.kv_stride = kv_stride;
        a.N = N;
        a.pos0 = q_pos0 + b0;
        a.Lb = (int)Lb;
        a.H = H;
        a.top_k = top_k;
        a.scale = scale;
        hipError_t e = pack && dsa::sparse_attention_packable(a) ? dsa::launch_sparse_attention_packed(a, s)
                                                                 : dsa::launch_sparse_attention(a, s);
        if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    }
    return DSA_OK;
}

dsa_status_t dsa_sparse_prefill(const uint16_t* q, const uint16_t* kv, int64_t kv_stride, const int32_t* idx,
                                int64_t L, int64_t N, int32_t H, int32_t d_latent, int32_t d_rope, int32_t top_k,
                                int64_t q_pos0, float scale, int32_t q_block, uint16_t* out, float* lse,
                                dsa_stream_t stream) {
    return sparse_prefill_impl(q, kv, kv_stride, idx, L, N, H, d_latent, d_rope, top_k, q_pos0, scale, q_block, out,
                               lse, stream, false);
}

dsa_status_t dsa_sparse_prefill_packed(const uint16_t* q, const uint16_t* kv, int64_t kv_stride, const int32_t* idx,
                                       int64_t L, int64_t N, int32_t H, int32_t d_latent, int32_t d_rope,
                                       int32_t top_k, int64_t q_pos0, float scale, int32_t q_block, uint16_t* out,
                                       float* lse, dsa_stream_t stream) {
    return sparse_prefill_impl(q, kv, kv_stride, idx, L, N, H, d_latent, d_rope, top_k, q_pos0, scale, q_block, out,
                               lse, stream, true);
}

static int resolve_splits(int64_t L, int32_t top_k, int32_t splits) {
    const int n_tiles = (top_k + 31) / 32;
    if (splits > 0) return splits < n_tiles ? splits : n_tiles;
    const int64_t rows = L < dsa::kDecodeRows ? L : dsa::kDecodeRows;
    int64_t s = (512 + rows - 1) / (rows > 0 ? rows : 1);  // about 512 workgroups
    if (s > n_tiles) s = n_tiles;
    if (s > dsa::kMaxSplits) s = dsa::kMaxSplits;
    if (s < 1) s = 1;
    return (int)s;
}

size_t dsa_sparse_decode_workspace_bytes(int64_t L, int32_t H, int32_t top_k, int32_t splits) {
    if (L < 0 || H <= 0 || H % 16 != 0 || H > DSA_MAX_HEADS || top_k < 1 || splits < 0 || splits > dsa::kMaxSplits)
        return 0;
    if (L == 0) return 0;
    return dsa::decode_workspace_bytes(L, H, resolve_splits(L, top_k, splits));
}

dsa_status_t dsa_sparse_decode(const uint16_t* q, const uint16_t* kv, int64_t kv_stride, const int32_t* idx,
                               int64_t L, int64_t N, int32_t H, int32_t d_latent, int32_t d_rope, int32_t top_k,
                               int64_t q_pos0, float scale, int32_t splits, uint16_t* out, float* lse,
                               void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (L < 0) return fail(DSA_ERR_INVALID_ARG, "L must be >= 0 (got %lld)", (long long)L);
    if (N <= 0) return fail(DSA_ERR_INVALID_ARG, "N must be > 0 (got %lld)", (long long)N);
    if (N > (int64_t)INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "N above 2^31-1 is not supported");
    if (q_pos0 < 0 || q_pos0 + L > N)
        return fail(DSA_ERR_INVALID_ARG, "need 0 <= q_pos0 and q_pos0 + L <= N");
    if (top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (splits < 0 || splits > dsa::kMaxSplits)
        return fail(DSA_ERR_INVALID_ARG, "splits must be in 0..%d (got %d)", dsa::kMaxSplits, splits);
    if (d_latent != DSA_D_LATENT || d_rope != DSA_D_ROPE)
        return fail(DSA_ERR_UNSUPPORTED, "need d_latent=%d and d_rope=%d (got %d, %d)", DSA_D_LATENT, DSA_D_ROPE,
                    d_latent, d_rope);
    if (H <= 0 || H % 16 != 0 || H > DSA_MAX_HEADS)
        return fail(DSA_ERR_UNSUPPORTED, "H must be a positive multiple of 16 up to %d (got %d)", DSA_MAX_HEADS, H);
    if (kv_stride < d_latent + d_rope || kv_stride % 8 != 0)
        return fail(DSA_ERR_INVALID_ARG, "kv_stride must be >= %d and a multiple of 8 (got %lld)",
                    d_latent + d_rope, (long long)kv_stride);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DSA_ERR_INVALID_ARG, "scale must be finite");
    if (L == 0) return DSA_OK;
    if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(idx, 4) || !aligned(out, 8) || (lse && !aligned(lse, 4)))
        return fail(DSA_ERR_INVALID_ARG, "q/kv must be 16-byte aligned, out 8-byte, idx/lse 4-byte");
    const int S = resolve_splits(L, top_k, splits);
    const size_t need = dsa::decode_workspace_bytes(L, H, S);
    if (!workspace || workspace_bytes < need)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t rows = L < dsa::kDecodeRows ? L : dsa::kDecodeRows;
    float* part_o = static_cast<float*>(workspace);
    float* part_ml = part_o + (size_t)rows * S * H * 512;
    for (int64_t b0 = 0; b0 < L; b0 += dsa::kDecodeRows) {
        dsa::AttentionArgs a{};
        const int64_t Lb = (L - b0) < dsa::kDecodeRows ? (L - b0) : dsa::kDecodeRows;
        a.q = q + (size_t)b0 * H * (d_latent + d_rope);
        a.kv = kv;
        a.idx = idx + (size_t)b0 * top_k;
        a.out = out + (size_t)b0 * H * d_latent;
        a.lse = lse ? lse + (size_t)b0 * H : nullptr;
        a.kv_stride = kv_stride;
        a.N = N;
        a.pos0 = q_pos0 + b0;
        a.Lb = (int)Lb;
        a.H = H;
        a.top_k = top_k;
        a.scale = scale;
        a.splits = S;
        a.part_o = part_o;
        a.part_ml = part_ml;
        hipError_t e = dsa::launch_sparse_attention_split(a, s);
        if (e != hipSuccess) return hip_fail(e, "split attention launch");
    }
    return DSA_OK;
}


size_t dsa_indexer_topk_varlen_workspace_bytes(int64_t B, const int64_t* cu_q, const int64_t* cu_k,
                                               const int64_t* pos0, int32_t top_k, int32_t q_block) {
    if (top_k < 1 || top_k > DSA_MAX_TOPK || q_block < 0) return 0;
    Batch bt;
    if (check_batch(B, cu_q, cu_k, pos0, &bt) != DSA_OK) {
        g_last_error[0] = 0;
        return 0;
    }
    if (bt.T == 0) return 0;
    return batch_indexer_layout(bt, top_k, q_block).total;
}

dsa_status_t dsa_indexer_topk_varlen(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t B,
                                     const int64_t* cu_q, const int64_t* cu_k, const int64_t* pos0,
                                     int32_t n_heads, int32_t head_dim, int32_t top_k, int32_t q_block,
                                     int32_t* out_idx, void* workspace, size_t workspace_bytes,
                                     dsa_stream_t stream) {
    g_last_error[0] = 0;
    Batch bt;
    dsa_status_t st = check_batch(B, cu_q, cu_k, pos0, &bt);
    if (st != DSA_OK) return st;
    if (top_k < 1 || top_k > DSA_MAX_TOPK)
        return fail(DSA_ERR_INVALID_ARG, "top_k must be in 1..%d (got %d)", DSA_MAX_TOPK, top_k);
    if (q_block < 0) return fail(DSA_ERR_INVALID_ARG, "q_block must be >= 0 (got %d)", q_block);
    if (n_heads != DSA_INDEX_HEADS || head_dim != DSA_INDEX_DIM)
        return fail(DSA_ERR_UNSUPPORTED, "indexer needs %d heads x %d dims (got %d x %d)", DSA_INDEX_HEADS,
                    DSA_INDEX_DIM, n_heads, head_dim);
    if (bt.T == 0) return DSA_OK;
    if (!q_idx || !k_idx || !w || !out_idx) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w, 4) || !aligned(out_idx, 4))
        return fail(DSA_ERR_INVALID_ARG, "q_idx/k_idx must be 16-byte aligned, w/out_idx 4-byte aligned");
    const dsa::IndexerLayout lay = batch_indexer_layout(bt, top_k, q_block);
    if (!workspace || workspace_bytes < lay.total)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", lay.total, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    dsa::IndexerArgs a{};
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.w = w;
    a.out = out_idx;
    a.N = bt.n_max;
    a.top_k = top_k;
    a.cap = lay.cap;
    a.sample_stride = lay.sample_stride;
    a.fold_cap = lay.fold_cap;
    a.force_fallback = debug_force_fallback() ? 1 : 0;
    a.diag = reinterpret_cast<unsigned long long*>(ws + lay.off_diag);
    a.kstats = reinterpret_cast<dsa::KeyStats*>(ws + lay.off_kstats);
    a.qstat = reinterpret_cast<dsa::QHeadStat*>(ws + lay.off_qstat);
    a.tau = reinterpret_cast<float*>(ws + lay.off_tau);
    a.delta = reinterpret_cast<float*>(ws + lay.off_delta);
    a.mode = reinterpret_cast<int*>(ws + lay.off_mode);
    a.count = reinterpret_cast<int*>(ws + lay.off_count);
    a.fb_ctrl = reinterpret_cast<int*>(ws + lay.off_fbctrl);
    a.fb_list = reinterpret_cast<int*>(ws + lay.off_fblist);
    a.sample = reinterpret_cast<float*>(ws + lay.off_sample);
    a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
    a.fold_s = reinterpret_cast<float*>(ws + lay.off_fold_s);
    a.fold_i = reinterpret_cast<int*>(ws + lay.off_fold_i);
    a.fold_bi = reinterpret_cast<int*>(ws + lay.off_fold_bi);
    a.fold_bs = reinterpret_cast<double*>(ws + lay.off_fold_bs);
    a.fold_bf = reinterpret_cast<float*>(ws + lay.off_fold_bf);
    a.fold_ms = reinterpret_cast<float*>(ws + lay.off_fold_ms);
    a.fold_mi = reinterpret_cast<int*>(ws + lay.off_fold_mi);
    dsa::RowInfo* rows = reinterpret_cast<dsa::RowInfo*>(ws + lay.off_rowinfo);
    dsa::SeqKeys* seqs = reinterpret_cast<dsa::SeqKeys*>(ws + lay.off_seqkeys);
    uint16_t* k_tile = reinterpret_cast<uint16_t*>(ws + lay.off_ktile);
    a.k_tile = k_tile;
    a.n_ktiles = bt.tiles;

    // Tables, then the key statistics (over the whole batch) and every sequence's tiled keys.
    hipError_t e = write_batch_tables(B, cu_q, cu_k, pos0, rows, seqs, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "batch table launch");
    a.n_kstats = dsa::key_stats_blocks(bt.tiles * dsa::kKeyTileKeys);
    e = dsa::launch_key_stats_batch(k_idx, seqs, (int)B, bt.tiles, a.kstats, k_tile, a.diag, s);
    if (e != hipSuccess) return hip_fail(e, "key statistics launch");

    // Blocks of the padded row space; sequence sq is the first one a block may hold.
    const int64_t qb = resolve_q_block8(q_block);
    int64_t sq = 0, sq_row0 = 0;
    for (int64_t b0 = 0; b0 < bt.P; b0 += qb) {
        const int64_t Lb = (bt.P - b0) < qb ? (bt.P - b0) : qb;
        while (sq < B && sq_row0 + round8(cu_q[sq + 1] - cu_q[sq]) <= b0) {
            sq_row0 += round8(cu_q[sq + 1] - cu_q[sq]);
            ++sq;
        }
        // The most keys a row of this block sees: a sample is needed if its group needs one.
        // Also count the block's query rows: mostly padding means groups of few rows.
        int64_t n_last = 0, live = 0;
        for (int64_t b = sq, r0 = sq_row0; b < B && r0 < b0 + Lb; r0 += round8(cu_q[b + 1] - cu_q[b]), ++b) {
            const int64_t L = cu_q[b + 1] - cu_q[b];
            const int64_t i_first = b0 > r0 ? b0 - r0 : 0;
            const int64_t i_last = (b0 + Lb - r0 < L ? b0 + Lb - r0 : L) - 1;
            if (i_last >= 0 && pos0[b] + i_last + 1 > n_last) n_last = pos0[b] + i_last + 1;
            if (i_last >= i_first) live += i_last - i_first + 1;
        }
        a.rows = rows + b0;
        a.Lb = (int)Lb;
        a.parts = dsa::key_parts((int)(Lb / dsa::kRowsPerGroup));
        e = dsa::launch_indexer_block(a, dsa::sample_size(n_last, top_k, lay.cap) > 0, s, 2 * live <= Lb);
        if (e != hipSuccess) return hip_fail(e, "indexer launch");
    }
    return DSA_OK;
}

static size_t varlen_attention_bytes(const Batch& bt, int32_t H, int S, size_t* qinfo_bytes) {
    const size_t qi = ((size_t)bt.T * sizeof(dsa::QueryInfo) + 255) & ~(size_t)255;
    if (qinfo_bytes) *qinfo_bytes = qi;
    return qi + (S > 1 ? dsa::decode_workspace_bytes(bt.T, H, S) : 0);
}

size_t dsa_sparse_prefill_varlen_workspace_bytes(int64_t B, const int64_t* cu_q, const int64_t* cu_k,
                                                 const int64_t* pos0, int32_t H, int32_t top_k, int32_t splits) {
    if (H <= 0 || H % 16 != 0 || H > DSA_MAX_HEADS || top_k < 1 || splits < 0 || splits > dsa::kMaxSplits) return 0;
    Batch bt;
    if (check_batch(B, cu_q, cu_k, pos0, &bt) != DSA_OK) {
        g_last_error[0] = 0;
        return 0;
    }
    if (bt.T == 0) return 0;
    return varlen_attention_bytes(bt, H, resolve_splits(bt.T, top_k, splits), nullptr);
}

dsa_status_t dsa_sparse_prefill_varlen(const uint16_t* q, const uint16_t* kv, int64_t kv_stride, const int32_t* idx,
                                       int64_t B, const int64_t* cu_q, const int64_t* cu_k, const int64_t* pos0,
                                       int32_t H, int32_t d_latent, int32_t d_rope, int32_t top_k, float scale,
                                       int32_t splits, uint16_t* out, float* lse, void* workspace,
                                       size_t workspace_bytes, dsa_stream_t stream) {
    g_last_error[0] = 0;
    Batch bt;
    dsa_status_t st = check_batch(B, cu_q, cu_k, pos0, &bt);
    if (st != DSA_OK) return st;
    st = check_attention_shape(H, d_latent, d_rope, top_k, kv_stride, scale);
    if (st != DSA_OK) return st;
    if (splits < 0 || splits > dsa::kMaxSplits)
        return fail(DSA_ERR_INVALID_ARG, "splits must be in 0..%d (got %d)", dsa::kMaxSplits, splits);
    if (bt.T == 0) return DSA_OK;
    if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(idx, 4) || !aligned(out, 8) || (lse && !aligned(lse, 4)))
        return fail(DSA_ERR_INVALID_ARG, "q/kv must be 16-byte aligned, out 8-byte, idx/lse 4-byte");
    const int S = resolve_splits(bt.T, top_k, splits);
    size_t qi_bytes = 0;
    const size_t need = varlen_attention_bytes(bt, H, S, &qi_bytes);
    if (!workspace || workspace_bytes < need)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    dsa::QueryInfo* qinfo = static_cast<dsa::QueryInfo*>(workspace);
    hipError_t e = write_batch_tables(B, cu_q, cu_k, pos0, nullptr, nullptr, qinfo, s);
    if (e != hipSuccess) return hip_fail(e, "batch table launch");
    float* part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + qi_bytes);
    const int64_t rows = bt.T < dsa::kDecodeRows ? bt.T : dsa::kDecodeRows;
    float* part_ml = part_o + (size_t)rows * S * H * 512;
    const int64_t qb = S > 1 ? dsa::kDecodeRows : DSA_DEFAULT_Q_BLOCK;
    for (int64_t b0 = 0; b0 < bt.T; b0 += qb) {
        dsa::AttentionArgs a{};
        const int64_t Lb = (bt.T - b0) < qb ? (bt.T - b0) : qb;
        a.q = q + (size_t)b0 * H * (d_latent + d_rope);
        a.kv = kv;
        a.idx = idx + (size_t)b0 * top_k;
        a.out = out + (size_t)b0 * H * d_latent;
        a.lse = lse ? lse + (size_t)b0 * H : nullptr;
        a.kv_stride = kv_stride;
        a.N = bt.n_max;
        a.qinfo = qinfo + b0;
        a.Lb = (int)Lb;
        a.H = H;
        a.top_k = top_k;
        a.scale = scale;
        a.splits = S;
        a.part_o = part_o;
        a.part_ml = part_ml;
        e = S > 1 ? dsa::launch_sparse_attention_split(a, s) : dsa::launch_sparse_attention(a, s);
        if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    }
    return DSA_OK;
}


// Vector retrieval: the indexer's workspace for min(M, q_block) rows (rounded up to a row
// group), plus the row table and each row's two-head form and weights.
struct RetrievalExtra {
    size_t off_qemb, off_wemb, off_runs, off_ids, off_segcnt, total;
    int64_t rows_pad;
};

// Run slots (rows x segments x capacity) and segment counters of the filter's per-lane lists
// for a block of Lb queries.
static size_t retrieval_run_slots(int64_t Lb, int64_t N, int32_t top_k, int cap, size_t* n_counters) {
    const int64_t n_tiles = (N + dsa::kKeyTileKeys - 1) / dsa::kKeyTileKeys;
    const int parts = dsa::retrieval_parts(dsa::retrieval_groups((int)Lb), n_tiles);
    const bool keep_all = dsa::sample_size(N, top_k, cap) == 0;
    const int seg_cap = dsa::retrieval_seg_cap(parts, n_tiles, top_k, keep_all);
    *n_counters = (size_t)Lb * parts * 8;
    return (size_t)Lb * parts * 8 * (size_t)seg_cap;
}

static dsa::IndexerLayout retrieval_layout(int64_t M, int64_t N, int32_t top_k, int32_t q_block, RetrievalExtra* x) {
    const int64_t qb = resolve_q_block(q_block);
    int64_t rows = M < qb ? M : qb;
    if (rows < 1) rows = 1;
    const int64_t rp = round8(rows);
    const dsa::IndexerLayout lay = dsa::IndexerLayout::make(rows, N, top_k, 0, rp, 0);  // no tiled copy
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    // the full block and the last (shorter) block may split the corpus differently
    size_t c_full, c_tail = 0;
    size_t slots = retrieval_run_slots(rows, N, top_k, lay.cap, &c_full);
    if (M > qb && M % qb) {
        const size_t t = retrieval_run_slots(M % qb, N, top_k, lay.cap, &c_tail);
        slots = t > slots ? t : slots;
    }
    const size_t counters = c_full > c_tail ? c_full : c_tail;
    x->off_qemb = lay.total;
    x->off_wemb = al(x->off_qemb + (size_t)rp * DSA_INDEX_HEADS * DSA_INDEX_DIM * 2);
    x->off_runs = al(x->off_wemb + (size_t)rp * DSA_INDEX_HEADS * 4);
    x->off_ids = al(x->off_runs + slots * 16);
    x->off_segcnt = al(x->off_ids + slots * 4);
    x->total = al(x->off_segcnt + counters * 4);
    x->rows_pad = rp;
    return lay;
}

size_t dsa_retrieval_topk_workspace_bytes(int64_t M, int64_t N, int32_t top_k, int32_t q_block) {
    if (M <= 0 || N <= 0 || N > (int64_t)INT32_MAX || top_k < 1 || top_k > DSA_MAX_TOPK || q_block < 0) return 0;
    RetrievalExtra x;
    retrieval_layout(M, N, top_k, q_block, &x);
    return x.total;
}

dsa_status_t dsa_retrieval_topk(const uint16_t* q, const uint16_t* x, int64_t M, int64_t N, int32_t dim,
                                int32_t top_k, int32_t q_block, int32_t* out_idx, void* workspace,
                                size_t workspace_bytes, dsa_stream_t stream) {
    g_last_error[0] = 0;
    if (M < 0) return fail(DSA_ERR_INVALID_ARG, "M must be >= 0 (got %lld)", (long long)M);
    if (N <= 0) return fail(DSA_ERR_INVALID_ARG, "N must be > 0 (got %lld)", (long long)N);
    if (N > (int64_t)INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "N above 2^31-1 is not supported");
    if (top_k < 1 || top_k > DSA_MAX_TOPK)
        return fail(DSA_ERR_INVALID_ARG, "top_k must be in 1..%d (got %d)", DSA_MAX_TOPK, top_k);
    if (q_block < 0) return fail(DSA_ERR_INVALID_ARG, "q_block must be >= 0 (got %d)", q_block);
    if (dim != DSA_INDEX_DIM) return fail(DSA_ERR_UNSUPPORTED, "dim must be %d (got %d)", DSA_INDEX_DIM, dim);
    if (M == 0) return DSA_OK;
    if (!q || !x || !out_idx) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q, 16) || !aligned(x, 16) || !aligned(out_idx, 4))
        return fail(DSA_ERR_INVALID_ARG, "q/x must be 16-byte aligned, out_idx 4-byte aligned");
    RetrievalExtra rx;
    const dsa::IndexerLayout lay = retrieval_layout(M, N, top_k, q_block, &rx);
    if (!workspace || workspace_bytes < rx.total)
        return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", rx.total, workspace_bytes,
                    workspace ? "" : ", null");
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    dsa::IndexerArgs a{};
    a.q_idx = reinterpret_cast<const uint16_t*>(ws + rx.off_qemb);
    a.w = reinterpret_cast<const float*>(ws + rx.off_wemb);
    a.k_idx = x;
    a.N = N;
    a.top_k = top_k;
    a.cap = lay.cap;
    a.sample_stride = lay.sample_stride;
    a.fold_cap = lay.fold_cap;
    a.force_fallback = debug_force_fallback() ? 1 : 0;
    a.parts = 4;  // one appended candidate list per row
    a.diag = reinterpret_cast<unsigned long long*>(ws + lay.off_diag);
    a.kstats = reinterpret_cast<dsa::KeyStats*>(ws + lay.off_kstats);
    a.qstat = reinterpret_cast<dsa::QHeadStat*>(ws + lay.off_qstat);
    a.tau = reinterpret_cast<float*>(ws + lay.off_tau);
    a.delta = reinterpret_cast<float*>(ws + lay.off_delta);
    a.mode = reinterpret_cast<int*>(ws + lay.off_mode);
    a.count = reinterpret_cast<int*>(ws + lay.off_count);
    a.fb_ctrl = reinterpret_cast<int*>(ws + lay.off_fbctrl);
    a.fb_list = reinterpret_cast<int*>(ws + lay.off_fblist);
    a.sample = reinterpret_cast<float*>(ws + lay.off_sample);
    a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
    a.fold_s = reinterpret_cast<float*>(ws + lay.off_fold_s);
    a.fold_i = reinterpret_cast<int*>(ws + lay.off_fold_i);
    a.fold_bi = reinterpret_cast<int*>(ws + lay.off_fold_bi);
    a.fold_bs = reinterpret_cast<double*>(ws + lay.off_fold_bs);
    a.fold_bf = reinterpret_cast<float*>(ws + lay.off_fold_bf);
    a.fold_ms = reinterpret_cast<float*>(ws + lay.off_fold_ms);
    a.fold_mi = reinterpret_cast<int*>(ws + lay.off_fold_mi);
    a.rows = reinterpret_cast<const dsa::RowInfo*>(ws + lay.off_rowinfo);
    a.n_kstats = dsa::key_stats_blocks(N);
    hipError_t e = dsa::launch_key_stats(x, N, a.kstats, nullptr, a.diag, s);  // statistics only
    if (e != hipSuccess) return hip_fail(e, "key statistics launch");

    dsa::RetrievalArgs r{};
    r.x = x;
    r.N = N;
    r.sample = a.sample;
    r.sample_stride = lay.sample_stride;
    r.sample_n = dsa::sample_size(N, top_k, lay.cap);
    r.tau = a.tau;
    r.mode = a.mode;
    r.cand = a.cand;
    r.count = a.count;
    r.cap = lay.cap;
    r.seg_runs = reinterpret_cast<float4*>(ws + rx.off_runs);
    r.seg_ids = reinterpret_cast<uint32_t*>(ws + rx.off_ids);
    r.seg_count = reinterpret_cast<int*>(ws + rx.off_segcnt);
    const int64_t qb = resolve_q_block(q_block);
    for (int64_t b0 = 0; b0 < M; b0 += qb) {
        const int64_t Lb = (M - b0) < qb ? (M - b0) : qb;
        a.out = out_idx + (size_t)b0 * top_k;
        a.Lb = (int)Lb;
        r.q = q + (size_t)b0 * DSA_INDEX_DIM;
        r.Lb = (int)Lb;
        e = dsa::launch_retrieval_block(r, a, r.sample_n > 0, (int)rx.rows_pad, s);
        if (e != hipSuccess) return hip_fail(e, "retrieval launch");
    }
    return DSA_OK;
}

}  // extern "C"
