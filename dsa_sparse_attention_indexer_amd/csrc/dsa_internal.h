// dsa_internal.h -- host/device interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

enum : int { kModeNormal = 0, kModeAll = 1, kModePad = 2 };

struct KeyStats {
    unsigned knorm_bits;  // max ||k_s||_2 (fp32 bits, rounded up)
    unsigned kinf_bits;   // max |k_s,i|
    int kexp_min;         // min exponent of the lowest set bit over nonzero k elements
    int pad;
};

// Every key-statistics block writes its partial result to its own slot (no atomics, no
// initialisation); the consumer reduces the slots.  One block per four 32-key tiles, at
// most kStatSlots blocks.
constexpr int kStatSlots = 1024;
__host__ __device__ inline int key_stats_blocks(int64_t n_keys) {
    const int64_t tiles = (n_keys + 31) / 32;
    int64_t b = (tiles + 3) / 4;
    if (b > kStatSlots) b = kStatSlots;
    if (b < 1) b = 1;
    return (int)b;
}

// Candidate capacity per query row: expected candidates are 2.5 * top_k.  A multiple of
// 2,048, so select (cap / 32 threads) runs whole waves.
__host__ __device__ inline int cand_capacity(int top_k) {
    int c = 4 * top_k;
    if (c < 8192) c = 8192;
    return (c + 2047) & ~2047;
}

constexpr int kRowsPerGroup = 8;  // indexer query rows scored together (one sample each)

// Sample keys expected above the threshold: the threshold is the sample's rank-r score
// with r about kSampleRank, estimating the 2.5 k-th score of the row.  The true k-th score
// sits near sample rank kSampleRank / 2.5 (~51, std ~7), so the threshold falls below it
// with overwhelming probability.  The candidate count (2.5 k, relative std ~1/11) fills a
// list of cap = 1.56 x its mean (about 6 std); smaller samples (r = 64, 96) were measured
// to bring the largest rows too close to that capacity.
constexpr int kSampleRank = 128;

// Keys scored in the threshold sample of a row group whose first row sees n_t keys.
// Groups whose first row sees at most cap - kRowsPerGroup keys are not sampled: every row
// of such a group sees at most cap keys, so all its causal keys fit the candidate buffer.
__host__ __device__ inline int sample_size(int64_t n_t, int top_k, int cap) {
    if (n_t <= cap - kRowsPerGroup) return 0;
    int64_t s = (int64_t)((n_t * kSampleRank + (int64_t)(2.5 * top_k) - 1) / (int64_t)(2.5 * top_k));
    if (s < 1024) s = 1024;
    if (s > 16384) s = 16384;
    if (s > n_t) s = n_t;
    return (int)s;
}

// Rank (1 = largest) of the sample score used as the row's threshold estimate.
__host__ __device__ inline int sample_rank(int64_t n_t, int s, int top_k) {
    double r = 2.5 * (double)top_k * (double)s / (double)n_t;
    int ri = (int)r;
    if ((double)ri < r) ++ri;
    if (ri < 1) ri = 1;
    if (ri > s) ri = s;
    return ri;
}

// Key parts per row group: the two halves while the groups fill 256 compute units (128 or
// more groups), else a power of two giving about 256 workgroups (at most 256 parts).
inline int key_parts(int groups) {
    if (groups >= 128) return 2;
    int p = 4;
    while (p < 256 && p * groups < 256) p <<= 1;
    return p;
}

constexpr int kFallbackSlots = 32;
constexpr int kFoldKeys = 4096;
// The first kFoldSplitRows rows of a block that fall back are each folded as up to kFoldParts
// key ranges by different fold workgroups; the last range to finish merges the ranges' exact
// top-k lists.  Later rows are folded whole, one per workgroup.
constexpr int kFoldSplitRows = 16;
constexpr int kFoldParts = 16;
// Fold control words: [0] rows handed over, [1] next work item, [4 + j] ranges finished of
// split row j, [4 + kFoldSplitRows + j] flags of split row j's ranges (1: one failed, 2: one
// needed the radix select).
constexpr int kFbCtrlWords = 4 + 2 * kFoldSplitRows;
constexpr int kCandSegs = 8;  // count words per row; key ranges per row group: 2 key halves x 4 scoring waves

// Indexer keys are re-laid out once per call as 32-key tiles of 8 KB in the order the
// scoring MFMA's B operand is loaded: [tile][k-step 0..7][lane 0..63][8 bf16], where lane
// l = 32*hf + c holds key 32*tile + c, dims 64*hf + 8*kstep .. +7.  Every scoring load
// instruction then reads 1 KB of consecutive bytes.
constexpr int kKeyTileKeys = 32;
constexpr size_t kKeyTileBytes = (size_t)kKeyTileKeys * 128 * 2;
__host__ __device__ inline size_t key_tile_bytes(int64_t n_keys) {
    return (size_t)((n_keys + kKeyTileKeys - 1) / kKeyTileKeys) * kKeyTileBytes;
}

// Per (query row, head) statistics of q_idx that the exact re-score needs: an upper bound
// of sum_i |q_h,i| and the lowest set-bit exponent over the nonzero q_h,i (INT_MAX: none).
struct QHeadStat {
    double l1;
    int e;
    int pad;
};

// Selection counters of one indexer call, the first bytes of its workspace.  The call's
// first kernel (key statistics) clears them; select and the fold add to them with device
// atomics; dsa_indexer_topk_stats copies them out.
enum DiagSlot : int {
    kDiagRows = 0,      // rows finished by the candidate path
    kDiagRowsAll,       // rows with at most top_k causal keys (no selection)
    kDiagFallback,      // rows handed to the blocked fold ...
    kDiagFbOverflow,    // ... because the row's candidate list overflowed (or the fold was forced)
    kDiagFbIncomplete,  // ... because the candidates were not provably a superset of the top-k
    kDiagFbBand,        // ... because the band outgrew select's buffer
    kDiagFailed,        // rows no path could finish (emitted as -1; never expected)
    kDiagCandSum,       // candidates, summed over the candidate-path rows
    kDiagCandMax,       // most candidates of one such row
    kDiagBandSum,       // keys re-scored in fp64, summed over those rows
    kDiagBandMax,       // most re-scored keys of one row
    kDiagRadix,         // fold rows whose k-th searches needed the radix select
    kDiagSlots = 16
};
constexpr size_t kDiagBytes = 256;

struct IndexerLayout {
    int rows, cap, sample_stride, fold_cap;
    size_t off_diag, off_kstats, off_tau, off_delta, off_mode, off_count, off_fbctrl, off_fblist;
    size_t off_sample, off_cand, off_ktile, off_qstat;
    size_t off_fold_s, off_fold_i, off_fold_bi, off_fold_bs, off_fold_bf, off_fold_ms, off_fold_mi;
    size_t total;

    // rows: block rows; N: the most keys a query may see.  A batch of sequences also needs
    // the tiled copies of all of them (key_tiles), its row table (row_infos) and its
    // per-sequence key table (n_seqs).
    size_t off_rowinfo, off_seqkeys;
    static IndexerLayout make(int64_t rows, int64_t N, int top_k, int64_t key_tiles = -1, int64_t row_infos = 0,
                              int64_t n_seqs = 0) {
        IndexerLayout l{};
        auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
        l.rows = (int)((rows + kRowsPerGroup - 1) & ~(int64_t)(kRowsPerGroup - 1));
        l.cap = cand_capacity(top_k);
        l.sample_stride = (sample_size(N, top_k, l.cap) + 3) & ~3;  // rows 16-byte aligned
        l.fold_cap = top_k + 2 * kFoldKeys;  // the fold's list: its top-k plus up to two blocks' admissions
        size_t o = 0;
        l.off_diag = o; o = al(o + kDiagBytes);
        l.off_kstats = o; o = al(o + sizeof(KeyStats) * kStatSlots);
        l.off_tau = o; o = al(o + 4 * (size_t)l.rows);
        l.off_delta = o; o = al(o + 4 * (size_t)l.rows);
        l.off_mode = o; o = al(o + 4 * (size_t)l.rows);
        l.off_count = o; o = al(o + 4 * (size_t)l.rows * kCandSegs);
        l.off_fbctrl = o; o = al(o + 4 * (size_t)kFbCtrlWords);
        l.off_fblist = o; o = al(o + 4 * (size_t)l.rows);
        l.off_sample = o; o = al(o + 4 * (size_t)l.rows * (size_t)l.sample_stride);
        l.off_cand = o; o = al(o + 8 * (size_t)l.rows * (size_t)l.cap);
        l.off_ktile = o; o = al(o + (key_tiles < 0 ? key_tile_bytes(N) : (size_t)key_tiles * kKeyTileBytes));
        l.off_qstat = o; o = al(o + sizeof(QHeadStat) * 32 * (size_t)l.rows);
        l.off_fold_s = o; o = al(o + 4 * (size_t)kFallbackSlots * 2 * l.fold_cap);
        l.off_fold_i = o; o = al(o + 4 * (size_t)kFallbackSlots * 2 * l.fold_cap);
        l.off_fold_bi = o; o = al(o + 4 * (size_t)kFallbackSlots * l.fold_cap);
        l.off_fold_bs = o; o = al(o + 8 * (size_t)kFallbackSlots * l.fold_cap);
        l.off_fold_bf = o; o = al(o + 4 * (size_t)kFallbackSlots * l.fold_cap);
        l.off_fold_ms = o; o = al(o + 4 * (size_t)kFoldSplitRows * kFoldParts * (size_t)top_k);
        l.off_fold_mi = o; o = al(o + 4 * (size_t)kFoldSplitRows * kFoldParts * (size_t)top_k);
        l.off_rowinfo = o; o = al(o + 40 * (size_t)row_infos);
        l.off_seqkeys = o; o = al(o + 32 * (size_t)n_seqs);
        l.total = o;
        return l;
    }
};

// A batched block packs the query rows of one or more sequences, each sequence's run padded
// to a multiple of the row group, so row groups never straddle sequences.  Per block row:
struct RowInfo {
    int64_t qrow;   // row of q_idx / w / out (of the whole batch); -1 for a padding row
    int64_t pos;    // the query's position in its sequence
    int64_t kbase;  // the sequence's first key in k_idx
    int64_t tbase;  // the sequence's first 32-key tile in the tiled key copy
    int64_t nkeys;  // keys of the sequence that any of its queries may see (last position + 1)
};

static_assert(sizeof(RowInfo) == 40, "row table entry");

// A sequence's keys in a batch: where they start in k_idx, how many any of its queries may
// see, and the range [tbase, tend) of its 32-key tiles in the tiled copy.
struct SeqKeys {
    int64_t kbase, nkeys, tbase, tend;
};
static_assert(sizeof(SeqKeys) == 32, "sequence table entry");

// Per query row of a batch, for the attention: the sequence's first kv row and the query's position.
struct QueryInfo {
    int64_t kbase, pos;
};

// Up to kVarlenChunk sequences of a batch, passed by value to the kernel that writes the
// tables above (so the tables need no host-to-device copy).
constexpr int kVarlenChunk = 32;
struct VarlenChunk {
    int n;
    int64_t qrow0[kVarlenChunk];  // first query row of the sequence in the batch
    int64_t L[kVarlenChunk];      // its query rows
    int64_t row0[kVarlenChunk];   // its first row in the padded row space of the indexer
    int64_t pos0[kVarlenChunk];   // position of its first query
    int64_t kbase[kVarlenChunk];  // its first key (kv row)
    int64_t nvis[kVarlenChunk];   // keys its queries may see: pos0 + L (0 if L == 0)
    int64_t tbase[kVarlenChunk];  // its first tile in the tiled key copy
};
// Writes, for sequences seq0 .. seq0 + c.n - 1: their rows of the padded row table (rows,
// padding rows qrow = -1), their SeqKeys entries (seqs) and their query rows of the
// attention table (qinfo); null outputs are skipped.
hipError_t launch_varlen_tables(const VarlenChunk& c, int64_t seq0, RowInfo* rows, SeqKeys* seqs,
                                QueryInfo* qinfo, hipStream_t s);

struct IndexerArgs {
    const uint16_t* q_idx;  // rows of this block: [Lb][32][128] (batched: the whole batch's rows)
    const uint16_t* k_idx;  // [N][128]
    const uint16_t* k_tile; // keys 0..n_ktiles*32-1 in scoring tile order (pad keys zero)
    int64_t n_ktiles;
    const float* w;         // [Lb][32]
    int32_t* out;           // [Lb][top_k]
    int64_t N;
    int64_t pos0;           // position of the block's first query
    const RowInfo* rows;    // batched: [Lb] per block row (null: one sequence, row r at pos0 + r)
    int Lb;
    int top_k;
    int cap;
    int sample_stride;
    int fold_cap;
    int force_fallback;     // debug: send every scored row through the fallback fold
    int clear_diag;         // row_prep clears diag (the call's first block, when key_stats did not run)
    // Key parts per row group.  2 (the key halves, XCD-mapped): each half's 4 scoring waves
    // append to the row's list through the workgroup's LDS counter, half 0 from the list's
    // bottom and half 1 from its top.  More parts (few row groups): every wave of every part
    // appends to the row's list from its bottom through a global counter (count[r][0]).
    // Either way the selection puts its output in key order through a bitmap.
    int parts;
    unsigned long long* diag;  // [kDiagSlots] selection counters of the call
    KeyStats* kstats;       // [n_kstats] partial key statistics, one per key-statistics block
    QHeadStat* qstat;       // [Lb][32] per-head q statistics (row prep)
    int n_kstats;
    float* tau;
    float* delta;
    int* mode;
    int* count;             // [Lb][kCandSegs]: list entries of key half 0 ([0]) and half 1 ([1]);
                            // more key parts: [0] counts the row's appended list
    int* fb_ctrl;           // [0] flagged rows, [1] next row to take
    int* fb_list;
    float* sample;
    uint32_t* cand;         // [Lb][2][cap] words: a row's candidate scores (fp32 bits) in its
                            // first cap words, their keys in the next cap; key half 0 fills
                            // slots from 0 up, half 1 from cap - 1 down
    float* fold_s;          // [slots][2][fold_cap]
    int* fold_i;            // [slots][2][fold_cap]
    int* fold_bi;           // [slots][fold_cap]
    double* fold_bs;        // [slots][fold_cap]
    float* fold_bf;         // [slots][fold_cap]
    float* fold_ms;         // [kFoldSplitRows][kFoldParts][top_k]: split rows' range top-k scores
    int* fold_mi;           // ... and keys
};

// Optional per-launch event timing (dsa_profile_enable).  A ProfScope records an
// event before its launch and another after it on the same stream.
enum ProfKernel : int {
    kProfKeyStats = 0, kProfScoreSample, kProfRowPrep, kProfScoreFilter, kProfSelect, kProfFold,
    kProfAttention, kProfCausalMask, kProfAttnSplit, kProfAttnMerge, kProfRetrievalPrep,
    kProfRetrievalSample, kProfRetrievalFilter, kProfRetrievalGather, kProfCeilingMfma, kProfCeilingCopy,
    kProfCount
};
struct ProfScope {
    ProfScope(hipStream_t s, int kernel);
    ~ProfScope();
    hipStream_t stream;
    int kernel;
    hipEvent_t start;
    bool on;
};

// Kernel launchers (indexer.hip).  Each returns the launch status.
// k_tile may be null: statistics only.
// It also clears the call's selection counters (diag).
hipError_t launch_key_stats(const uint16_t* k_idx, int64_t n_keys, KeyStats* ks, uint16_t* k_tile,
                            unsigned long long* diag, hipStream_t s);
// The same over a batch: seqs[0 .. n_seqs) (device), n_tiles tiles in all.
hipError_t launch_key_stats_batch(const uint16_t* k_idx, const SeqKeys* seqs, int n_seqs, int64_t n_tiles,
                                  KeyStats* ks, uint16_t* k_tile, unsigned long long* diag, hipStream_t s);
// Appends keys [n_old, n_new) of k_idx to a key cache: their tiled copy (the tile holding key
// n_old is redone whole) and the running statistics in *stats (reset first when n_old == 0).
hipError_t launch_key_cache_append(const uint16_t* k_idx, int64_t n_old, int64_t n_new, KeyStats* stats,
                                   uint16_t* k_tile, hipStream_t s);

// An append-only key cache: a 256-byte header (the KeyStats of every appended key) and the
// tiled copy of capacity keys.
constexpr size_t kKeyCacheHeader = 256;
inline size_t key_cache_bytes(int64_t capacity) { return kKeyCacheHeader + key_tile_bytes(capacity); }
// sparse_rows: most row groups hold few query rows (decode, short chunks, batches of single
// queries): the scoring skips the MFMAs of row pairs without a live row.
hipError_t launch_indexer_block(const IndexerArgs& a, bool need_sample, hipStream_t s, bool sparse_rows = false);
// The stages of launch_indexer_block that follow a scoring kernel: row_prep (error bound,
// threshold from the sample), then select and the fold.
hipError_t launch_row_prep(const IndexerArgs& a, hipStream_t s);
hipError_t launch_select_fold(const IndexerArgs& a, hipStream_t s);

// Inner-product top-k over a corpus: the scoring kernels' arguments.  The selection runs
// on an IndexerArgs whose rows are the two-head form (q, -q), weights (1, -1), of each query.
struct RetrievalArgs {
    const uint16_t* q;       // [Lb][128] this block's query rows
    const uint16_t* x;       // [N][128] corpus (the sample reads it row-major)
    int64_t N;
    int Lb, n_groups, parts;
    float* sample;           // [Lb][sample_stride]
    int sample_stride, sample_n;
    const float* tau;        // [Lb] filter threshold (row_prep)
    const int* mode;         // [Lb]
    uint32_t* cand;          // [Lb][2][cap] appended candidate lists (scores, then keys)
    int* count;              // [Lb][kCandSegs]: entry 0 counts a row's list
    int cap;
    // The filter's per-lane lists: segment (part, wave, lane half) of each row holds up to
    // seg_cap runs of 4 consecutive corpus rows (their 4 fp32 scores and the run's id =
    // first row / 4) of which at least one passed the threshold; gathered into cand afterwards.
    float4* seg_runs;        // [Lb][n_segs][seg_cap]
    uint32_t* seg_ids;       // [Lb][n_segs][seg_cap]
    int* seg_count;          // [Lb][n_segs]
    int seg_cap;
};
// Key parts of the retrieval filter for a block of Lb queries over n_tiles corpus tiles, and
// the segment capacity its workspace needs (each row has 8 segments per part).
int retrieval_parts(int n_groups, int64_t n_tiles);
int retrieval_groups(int Lb);
int retrieval_seg_cap(int parts, int64_t n_tiles, int top_k, bool keep_all);
// Prep (two-head rows into a.q_idx / a.w, row table a.rows of n_table_rows entries), sample,
// row_prep, filter, select and fold for one block of queries.
hipError_t launch_retrieval_block(RetrievalArgs r, const IndexerArgs& a, bool need_sample, int n_table_rows,
                                  hipStream_t s);
hipError_t launch_causal_mask(int32_t* idx, int64_t L, int top_k, int64_t q_pos0, hipStream_t s);
// Diagnostic: row_prep and the production filter kernel (two key halves, parts = 2) with every
// row's threshold at -inf, then each row's stored (score, key) entries scattered into
// scores[row][key] (NaN elsewhere) and the rows' error bounds into delta_out.  The caller
// sets a.top_k = 1 and a.cap large enough that no row samples and every row's list holds
// all of its keys.
hipError_t launch_score_dump(const IndexerArgs& a, float* scores, int64_t n_cols, float* delta_out, hipStream_t s);

struct AttentionArgs {
    const uint16_t* q;    // [Lb][H][576]
    const uint16_t* kv;   // [N][kv_stride]
    const int32_t* idx;   // [Lb][top_k]
    uint16_t* out;        // [Lb][H][512]
    float* lse;           // [Lb][H] or null
    int64_t kv_stride;
    int64_t N;
    int64_t pos0;
    const QueryInfo* qinfo;  // batch: [Lb] per query (null: one sequence, query t at pos0 + t)
    int Lb, H, top_k;
    float scale;
    // Split over the keys (decode): splits > 1 sends split s of query t to workgroup (t, s),
    // which writes its unnormalised partial into part_o / part_ml for the merge.
    int splits;
    float* part_o;        // [Lb][splits][H][512] fp32
    float* part_ml;       // [Lb][splits][H][4]: reference max (base 2), bf16-weight sum, fp32-weight sum
};
hipError_t launch_sparse_attention(const AttentionArgs& a, hipStream_t s);
// Neighbour packing: pairs of consecutive queries over the union of their rows (one sequence,
// H <= 64, top_k <= 2048: sparse_attention_packable).
bool sparse_attention_packable(const AttentionArgs& a);
hipError_t launch_sparse_attention_packed(const AttentionArgs& a, hipStream_t s);
// Split-key attention and the log-sum-exp merge of its partials.
hipError_t launch_sparse_attention_split(const AttentionArgs& a, hipStream_t s);

// Measured ceilings (ceiling.hip): an MFMA-only bf16 loop on n_cu workgroups of 4 * waves_per_simd
// waves, iters x 8 MFMAs per wave, one value per thread to out; a 16-byte streaming copy.
hipError_t launch_ceiling_mfma(float* out, int n_cu, int iters, bool random, int waves_per_simd, hipStream_t s);
constexpr int kCeilingCopyBlocks = 2048;  // workgroups of 256 threads of the copy / read stream
hipError_t launch_ceiling_copy(const void* src, void* dst, size_t bytes, uint32_t* sink, bool nontemporal,
                               hipStream_t s);

// Workspace of the split-key attention: the partials of min(L, 1024) queries.
constexpr int kDecodeRows = 1024;
constexpr int kMaxSplits = 128;
__host__ __device__ inline size_t decode_workspace_bytes(int64_t rows, int H, int splits) {
    const size_t r = (size_t)(rows < kDecodeRows ? rows : kDecodeRows);
    return r * (size_t)splits * (size_t)H * (512 + 4) * sizeof(float);
}

}  // namespace dsa
