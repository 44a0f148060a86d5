/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-sparse-attention prefill path.
 *
 * Three operations, one sequence per call (batch 1):
 *   dsa_indexer_topk     indexer scores + exact top-k with causal masking
 *   dsa_causal_mask_topk causal masking of an externally supplied index tensor
 *   dsa_sparse_prefill   sparse absorbed-MLA attention over the selected keys
 * plus the split-key attention for decode and short chunks (dsa_sparse_decode)
 * and a batch of sequences of any lengths per call (the *_varlen entry points),
 * and the same top-k as an inner-product search over a corpus (dsa_retrieval_topk).
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense,
 *     row-major, and live in device memory owned by the caller.  Inputs are
 *     never written.
 *   - Key index = sequence position.  Query t of the chunk sits at position
 *     q_pos0 + t; it may only use keys 0 .. q_pos0 + t.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns without
 *     waiting for the device.  The library keeps no pointer after return
 *     beyond stream-ordered use, and allocates nothing on these paths.
 *   - Arguments are validated before anything is enqueued; on a non-OK
 *     status no output byte has been written.  Asynchronous device faults show
 *     up at the caller's next synchronisation.  No exception crosses the ABI
 *     and the library never aborts.
 *   - Results are deterministic and identical run to run and for every
 *     q_block value.  Calls may run concurrently on different streams when
 *     each has its own workspace.
 *   - Inputs are finite, and the indexer's fp32 work stays in fp32 range:
 *     key elements below 2^60 in magnitude (so that squared key norms are
 *     finite) and indexer scores below 2^120.  Outside that (or with NaN or
 *     infinite inputs) the indices are unspecified.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dsa_stream_t; /* a hipStream_t */

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size or position          */
    DSA_ERR_UNSUPPORTED = 2, /* a shape this build has no kernel for        */
    DSA_ERR_WORKSPACE = 3,   /* workspace null or smaller than required     */
    DSA_ERR_HIP = 4          /* a HIP runtime call failed (see last_error)  */
} dsa_status_t;

#define DSA_INDEX_HEADS 32   /* indexer heads                                 */
#define DSA_INDEX_DIM 128    /* indexer head dimension                        */
#define DSA_MAX_TOPK 4096    /* largest supported top_k                       */
#define DSA_D_LATENT 512     /* latent width = value width                    */
#define DSA_D_ROPE 64        /* rope width; key/query width is 576            */
#define DSA_MAX_HEADS 128    /* attention heads: a multiple of 16, <= 128     */
#define DSA_DEFAULT_Q_BLOCK 1024
#define DSA_MAX_BATCH 65536  /* sequences per *_varlen call                   */

/*
 * Bytes of device workspace dsa_indexer_topk needs for these sizes.  The
 * figure depends on N, top_k and min(L, q_block), never on L*N.  Returns 0 for
 * arguments dsa_indexer_topk would reject.
 */
size_t dsa_indexer_topk_workspace_bytes(int64_t L, int64_t N, int32_t top_k, int32_t q_block);

/*
 * Indexer + top-k ("GLM prefill now attends only to the keys its indexer
 * picks", How it works: the indexer scores every cached key with 32 heads and
 * keeps the top-k per query; the blocked form folds 4,096-key blocks into a
 * running list and never builds the B x 32 x L x N score tensor.  The
 * LiteTopK abstract supplies the threshold scheme: sample the score range,
 * keep a tight threshold, write back only promising candidates, stay exact).
 *
 *   score(t, s) = sum_h w[t,h] * max(0, q_idx[t,h,:] . k_idx[s,:])
 *
 * Selection is over the causal keys s <= q_pos0 + t, highest score first,
 * lower key index first among equal scores.  Scores are ranked exactly as
 * the fp64 evaluation  d_h = sum_i q*k (i ascending), r_h = max(d_h, +0),
 * s = sum_h fl64(w_h * r_h) (h ascending)  ranks them: fp32 matrix-core
 * scores select, and every key whose fp32 score lies within a proven error
 * bound of the k-th is re-scored in that fp64 order.
 *
 *   q_idx   bf16 [L][n_heads][head_dim]
 *   k_idx   bf16 [N][head_dim]
 *   w       fp32 [L][n_heads]
 *   n_heads must be 32, head_dim must be 128 (else DSA_ERR_UNSUPPORTED)
 *   q_pos0  0 <= q_pos0 and q_pos0 + L <= N
 *   top_k   1 .. DSA_MAX_TOPK
 *   q_block queries per internal block; 0 selects 1024
 *   out_idx int32 [L][top_k]: selected keys in ascending order; a row with
 *           fewer than top_k causal keys is padded with -1
 *   workspace / workspace_bytes: device scratch of at least
 *           dsa_indexer_topk_workspace_bytes(L, N, top_k, q_block) bytes,
 *           256-byte aligned; contents need not be initialised
 * L == 0 is a no-op returning DSA_OK.
 */
dsa_status_t dsa_indexer_topk(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                              int64_t L, int64_t N, int32_t n_heads, int32_t head_dim,
                              int64_t q_pos0, int32_t top_k, int32_t q_block, int32_t* out_idx,
                              void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * An append-only cache of the indexer keys in the layout the scoring kernel reads, for
 * decode and chunked prefill over a growing cache ("GLM prefill now attends only to the
 * keys its indexer picks", Evidence: decode continues after a sparse prefill).
 * dsa_indexer_topk lays out all the keys its queries see on every call; a caller that keeps
 * a key cache lays out only the keys appended since its last step.
 *
 *   dsa_indexer_key_cache_bytes(capacity): device bytes of a cache for up to capacity keys
 *       (0 for capacity outside 1 .. 2^31-1).
 *   dsa_indexer_key_cache_append(k_idx, n_old, n_new, cache, bytes, stream): keys n_old ..
 *       n_new-1 of k_idx (bf16 [n_new][128], rows 0 .. n_old-1 unchanged since they were
 *       appended) join the cache; n_old = 0 starts it afresh.  The cache also keeps the
 *       error-bound statistics (largest key norm and element, lowest set bit) of every key
 *       appended since the last restart.  cache: caller-owned device memory, 256-byte
 *       aligned, at least dsa_indexer_key_cache_bytes(n_new) bytes; contents need no
 *       initialisation before a restart.  Asynchronous on `stream`.
 *   dsa_indexer_topk_cached(..., cache, bytes, cached_keys, workspace, ...): dsa_indexer_topk
 *       (same arguments, results and errors) with the keys' layout and statistics taken from
 *       the cache, which holds cached_keys keys (at least the min(N, q_pos0 + L) keys the
 *       queries see, at most N; else DSA_ERR_INVALID_ARG).  k_idx is still read (the exact
 *       re-score reads key rows).  Workspace: at least
 *       dsa_indexer_topk_cached_workspace_bytes(L, N, top_k, q_block) bytes (no key copy).
 * The indices equal dsa_indexer_topk's bit for bit.  A cache is used by one stream at a time.
 */
size_t dsa_indexer_key_cache_bytes(int64_t capacity);
dsa_status_t dsa_indexer_key_cache_append(const uint16_t* k_idx, int64_t n_old, int64_t n_new, void* key_cache,
                                          size_t key_cache_bytes, dsa_stream_t stream);
size_t dsa_indexer_topk_cached_workspace_bytes(int64_t L, int64_t N, int32_t top_k, int32_t q_block);
dsa_status_t dsa_indexer_topk_cached(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                                     int64_t N, int32_t n_heads, int32_t head_dim, int64_t q_pos0, int32_t top_k,
                                     int32_t q_block, int32_t* out_idx, const void* key_cache,
                                     size_t key_cache_bytes, int64_t cached_keys, void* workspace,
                                     size_t workspace_bytes, dsa_stream_t stream);

/*
 * dsa_indexer_topk without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The scratch is a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until the
 * process ends; this call allocates nothing and calls no allocating routine (with
 * kernel timing, dsa_profile_enable, off).  Arguments, results and errors are those
 * of dsa_indexer_topk; sizes whose dsa_indexer_topk_workspace_bytes exceeds
 * DSA_NOALLOC_SCRATCH_BYTES return DSA_ERR_WORKSPACE (a smaller q_block may fit:
 * the decode step at N = 131,072 needs about 39 MiB, a 512-query chunk at 16,384 keys
 * about 44 MiB).  Every call on one GPU uses that GPU's one array, so calls that
 * overlap on one GPU (other streams, other host threads) race and give wrong
 * results; calls in one stream's order are safe.  The scratch needs no clearing:
 * every counter the kernels read is set by an earlier kernel of the same call.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status_t dsa_indexer_topk_noalloc(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                                      int64_t L, int64_t N, int32_t n_heads, int32_t head_dim,
                                      int64_t q_pos0, int32_t top_k, int32_t q_block, int32_t* out_idx,
                                      dsa_stream_t stream);

/*
 * Selection counters of the last dsa_indexer_topk, dsa_indexer_topk_varlen or
 * dsa_retrieval_topk call made with this workspace (diagnostics; no result
 * depends on them).  They show how the LiteTopK abstract's threshold scheme
 * behaved on the call's inputs: how many candidates each row wrote back above
 * its sampled threshold, how many keys within the error bound of the k-th score
 * were re-scored in fp64, and how many rows needed the GLM page's blocked
 * 4,096-key fold (How it works) because their candidates could not be proven to
 * hold the top-k.  Counts run over the whole call (every query block).
 */
typedef struct {
    int64_t rows;                /* rows finished from their candidate lists            */
    int64_t rows_all_keys;       /* rows with at most top_k causal keys (no selection)  */
    int64_t rows_fallback;       /* rows finished by the blocked fold, because ...      */
    int64_t fallback_overflow;   /*   the row's candidate list overflowed               */
    int64_t fallback_incomplete; /*   the candidates could miss a top-k key             */
    int64_t fallback_band;       /*   the fp64 band outgrew the selection buffer        */
    int64_t rows_failed;         /* rows no path finished (written as -1): 0 expected   */
    int64_t candidates;          /* candidates summed over `rows`                       */
    int64_t candidates_max;      /* most candidates of one of those rows                */
    int64_t band;                /* keys re-scored in fp64, summed over `rows`          */
    int64_t band_max;            /* most keys re-scored for one row                     */
    int64_t kth_radix;           /* fold rows whose k-th search took the radix pass     */
} dsa_indexer_stats_t;

/*
 * Copies the counters above out of `workspace` (the device workspace of the
 * call) into *out.  Enqueued on `stream` after the call and waits for the
 * stream: a host synchronisation, unlike the entry points.  workspace must be
 * non-null and 256-byte aligned (else DSA_ERR_INVALID_ARG).
 */
dsa_status_t dsa_indexer_topk_stats(const void* workspace, dsa_indexer_stats_t* out, dsa_stream_t stream);

/*
 * The fp32 indexer scores that the selection starts from, for up to
 * DSA_MAX_SCORE_ROWS query rows (a diagnostic: it lets a caller check the error
 * bound that makes the selection exact, "GLM prefill now attends only to the
 * keys its indexer picks", How it works: the sparse path picks the same keys as
 * the stock indexer).  The production scoring kernel (bf16 matrix cores, ReLU,
 * weighted head sum) runs with every row's threshold at -infinity, so it keeps
 * every causal key, and the kept scores are scattered out:
 *
 *   scores fp32 [L][N]: row t holds score(t, s) for s <= q_pos0 + t, NaN after
 *   delta  fp32 [L] or NULL: the bound delta_t on |fp32 score - fp64 score| the
 *          selection uses for row t (0 when the row's fp32 scores are exact)
 *
 * Arguments as dsa_indexer_topk, with 1 <= q_pos0 and L <= DSA_MAX_SCORE_ROWS
 * (else DSA_ERR_INVALID_ARG); workspace: at least
 * dsa_indexer_scores_workspace_bytes(L, N) bytes, 256-byte aligned (it holds
 * every key of every row as a candidate).  Not a hot-path call.
 */
#define DSA_MAX_SCORE_ROWS 64
size_t dsa_indexer_scores_workspace_bytes(int64_t L, int64_t N);
dsa_status_t dsa_indexer_scores(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                                int64_t N, int32_t n_heads, int32_t head_dim, int64_t q_pos0, float* scores,
                                float* delta, void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * Causal masking of an index tensor ("cuda : support for sparse KV indices in
 * MMA flash attention kernel", review thread: apply causality to the top-k
 * indices with a separate op, masked entries becoming -1, assuming key index =
 * sequence position).  In place: idx[t][j] > q_pos0 + t becomes -1; every
 * other entry (including -1) is left as is.  Idempotent.
 *   idx int32 [L][top_k] (device); L >= 0, top_k >= 1, q_pos0 >= 0
 */
dsa_status_t dsa_causal_mask_topk(int32_t* idx, int64_t L, int32_t top_k, int64_t q_pos0,
                                  dsa_stream_t stream);

/*
 * Sparse prefill attention in the absorbed latent space ("GLM prefill now
 * attends only to the keys its indexer picks", How it works: join the 512-wide
 * latent and 64-wide rope caches into one 576-wide key, gather the top-k rows
 * each query picked, all heads share that block, the latent is also the
 * value; chunks above 1,024 queries run as query blocks).
 *
 *   for each query t and head h, over J = { idx[t][j] : idx != -1, idx <= q_pos0+t }:
 *     l_j = scale * q[t,h,:] . kv[j, 0:576]
 *     out[t,h,:] = sum_j softmax(l)_j * kv[j, 0:512]      (fp32 accumulate, bf16 out)
 *     lse[t,h]   = log(sum_j exp(l_j))                    (natural log)
 *   an empty J gives out = 0 and lse = -inf.
 *
 *   q        bf16 [L][H][d_latent + d_rope]
 *   kv       bf16 [N][kv_stride]: latent in 0..d_latent-1, rope after it
 *   kv_stride elements per kv row, >= d_latent + d_rope, a multiple of 8
 *   idx      int32 [L][top_k]; indices must be < N (or -1); repeats are out of contract
 *   H        a multiple of 16, <= DSA_MAX_HEADS (else DSA_ERR_UNSUPPORTED)
 *   d_latent must be 512 and d_rope 64 (else DSA_ERR_UNSUPPORTED)
 *   q_pos0   0 <= q_pos0, q_pos0 + L <= N
 *   scale    logit scale (1/sqrt(192) for the GLM/DeepSeek shapes)
 *   q_block  queries per launch; 0 selects 1024
 *   out      bf16 [L][H][d_latent]
 *   lse      fp32 [L][H] or NULL
 * L == 0 is a no-op returning DSA_OK.
 */
dsa_status_t dsa_sparse_prefill(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                                const int32_t* idx, int64_t L, int64_t N, int32_t H,
                                int32_t d_latent, int32_t d_rope, int32_t top_k, int64_t q_pos0,
                                float scale, int32_t q_block, uint16_t* out, float* lse,
                                dsa_stream_t stream);

/*
 * dsa_sparse_prefill with neighbour packing (LiteDSA, in the LiteTopK page's
 * abstract and Fig. 3: neighbouring tokens' candidate sets are similar, so they
 * are packed for joint computation and each query masks the scores it did not
 * select).  Queries 2b and 2b + 1 of each query block share one workgroup: the
 * rows of the union of their index rows are gathered once, and each query
 * attends only over its own entries.  The result is the dsa_sparse_prefill
 * result (same definition and arguments) up to the rounding order of the
 * softmax sums.  Rows that are ascending with a -1 tail (dsa_indexer_topk's
 * output) are merged with repeats removed, which is where the gather saves
 * bytes; other rows are concatenated.  H > 64 or top_k > 2048 run the unpacked
 * kernel.  Arguments and errors as dsa_sparse_prefill.
 * Performance: on MI355X this is slower than dsa_sparse_prefill at every overlap
 * measured (0.59x of its speed with no shared rows, 0.88x when neighbours share
 * 80% of their rows, 0.96x at 95%): the attention's per-key compute, which
 * packing does not reduce, outweighs the gather it saves.  dsa_sparse_prefill is
 * the default path.
 */
dsa_status_t dsa_sparse_prefill_packed(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                                       const int32_t* idx, int64_t L, int64_t N, int32_t H,
                                       int32_t d_latent, int32_t d_rope, int32_t top_k,
                                       int64_t q_pos0, float scale, int32_t q_block, uint16_t* out,
                                       float* lse, dsa_stream_t stream);

/*
 * Sparse attention split over the selected keys, for decode (L = 1) and short
 * chunks ("GLM prefill now attends only to the keys its indexer picks", How it
 * works: the sparse path uses the same absorbed form decode already uses; and
 * Evidence: decode continues after a sparse prefill).  Each query's top-k list
 * is cut into `splits` contiguous parts attended by separate workgroups; each
 * part's unnormalised output and softmax sums are merged by log-sum-exp.  The
 * result is the dsa_sparse_prefill result (same definition, same arguments),
 * up to the rounding order of the merge.
 *
 *   splits   1 .. 128 parts per query (clamped to ceil(top_k/32)); 0 picks a count
 *            that gives about 512 workgroups
 *   workspace / workspace_bytes: device scratch of at least
 *            dsa_sparse_decode_workspace_bytes(L, H, top_k, splits) bytes, 256-byte
 *            aligned, caller-owned; it holds the partials of up to 1,024 queries
 *            (longer chunks run in blocks of 1,024 queries reusing it)
 *   other arguments and the errors as dsa_sparse_prefill; a short or null
 *   workspace gives DSA_ERR_WORKSPACE, splits outside 0..128 DSA_ERR_INVALID_ARG.
 * L == 0 is a no-op returning DSA_OK.
 */
size_t dsa_sparse_decode_workspace_bytes(int64_t L, int32_t H, int32_t top_k, int32_t splits);
dsa_status_t dsa_sparse_decode(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                               const int32_t* idx, int64_t L, int64_t N, int32_t H,
                               int32_t d_latent, int32_t d_rope, int32_t top_k, int64_t q_pos0,
                               float scale, int32_t splits, uint16_t* out, float* lse,
                               void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * A batch of sequences in one call (the GLM page's Evidence section names batched
 * sparse prefill as the next step after the single-sequence path; the indexer
 * and attention definitions above apply to each sequence on its own).  The
 * batch is described by three HOST arrays, in the packed ("varlen") layout:
 *
 *   cu_q  int64 [B+1]: sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 of every
 *         per-query tensor (q_idx, w, q, idx, out, lse, out_idx); cu_q[0] = 0
 *   cu_k  int64 [B+1]: sequence b owns key rows cu_k[b] .. cu_k[b+1]-1 of k_idx
 *         and kv (N_b = cu_k[b+1] - cu_k[b] keys); cu_k[0] = 0
 *   pos0  int64 [B]: position of sequence b's first query; query row cu_q[b]+i
 *         sits at position pos0[b]+i and may use the sequence's keys 0 .. pos0[b]+i
 *
 * Both arrays must be non-decreasing, with 0 <= pos0[b] and pos0[b] + L_b <= N_b
 * (L_b = cu_q[b+1] - cu_q[b]; L_b = 0 and N_b = 0 are allowed), B in
 * 0 .. DSA_MAX_BATCH, else DSA_ERR_INVALID_ARG.  Key indices (out_idx, idx)
 * are positions within the sequence, 0 .. N_b-1, as in the one-sequence calls;
 * each query row's result equals the one-sequence call on its sequence alone.
 * The host arrays are read during the call only.  A batch with no query rows
 * is a no-op returning DSA_OK; the *_workspace_bytes functions return 0 for it
 * and for arguments the call would reject.
 *
 * dsa_indexer_topk_varlen: q_idx bf16 [T][32][128], w fp32 [T][32], k_idx
 *   bf16 [cu_k[B]][128], out_idx int32 [T][top_k] (T = cu_q[B]); n_heads,
 *   head_dim, top_k, q_block and the errors as dsa_indexer_topk.  Workspace:
 *   256-byte aligned, at least dsa_indexer_topk_varlen_workspace_bytes(...).
 */
size_t dsa_indexer_topk_varlen_workspace_bytes(int64_t B, const int64_t* cu_q, const int64_t* cu_k,
                                               const int64_t* pos0, int32_t top_k, int32_t q_block);
dsa_status_t dsa_indexer_topk_varlen(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                                     int64_t B, const int64_t* cu_q, const int64_t* cu_k,
                                     const int64_t* pos0, int32_t n_heads, int32_t head_dim,
                                     int32_t top_k, int32_t q_block, int32_t* out_idx,
                                     void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * dsa_sparse_prefill_varlen: the attention of dsa_sparse_prefill for each
 * sequence of a batch (layout as above): q bf16 [T][H][576], kv bf16
 * [cu_k[B]][kv_stride], idx int32 [T][top_k], out bf16 [T][H][512], lse fp32
 * [T][H] or NULL.  splits as dsa_sparse_decode (1 = one workgroup per query, the
 * dsa_sparse_prefill kernel; 0 picks a count from T, which is 1 for T >= 512).
 * Workspace: 256-byte aligned, at least
 * dsa_sparse_prefill_varlen_workspace_bytes(...) bytes (a per-query table, plus
 * the split partials when splits > 1).  Other arguments and errors as
 * dsa_sparse_decode.
 */
size_t dsa_sparse_prefill_varlen_workspace_bytes(int64_t B, const int64_t* cu_q, const int64_t* cu_k,
                                                 const int64_t* pos0, int32_t H, int32_t top_k,
                                                 int32_t splits);
dsa_status_t dsa_sparse_prefill_varlen(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                                       const int32_t* idx, int64_t B, const int64_t* cu_q,
                                       const int64_t* cu_k, const int64_t* pos0, int32_t H,
                                       int32_t d_latent, int32_t d_rope, int32_t top_k, float scale,
                                       int32_t splits, uint16_t* out, float* lse, void* workspace,
                                       size_t workspace_bytes, dsa_stream_t stream);

/*
 * Inner-product top-k over a corpus, for vector retrieval (LiteTopK abstract:
 * the Indexer-TopK operation also serves vector retrieval in recommendation
 * systems and vector databases).  For each query row t, over every corpus row j:
 *
 *   score(t, j) = q[t,:] . x[j,:]       (one head, no ReLU, no weights, no causality)
 *
 * ranked exactly as the fp64 left-to-right sum of the dim products ranks them,
 * highest first, lower row first among equal scores (the indexer's rule; the
 * same sample -> threshold -> candidates -> exact band re-score scheme).
 *
 *   q        bf16 [M][dim] queries;  x bf16 [N][dim] corpus;  dim must be 128
 *   top_k    1 .. DSA_MAX_TOPK
 *   q_block  queries per internal block; 0 selects 1024
 *   out_idx  int32 [M][top_k]: selected corpus rows in ascending order, -1 padded
 *            when N < top_k
 *   workspace / workspace_bytes: at least
 *            dsa_retrieval_topk_workspace_bytes(M, N, top_k, q_block) bytes,
 *            256-byte aligned; it grows with min(M, q_block) and N / top_k-sized
 *            candidate lists, not with N alone (the corpus is read in place)
 * Errors as dsa_indexer_topk (dim != 128 gives DSA_ERR_UNSUPPORTED).  M == 0 is a
 * no-op returning DSA_OK.
 */
size_t dsa_retrieval_topk_workspace_bytes(int64_t M, int64_t N, int32_t top_k, int32_t q_block);
dsa_status_t dsa_retrieval_topk(const uint16_t* q, const uint16_t* x, int64_t M, int64_t N, int32_t dim,
                                int32_t top_k, int32_t q_block, int32_t* out_idx, void* workspace,
                                size_t workspace_bytes, dsa_stream_t stream);

/*
 * The sparse-prefill gate of the GLM page ("How it works": sparse only for a
 * single sequence, only in prefill, and only once the cache holds at least
 * min_context tokens; 16,384 by default).  Returns 1 when the sparse path
 * applies to (B, L, N), else 0.  min_context <= 0 selects 16384.  Host only.
 */
int dsa_sparse_prefill_gate(int64_t B, int64_t L, int64_t N, int64_t min_context);

/*
 * Measured ceilings beside the published peaks (not part of the DSA path; bench.py
 * reports them): what the GPU actually reaches on a plain stream of the same kind of
 * work as a kernel, to set its roofline fraction beside:
 *
 * dsa_ceiling_mfma_bf16: bf16 32x32x16 MFMA chains and nothing else (operands in
 * registers, eight independent accumulators per wave, no memory traffic in the loop),
 * one workgroup per compute unit with 4 * waves_per_simd waves, i.e. one or two waves
 * per SIMD (the indexer's scoring kernel runs one).  random_operands != 0 draws the
 * operands as bf16 values of random sign and mantissa (exponents in [2^-3, 2^1)),
 * else every operand is 1.0: the matrix units draw more power on random data and the
 * clock drops.  Each wave runs iters x 8 MFMAs; one float per thread is written to
 * out (device memory, out_len >= dsa_ceiling_mfma_threads(waves_per_simd)) so that no
 * work is dropped.  *flops (host) receives the launch's MFMA flops (32768 per MFMA).
 * Errors: waves_per_simd outside {1, 2}, iters < 1, null pointers or a short out give
 * DSA_ERR_INVALID_ARG.  Asynchronous on stream; time it with the "ceiling_mfma"
 * timing class below.
 *
 * dsa_ceiling_stream: streams bytes (a multiple of 16; 16-byte aligned device
 * pointers) from src with 16-byte loads, eight in flight per lane, one contiguous chunk
 * per workgroup (timing class "ceiling_copy").  dst non-null: a copy to dst (bytes read and bytes written).  dst
 * null: reads only; each thread writes the XOR of what it read to sink (device,
 * sink_len >= dsa_ceiling_stream_sink_words() words) so that no load is dropped.
 * nontemporal != 0 marks the loads and stores nontemporal.  Bad pointers, alignment or
 * sizes give DSA_ERR_INVALID_ARG; bytes == 0 is a no-op.
 */
int64_t dsa_ceiling_mfma_threads(int32_t waves_per_simd);
dsa_status_t dsa_ceiling_mfma_bf16(float* out, int64_t out_len, int32_t iters, int32_t random_operands,
                                   int32_t waves_per_simd, double* flops, dsa_stream_t stream);
int64_t dsa_ceiling_stream_sink_words(void);
dsa_status_t dsa_ceiling_stream(const void* src, void* dst, size_t bytes, uint32_t* sink, int64_t sink_len,
                                int32_t nontemporal, dsa_stream_t stream);

/*
 * Kernel timing diagnostics.  While enabled (on != 0), every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the caller's stream;
 * the events add no synchronisation.  dsa_profile_read waits for the recorded
 * events of one kernel class, returns the summed duration in milliseconds and
 * the number of launches since the last read of that class, and forgets them.
 * Kernel classes: "key_stats", "score_sample", "row_prep", "score_filter",
 * "select", "fold", "sparse_attention", "causal_mask", "attn_split",
 * "attn_merge", "retr_prep", "retr_sample", "retr_filter", "retr_gather", "ceiling_mfma",
 * "ceiling_copy".  Unknown names give
 * DSA_ERR_INVALID_ARG.  Host only; safe to
 * call from one thread at a time.
 */
dsa_status_t dsa_profile_enable(int on);
/* Brackets only the listed kernel classes (comma-separated names as above; NULL or
 * "" = all of them) and turns timing on; fewer events disturb the stream less.
 * An unknown name gives DSA_ERR_INVALID_ARG and changes nothing.  Host only. */
dsa_status_t dsa_profile_set(const char* kernels);
dsa_status_t dsa_profile_read(const char* kernel, double* total_ms, int64_t* launches);

/* Static description of a status code. */
const char* dsa_status_string(dsa_status_t s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* Library version string. */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
