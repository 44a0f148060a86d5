/*
 * oracle.c -- plain, slow fp64 CPU oracle for the DSA prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes, and where the pages define it:
 *
 *  - Indexer score (mlx-lm PR 1997, "How it works": the indexer scores every
 *    cached key with 32 heads; the per-head form sum_h w[t,h] * ReLU(q[t,h].k[s])
 *    is the lightning-indexer score of the DSA problem statement).  Canonical
 *    evaluation order, all in fp64 with no fused multiply-add:
 *        d_h = sum_{i=0..d-1} q[t,h,i]*k[s,i]     (left to right; bf16*bf16 is exact)
 *        r_h = d_h > 0 ? d_h : +0
 *        s   = sum_{h=0..H-1} (w[t,h]*r_h)        (each product rounded, then added)
 *        -0 -> +0
 *  - Top-k selection (same page: the stock indexer's full argpartition, and
 *    "blocked top-k", which folds 4,096-key blocks into a running list and
 *    selects the same keys up to the order of equal scores).  Order used:
 *    score descending, then key index ascending (lower index wins a tie), over
 *    the causal keys 0..p_t only.  Output row = selected keys ascending, then -1.
 *  - Causal masking of an index tensor (llama.cpp PR 25917, review thread:
 *    apply causality on the top-k indices with a separate op, masked = -1,
 *    assuming key index = sequence position).
 *  - Inner-product top-k for vector retrieval (LiteTopK abstract: the same
 *    Indexer-TopK operation serves vector retrieval in recommendation systems
 *    and vector databases).  One query vector against every corpus vector, no
 *    ReLU, no head weights, no causality:
 *        s = sum_{i=0..d-1} q[i]*x[j,i]          (fp64, left to right), -0 -> +0
 *    then the same order as the indexer's top-k (score descending, lower index
 *    first) over all N corpus rows; output ascending, -1 padded.
 *  - Sparse prefill attention (mlx-lm PR 1997, "How it works": 576-wide joined
 *    latent|rope key, gathered top-k rows shared by all heads, absorbed latent
 *    space, value = the 512-wide latent) and the dense boolean-masked form it
 *    replaces ("The change": an L x N mask over every key).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (see build.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FP_FAST_FMA) && defined(__FAST_MATH__)
#error "oracle must be built without fast-math"
#endif

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------- scores */

/* Canonical indexer score of key row k_row for query row q_row ([H][d] bf16). */
double dsa_oracle_score(const uint16_t* q_row, const uint16_t* k_row, const float* w_row,
                        int n_heads, int head_dim) {
    double s = 0.0;
    for (int h = 0; h < n_heads; ++h) {
        const uint16_t* qh = q_row + (size_t)h * head_dim;
        double d = 0.0;
        for (int i = 0; i < head_dim; ++i) {
            double prod = bf16_to_double(qh[i]) * bf16_to_double(k_row[i]);
            d = d + prod;
        }
        double r = d > 0.0 ? d : 0.0;
        double term = (double)w_row[h] * r;
        s = s + term;
    }
    if (s == 0.0) s = 0.0; /* -0 -> +0 */
    return s;
}

/* Per-head dot products only (used by tests to pin the head layout). */
void dsa_oracle_head_dots(const uint16_t* q_row, const uint16_t* k_row, int n_heads,
                          int head_dim, double* out) {
    for (int h = 0; h < n_heads; ++h) {
        double d = 0.0;
        for (int i = 0; i < head_dim; ++i)
            d = d + bf16_to_double(q_row[(size_t)h * head_dim + i]) * bf16_to_double(k_row[i]);
        out[h] = d;
    }
}

/* ------------------------------------------------------------- selection */

typedef struct {
    double score;
    int64_t idx;
} scored_t;

/* score descending, then index ascending */
static int cmp_rank(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

typedef struct {
    const uint16_t* q_idx;
    const uint16_t* k_idx;
    const float* w;
    int64_t L, N, q_pos0, block;
    int n_heads, head_dim, top_k;
    const int64_t* rows;
    int64_t n_rows;
    int32_t* out_idx;
    double* out_kth;
    int64_t next; /* shared row counter */
    pthread_mutex_t mu;
} topk_job_t;

/* One query row.  block == 0: score every causal key, sort, take the first k.
 * block > 0: the pages' blocked fold -- keep a running list of at most k
 * entries, append the next `block` keys, re-rank the k+block entries, keep k. */
static void topk_row(const topk_job_t* J, int64_t t, int32_t* out, double* kth) {
    const int64_t p = J->q_pos0 + t;
    const int64_t n_causal = (p < J->N - 1 ? p : J->N - 1) + 1;
    const int k = J->top_k;
    const uint16_t* q_row = J->q_idx + (size_t)t * J->n_heads * J->head_dim;
    const float* w_row = J->w + (size_t)t * J->n_heads;
    int64_t n_sel;
    scored_t* list;

    if (J->block <= 0) {
        list = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n_causal > 0 ? n_causal : 1));
        for (int64_t s = 0; s < n_causal; ++s) {
            list[s].score = dsa_oracle_score(q_row, J->k_idx + (size_t)s * J->head_dim, w_row,
                                             J->n_heads, J->head_dim);
            list[s].idx = s;
        }
        qsort(list, (size_t)n_causal, sizeof(scored_t), cmp_rank);
        n_sel = n_causal < k ? n_causal : k;
    } else {
        const int64_t B = J->block;
        list = (scored_t*)malloc(sizeof(scored_t) * (size_t)(k + B));
        int64_t n_run = 0;
        for (int64_t b0 = 0; b0 < n_causal; b0 += B) {
            int64_t b1 = b0 + B < n_causal ? b0 + B : n_causal;
            int64_t n = n_run;
            for (int64_t s = b0; s < b1; ++s) {
                list[n].score = dsa_oracle_score(q_row, J->k_idx + (size_t)s * J->head_dim,
                                                 w_row, J->n_heads, J->head_dim);
                list[n].idx = s;
                ++n;
            }
            qsort(list, (size_t)n, sizeof(scored_t), cmp_rank);
            n_run = n < k ? n : k;
        }
        n_sel = n_run;
    }
    if (kth) *kth = n_sel > 0 ? list[n_sel - 1].score : -INFINITY;
    for (int64_t j = 0; j < n_sel; ++j) out[j] = (int32_t)list[j].idx;
    qsort(out, (size_t)n_sel, sizeof(int32_t), cmp_i32);
    for (int64_t j = n_sel; j < k; ++j) out[j] = -1;
    free(list);
}

static void* topk_worker(void* arg) {
    topk_job_t* J = (topk_job_t*)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->n_rows) break;
        int64_t t = J->rows ? J->rows[r] : r;
        topk_row(J, t, J->out_idx + (size_t)r * J->top_k, J->out_kth ? J->out_kth + r : NULL);
    }
    return NULL;
}

static void run_threads(void* (*fn)(void*), void* job, int n_threads) {
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    for (int i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, fn, job);
    for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
}

/* Top-k indices of the listed rows (all rows if rows == NULL, n_rows = L).
 * out_idx: [n_rows][top_k].  out_kth (optional): the k-th selected score.
 * Returns 0, or -1 on a bad argument. */
int dsa_oracle_topk(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L,
                    int64_t N, int n_heads, int head_dim, int64_t q_pos0, int top_k,
                    int64_t block, const int64_t* rows, int64_t n_rows, int32_t* out_idx,
                    double* out_kth, int n_threads) {
    if (!q_idx || !k_idx || !w || !out_idx || L < 0 || N <= 0 || top_k <= 0 || q_pos0 < 0 ||
        q_pos0 + L > N || n_heads <= 0 || head_dim <= 0)
        return -1;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    topk_job_t J;
    memset(&J, 0, sizeof J);
    J.q_idx = q_idx; J.k_idx = k_idx; J.w = w;
    J.L = L; J.N = N; J.q_pos0 = q_pos0; J.block = block;
    J.n_heads = n_heads; J.head_dim = head_dim; J.top_k = top_k;
    J.rows = rows; J.n_rows = rows ? n_rows : L;
    J.out_idx = out_idx; J.out_kth = out_kth;
    pthread_mutex_init(&J.mu, NULL);
    run_threads(topk_worker, &J, n_threads);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* Canonical scores of the listed rows against every key (all rows if rows == NULL):
 * out[r][s] = dsa_oracle_score(row, key s) for s <= p_t, NaN for the later keys.  Used by
 * the tests that compare the GPU's fp32 scores with the canonical order. */
typedef struct {
    const topk_job_t* J;
    double* out;
    int64_t next;
    pthread_mutex_t mu;
} scores_job_t;

static void* scores_worker(void* arg) {
    scores_job_t* S = (scores_job_t*)arg;
    const topk_job_t* J = S->J;
    for (;;) {
        pthread_mutex_lock(&S->mu);
        int64_t r = S->next++;
        pthread_mutex_unlock(&S->mu);
        if (r >= J->n_rows) break;
        const int64_t t = J->rows ? J->rows[r] : r;
        const int64_t p = J->q_pos0 + t;
        const uint16_t* q_row = J->q_idx + (size_t)t * J->n_heads * J->head_dim;
        const float* w_row = J->w + (size_t)t * J->n_heads;
        double* o = S->out + (size_t)r * J->N;
        for (int64_t s = 0; s < J->N; ++s)
            o[s] = s <= p ? dsa_oracle_score(q_row, J->k_idx + (size_t)s * J->head_dim, w_row, J->n_heads,
                                             J->head_dim)
                          : NAN;
    }
    return NULL;
}

int dsa_oracle_scores(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, int64_t L, int64_t N,
                      int n_heads, int head_dim, int64_t q_pos0, const int64_t* rows, int64_t n_rows,
                      double* out, int n_threads) {
    if (!q_idx || !k_idx || !w || !out || L < 0 || N <= 0 || q_pos0 < 0 || q_pos0 + L > N || n_heads <= 0 ||
        head_dim <= 0)
        return -1;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    topk_job_t J;
    memset(&J, 0, sizeof J);
    J.q_idx = q_idx; J.k_idx = k_idx; J.w = w;
    J.L = L; J.N = N; J.q_pos0 = q_pos0;
    J.n_heads = n_heads; J.head_dim = head_dim;
    J.rows = rows; J.n_rows = rows ? n_rows : L;
    scores_job_t S;
    memset(&S, 0, sizeof S);
    S.J = &J;
    S.out = out;
    pthread_mutex_init(&S.mu, NULL);
    run_threads(scores_worker, &S, n_threads);
    pthread_mutex_destroy(&S.mu);
    return 0;
}

/* Causal mask on an index tensor: any index greater than the query's position
 * becomes -1 (idempotent; -1 stays -1). */
void dsa_oracle_causal_mask(int32_t* idx, int64_t L, int top_k, int64_t q_pos0) {
    for (int64_t t = 0; t < L; ++t) {
        int64_t p = q_pos0 + t;
        for (int j = 0; j < top_k; ++j) {
            int32_t v = idx[(size_t)t * top_k + j];
            if (v > p) idx[(size_t)t * top_k + j] = -1;
        }
    }
}

/* ------------------------------------------------------------- attention */

typedef struct {
    const uint16_t* q;
    const uint16_t* kv;
    int64_t kv_stride;
    const int32_t* idx;
    int64_t L, N, q_pos0;
    int H, d_latent, d_rope, top_k, dense;
    double scale;
    const int64_t* rows;
    int64_t n_rows;
    double* out;
    double* lse;
    int64_t next;
    pthread_mutex_t mu;
} attn_job_t;

static double logit(const attn_job_t* J, const uint16_t* q_h, int64_t key) {
    const uint16_t* kr = J->kv + (size_t)key * J->kv_stride;
    const int dqk = J->d_latent + J->d_rope;
    double d = 0.0;
    for (int i = 0; i < dqk; ++i) d = d + bf16_to_double(q_h[i]) * bf16_to_double(kr[i]);
    return J->scale * d;
}

/* Sparse form: softmax over the gathered valid keys J = {idx_j : idx_j != -1,
 * idx_j <= p_t}; o = sum_j softmax_j * latent(idx_j); lse = natural log of the
 * softmax denominator.  Dense form: logits for all N keys, -inf where the
 * boolean mask (key selected for this row and causal) is false, softmax over
 * all N.  Empty set: o = 0, lse = -inf. */
static void attn_row(const attn_job_t* J, int64_t t, double* out, double* lse) {
    const int64_t p = J->q_pos0 + t;
    const int k = J->top_k;
    const int32_t* row = J->idx + (size_t)t * k;
    const int dqk = J->d_latent + J->d_rope;
    int64_t n_keys = J->dense ? J->N : k;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_keys > 0 ? n_keys : 1));
    unsigned char* mask = NULL;
    if (J->dense) {
        mask = (unsigned char*)calloc((size_t)J->N, 1);
        for (int j = 0; j < k; ++j)
            if (row[j] >= 0 && row[j] <= p && row[j] < J->N) mask[row[j]] = 1;
    }
    for (int h = 0; h < J->H; ++h) {
        const uint16_t* q_h = J->q + ((size_t)t * J->H + h) * dqk;
        int64_t n = 0;
        double m = -INFINITY;
        if (J->dense) {
            for (int64_t s = 0; s < J->N; ++s) {
                key[n] = s;
                lg[n] = mask[s] ? logit(J, q_h, s) : -INFINITY;
                if (lg[n] > m) m = lg[n];
                ++n;
            }
        } else {
            for (int j = 0; j < k; ++j) {
                int32_t s = row[j];
                if (s < 0 || s > p) continue;
                key[n] = s;
                lg[n] = logit(J, q_h, s);
                if (lg[n] > m) m = lg[n];
                ++n;
            }
        }
        double* o = out + ((size_t)0 + h) * J->d_latent;
        for (int c = 0; c < J->d_latent; ++c) o[c] = 0.0;
        if (m == -INFINITY) {
            lse[h] = -INFINITY;
            continue;
        }
        double den = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double e = exp(lg[j] - m);
            if (e == 0.0) continue;
            den = den + e;
            const uint16_t* v = J->kv + (size_t)key[j] * J->kv_stride;
            for (int c = 0; c < J->d_latent; ++c) o[c] = o[c] + e * bf16_to_double(v[c]);
        }
        for (int c = 0; c < J->d_latent; ++c) o[c] = o[c] / den;
        lse[h] = m + log(den);
    }
    free(lg);
    free(key);
    free(mask);
}

static void* attn_worker(void* arg) {
    attn_job_t* J = (attn_job_t*)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->n_rows) break;
        int64_t t = J->rows ? J->rows[r] : r;
        attn_row(J, t, J->out + (size_t)r * J->H * J->d_latent, J->lse + (size_t)r * J->H);
    }
    return NULL;
}

/* out: [n_rows][H][d_latent] fp64; lse: [n_rows][H] fp64. dense != 0 selects
 * the boolean-masked form over all N keys. Returns 0 or -1. */
int dsa_oracle_attention(const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                         const int32_t* idx, int64_t L, int64_t N, int H, int d_latent,
                         int d_rope, int top_k, int64_t q_pos0, double scale, int dense,
                         const int64_t* rows, int64_t n_rows, double* out, double* lse,
                         int n_threads) {
    if (!q || !kv || !idx || !out || !lse || L < 0 || N <= 0 || H <= 0 || top_k <= 0 ||
        kv_stride < d_latent + d_rope || q_pos0 < 0 || q_pos0 + L > N)
        return -1;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    attn_job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.kv = kv; J.kv_stride = kv_stride; J.idx = idx;
    J.L = L; J.N = N; J.q_pos0 = q_pos0;
    J.H = H; J.d_latent = d_latent; J.d_rope = d_rope; J.top_k = top_k; J.dense = dense;
    J.scale = scale; J.rows = rows; J.n_rows = rows ? n_rows : L;
    J.out = out; J.lse = lse;
    pthread_mutex_init(&J.mu, NULL);
    run_threads(attn_worker, &J, n_threads);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* ------------------------------------------------------- vector retrieval */

/* Canonical inner product of two bf16 rows of length d (left to right). */
double dsa_oracle_dot(const uint16_t* a, const uint16_t* b, int d) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) {
        double prod = bf16_to_double(a[i]) * bf16_to_double(b[i]);
        s = s + prod;
    }
    if (s == 0.0) s = 0.0;
    return s;
}

typedef struct {
    const uint16_t* q;
    const uint16_t* x;
    int64_t M, N;
    int d, top_k;
    const int64_t* rows;
    int64_t n_rows;
    int32_t* out_idx;
    double* out_kth;
    int64_t next;
    pthread_mutex_t mu;
} retr_job_t;

static void retr_row(const retr_job_t* J, int64_t t, int32_t* out, double* kth) {
    const int k = J->top_k;
    scored_t* list = (scored_t*)malloc(sizeof(scored_t) * (size_t)J->N);
    for (int64_t j = 0; j < J->N; ++j) {
        list[j].score = dsa_oracle_dot(J->q + (size_t)t * J->d, J->x + (size_t)j * J->d, J->d);
        list[j].idx = j;
    }
    qsort(list, (size_t)J->N, sizeof(scored_t), cmp_rank);
    const int64_t n_sel = J->N < k ? J->N : k;
    if (kth) *kth = n_sel > 0 ? list[n_sel - 1].score : -INFINITY;
    for (int64_t j = 0; j < n_sel; ++j) out[j] = (int32_t)list[j].idx;
    qsort(out, (size_t)n_sel, sizeof(int32_t), cmp_i32);
    for (int64_t j = n_sel; j < k; ++j) out[j] = -1;
    free(list);
}

static void* retr_worker(void* arg) {
    retr_job_t* J = (retr_job_t*)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->n_rows) break;
        int64_t t = J->rows ? J->rows[r] : r;
        retr_row(J, t, J->out_idx + (size_t)r * J->top_k, J->out_kth ? J->out_kth + r : NULL);
    }
    return NULL;
}

/* Inner-product top-k of the listed query rows (all if rows == NULL).
 * q: [M][d], x: [N][d] bf16; out_idx: [n_rows][top_k]. Returns 0 or -1. */
int dsa_oracle_retrieval_topk(const uint16_t* q, const uint16_t* x, int64_t M, int64_t N, int d,
                              int top_k, const int64_t* rows, int64_t n_rows, int32_t* out_idx,
                              double* out_kth, int n_threads) {
    if (!q || !x || !out_idx || M < 0 || N <= 0 || d <= 0 || top_k <= 0) return -1;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return -1;
    retr_job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.x = x; J.M = M; J.N = N; J.d = d; J.top_k = top_k;
    J.rows = rows; J.n_rows = rows ? n_rows : M;
    J.out_idx = out_idx; J.out_kth = out_kth;
    pthread_mutex_init(&J.mu, NULL);
    run_threads(retr_worker, &J, n_threads);
    pthread_mutex_destroy(&J.mu);
    return 0;
}
