/*
 * snapkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU oracle for SnapKV prefill-time KV-cache
 * compression, in fp64.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only at the seeded synthetic inputs.
 *
 * Source: the page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮"
 * (0h-n0.github.io/posts/paper-2404-14469/), sections
 *   - プロンプトの分割 (prompt split, L_prompt = L_prefix + L_obs),
 *   - 投票メカニズム (voting: C = sum over window rows of W_obs; I = Top_k(C, k),
 *     k = floor(p * L_prefix)),
 *   - クラスタリングによる文脈保持 (1-D max pooling of C before top-k),
 *   - Hit Rate（適中率）の定式化 (M_threshold, O, H, theta = 0.05),
 *   - アルゴリズム (the algorithm listing: split, softmax of window queries
 *     times keys over sqrt(d_k), sum, max pooling with padding kernel//2 and
 *     stride 1, top-k, ascending sort of indices, per-head gather, concat).
 *
 * Readings where the page is silent or differs:
 *   - softmax denominator: every key visible to the window row, i.e. the
 *     prefix plus the window up to and including the row's own position
 *     (causal inside the window).  The listing's prefix-only variant is
 *     available with variant = 1.
 *   - the vote sum runs over the L_obs window rows i = 0..L_obs-1 (the printed
 *     upper bound is garbled), and under GQA over the G query heads that share
 *     a KV head (head h uses KV head h / G).
 *   - the pool's padding is -infinity: windows are clipped to [0, P).
 *   - k = floor(ratio * P) in double, or min(budget, P).
 *   - ties in top-k: larger value first, then lower position first.
 *
 * Every floating-point step is fp64; fp32 and bf16 inputs widen exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of the raw input arrays handed to the oracle */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Widen element e of a row of `dtype` to double, exactly. */
static double widen(const void *row, int dtype, int64_t e)
{
    if (dtype == ORACLE_F32) {
        return (double)((const float *)row)[e];
    } else {
        uint32_t bits = ((uint32_t)((const uint16_t *)row)[e]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static const void *row_ptr(const void *base, int dtype, int64_t row, int64_t stride_elems)
{
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    return (const char *)base + (size_t)row * (size_t)stride_elems * esz;
}

/*
 * Votes of one (request, KV head).
 *   q      : n_rows = G * w window queries, row r = (query head r / w, window row r % w),
 *            rows contiguous with d elements each.
 *   keys   : L key rows of this request and KV head, row stride key_stride elements.
 *   variant: 0 = causal window (window row i sees keys j <= P + i),
 *            1 = prefix-only denominator (every row sees keys j < P only).
 *   votes  : out, L doubles.  votes[j] = sum over rows of softmax weight of key j.
 *            Entries j >= P hold the window's own share (variant 0) or 0.
 * Section 投票メカニズム (C = sum over window rows of W_obs) and the アルゴリズム
 * listing's softmax of q_obs k^T / sqrt(d_k).
 */
void snapkv_oracle_votes(const void *q, int dtype, int64_t n_rows, int32_t w, int32_t d,
                         const void *keys, int64_t key_stride, int64_t L, int32_t variant,
                         double *votes, double *row_buf)
{
    int64_t P = L - w;
    double scale = 1.0 / sqrt((double)d);
    for (int64_t j = 0; j < L; ++j) votes[j] = 0.0;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = r % w;                                   /* window row of this query */
        int64_t n_vis = variant == 0 ? P + i + 1 : P;         /* keys 0 .. n_vis-1 are visible */
        if (n_vis <= 0) continue;                             /* prefix-only variant with P = 0 */
        const void *qr = row_ptr(q, dtype, r, d);
        /* logits */
        for (int64_t j = 0; j < n_vis; ++j) {
            const void *kj = row_ptr(keys, dtype, j, key_stride);
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += widen(qr, dtype, c) * widen(kj, dtype, c);
            row_buf[j] = s * scale;
        }
        /* softmax over the visible keys */
        double m = row_buf[0];
        for (int64_t j = 1; j < n_vis; ++j) if (row_buf[j] > m) m = row_buf[j];
        double l = 0.0;
        for (int64_t j = 0; j < n_vis; ++j) l += exp(row_buf[j] - m);
        /* add this row's weights to the vote */
        for (int64_t j = 0; j < n_vis; ++j) votes[j] += exp(row_buf[j] - m) / l;
    }
}

/*
 * Log-sum-exp of each window row's logits over the keys it sees (the softmax
 * denominator of 投票メカニズム and of the アルゴリズム listing's softmax, in log
 * form): lse[r] = ln sum_j exp(q_r . k_j / sqrt(d)), -infinity for a row that
 * sees no key.  Same visibility rule and row numbering as snapkv_oracle_votes.
 */
void snapkv_oracle_row_lse(const void *q, int dtype, int64_t n_rows, int32_t w, int32_t d,
                           const void *keys, int64_t key_stride, int64_t L, int32_t variant,
                           double *lse, double *row_buf)
{
    int64_t P = L - w;
    double scale = 1.0 / sqrt((double)d);
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = r % w;
        int64_t n_vis = variant == 0 ? P + i + 1 : P;
        if (n_vis <= 0) { lse[r] = -INFINITY; continue; }
        const void *qr = row_ptr(q, dtype, r, d);
        for (int64_t j = 0; j < n_vis; ++j) {
            const void *kj = row_ptr(keys, dtype, j, key_stride);
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += widen(qr, dtype, c) * widen(kj, dtype, c);
            row_buf[j] = s * scale;
        }
        double m = row_buf[0];
        for (int64_t j = 1; j < n_vis; ++j) if (row_buf[j] > m) m = row_buf[j];
        double l = 0.0;
        for (int64_t j = 0; j < n_vis; ++j) l += exp(row_buf[j] - m);
        lse[r] = m + log(l);
    }
}

/*
 * 1-D max pooling of width K_pool (odd), stride 1, padding K_pool/2 with
 * -infinity, over C[0..P).  Section クラスタリングによる文脈保持; the
 * アルゴリズム listing's pooling call.
 */
void snapkv_oracle_pool(const double *c, int64_t P, int32_t K_pool, double *pooled)
{
    int64_t h = K_pool / 2;
    for (int64_t j = 0; j < P; ++j) {
        int64_t lo = j - h < 0 ? 0 : j - h;
        int64_t hi = j + h > P - 1 ? P - 1 : j + h;
        double m = c[lo];
        for (int64_t t = lo + 1; t <= hi; ++t) if (c[t] > m) m = c[t];
        pooled[j] = m;
    }
}

/* k for a prefix of P positions: floor(ratio * P) (mode 0) or min(budget, P) (mode 1). */
int64_t snapkv_oracle_k(int64_t P, int32_t mode, double ratio, int64_t budget)
{
    if (mode == 0) {
        int64_t k = (int64_t)floor(ratio * (double)P);
        if (k > P) k = P;
        if (k < 0) k = 0;
        return k;
    }
    return budget < P ? budget : P;
}

/* qsort comparators: (value desc, index asc), then plain ascending index. */
typedef struct { double v; int64_t j; } vj_t;
static int cmp_value_desc_index_asc(const void *a, const void *b)
{
    const vj_t *x = (const vj_t *)a, *y = (const vj_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->j > y->j) - (x->j < y->j);
}
static int cmp_i32_asc(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Top-k with ascending output: order positions by (pooled desc, position asc),
 * keep the first k, sort them ascending.  Section 投票メカニズム
 * (I = Top_k(C, k)); the アルゴリズム listing sorts the chosen indices.
 * scratch: P entries of 16 bytes.
 */
void snapkv_oracle_select(const double *pooled, int64_t P, int64_t k, int32_t *idx, void *scratch)
{
    vj_t *vj = (vj_t *)scratch;
    for (int64_t j = 0; j < P; ++j) { vj[j].v = pooled[j]; vj[j].j = j; }
    qsort(vj, (size_t)P, sizeof(vj_t), cmp_value_desc_index_asc);
    for (int64_t t = 0; t < k; ++t) idx[t] = (int32_t)vj[t].j;
    qsort(idx, (size_t)k, sizeof(int32_t), cmp_i32_asc);
}

/*
 * Gather of one (request, KV head): rows idx[0..k) of the prefix, then the w
 * window rows P..P+w-1, copied byte for byte.  アルゴリズム listing: gather
 * per head, then concat with the window.
 */
void snapkv_oracle_gather(const void *rows, int64_t row_bytes, int64_t row_stride_bytes,
                          int64_t P, int32_t w, const int32_t *idx, int64_t k, void *out)
{
    char *o = (char *)out;
    for (int64_t t = 0; t < k; ++t)
        memcpy(o + t * row_bytes, (const char *)rows + (int64_t)idx[t] * row_stride_bytes, (size_t)row_bytes);
    for (int32_t i = 0; i < w; ++i)
        memcpy(o + (k + i) * row_bytes, (const char *)rows + (P + i) * row_stride_bytes, (size_t)row_bytes);
}

/*
 * Section Hit Rate（適中率）の定式化: M_thr = 1(a_cur > theta), O = M_thr AND M_vote,
 * H = sum(O) / sum(M_thr).  Returns NaN when no position passes the threshold.
 */
double snapkv_oracle_hit_rate(const double *a_cur, const uint8_t *vote_mask, int64_t n, double theta)
{
    int64_t n_thr = 0, n_hit = 0;
    for (int64_t j = 0; j < n; ++j) {
        int thr = a_cur[j] > theta;
        n_thr += thr;
        n_hit += thr && vote_mask[j];
    }
    if (n_thr == 0) return NAN;
    return (double)n_hit / (double)n_thr;
}

/*
 * One whole (request, KV head) job: votes, pool, k, select.  The gather is a
 * byte copy the caller does with snapkv_oracle_gather.
 */
typedef struct {
    const void *q;        /* [G*w][d] window queries of the group */
    const void *keys;     /* first key row of the request for this KV head */
    int64_t key_stride;   /* elements between key rows */
    int64_t L;            /* request length */
    int32_t n_rows;       /* G*w */
    int32_t w, d, dtype, K_pool, mode, variant, _pad;
    double ratio;
    int64_t budget;
    double *votes;        /* out [L] */
    double *pooled;       /* out [P] */
    int32_t *idx;         /* out [P] capacity; first k entries valid */
    int64_t k;            /* out */
} snapkv_oracle_job;

static void run_job(snapkv_oracle_job *jb)
{
    int64_t P = jb->L - jb->w;
    double *row_buf = (double *)malloc(sizeof(double) * (size_t)(jb->L > 0 ? jb->L : 1));
    void *scratch = malloc(sizeof(vj_t) * (size_t)(P > 0 ? P : 1));
    snapkv_oracle_votes(jb->q, jb->dtype, jb->n_rows, jb->w, jb->d, jb->keys, jb->key_stride,
                        jb->L, jb->variant, jb->votes, row_buf);
    if (P > 0) snapkv_oracle_pool(jb->votes, P, jb->K_pool, jb->pooled);
    jb->k = snapkv_oracle_k(P, jb->mode, jb->ratio, jb->budget);
    if (P > 0) snapkv_oracle_select(jb->pooled, P, jb->k, jb->idx, scratch);
    free(row_buf);
    free(scratch);
}

/*
 * Decode attention over a (compressed) cache: the step after the compression (page
 * "論文解説: SnapKV ..." section デコード速度とメモリ効率, and the KV-cache chapter's decode
 * step, where one new query attends to every cached key).  For G query rows q[G][d] of
 * one KV head and n_rows cached rows: out[h] = sum_j softmax_j(q_h . k_j / sqrt(d)) v_j,
 * in fp64.  out is zero when n_rows = 0.
 */
void snapkv_oracle_decode(const void *q, int dtype, int32_t G, int32_t d, const void *keys, const void *values,
                          int64_t row_stride, int64_t n_rows, double *out, double *row_buf)
{
    double scale = 1.0 / sqrt((double)d);
    for (int32_t h = 0; h < G; ++h) {
        double *o = out + (int64_t)h * d;
        for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
        if (n_rows <= 0) continue;
        const void *qh = row_ptr(q, dtype, h, d);
        for (int64_t j = 0; j < n_rows; ++j) {
            const void *kj = row_ptr(keys, dtype, j, row_stride);
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += widen(qh, dtype, c) * widen(kj, dtype, c);
            row_buf[j] = s * scale;
        }
        double m = row_buf[0];
        for (int64_t j = 1; j < n_rows; ++j) if (row_buf[j] > m) m = row_buf[j];
        double l = 0.0;
        for (int64_t j = 0; j < n_rows; ++j) l += exp(row_buf[j] - m);
        for (int64_t j = 0; j < n_rows; ++j) {
            const void *vj = row_ptr(values, dtype, j, row_stride);
            double p = exp(row_buf[j] - m) / l;
            for (int32_t c = 0; c < d; ++c) o[c] += p * widen(vj, dtype, c);
        }
    }
}

/* Run independent jobs, one OpenMP thread per job at a time.  Returns the thread count used. */
int snapkv_oracle_run_jobs(snapkv_oracle_job *jobs, int64_t n_jobs, int n_threads)
{
    int used = 1;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
    used = n_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (int64_t t = 0; t < n_jobs; ++t) run_job(&jobs[t]);
    return used;
}

int snapkv_oracle_job_size(void) { return (int)sizeof(snapkv_oracle_job); }
