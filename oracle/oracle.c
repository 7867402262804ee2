/*
 * CPU oracle for tree-verification attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the CPU-baseline leg of the benchmark may
 * load this library. It shares no code, header or constant with the HIP path.
 *
 * What it computes is the plain definition that LongSpec's Hybrid Tree Attention reaches
 * exactly (LongSpec page, "Fast tree attention" section, and the appendix "Correctness of
 * attention aggregation", Proposition and proof): for every tree node i, q-head h,
 *
 *     softmax attention of q[b,i,h] over the keys [ prefix 0..L_b-1  ||  tree nodes anc(i) ],
 *
 * where anc(i) is i together with its ancestors in the draft tree (textbook page, "Linear chains
 * and candidate trees consume work differently": a node may only attend to its ancestors; the
 * node itself is included, which is the reading under which a chain reproduces causal scoring,
 * textbook page "Generation is sequential, verification can be parallel").
 *
 * Everything is evaluated in double precision from the exact inputs (bf16 / fp32 bit patterns
 * widened without rounding). The softmax is two-pass: maximum, then sum of exponentials; the
 * log-sum-exp is natural-log and covers the scaled logits s = scale * q.k.
 *
 * Threads split the list of output rows; every row is computed serially by one thread, so the
 * thread count never changes a result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

#define OR_FULL 0   /* prefix || masked tree */
#define OR_PREFIX 1 /* prefix keys only */
#define OR_TREE 2   /* masked tree keys only */

#define OR_OK 0
#define OR_EBAD_PARENT 1
#define OR_EBAD_LEN 2
#define OR_EBAD_ARG 3
#define OR_ENOMEM 4

static double widen(const void *base, int dtype, size_t idx) {
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* A node's parent must precede it (topological numbering, DFlash-TfM summary page,
 * "Rollback-free tree verification"); -1 attaches it to the committed prefix. */
int oracle_check_parents(const int32_t *parent, int B, int T) {
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < T; ++i) {
            int32_t p = parent[(size_t)b * T + i];
            if (p < -1 || p >= i) return OR_EBAD_PARENT;
        }
    return OR_OK;
}

/* Ancestor-or-self mask, one row per node: bit (j % 64) of word j / 64 of row i is set when j is
 * i or an ancestor of i. Built by walking parent pointers from every node up to the prefix. */
int oracle_tree_mask(const int32_t *parent, int B, int T, uint64_t *mask) {
    if (B < 0 || T < 0) return OR_EBAD_ARG;
    int rc = oracle_check_parents(parent, B, T);
    if (rc) return rc;
    int W = (T + 63) / 64;
    memset(mask, 0, sizeof(uint64_t) * (size_t)B * T * W);
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < T; ++i) {
            uint64_t *row = mask + ((size_t)b * T + i) * W;
            for (int j = i; j >= 0; j = parent[(size_t)b * T + j]) row[j / 64] |= 1ull << (j % 64);
        }
    return OR_OK;
}

typedef struct {
    int B, T, Hq, Hkv, D, dtype, which;
    double scale;
    const void *q, *k_cache, *v_cache, *k_tree, *v_tree;
    int Lmax;
    const int32_t *seq_lens, *block_table, *parent;
    int page_size, max_blocks;
    const int32_t *rows;
    int n_rows;
    double *o, *lse;
    /* per-thread work split */
    int row_lo, row_hi;
} job_t;

/* Element offset of prefix key j of sequence b, kv-head g. Contiguous storage is
 * [B][Lmax][Hkv][D]; paged storage is a pool [pages][page_size][Hkv][D] addressed through the
 * block table [B][max_blocks]: key j lives in block j / page_size at row j % page_size. */
static size_t prefix_offset(const job_t *jb, int b, int j, int g) {
    size_t row;
    if (jb->block_table) {
        int32_t page = jb->block_table[(size_t)b * jb->max_blocks + j / jb->page_size];
        row = (size_t)page * jb->page_size + (size_t)(j % jb->page_size);
    } else {
        row = (size_t)b * jb->Lmax + (size_t)j;
    }
    return (row * jb->Hkv + g) * (size_t)jb->D;
}

static void one_row(const job_t *jb, int b, int i, int h, double *o, double *lse, double *logit,
                    int32_t *keys_tree) {
    const int D = jb->D, T = jb->T, G = jb->Hq / jb->Hkv;
    const int g = h / G; /* q-head h reads kv-head floor(h / G) */
    const size_t qoff = (((size_t)b * T + i) * jb->Hq + h) * (size_t)D;
    const int L = (jb->which == OR_TREE) ? 0 : jb->seq_lens[b];

    /* tree keys visible from node i: i and its ancestors */
    int n_tree = 0;
    if (jb->which != OR_PREFIX)
        for (int j = i; j >= 0; j = jb->parent[(size_t)b * T + j]) keys_tree[n_tree++] = j;

    const int n = L + n_tree;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    /* pass 1: logits and their maximum */
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        const void *kb;
        size_t koff;
        if (t < L) {
            kb = jb->k_cache;
            koff = prefix_offset(jb, b, t, g);
        } else {
            kb = jb->k_tree;
            koff = (((size_t)b * T + keys_tree[t - L]) * jb->Hkv + g) * (size_t)D;
        }
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += widen(jb->q, jb->dtype, qoff + d) * widen(kb, jb->dtype, koff + d);
        s *= jb->scale;
        logit[t] = s;
        if (s > m) m = s;
    }
    /* pass 2: normaliser and weighted sum of values */
    double z = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(logit[t] - m);
        z += w;
        const void *vb;
        size_t voff;
        if (t < L) {
            vb = jb->v_cache;
            voff = prefix_offset(jb, b, t, g);
        } else {
            vb = jb->v_tree;
            voff = (((size_t)b * T + keys_tree[t - L]) * jb->Hkv + g) * (size_t)D;
        }
        for (int d = 0; d < D; ++d) o[d] += w * widen(vb, jb->dtype, voff + d);
    }
    for (int d = 0; d < D; ++d) o[d] /= z;
    *lse = m + log(z);
}

static void *run_job(void *arg) {
    job_t *jb = (job_t *)arg;
    int maxL = 0;
    if (jb->which != OR_TREE)
        for (int b = 0; b < jb->B; ++b)
            if (jb->seq_lens[b] > maxL) maxL = jb->seq_lens[b];
    double *logit = (double *)malloc(sizeof(double) * ((size_t)maxL + jb->T + 1));
    int32_t *keys = (int32_t *)malloc(sizeof(int32_t) * ((size_t)jb->T + 1));
    if (!logit || !keys) {
        free(logit);
        free(keys);
        return (void *)1;
    }
    for (int r = jb->row_lo; r < jb->row_hi; ++r) {
        int b, i, h;
        if (jb->rows) {
            b = jb->rows[3 * (size_t)r];
            i = jb->rows[3 * (size_t)r + 1];
            h = jb->rows[3 * (size_t)r + 2];
        } else {
            h = r % jb->Hq;
            i = (r / jb->Hq) % jb->T;
            b = r / (jb->Hq * jb->T);
        }
        one_row(jb, b, i, h, jb->o + (size_t)r * jb->D, jb->lse + r, logit, keys);
    }
    free(logit);
    free(keys);
    return NULL;
}

/*
 * Attention of the selected rows. ``which`` picks the key set: OR_FULL (prefix || masked tree),
 * OR_PREFIX (unmasked prefix only) or OR_TREE (masked tree only). ``rows`` lists (b, i, h)
 * triples, or is NULL for every row in (b, i, h) order. Outputs: o[n_rows][D], lse[n_rows].
 * A row with no visible key gets o = 0 and lse = -inf.
 */
int oracle_attend(int B, int T, int Hq, int Hkv, int D, int dtype, double scale, const void *q,
                  const void *k_cache, const void *v_cache, int Lmax, const int32_t *seq_lens,
                  const int32_t *block_table, int page_size, int max_blocks, int num_pages,
                  const void *k_tree, const void *v_tree, const int32_t *parent, int which,
                  const int32_t *rows, int n_rows, double *o, double *lse, int nthreads) {
    if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0) return OR_EBAD_ARG;
    if (dtype != OR_F32 && dtype != OR_BF16) return OR_EBAD_ARG;
    if (which < OR_FULL || which > OR_TREE) return OR_EBAD_ARG;
    if (T > 0) {
        int rc = oracle_check_parents(parent, B, T);
        if (rc) return rc;
    }
    if (which != OR_TREE) {
        long cap = block_table ? (long)max_blocks * page_size : (long)Lmax;
        for (int b = 0; b < B; ++b)
            if (seq_lens[b] < 0 || seq_lens[b] > cap) return OR_EBAD_LEN;
        if (block_table) {
            if (page_size <= 0) return OR_EBAD_ARG;
            for (int b = 0; b < B; ++b)
                for (int blk = 0; blk < (seq_lens[b] + page_size - 1) / page_size; ++blk) {
                    int32_t pg = block_table[(size_t)b * max_blocks + blk];
                    if (pg < 0 || pg >= num_pages) return OR_EBAD_LEN;
                }
        }
    }
    if (!rows) n_rows = B * T * Hq;
    for (int r = 0; rows && r < n_rows; ++r) {
        int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
        if (b < 0 || b >= B || i < 0 || i >= T || h < 0 || h >= Hq) return OR_EBAD_ARG;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_rows) nthreads = n_rows > 0 ? n_rows : 1;

    job_t base = {B, T, Hq, Hkv, D, dtype, which, scale, q, k_cache, v_cache, k_tree, v_tree,
                  Lmax, seq_lens, block_table, parent, page_size, max_blocks, rows, n_rows, o,
                  lse, 0, 0};
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return OR_ENOMEM;
    }
    char *created = (char *)calloc((size_t)nthreads, 1);
    if (!created) {
        free(jobs);
        free(th);
        return OR_ENOMEM;
    }
    int failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].row_lo = (int)((long)n_rows * t / nthreads);
        jobs[t].row_hi = (int)((long)n_rows * (t + 1) / nthreads);
    }
    for (int t = 0; t + 1 < nthreads; ++t)
        created[t] = pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0;
    if (run_job(&jobs[nthreads - 1])) failed = 1;
    for (int t = 0; t + 1 < nthreads; ++t) {
        if (created[t]) {
            void *ret = NULL;
            pthread_join(th[t], &ret);
            if (ret) failed = 1;
        } else if (run_job(&jobs[t])) {
            failed = 1; /* a thread that could not start: its rows run here */
        }
    }
    free(created);
    free(jobs);
    free(th);
    return failed ? OR_ENOMEM : OR_OK;
}

/*
 * Merge of two partial attention results over disjoint key sets (LongSpec page, "Fast tree
 * attention", aggregation step; appendix Proposition):
 *     LSE = log(exp(LSE_a) + exp(LSE_b)),
 *     o   = o_a * exp(LSE_a - LSE) + o_b * exp(LSE_b - LSE).
 * The logarithm of the sum is evaluated after factoring out the larger exponent, which changes
 * nothing mathematically and keeps exp() finite. Two empty parts (both -inf) give o = 0,
 * LSE = -inf.
 */
void oracle_merge(int n, int D, const double *o_a, const double *lse_a, const double *o_b,
                  const double *lse_b, double *o, double *lse) {
    for (int r = 0; r < n; ++r) {
        double a = lse_a[r], b = lse_b[r];
        if (isinf(a) && a < 0 && isinf(b) && b < 0) {
            for (int d = 0; d < D; ++d) o[(size_t)r * D + d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double mx = a > b ? a : b;
        double l = mx + log(exp(a - mx) + exp(b - mx));
        double wa = exp(a - l), wb = exp(b - l);
        for (int d = 0; d < D; ++d)
            o[(size_t)r * D + d] = o_a[(size_t)r * D + d] * wa + o_b[(size_t)r * D + d] * wb;
        lse[r] = l;
    }
}
