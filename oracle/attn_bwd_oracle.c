/*
 * attn_bwd_oracle.c -- plain fp64 CPU oracle for the gradients of the exact attention forward.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code. It shares no code
 * with the GPU path and the GPU path never calls it.
 *
 * The pages name a faster backward pass and the recomputation of attention
 * from stored statistics instead of storing the attention matrix (unite.ai page
 * "Flash Attention: revolutionizing transformer efficiency": the list of key
 * ideas after "Enter Flash Attention", item 2, and "FlashAttention-2", item 2)
 * but print no formula. What is computed here is the gradient of the forward
 * that attn_oracle.c computes, by the chain rule, for an upstream gradient dO
 * of o (lse receives no upstream gradient):
 *
 *   p_ij  = exp(s_ij - lse_i)                  (the softmax of row i; 0 outside J_i)
 *   o_i   = sum_j p_ij v_j,    D_i = sum_c dO_ic o_ic
 *   dP_ij = sum_c dO_ic v_jc
 *   dS_ij = p_ij (dP_ij - D_i)                 (softmax Jacobian applied to dP)
 *   dq_i  = scale sum_j dS_ij k_j
 *   dk_j  = scale sum_i dS_ij q_i              (summed over the query heads that share k_j)
 *   dv_j  = sum_i p_ij dO_i                    (likewise)
 *
 * with s_ij, J_i, lse_i and the key/value head g of query head h exactly as in
 * attn_oracle.c, including its key-padding lengths: with a length L_b for batch
 * b, J_i keeps only the keys j < L_b, so a key j >= L_b gets dk_j = dv_j = 0
 * and a query row with no visible key (L_b = 0) has o_i = 0, D_i = 0 and
 * dq_i = 0 (its lse is -inf and never used). Everything is fp64, sums sequential in
 * index order. The statistics lse_i and D_i of a head are computed from a
 * materialised score row, as the forward oracle does, before the gradient rows.
 *
 * Threads (pthreads) split independent rows.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *dout;
    long B, H, Hkv, N, d;
    int causal;
    double scale;
    const int *kv_len;     /* [B] valid keys per batch (clamped to [0, N]), or NULL: all N */
    double *lse, *D;       /* [B*H*N]: statistics of every query row of the needed heads */
    const long *items;     /* work items of the current phase */
    long n_items;
    double *out0, *out1, *out2;
} ctx_t;

typedef struct {
    const ctx_t *C;
    void (*fn)(const ctx_t *, long, double *);
    long first, stride;
    int status;
} job_t;

/* valid keys of batch b: the prefix j < L_b */
static long len_of(const ctx_t *C, long b) {
    if (!C->kv_len) return C->N;
    const long L = C->kv_len[b];
    return L < 0 ? 0 : (L > C->N ? C->N : L);
}

/* visible keys of query row i of batch b: j < nvis_of (causal: j <= i; key padding: j < L_b) */
static long nvis_of(const ctx_t *C, long b, long i) {
    const long n = (C->causal && i + 1 < C->N) ? i + 1 : C->N, L = len_of(C, b);
    return n < L ? n : L;
}

static double dot(const float *a, const float *b, long d) {
    double s = 0.0;
    for (long c = 0; c < d; ++c) s += (double)a[c] * (double)b[c];
    return s;
}

/* Phase 1, item = flat query row (b*H + h)*N + i: lse_i and D_i = dO_i . o_i. */
static void row_stats(const ctx_t *C, long fr, double *s) {
    const long N = C->N, d = C->d, bh = fr / N, i = fr % N, b = bh / C->H, h = bh % C->H;
    const long g = h / (C->H / C->Hkv);
    const float *qi = C->q + fr * d, *doi = C->dout + fr * d;
    const float *kh = C->k + (b * C->Hkv + g) * N * d, *vh = C->v + (b * C->Hkv + g) * N * d;
    const long nv = nvis_of(C, b, i);
    if (nv == 0) { /* the empty softmax: o_i = 0, lse_i = ln 0 */
        C->lse[fr] = -INFINITY;
        C->D[fr] = 0.0;
        return;
    }
    double m = -INFINITY, l = 0.0;
    for (long j = 0; j < nv; ++j) {
        s[j] = C->scale * dot(qi, kh + j * d, d);
        if (s[j] > m) m = s[j];
    }
    for (long j = 0; j < nv; ++j) l += exp(s[j] - m);
    const double lse = m + log(l);
    /* D_i = sum_c dO_ic o_ic with o_i = sum_j p_ij v_j */
    double D = 0.0;
    for (long c = 0; c < d; ++c) {
        double oc = 0.0;
        for (long j = 0; j < nv; ++j) oc += exp(s[j] - lse) * (double)vh[j * d + c];
        D += (double)doi[c] * oc;
    }
    C->lse[fr] = lse;
    C->D[fr] = D;
}

/* Phase 2, item = index r into the query-row list: dq of that row into out0[r*d ..]. */
static void dq_row(const ctx_t *C, long r, double *unused) {
    (void)unused;
    const long N = C->N, d = C->d, fr = C->items[r], bh = fr / N, i = fr % N, b = bh / C->H, h = bh % C->H;
    const long g = h / (C->H / C->Hkv);
    const float *qi = C->q + fr * d, *doi = C->dout + fr * d;
    const float *kh = C->k + (b * C->Hkv + g) * N * d, *vh = C->v + (b * C->Hkv + g) * N * d;
    double *dq = C->out0 + r * d;
    for (long c = 0; c < d; ++c) dq[c] = 0.0;
    for (long j = 0; j < nvis_of(C, b, i); ++j) {
        const double p = exp(C->scale * dot(qi, kh + j * d, d) - C->lse[fr]);
        const double ds = p * (dot(doi, vh + j * d, d) - C->D[fr]);
        for (long c = 0; c < d; ++c) dq[c] += C->scale * ds * (double)kh[j * d + c];
    }
}

/* Phase 3, item = index r into the key-row list, flat key row (b*Hkv + g)*N + j: dk, dv into out1, out2. */
static void dkdv_row(const ctx_t *C, long r, double *unused) {
    (void)unused;
    const long N = C->N, d = C->d, fk = C->items[r], bg = fk / N, j = fk % N, b = bg / C->Hkv, g = bg % C->Hkv;
    const long group = C->H / C->Hkv;
    const float *kj = C->k + fk * d, *vj = C->v + fk * d;
    double *dk = C->out1 + r * d, *dv = C->out2 + r * d;
    for (long c = 0; c < d; ++c) dk[c] = dv[c] = 0.0;
    if (j >= len_of(C, b)) return; /* a padded key is visible to no query */
    for (long h = g * group; h < (g + 1) * group; ++h) {
        const long bh = b * C->H + h;
        for (long i = C->causal ? j : 0; i < N; ++i) { /* queries that see key j */
            const long fr = bh * N + i;
            const float *qi = C->q + fr * d, *doi = C->dout + fr * d;
            const double p = exp(C->scale * dot(qi, kj, d) - C->lse[fr]);
            const double ds = p * (dot(doi, vj, d) - C->D[fr]);
            for (long c = 0; c < d; ++c) {
                dk[c] += C->scale * ds * (double)qi[c];
                dv[c] += p * (double)doi[c];
            }
        }
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->C->N);
    if (!s) {
        J->status = 2;
        return NULL;
    }
    for (long r = J->first; r < J->C->n_items; r += J->stride) J->fn(J->C, r, s);
    free(s);
    J->status = 0;
    return NULL;
}

static int parallel_for(const ctx_t *C, void (*fn)(const ctx_t *, long, double *), int threads) {
    if (threads > C->n_items) threads = C->n_items > 0 ? (int)C->n_items : 1;
    job_t *jobs = (job_t *)calloc((size_t)threads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 2;
    }
    for (int t = 0; t < threads; ++t) {
        job_t j = {C, fn, t, threads, 0};
        jobs[t] = j;
    }
    for (int t = 1; t < threads; ++t)
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) jobs[t].status = -1;
    worker(&jobs[0]);
    int rc = 0;
    for (int t = 1; t < threads; ++t) {
        if (jobs[t].status == -1) {
            worker(&jobs[t]);
            continue;
        }
        pthread_join(tids[t], NULL);
    }
    for (int t = 0; t < threads; ++t)
        if (jobs[t].status) rc = jobs[t].status;
    free(jobs);
    free(tids);
    return rc;
}

/* Item (index into the per-row item function) for phase 1 uses the flat row itself: wrap it. */
static void row_stats_item(const ctx_t *C, long r, double *s) { row_stats(C, C->items[r], s); }

/*
 * oracle_attn_bwd_rows: gradients of the attention forward for listed rows.
 *   q, dout : [B, H, N, d] fp32;  k, v : [B, Hkv, N, d] fp32 (Hkv divides H)
 *   q_rows  : n_q flat query rows (b*H + h)*N + i  -> dq [n_q, d]
 *   kv_rows : n_kv flat key rows (b*Hkv + g)*N + j -> dk, dv [n_kv, d]
 *   (NULL with n = the full count: every row in order)
 *   kv_len  : [B] valid keys per batch (clamped to [0, N]), or NULL for all N
 * Returns 0 on success, 1 on a bad argument, 2 when memory runs out.
 */
int oracle_attn_bwd_rows(const float *q, const float *k, const float *v, const float *dout, long B, long H, long Hkv,
                         long N, long d, int causal, double scale, const int *kv_len, const long *q_rows, long n_q,
                         const long *kv_rows, long n_kv, double *dq, double *dk, double *dv, int threads) {
    if (!q || !k || !v || !dout || B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || N < 1 || d < 1 || threads < 1 ||
        n_q < 0 || n_kv < 0 || (n_q && !dq) || (n_kv && (!dk || !dv)))
        return 1;
    if ((!q_rows && n_q && n_q != B * H * N) || (!kv_rows && n_kv && n_kv != B * Hkv * N)) return 1;
    for (long r = 0; q_rows && r < n_q; ++r)
        if (q_rows[r] < 0 || q_rows[r] >= B * H * N) return 1;
    for (long r = 0; kv_rows && r < n_kv; ++r)
        if (kv_rows[r] < 0 || kv_rows[r] >= B * Hkv * N) return 1;

    const long group = H / Hkv, rows = B * H * N;
    char *need = (char *)calloc((size_t)(B * H), 1);
    double *lse = (double *)malloc(sizeof(double) * (size_t)rows);
    double *D = (double *)malloc(sizeof(double) * (size_t)rows);
    long *items = (long *)malloc(sizeof(long) * (size_t)(rows + n_q + n_kv + 1));
    if (!need || !lse || !D || !items) {
        free(need), free(lse), free(D), free(items);
        return 2;
    }
    /* heads whose statistics are needed: those of the query rows, and every query head of a key row's group */
    for (long r = 0; r < n_q; ++r) need[(q_rows ? q_rows[r] : r) / N] = 1;
    for (long r = 0; r < n_kv; ++r) {
        const long bg = (kv_rows ? kv_rows[r] : r) / N, b = bg / Hkv, g = bg % Hkv;
        for (long h = g * group; h < (g + 1) * group; ++h) need[b * H + h] = 1;
    }
    ctx_t C = {q, k, v, dout, B, H, Hkv, N, d, causal, scale, kv_len, lse, D, items, 0, dq, dk, dv};
    int rc = 0;
    /* phase 1: statistics of every row of the needed heads */
    for (long bh = 0; bh < B * H; ++bh)
        if (need[bh])
            for (long i = 0; i < N; ++i) items[C.n_items++] = bh * N + i;
    rc = parallel_for(&C, row_stats_item, threads);
    /* phase 2: dq rows */
    if (!rc && n_q) {
        for (long r = 0; r < n_q; ++r) items[r] = q_rows ? q_rows[r] : r;
        C.n_items = n_q;
        rc = parallel_for(&C, dq_row, threads);
    }
    /* phase 3: dk, dv rows */
    if (!rc && n_kv) {
        for (long r = 0; r < n_kv; ++r) items[r] = kv_rows ? kv_rows[r] : r;
        C.n_items = n_kv;
        rc = parallel_for(&C, dkdv_row, threads);
    }
    free(need), free(lse), free(D), free(items);
    return rc;
}
