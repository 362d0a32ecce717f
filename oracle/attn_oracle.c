/*
 * attn_oracle.c -- plain fp64 CPU oracle for the exact attention forward.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code. It shares no code
 * with the GPU path and the GPU path never calls it.
 *
 * What it computes is the plain definition of attention as the unite.ai page
 * ("Flash Attention: revolutionizing transformer efficiency") states it in its
 * opening code block and in "The Math Behind Flash Attention", item 1 (softmax
 * with the row maximum subtracted): for every batch b, head h and query row i,
 *
 *   s_ij   = scale * sum_c q[b,h,i,c] * k[b,g,j,c]      for j in J_i
 *   J_i    = {j : j < L_b}, and j <= i as well when causal
 *   m_i    = max_{j in J_i} s_ij
 *   l_i    = sum_{j in J_i} exp(s_ij - m_i)
 *   p_ij   = exp(s_ij - m_i) / l_i          (0 for j outside J_i)
 *   o_ic   = sum_j p_ij * v[b,g,j,c]
 *   lse_i  = m_i + ln(l_i)
 * and, when J_i is empty (only possible with L_b = 0), o_i = 0 and lse_i = -inf
 * (the log of an empty sum).
 *
 * g is the key/value head of query head h. With as many key/value heads as
 * query heads (Hkv = H) g = h; with fewer (grouped-query attention, Hkv
 * dividing H; multi-query attention, Hkv = 1) the H/Hkv consecutive query heads
 * h of a group share head g = h / (H/Hkv). The unite.ai page lists grouped and
 * multi-query attention among the FlashAttention-2 improvements (section
 * "FlashAttention-2", item 3) without defining the grouping; consecutive
 * grouping is a reading.
 *
 * L_b is the number of valid keys of batch b (a key-padding mask whose valid
 * keys are a prefix, as right padding makes): keys j >= L_b are invisible to
 * every query of that batch. Without lengths L_b = Nk. The mask itself appears
 * only as a usage example (triton-transformer README, "ex. BERT": a boolean
 * (batch, seq) mask passed to the model); the prefix form is a reading.
 *
 * The causal rule j <= i is a reading: the pages only say "causal" and
 * "triangular" (triton-transformer README, usage and to-do list). lse is the
 * natural-log form of the running statistics M and L of the blockwise code on
 * the unite.ai page ("Implementation Details").
 *
 * Everything is fp64. Inputs arrive as fp32 arrays (every bf16 and fp32 input
 * value is exact in fp32) and are widened to double exactly. The row s_i. of
 * the score matrix is materialised in full before the softmax, as the
 * definition does; sums run sequentially in index order. No blocking, no
 * online softmax, no BLAS.
 *
 * Threads (pthreads) split the list of rows; each row is independent.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v;
    long B, H, Hkv, Nq, Nk, d;
    int causal;
    double scale;
    const long *kv_len; /* NULL: every batch has Nk valid keys */
    const long *rows; /* NULL: row r of the output is flat row r */
    long n_rows;
    double *o, *lse;
    long first, stride; /* this thread handles r = first, first+stride, ... */
    int status;
} job_t;

/* One query row: flat index fr = (b*H + h)*Nq + i. Writes o_out[0..d) and *lse_out. */
static int one_row(const job_t *J, long fr, double *s, double *o_out, double *lse_out) {
    const long Nq = J->Nq, Nk = J->Nk, d = J->d;
    const long bh = fr / Nq, i = fr % Nq;
    const long b = bh / J->H, h = bh % J->H;
    const long g = h / (J->H / J->Hkv); /* key/value head of query head h */
    const float *qi = J->q + fr * d;
    const float *kh = J->k + (b * J->Hkv + g) * Nk * d;
    const float *vh = J->v + (b * J->Hkv + g) * Nk * d;
    /* J_i = {0 .. nvis-1}: keys below L_b, and up to i when causal */
    long nvis = J->kv_len ? J->kv_len[b] : Nk;
    if (J->causal && i + 1 < nvis) nvis = i + 1;

    if (nvis == 0) { /* empty softmax */
        for (long c = 0; c < d; ++c) o_out[c] = 0.0;
        *lse_out = -INFINITY;
        return 0;
    }

    /* s_ij for every visible key */
    for (long j = 0; j < nvis; ++j) {
        const float *kj = kh + j * d;
        double dot = 0.0;
        for (long c = 0; c < d; ++c) dot += (double)qi[c] * (double)kj[c];
        s[j] = J->scale * dot;
    }
    /* m_i */
    double m = -INFINITY;
    for (long j = 0; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    /* l_i and the unnormalised weights exp(s_ij - m_i) */
    double l = 0.0;
    for (long j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* p_ij and o_i */
    for (long c = 0; c < d; ++c) o_out[c] = 0.0;
    for (long j = 0; j < nvis; ++j) {
        const double p = s[j] / l;
        const float *vj = vh + j * d;
        for (long c = 0; c < d; ++c) o_out[c] += p * (double)vj[c];
    }
    *lse_out = m + log(l);
    return 0;
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->Nk);
    if (!s) {
        J->status = 2;
        return NULL;
    }
    for (long r = J->first; r < J->n_rows; r += J->stride) {
        const long fr = J->rows ? J->rows[r] : r;
        one_row(J, fr, s, J->o + r * J->d, J->lse + r);
    }
    free(s);
    J->status = 0;
    return NULL;
}

/*
 * oracle_attn_rows_ex: attention forward for a list of query rows.
 *   q       : [B, H, Nq, d] fp32, contiguous;  k, v : [B, Hkv, Nk, d] fp32, contiguous
 *             (the attention problems of interest have Nq == Nk; Nq != Nk serves the key-block tests)
 *   Hkv     : key/value heads, dividing H (query head h reads key/value head h / (H / Hkv))
 *   causal  : key j visible to query i iff j <= i
 *   kv_len  : B valid-key counts in [0, Nk] (keys j >= kv_len[b] are masked), or NULL (all Nk keys valid)
 *   rows    : n_rows flat row ids (b*H + h)*Nq + i, or NULL for all B*H*Nq rows in order
 *   o       : [n_rows, d] fp64 out;  lse : [n_rows] fp64 out
 *   threads : worker threads (>= 1)
 * Returns 0 on success, 1 on a bad argument, 2 when memory runs out.
 */
int oracle_attn_rows_ex(const float *q, const float *k, const float *v, long B, long H, long Hkv, long Nq, long Nk,
                        long d, int causal, double scale, const long *kv_len, const long *rows, long n_rows,
                        double *o, double *lse, int threads) {
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || n_rows < 0 || threads < 1)
        return 1;
    if (Hkv < 1 || H % Hkv != 0) return 1;
    if (kv_len)
        for (long b = 0; b < B; ++b)
            if (kv_len[b] < 0 || kv_len[b] > Nk) return 1;
    if (!rows && n_rows != B * H * Nq) return 1;
    if (rows)
        for (long r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= B * H * Nq) return 1;
    if (threads > n_rows) threads = n_rows > 0 ? (int)n_rows : 1;

    job_t *jobs = (job_t *)calloc((size_t)threads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 2;
    }
    for (int t = 0; t < threads; ++t) {
        job_t j = {q, k, v, B, H, Hkv, Nq, Nk, d, causal, scale, kv_len, rows, n_rows, o, lse, t, threads, 0};
        jobs[t] = j;
    }
    int rc = 0;
    for (int t = 1; t < threads; ++t)
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) jobs[t].status = -1;
    worker(&jobs[0]);
    for (int t = 1; t < threads; ++t) {
        if (jobs[t].status == -1) { /* thread did not start: do its share here */
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

/* oracle_attn_rows: oracle_attn_rows_ex with one key/value head per query head and no key-padding mask. */
int oracle_attn_rows(const float *q, const float *k, const float *v, long B, long H, long Nq, long Nk, long d,
                     int causal, double scale, const long *rows, long n_rows, double *o, double *lse, int threads) {
    return oracle_attn_rows_ex(q, k, v, B, H, H, Nq, Nk, d, causal, scale, NULL, rows, n_rows, o, lse, threads);
}
