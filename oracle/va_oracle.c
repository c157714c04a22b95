/*
 * va_oracle.c -- plain fp64 CPU oracle for paged GQA target-verify attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  It shares no code,
 * header, table or helper with the HIP library; it is written directly from the
 * definition of the operation, slowly and obviously, in double precision.
 *
 * What it computes (sources, cited by page and section):
 *  - The call being modelled is the verify-attention wrapper of the sglang
 *    PR #36330 summary page ("Key source snippets": the aiter_backend.py gate
 *    and the test _check_matches_aiter).  Inputs: q [total_q, Hq, D] bf16,
 *    paged k/v pools [num_blocks, page, Hkv, D] (fp8 e4m3 or bf16),
 *    block_table [B, max_blocks_per_seq], cu_seqlens_q [B+1], seqused_k [B],
 *    softmax_scale, per-tensor k/v descale.
 *  - Attention is causal (the reference call passes causal=True, same
 *    section) and seqused_k already counts the verify tokens (the gate passes
 *    seq_lens + max_q_len), so the query block sits at the bottom-right of the
 *    key range: query token t of a sequence with Lq queries and Lk keys sees
 *    keys 0 .. Lk-Lq+t.
 *  - GQA: the number of query heads per kv head is Hq/Hkv (the gate's
 *    num_queries_per_kv); q head h reads kv head h / (Hq/Hkv).
 *  - Logits are scaled by softmax_scale * k_scale and masked keys get -inf
 *    (sglang PR #34517 summary page, "Key source snippets": the shared-KV verify
 *    kernel's inner loop).  The value descale multiplies the dequantised V.
 *  - Split mode: the method splits the key range into segments and merges the
 *    per-segment results (PR #36330 summary, "Implementation breakdown", item 1:
 *    segments plus a reduce-segments kernel).  The merge of softmax partials by
 *    log-sum-exp is exact algebra: with lse_s = log sum_{j in s} exp(s_j),
 *    O = sum_s exp(lse_s - lse) * o_s, lse = log sum_s exp(lse_s).
 *
 * Optional features, as the verify call of the PR #30105 summary page passes
 * them to the shared attention kernel ("Key source snippets": window_size,
 * softcap, sinks; the PR #36330 gate excludes all three):
 *  - sliding window: window_size = (window_left, 0), window_left = sliding
 *    window - 1; a query at absolute position i = Lk-Lq+t also needs key
 *    j >= i - window_left (keys i-window_left .. i).  -1 = no window;
 *  - logit softcap: s <- softcap * tanh(s / softcap) on the scaled logit
 *    (0 = off);
 *  - attention sinks: one logit per query head that joins the softmax
 *    denominator and carries no value: out = sum_j e^s_j V_j / (sum_j e^s_j
 *    + e^sink_h).
 * The pages name these features but do not define them; the readings above
 * are the ones their parameter names carry in common attention APIs.
 *
 * FP8 format: OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, S.1111.111 = NaN, subnormals m/8 * 2^-6).  The pages only say
 * "FP8 KV"; this is the e4m3 variant that gfx950 converts and multiplies natively.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codecs -- */

double va_oracle_fp8e4m3fn_to_double(uint8_t x)
{
    int sign = (x >> 7) & 1;
    int e = (x >> 3) & 0xF;
    int m = x & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);            /* subnormal */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);   /* normal, bias 7 */
    return sign ? -v : v;
}

double va_oracle_bf16_to_double(uint16_t x)
{
    /* bf16 is the top half of an IEEE binary32 */
    uint32_t u = (uint32_t)x << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------- the problem -- */

typedef struct {
    const uint16_t *q;          /* [total_q, Hq, D] bf16 bits */
    const void *k_pool;         /* [num_blocks, page, Hkv, D] */
    const void *v_pool;
    int kv_is_fp8;              /* 1: fp8 e4m3fn bytes, 0: bf16 bits */
    const int32_t *block_table; /* [B, bt_stride] */
    int64_t bt_stride;
    const int32_t *cu_seqlens_q;/* [B+1] */
    const int32_t *seqused_k;   /* [B] */
    int num_seqs, num_q_heads, num_kv_heads, head_dim, page_size;
    double scale, k_descale, v_descale;
    int window_left;            /* -1: no sliding window */
    double softcap;             /* 0: no logit softcap */
    const double *sinks;        /* [Hq] sink logits, or NULL */
    /* split mode (optional): segments of sequence b are
     * seg_start[seg_ptr[b] .. seg_ptr[b+1]), each running to the next start
     * (or to seqused_k[b] for the last one).  NULL = one segment. */
    const int32_t *seg_start;
    const int32_t *seg_ptr;
    /* rows to compute: flat (q_row * Hq + head) indices, or NULL = all */
    const int64_t *rows;
    int64_t n_rows;
    double *out;                /* [n_rows, D] */
    double *lse;                /* [n_rows]   natural-log LSE of the scaled logits */
} va_oracle_problem;

/* the 256 fp8 codes decoded once by the function above (filled before any
 * worker thread starts; only a cache of va_oracle_fp8e4m3fn_to_double) */
static double fp8_value[256];

static double kv_at(const va_oracle_problem *p, const void *pool, int64_t idx)
{
    if (p->kv_is_fp8)
        return fp8_value[((const uint8_t *)pool)[idx]];
    return va_oracle_bf16_to_double(((const uint16_t *)pool)[idx]);
}

/* element offset of (key j of sequence b, kv head g, dim 0) in a pool */
static int64_t kv_row(const va_oracle_problem *p, int b, int64_t j, int g)
{
    int64_t page = p->block_table[(int64_t)b * p->bt_stride + j / p->page_size];
    int64_t slot = j % p->page_size;
    return ((page * p->page_size + slot) * p->num_kv_heads + g) * p->head_dim;
}

/*
 * Softmax statistics of one query row over the keys [lo, hi) (already clipped
 * to the visible range): m = max logit, L = sum exp(s - m),
 * acc[d] = sum exp(s - m) * V[d].  Returns the number of keys used.
 */
static int64_t row_segment(const va_oracle_problem *p, int b, int g,
                           const uint16_t *qrow, int64_t lo, int64_t hi,
                           double *m_out, double *L_out, double *acc,
                           double *logits)
{
    const int D = p->head_dim;
    int64_t n = hi - lo, j;
    int d;
    double m = -INFINITY, L = 0.0;
    for (d = 0; d < D; ++d)
        acc[d] = 0.0;
    if (n <= 0) {
        *m_out = -INFINITY;
        *L_out = 0.0;
        return 0;
    }
    for (j = 0; j < n; ++j) {
        int64_t base = kv_row(p, b, lo + j, g);
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += va_oracle_bf16_to_double(qrow[d]) * kv_at(p, p->k_pool, base + d);
        logits[j] = p->scale * p->k_descale * dot;
        if (p->softcap > 0.0)
            logits[j] = p->softcap * tanh(logits[j] / p->softcap);
        if (logits[j] > m)
            m = logits[j];
    }
    for (j = 0; j < n; ++j) {
        int64_t base = kv_row(p, b, lo + j, g);
        double w = exp(logits[j] - m);
        L += w;
        for (d = 0; d < D; ++d)
            acc[d] += w * kv_at(p, p->v_pool, base + d);
    }
    *m_out = m;
    *L_out = L;
    return n;
}

/* locate the sequence that owns q row qr (cu_seqlens_q is a prefix sum) */
static int seq_of_row(const va_oracle_problem *p, int64_t qr)
{
    int b;
    for (b = 0; b < p->num_seqs; ++b)
        if (qr >= p->cu_seqlens_q[b] && qr < p->cu_seqlens_q[b + 1])
            return b;
    return -1;
}

static int compute_row(const va_oracle_problem *p, int64_t flat, double *out,
                       double *lse, double *acc, double *acc2, double *logits)
{
    const int D = p->head_dim;
    const int G = p->num_q_heads / p->num_kv_heads;
    int64_t qr = flat / p->num_q_heads;
    int h = (int)(flat % p->num_q_heads);
    int b = seq_of_row(p, qr);
    int g = h / G, d;
    int64_t Lq, Lk, t, visible, first;
    double sink = -INFINITY;
    const uint16_t *qrow = p->q + flat * D;
    if (b < 0)
        return -1;
    Lq = p->cu_seqlens_q[b + 1] - p->cu_seqlens_q[b];
    Lk = p->seqused_k[b];
    t = qr - p->cu_seqlens_q[b];
    visible = Lk - Lq + t + 1;          /* keys 0 .. Lk-Lq+t (bottom-right causal) */
    if (visible > Lk)
        visible = Lk;
    first = 0;                          /* sliding window: keys from i - window_left on */
    if (p->window_left >= 0 && visible - 1 - p->window_left > 0)
        first = visible - 1 - p->window_left;
    if (p->sinks)
        sink = p->sinks[h];

    if (p->seg_start == NULL) {
        double m, L;
        row_segment(p, b, g, qrow, first, visible, &m, &L, acc, logits);
        if (sink > -INFINITY) {         /* the sink joins the denominator only */
            double mm = m > sink ? m : sink;
            double f = L > 0.0 ? exp(m - mm) : 0.0;
            L = L * f + exp(sink - mm);
            for (d = 0; d < D; ++d)
                acc[d] *= f;
            m = mm;
        }
        if (L > 0.0) {
            for (d = 0; d < D; ++d)
                out[d] = p->v_descale * acc[d] / L;
            *lse = m + log(L);
        } else {
            for (d = 0; d < D; ++d)
                out[d] = 0.0;
            *lse = -INFINITY;
        }
        return 0;
    }

    /* split mode: per-segment (lse_s, o_s), then the log-sum-exp merge */
    {
        int32_t s0 = p->seg_ptr[b], s1 = p->seg_ptr[b + 1], s;
        double lse_max = -INFINITY, denom = 0.0;
        double *seg_lse = (double *)malloc(sizeof(double) * (size_t)(s1 - s0 + 1));
        double *seg_o = (double *)malloc(sizeof(double) * (size_t)(s1 - s0 + 1) * D);
        if (!seg_lse || !seg_o) {
            free(seg_lse);
            free(seg_o);
            return -2;
        }
        for (s = s0; s < s1; ++s) {
            int64_t lo = p->seg_start[s];
            int64_t hi = (s + 1 < s1) ? p->seg_start[s + 1] : Lk;
            double m, L;
            if (hi > visible)
                hi = visible;
            if (lo < first)
                lo = first;
            row_segment(p, b, g, qrow, lo, hi, &m, &L, acc, logits);
            if (L > 0.0) {
                seg_lse[s - s0] = m + log(L);
                for (d = 0; d < D; ++d)
                    seg_o[(int64_t)(s - s0) * D + d] = acc[d] / L;
            } else {                        /* no visible key: weight zero */
                seg_lse[s - s0] = -INFINITY;
                for (d = 0; d < D; ++d)
                    seg_o[(int64_t)(s - s0) * D + d] = 0.0;
            }
            if (seg_lse[s - s0] > lse_max)
                lse_max = seg_lse[s - s0];
        }
        if (sink > lse_max)
            lse_max = sink;
        for (d = 0; d < D; ++d)
            acc2[d] = 0.0;
        if (lse_max > -INFINITY) {
            for (s = s0; s < s1; ++s) {
                double w = exp(seg_lse[s - s0] - lse_max);
                denom += w;
                for (d = 0; d < D; ++d)
                    acc2[d] += w * seg_o[(int64_t)(s - s0) * D + d];
            }
            if (sink > -INFINITY)       /* the sink joins the denominator once */
                denom += exp(sink - lse_max);
            for (d = 0; d < D; ++d)
                out[d] = p->v_descale * acc2[d] / denom;
            *lse = lse_max + log(denom);
        } else {
            for (d = 0; d < D; ++d)
                out[d] = 0.0;
            *lse = -INFINITY;
        }
        free(seg_lse);
        free(seg_o);
    }
    return 0;
}

typedef struct {
    const va_oracle_problem *p;
    int64_t begin, end, max_keys;
    int status;
} worker_arg;

static void *worker(void *vp)
{
    worker_arg *a = (worker_arg *)vp;
    const va_oracle_problem *p = a->p;
    const int D = p->head_dim;
    double *acc = (double *)malloc(sizeof(double) * D);
    double *acc2 = (double *)malloc(sizeof(double) * D);
    double *logits = (double *)malloc(sizeof(double) * (size_t)(a->max_keys + 1));
    int64_t i;
    a->status = 0;
    if (!acc || !acc2 || !logits) {
        a->status = -2;
    } else {
        for (i = a->begin; i < a->end && a->status == 0; ++i) {
            int64_t flat = p->rows ? p->rows[i] : i;
            a->status = compute_row(p, flat, p->out + i * D, p->lse + i, acc, acc2, logits);
        }
    }
    free(acc);
    free(acc2);
    free(logits);
    return NULL;
}

/*
 * Exported entry.  Returns 0 on success, -1 on a row that belongs to no
 * sequence, -2 on allocation failure, -3 on bad arguments, -4 when a
 * sequence has more query tokens than keys (q_len > seqused_k).  seqused_k
 * counts the verify tokens themselves (the PR #36330 summary page's gate
 * passes seq_lens + max_q_len), so such a call is outside the operation's
 * domain and has no defined result.
 * window_left: -1 or >= 0; softcap: 0 or > 0; sinks: NULL or [num_q_heads].
 */
int va_oracle_attn_ex(const uint16_t *q, const void *k_pool, const void *v_pool,
                      int kv_is_fp8, const int32_t *block_table, int64_t bt_stride,
                      const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                      int num_seqs, int num_q_heads, int num_kv_heads,
                      int head_dim, int page_size, double scale,
                      double k_descale, double v_descale,
                      int window_left, double softcap, const double *sinks,
                      const int32_t *seg_start, const int32_t *seg_ptr,
                      const int64_t *rows, int64_t n_rows,
                      double *out, double *lse, int num_threads)
{
    va_oracle_problem p;
    pthread_t *th;
    worker_arg *args;
    int64_t max_keys = 0, per;
    int b, i, status = 0;
    if (!q || !k_pool || !v_pool || !block_table || !cu_seqlens_q || !seqused_k ||
        !out || !lse || num_seqs < 1 || num_kv_heads < 1 || num_q_heads < 1 ||
        num_q_heads % num_kv_heads != 0 || head_dim < 1 || page_size < 1 || n_rows < 0)
        return -3;
    if ((seg_start == NULL) != (seg_ptr == NULL))
        return -3;
    if (window_left < -1 || !(softcap >= 0.0))
        return -3;
    for (b = 0; b < num_seqs; ++b)
        if (cu_seqlens_q[b + 1] - cu_seqlens_q[b] > seqused_k[b])
            return -4;
    p.q = q; p.k_pool = k_pool; p.v_pool = v_pool; p.kv_is_fp8 = kv_is_fp8;
    p.block_table = block_table; p.bt_stride = bt_stride;
    p.cu_seqlens_q = cu_seqlens_q; p.seqused_k = seqused_k;
    p.num_seqs = num_seqs; p.num_q_heads = num_q_heads; p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim; p.page_size = page_size;
    p.scale = scale; p.k_descale = k_descale; p.v_descale = v_descale;
    p.window_left = window_left; p.softcap = softcap; p.sinks = sinks;
    p.seg_start = seg_start; p.seg_ptr = seg_ptr;
    p.rows = rows; p.n_rows = n_rows; p.out = out; p.lse = lse;
    for (i = 0; i < 256; ++i)
        fp8_value[i] = va_oracle_fp8e4m3fn_to_double((uint8_t)i);
    for (b = 0; b < num_seqs; ++b)
        if (seqused_k[b] > max_keys)
            max_keys = seqused_k[b];
    if (num_threads < 1)
        num_threads = 1;
    if (num_threads > n_rows && n_rows > 0)
        num_threads = (int)n_rows;
    th = (pthread_t *)malloc(sizeof(pthread_t) * num_threads);
    args = (worker_arg *)malloc(sizeof(worker_arg) * num_threads);
    if (!th || !args) {
        free(th);
        free(args);
        return -2;
    }
    per = (n_rows + num_threads - 1) / (num_threads > 0 ? num_threads : 1);
    for (i = 0; i < num_threads; ++i) {
        args[i].p = &p;
        args[i].begin = (int64_t)i * per;
        args[i].end = args[i].begin + per < n_rows ? args[i].begin + per : n_rows;
        args[i].max_keys = max_keys;
        args[i].status = 0;
        pthread_create(&th[i], NULL, worker, &args[i]);
    }
    for (i = 0; i < num_threads; ++i) {
        pthread_join(th[i], NULL);
        if (args[i].status != 0)
            status = args[i].status;
    }
    free(th);
    free(args);
    return status;
}

/* The plain call: no window, softcap or sinks. */
int va_oracle_attn(const uint16_t *q, const void *k_pool, const void *v_pool,
                   int kv_is_fp8, const int32_t *block_table, int64_t bt_stride,
                   const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                   int num_seqs, int num_q_heads, int num_kv_heads,
                   int head_dim, int page_size, double scale,
                   double k_descale, double v_descale,
                   const int32_t *seg_start, const int32_t *seg_ptr,
                   const int64_t *rows, int64_t n_rows,
                   double *out, double *lse, int num_threads)
{
    return va_oracle_attn_ex(q, k_pool, v_pool, kv_is_fp8, block_table, bt_stride, cu_seqlens_q,
                             seqused_k, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                             scale, k_descale, v_descale, -1, 0.0, NULL, seg_start, seg_ptr, rows,
                             n_rows, out, lse, num_threads);
}
