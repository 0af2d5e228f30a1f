/*
 * fp64 CPU oracle for one decode step of shared-prefix attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg call it; the attention library never does.  It
 * shares no code, header or constant with the GPU path.
 *
 * What it computes.  The shared-prefix method is exact in real arithmetic
 * ("Hydragen: High-Throughput LLM Inference with Shared Prefixes", section
 * "Attention Decomposition Across Subsequences", Eq. 5 and the proof it
 * summarises; "Shared Prefix KV Caching, in depth", section "Splitting
 * attention at the prefix boundary").  So the oracle is the plain definition:
 * for each sequence b and query head h, with KV head g = h / (Hq / Hkv), over
 * the concatenation of all key segments that sequence attends (its prefix
 * nodes, root first, then its own suffix):
 *
 *     s_j = scale * sum_c q_c k_{j,c}                  (scaled dot product)
 *     m   = max_j s_j
 *     l   = sum_j exp(s_j - m)
 *     O   = (sum_j exp(s_j - m) v_j) / l               (softmax(s) V)
 *     LSE = m + ln l                                   (= ln sum_j exp(s_j))
 *
 * in double precision, reading each stored element exactly (fp32, fp16 and
 * bf16 all widen to double without rounding).  The max shift is the one
 * ChunkAttention applies inside a chunk ("ChunkAttention: Efficient
 * Self-Attention with Prefix-Aware KV Cache and Two-Phase Partition", section
 * "The partial_attn Function", Eq. 1, steps 2-5), here with a single chunk
 * holding every key.  An empty key list gives O = 0 and LSE = -inf.
 *
 * oracle_merge() combines given (O, LSE) partials by the two-part
 * recombination of the Hydragen page (section "Attention Decomposition Across
 * Subsequences", Eq. 5, in the max-subtracted form its combine_lse
 * description gives), applied left to right; the merged LSE of two parts is
 * max + ln(w1 + w2), the log of the summed denominators.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

typedef struct {
    const void *k;        /* key of token t, head g at k + t*stride_tok + g*stride_head */
    const void *v;        /* same layout as k */
    int64_t len;          /* tokens in this segment */
    int64_t stride_tok;   /* elements */
    int64_t stride_head;  /* elements; the d elements of one head are contiguous */
} oracle_segment;

typedef struct {
    int32_t B, Hq, Hkv, d;
    int32_t dtype;                 /* storage type of q, k and v */
    float scale;                   /* widened to double before use */
    const void *q;                 /* [B][Hq][d] */
    const int64_t *seg_begin;      /* [B+1]: segments of sequence b are segs[seg_begin[b] .. seg_begin[b+1]) */
    const oracle_segment *segs;
    const int64_t *rows;           /* optional subset of rows r = b*Hq + h (NULL: all rows) */
    int64_t nrows;                 /* length of rows[] (ignored when rows is NULL) */
} oracle_problem;

static double f16_bits_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* (1024 + m) * 2^(e - 15 - 10) */
    return sign ? -v : v;
}

static double bf16_bits_to_double(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double elem(const void *base, int64_t i, int dtype)
{
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[i];
    case ORACLE_F16: return f16_bits_to_double(((const uint16_t *)base)[i]);
    default:         return bf16_bits_to_double(((const uint16_t *)base)[i]);
    }
}

static int check_problem(const oracle_problem *p)
{
    if (!p || !p->q || !p->seg_begin || p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->d <= 0)
        return 1;
    if (p->Hq % p->Hkv) return 2;
    if (p->dtype < ORACLE_F32 || p->dtype > ORACLE_BF16) return 3;
    return 0;
}

/* One (b, h) row: the plain definition above. */
static void one_row(const oracle_problem *p, int64_t r, double *o, double *lse, double *qd,
                    double *acc)
{
    const int64_t b = r / p->Hq, h = r % p->Hq, g = h / (p->Hq / p->Hkv);
    const int d = p->d;
    const double scale = (double)p->scale;
    for (int c = 0; c < d; c++) qd[c] = elem(p->q, (b * p->Hq + h) * d + c, p->dtype);

    int64_t n = 0;
    for (int64_t s = p->seg_begin[b]; s < p->seg_begin[b + 1]; s++) n += p->segs[s].len;
    for (int c = 0; c < d; c++) o[c] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double *sc = (double *)malloc((size_t)n * sizeof(double));

    /* scores */
    int64_t j = 0;
    for (int64_t s = p->seg_begin[b]; s < p->seg_begin[b + 1]; s++) {
        const oracle_segment *sg = &p->segs[s];
        for (int64_t t = 0; t < sg->len; t++) {
            const int64_t base = t * sg->stride_tok + g * sg->stride_head;
            double dot = 0.0;
            for (int c = 0; c < d; c++) dot += qd[c] * elem(sg->k, base + c, p->dtype);
            sc[j++] = scale * dot;
        }
    }
    /* max, then exponentials, denominator and weighted sum of values */
    double m = -INFINITY;
    for (j = 0; j < n; j++)
        if (sc[j] > m) m = sc[j];
    double l = 0.0;
    for (int c = 0; c < d; c++) acc[c] = 0.0;
    j = 0;
    for (int64_t s = p->seg_begin[b]; s < p->seg_begin[b + 1]; s++) {
        const oracle_segment *sg = &p->segs[s];
        for (int64_t t = 0; t < sg->len; t++) {
            const int64_t base = t * sg->stride_tok + g * sg->stride_head;
            const double e = exp(sc[j++] - m);
            l += e;
            for (int c = 0; c < d; c++) acc[c] += e * elem(sg->v, base + c, p->dtype);
        }
    }
    for (int c = 0; c < d; c++) o[c] = acc[c] / l;
    *lse = m + log(l);
    free(sc);
}

/*
 * o: [nrows][d] (or [B*Hq][d] when rows is NULL); lse: [nrows].
 * nthreads <= 0 uses every core OpenMP sees.  Returns 0 on success.
 */
int oracle_attention(const oracle_problem *p, double *o, double *lse, int32_t nthreads)
{
    int err = check_problem(p);
    if (err) return err;
    if (!o || !lse) return 1;
    const int64_t nr = p->rows ? p->nrows : (int64_t)p->B * p->Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *qd = (double *)malloc((size_t)p->d * sizeof(double));
        double *acc = (double *)malloc((size_t)p->d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nr; i++) {
            const int64_t r = p->rows ? p->rows[i] : i;
            if (r < 0 || r >= (int64_t)p->B * p->Hq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            one_row(p, r, o + i * p->d, lse + i, qd, acc);
        }
        free(qd);
        free(acc);
    }
    return bad ? 4 : 0;
}

/*
 * Merge n partials per row.  o_in[i]: [rows][d], lse_in[i]: [rows] (natural
 * log; -inf marks an empty partial), given in double so that fp32 partials
 * widen exactly and fp64 partials lose nothing.  o: [rows][d], lse: [rows].
 */
int oracle_merge(int32_t n, int64_t rows, int32_t d, const double *const *o_in,
                 const double *const *lse_in, double *o, double *lse)
{
    if (n < 0 || rows < 0 || d <= 0 || (n > 0 && (!o_in || !lse_in)) || !o || !lse) return 1;
    for (int64_t r = 0; r < rows; r++) {
        double cur_lse = -INFINITY;
        double *cur_o = o + r * d;
        for (int c = 0; c < d; c++) cur_o[c] = 0.0;
        for (int32_t i = 0; i < n; i++) {
            const double l2 = lse_in[i][r];
            const double *o2 = o_in[i] + r * d;
            const double mx = cur_lse > l2 ? cur_lse : l2;
            if (mx == -INFINITY) continue;              /* both parts empty */
            const double w1 = exp(cur_lse - mx), w2 = exp(l2 - mx);
            for (int c = 0; c < d; c++)
                cur_o[c] = (w1 * cur_o[c] + w2 * o2[c]) / (w1 + w2);
            cur_lse = mx + log(w1 + w2);
        }
        lse[r] = cur_lse;
    }
    return 0;
}
