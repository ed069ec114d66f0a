/*
 * CPU oracle for MLA varlen prefill attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is read by the tests, by the smoke
 * check and by the CPU-baseline leg of the benchmark; the product library
 * never links, loads or calls it, and it shares no code with the HIP path.
 *
 * What it computes follows the Ascend Transformer Boost "MLA Prefill" C API
 * page (Definition and the AtbMLAPreFillGetWorkspaceSize Members table):
 *   - Q / QRope / K / kRope / V rows: a query head carries a nope part of
 *     embeddimV elements and a separate 64-element rope part (rows Q, QRope,
 *     K, kRope, V of the Members table);
 *   - qkScale multiplies the whole query-key product (row qkScale), read here
 *     as covering the rope part too;
 *   - the mask is additive and applied after scaling (rows Mask, maskType);
 *   - causal masks are aligned bottom-right when qSeqLen < kvSeqLen;
 *   - maskType MASK_FREE takes one 512 x 512 tile (row Mask) that is placed
 *     on the diagonal 512-blocks of key-position space: blocks left of the
 *     diagonal are fully visible, blocks right of it fully masked.
 * A row that sees no key at all returns zeros (the page is silent there).
 *
 * Precision: every input element arrives as a double converted exactly from
 * its fp16/bf16 value; all arithmetic is IEEE double, summed in index order,
 * with libm exp(). Nothing is blocked, fused or reordered: each output row is
 * the textbook softmax(scale * q.k + mask) . V written out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Mask-type codes. The page names the modes but prints no integer values;
 * these are the values this project assigns. */
#define ORACLE_MASK_UNDEFINED 0
#define ORACLE_MASK_SPEC 1
#define ORACLE_MASK_CAUSAL 2
#define ORACLE_MASK_FREE 3

#define ORACLE_TILE 512

/* Additive mask entry for the query at key-position p and key j. */
static double mask_entry(int mask_type, long p, long j, const double *tile)
{
    if (mask_type == ORACLE_MASK_UNDEFINED)
        return 0.0;                                   /* all-0 mask */
    if (mask_type == ORACLE_MASK_SPEC || mask_type == ORACLE_MASK_CAUSAL)
        return (j <= p) ? 0.0 : -INFINITY;            /* key visible iff not in the future */
    /* ORACLE_MASK_FREE: the 512 x 512 tile repeated along the diagonal. */
    if (p < 0)
        return -INFINITY;
    long row_block = p / ORACLE_TILE;
    long col_block = j / ORACLE_TILE;
    if (col_block < row_block)
        return 0.0;
    if (col_block > row_block)
        return -INFINITY;
    return tile[(p % ORACLE_TILE) * ORACLE_TILE + (j % ORACLE_TILE)];
}

/*
 * One (sequence, query head) pair.
 *   q    [qlen, d_nope]     query nope part
 *   qr   [qlen, d_rope]     query rope part
 *   k    [kvlen, d_nope]    key nope part of the kv head this query head reads
 *   kr   [kvlen, d_rope]    key rope part
 *   v    [kvlen, d_v]       values
 *   rows [n_rows]           query rows (0 <= i < qlen) to evaluate
 *   out  [n_rows, d_v]      attention output for those rows
 *   weights [n_rows, kvlen] optional (NULL to skip): the softmax weights
 *   tile [512, 512]         only read for ORACLE_MASK_FREE
 * Query row i sits at key position p = kvlen - qlen + i.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention_head(const double *q, const double *qr, const double *k,
                          const double *kr, const double *v, long qlen, long kvlen,
                          int d_nope, int d_rope, int d_v, double scale, int mask_type,
                          const double *tile, const long *rows, long n_rows,
                          double *out, double *weights)
{
    if (qlen < 0 || kvlen < 0 || d_nope < 0 || d_rope < 0 || d_v < 0)
        return -1;
    if (mask_type == ORACLE_MASK_FREE && tile == NULL)
        return -1;
    if (mask_type < ORACLE_MASK_UNDEFINED || mask_type > ORACLE_MASK_FREE)
        return -1;
    for (long r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= qlen)
            return -1;

    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long r = 0; r < n_rows; ++r) {
        long i = rows[r];
        long p = kvlen - qlen + i;
        double *s = (double *)malloc(sizeof(double) * (size_t)(kvlen > 0 ? kvlen : 1));
        if (s == NULL) {
            failed = 1;
            continue;
        }
        /* scores: s_j = scale * (q_i . k_j + qr_i . kr_j) + m(p, j) */
        double row_max = -INFINITY;
        for (long j = 0; j < kvlen; ++j) {
            double dot = 0.0;
            for (int d = 0; d < d_nope; ++d)
                dot += q[i * d_nope + d] * k[j * d_nope + d];
            for (int d = 0; d < d_rope; ++d)
                dot += qr[i * d_rope + d] * kr[j * d_rope + d];
            double m = mask_entry(mask_type, p, j, tile);
            s[j] = (m == -INFINITY) ? -INFINITY : scale * dot + m;
            if (s[j] > row_max)
                row_max = s[j];
        }
        double *o = out + r * d_v;
        for (int d = 0; d < d_v; ++d)
            o[d] = 0.0;
        if (kvlen == 0 || row_max == -INFINITY) {
            /* no visible key: the row is defined as zeros */
            if (weights)
                for (long j = 0; j < kvlen; ++j)
                    weights[r * kvlen + j] = 0.0;
            free(s);
            continue;
        }
        /* softmax numerators e_j = exp(s_j - max) and their sum */
        double denom = 0.0;
        for (long j = 0; j < kvlen; ++j) {
            s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - row_max);
            denom += s[j];
        }
        /* O_i = sum_j (e_j / denom) v_j */
        for (long j = 0; j < kvlen; ++j) {
            double w = s[j] / denom;
            if (weights)
                weights[r * kvlen + j] = w;
            for (int d = 0; d < d_v; ++d)
                o[d] += w * v[j * d_v + d];
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Threads of the parallel regions the calling thread starts from now on (its
 * OpenMP thread-count setting); n < 1 is ignored. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
