/*
 * paged_attn_oracle.c -- fp64 CPU oracle for paged GQA decode attention.
 *
 * TEST INFRASTRUCTURE (see paged_attn_oracle.h for the definition it follows
 * and the passages of the pages behind it).  Deliberately plain: every score
 * is materialised, the softmax is the textbook two-pass one, and all sums are
 * straightforward left-to-right fp64 loops.
 */
#include "paged_attn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* A bfloat16 value is the upper half of an IEEE-754 binary32; widening it to
 * binary32 and then to binary64 is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_validate(const oracle_shape *s, const int32_t *block_table,
                    const int32_t *context_lens)
{
    if (!s || s->num_seqs < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
        s->head_dim <= 0 || s->page_size <= 0 || s->num_pages < 0 || s->max_blocks < 0)
        return ORACLE_EINVAL;
    if (s->num_q_heads % s->num_kv_heads != 0)
        return ORACLE_EINVAL;
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        const int32_t n = context_lens[b];
        if (n < 0 || (int64_t)n > (int64_t)s->max_blocks * s->page_size)
            return ORACLE_EINVAL;
        const int32_t blocks = (n + s->page_size - 1) / s->page_size;
        for (int32_t j = 0; j < blocks; ++j) {
            const int32_t page = block_table[(size_t)b * s->max_blocks + j];
            if (page < 0 || page >= s->num_pages)
                return ORACLE_EINVAL;
        }
    }
    return ORACLE_OK;
}

int oracle_attend_one(const oracle_shape *s, const uint16_t *q,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_table, const int32_t *context_lens,
                      double scale, int32_t b, int32_t h,
                      double *out_row, double *lse)
{
    const int32_t dim = s->head_dim;
    const int32_t group = s->num_q_heads / s->num_kv_heads; /* query heads per KV head */
    const int32_t kv = h / group;                            /* the KV head query head h reads */
    const int32_t n = context_lens[b];
    const size_t slot_stride = (size_t)s->num_kv_heads * dim; /* elements from one slot to the next */
    const uint16_t *qh = q + ((size_t)b * s->num_q_heads + h) * dim;

    for (int32_t d = 0; d < dim; ++d)
        out_row[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return ORACLE_OK;
    }

    double *z = (double *)malloc((size_t)n * sizeof *z);
    const uint16_t **vrow = (const uint16_t **)malloc((size_t)n * sizeof *vrow);
    if (!z || !vrow) {
        free(z);
        free((void *)vrow);
        return ORACLE_ENOMEM;
    }

    /* Walk the block table in logical token order and score every token. */
    for (int32_t t = 0; t < n; ++t) {
        const int32_t page = block_table[(size_t)b * s->max_blocks + t / s->page_size];
        const int32_t slot = t % s->page_size;
        const size_t row = ((size_t)page * s->page_size + slot) * slot_stride + (size_t)kv * dim;
        const uint16_t *k = k_pool + row;
        vrow[t] = v_pool + row;
        double dot = 0.0;
        for (int32_t d = 0; d < dim; ++d)
            dot += bf16_value(qh[d]) * bf16_value(k[d]);
        z[t] = scale * dot;
    }

    /* Softmax weights, shifted by the maximum score so exp cannot overflow. */
    double m = -INFINITY;
    for (int32_t t = 0; t < n; ++t)
        if (z[t] > m)
            m = z[t];
    double l = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        z[t] = exp(z[t] - m);
        l += z[t];
    }

    /* Weighted sum of the value rows, then normalise. */
    for (int32_t t = 0; t < n; ++t)
        for (int32_t d = 0; d < dim; ++d)
            out_row[d] += z[t] * bf16_value(vrow[t][d]);
    for (int32_t d = 0; d < dim; ++d)
        out_row[d] /= l;
    *lse = m + log(l);

    free(z);
    free((void *)vrow);
    return ORACLE_OK;
}

int oracle_paged_attn(const oracle_shape *s, const uint16_t *q,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_table, const int32_t *context_lens,
                      double scale, double *out, double *lse)
{
    int rc = oracle_validate(s, block_table, context_lens);
    if (rc != ORACLE_OK)
        return rc;
    const int64_t pairs = (int64_t)s->num_seqs * s->num_q_heads;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < pairs; ++i) {
        const int32_t b = (int32_t)(i / s->num_q_heads);
        const int32_t h = (int32_t)(i % s->num_q_heads);
        int r = oracle_attend_one(s, q, k_pool, v_pool, block_table, context_lens, scale,
                                  b, h, out + (size_t)i * s->head_dim, lse + i);
        if (r != ORACLE_OK) {
#pragma omp critical
            err = r;
        }
    }
    return err;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
