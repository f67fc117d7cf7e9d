/*
 * prefill_attn_oracle.c -- fp64 CPU oracle for chunked-prefill paged attention.
 *
 * TEST INFRASTRUCTURE (see prefill_attn_oracle.h).  Each (row, head) is the
 * decode-step definition of paged_attn_oracle.c applied to that row's query
 * with the context cut at the row's own position: the row is passed as
 * request 0 of a one-request view whose table row is the request's and whose
 * context length is position + 1.
 */
#include "prefill_attn_oracle.h"

#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_prefill_validate(const oracle_shape *s, int32_t num_rows, const int32_t *new_start,
                            const int32_t *block_table, const int32_t *context_lens)
{
    if (!s || !new_start || num_rows < 0)
        return ORACLE_EINVAL;
    const int rc = oracle_validate(s, block_table, context_lens);
    if (rc != ORACLE_OK)
        return rc;
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        const int32_t start = new_start[b];
        const int32_t n = new_start[b + 1] - start;
        if (start < 0 || n < 0 || (int64_t)start + n > num_rows || n > context_lens[b])
            return ORACLE_EINVAL;
    }
    return ORACLE_OK;
}

/* Request, position and row of (row r) if some request names it. */
static int find_row(const oracle_shape *s, const int32_t *new_start, const int32_t *context_lens,
                    int32_t r, int32_t *b_out, int32_t *pos_out)
{
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        const int32_t start = new_start[b];
        const int32_t n = new_start[b + 1] - start;
        if (r >= start && r < start + n) {
            *b_out = b;
            *pos_out = context_lens[b] - n + (r - start);
            return 1;
        }
    }
    return 0;
}

static int attend_row(const oracle_shape *s, const uint16_t *q, const uint16_t *k_pool,
                      const uint16_t *v_pool, const int32_t *block_table, int32_t b, int32_t pos,
                      int32_t r, int32_t h, double scale, double *out_row, double *lse)
{
    oracle_shape one = *s;
    one.num_seqs = 1;
    const int32_t visible = pos + 1;   /* the causal cut: tokens 0 .. pos */
    return oracle_attend_one(&one, q + (size_t)r * s->num_q_heads * s->head_dim, k_pool, v_pool,
                             block_table + (size_t)b * s->max_blocks, &visible, scale, 0, h,
                             out_row, lse);
}

int oracle_prefill_attn(const oracle_shape *s, int32_t num_rows, const uint16_t *q,
                        const uint16_t *k_pool, const uint16_t *v_pool, const int32_t *new_start,
                        const int32_t *block_table, const int32_t *context_lens, double scale,
                        double *out, double *lse)
{
    const int rc = oracle_prefill_validate(s, num_rows, new_start, block_table, context_lens);
    if (rc != ORACLE_OK)
        return rc;
    const int64_t total = (int64_t)num_rows * s->num_q_heads;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : failed)
    for (int64_t i = 0; i < total; ++i) {
        const int32_t r = (int32_t)(i / s->num_q_heads);
        const int32_t h = (int32_t)(i % s->num_q_heads);
        int32_t b, pos;
        if (!find_row(s, new_start, context_lens, r, &b, &pos))
            continue;
        failed |= attend_row(s, q, k_pool, v_pool, block_table, b, pos, r, h, scale,
                             out + (size_t)i * s->head_dim, lse + i) != ORACLE_OK;
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

int oracle_prefill_attn_pairs(const oracle_shape *s, int32_t num_rows, const uint16_t *q,
                              const uint16_t *k_pool, const uint16_t *v_pool,
                              const int32_t *new_start, const int32_t *block_table,
                              const int32_t *context_lens, double scale, const int32_t *pairs,
                              int32_t n_pairs, double *out, double *lse)
{
    const int rc = oracle_prefill_validate(s, num_rows, new_start, block_table, context_lens);
    if (rc != ORACLE_OK)
        return rc;
    for (int32_t i = 0; i < n_pairs; ++i) {
        int32_t b, pos;
        if (pairs[2 * i] < 0 || pairs[2 * i] >= num_rows || pairs[2 * i + 1] < 0 ||
            pairs[2 * i + 1] >= s->num_q_heads ||
            !find_row(s, new_start, context_lens, pairs[2 * i], &b, &pos))
            return ORACLE_EINVAL;
    }
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int32_t i = 0; i < n_pairs; ++i) {
        int32_t b, pos;
        find_row(s, new_start, context_lens, pairs[2 * i], &b, &pos);
        failed |= attend_row(s, q, k_pool, v_pool, block_table, b, pos, pairs[2 * i],
                             pairs[2 * i + 1], scale, out + (size_t)i * s->head_dim, lse + i) != ORACLE_OK;
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}
