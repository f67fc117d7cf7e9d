/*
 * kv_append_oracle.c -- fp64 CPU oracle for appending keys and values to a
 * paged KV cache, with optional RoPE.
 *
 * TEST INFRASTRUCTURE (see kv_append_oracle.h for the definition it follows,
 * the passages of the pages behind it and the readings taken where they are
 * silent).  Deliberately plain: one token, one head, one dimension pair at a
 * time, every rotation in fp64, one rounding to bf16 at the end.
 */
#include "kv_append_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t oracle_round_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    double r = x;
    if (x != 0.0 && !isinf(x)) {
        /* A bf16 number has 8 significant bits and the exponent range of
         * binary32, so around |x| in [2^(e-1), 2^e) neighbouring bf16 values
         * are 2^(e-8) apart, and never closer than the subnormal step 2^-133.
         * Scale x so that step is 1, round to the nearest integer (ties to
         * even under the default rounding mode), and scale back. */
        int e;
        frexp(x, &e);
        int step = e - 8;
        if (step < -133)
            step = -133;
        r = ldexp(nearbyint(ldexp(x, -step)), step);
        if (fabs(r) > 0x1.fep127)          /* past the largest finite bf16 */
            r = copysign(INFINITY, x);
    }
    const float f = (float)r;              /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_rope_f64(double *x, int32_t head_dim, double pos, double theta)
{
    const int32_t half = head_dim / 2;
    for (int32_t i = 0; i < half; ++i) {
        const double freq = pow(theta, -2.0 * (double)i / (double)head_dim);
        const double angle = pos * freq;
        const double c = cos(angle);
        const double s = sin(angle);
        const double first = x[i];
        const double second = x[i + half];
        x[i] = first * c - second * s;
        x[i + half] = second * c + first * s;
    }
}

/* Rows [*start, *start + *n) of the packed new-token arrays belong to b. */
static void new_rows(const int32_t *new_start, const int32_t *context_lens, int32_t b,
                     int32_t *start, int32_t *n)
{
    if (new_start) {
        *start = new_start[b];
        *n = new_start[b + 1] - new_start[b];
    } else {
        *start = b;
        *n = context_lens[b] > 0 ? 1 : 0;
    }
}

static int cmp_i64(const void *a, const void *b)
{
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

int oracle_kv_append_validate(const oracle_shape *s, int32_t num_rows,
                              const int32_t *new_start, const int32_t *block_table,
                              const int32_t *context_lens)
{
    if (!s || s->num_seqs < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
        s->head_dim <= 0 || s->head_dim % 2 != 0 || s->page_size <= 0 ||
        s->num_pages < 0 || s->max_blocks < 0 || num_rows < 0)
        return ORACLE_EINVAL;
    if (s->num_q_heads % s->num_kv_heads != 0)
        return ORACLE_EINVAL;
    if (!new_start && num_rows < s->num_seqs)
        return ORACLE_EINVAL;
    int64_t total = 0;
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        int32_t start, n;
        new_rows(new_start, context_lens, b, &start, &n);
        const int32_t c = context_lens[b];
        if (start < 0 || n < 0 || (int64_t)start + n > num_rows || n > c ||
            (int64_t)c > (int64_t)s->max_blocks * s->page_size)
            return ORACLE_EINVAL;
        for (int32_t p = c - n; p < c; ++p) {
            const int32_t page = block_table[(size_t)b * s->max_blocks + p / s->page_size];
            if (page < 0 || page >= s->num_pages)
                return ORACLE_EINVAL;
        }
        total += n;
    }
    /* No two new tokens may land in the same slot of the pool. */
    int64_t *slots = malloc((size_t)(total > 0 ? total : 1) * sizeof *slots);
    if (!slots)
        return ORACLE_ENOMEM;
    int64_t k = 0;
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        int32_t start, n;
        new_rows(new_start, context_lens, b, &start, &n);
        const int32_t c = context_lens[b];
        for (int32_t p = c - n; p < c; ++p) {
            const int32_t page = block_table[(size_t)b * s->max_blocks + p / s->page_size];
            slots[k++] = (int64_t)page * s->page_size + p % s->page_size;
        }
    }
    qsort(slots, (size_t)total, sizeof *slots, cmp_i64);
    int rc = ORACLE_OK;
    for (int64_t i = 1; i < total; ++i)
        if (slots[i] == slots[i - 1])
            rc = ORACLE_EINVAL;
    free(slots);
    return rc;
}

/* Rotates (or, with rope off, copies) one head vector of bf16 bits. */
static void rotate_head(const uint16_t *src, uint16_t *dst, int32_t dim, int32_t rope,
                        double pos, double theta, double *scratch)
{
    if (!rope) {
        memmove(dst, src, (size_t)dim * sizeof *dst);
        return;
    }
    for (int32_t d = 0; d < dim; ++d)
        scratch[d] = widen_bf16(src[d]);
    oracle_rope_f64(scratch, dim, pos, theta);
    for (int32_t d = 0; d < dim; ++d)
        dst[d] = oracle_round_bf16(scratch[d]);
}

int oracle_kv_append(const oracle_shape *s, int32_t num_rows, int32_t rope, double theta,
                     uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *new_start, const int32_t *block_table,
                     const int32_t *context_lens, uint16_t *k_pool, uint16_t *v_pool)
{
    const int rc = oracle_kv_append_validate(s, num_rows, new_start, block_table, context_lens);
    if (rc != ORACLE_OK)
        return rc;
    if (rope != 0 && rope != 1)
        return ORACLE_EINVAL;
    const int32_t dim = s->head_dim;
    double *scratch = malloc((size_t)dim * sizeof *scratch);
    if (!scratch)
        return ORACLE_ENOMEM;
    const size_t kv_row = (size_t)s->num_kv_heads * dim;   /* elements of one token's K (or V) */
    const size_t q_row = (size_t)s->num_q_heads * dim;
    for (int32_t b = 0; b < s->num_seqs; ++b) {
        int32_t start, n;
        new_rows(new_start, context_lens, b, &start, &n);
        const int32_t c = context_lens[b];
        for (int32_t j = 0; j < n; ++j) {
            const int32_t pos = c - n + j;
            const size_t row = (size_t)start + j;
            const int32_t page = block_table[(size_t)b * s->max_blocks + pos / s->page_size];
            const size_t slot = (size_t)page * s->page_size + pos % s->page_size;
            for (int32_t g = 0; g < s->num_kv_heads; ++g) {
                rotate_head(k_new + row * kv_row + (size_t)g * dim, k_pool + slot * kv_row + (size_t)g * dim,
                            dim, rope, (double)pos, theta, scratch);
                memcpy(v_pool + slot * kv_row + (size_t)g * dim, v_new + row * kv_row + (size_t)g * dim,
                       (size_t)dim * sizeof *v_pool);
            }
            if (q && rope)
                for (int32_t h = 0; h < s->num_q_heads; ++h) {
                    uint16_t *x = q + row * q_row + (size_t)h * dim;
                    rotate_head(x, x, dim, rope, (double)pos, theta, scratch);
                }
        }
    }
    free(scratch);
    return ORACLE_OK;
}
