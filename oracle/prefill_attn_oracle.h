/*
 * prefill_attn_oracle.h -- fp64 CPU oracle for chunked-prefill attention over
 * a paged KV cache.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The HIP library never includes,
 * links or calls it, and it includes nothing of the HIP library.
 *
 * What it computes.  Prefill builds the cache of a long prompt in chunks of
 * query tokens (MOSS-TD article, "Chunked prefill for long audio": 4096-token
 * blocks); each chunk's keys and values are appended first, and then every
 * query token of the chunk attends causally to the cache up to and including
 * its own position ("ASR model basics": prefill processes the prompt, decode
 * then extends it one token at a time).  For request b with n_b chunk tokens
 * and context length c_b (counting them), chunk token j sits at position
 * p = c_b - n_b + j, its query is row r = new_start[b] + j of q, and for every
 * query head h
 *
 *     out[r][h][:], lse[r][h] = the decode-step attention of q[r][h] over the
 *                               first p + 1 tokens of request b's cache
 *
 * that is, exactly what oracle_attend_one computes for a request whose
 * context length is p + 1 (see paged_attn_oracle.h).  The causal mask is that
 * shorter context; nothing else changes.
 *
 * Layouts (row-major): q uint16 bf16 bits [num_rows][num_q_heads][head_dim];
 * new_start int32 [num_seqs + 1]; out double [num_rows][num_q_heads][head_dim];
 * lse double [num_rows][num_q_heads]; the pools, block_table and
 * context_lens as in paged_attn_oracle.h.  Rows no request names are left
 * untouched.
 */
#ifndef PREFILL_ATTN_ORACLE_H
#define PREFILL_ATTN_ORACLE_H

#include <stdint.h>

#include "paged_attn_oracle.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Checks the chunk layout: counts within the contexts and rows within
 * num_rows, and the cache itself (oracle_validate). */
int oracle_prefill_validate(const oracle_shape *s, int32_t num_rows, const int32_t *new_start,
                            const int32_t *block_table, const int32_t *context_lens);

/* Every chunk row and query head, OpenMP-parallel over the (row, head) pairs. */
int oracle_prefill_attn(const oracle_shape *s, int32_t num_rows, const uint16_t *q,
                        const uint16_t *k_pool, const uint16_t *v_pool, const int32_t *new_start,
                        const int32_t *block_table, const int32_t *context_lens, double scale,
                        double *out, double *lse);

/* A chosen list of (row, query head) pairs, pairs[2*i] = row and pairs[2*i+1]
 * = h, each row named by some request; out is [n_pairs][head_dim]. */
int oracle_prefill_attn_pairs(const oracle_shape *s, int32_t num_rows, const uint16_t *q,
                              const uint16_t *k_pool, const uint16_t *v_pool,
                              const int32_t *new_start, const int32_t *block_table,
                              const int32_t *context_lens, double scale, const int32_t *pairs,
                              int32_t n_pairs, double *out, double *lse);

#ifdef __cplusplus
}
#endif

#endif
