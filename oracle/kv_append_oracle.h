/*
 * kv_append_oracle.h -- fp64 CPU oracle for appending new tokens' keys and
 * values to a paged KV cache, with optional rotary position embedding (RoPE).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The HIP library never includes,
 * links or calls it, and it includes nothing of the HIP library.
 *
 * What it computes.  Every decode step extends each request's KV cache by the
 * token it just produced, and prefill writes a whole chunk of the prompt's
 * tokens (MOSS-TD article, "ASR model basics" and "Chunked prefill for long
 * audio"); the cache is paged (FunASR vLLM guide, "Why vLLM?" table).  The
 * decoder is Qwen3-shaped with RoPE theta 1e6 ("Fun-ASR-Nano Native Runtime
 * Design", section "Decoder And Prompt").  For request b with n_b new tokens
 * and context length c_b (which already counts them), new token j in [0, n_b)
 * sits at position p = c_b - n_b + j, and
 *
 *     page = block_table[b][p / page_size],  slot = p % page_size
 *     K[page][slot][g][:] = R_p(k_new[row][g][:])     for every KV head g
 *     V[page][slot][g][:] = v_new[row][g][:]
 *     q[row][h][:]        = R_p(q[row][h][:])         for every query head h
 *
 * where row = new_start[b] + j (row = b, one token per request, when
 * new_start is NULL).  With rope off, R_p is the identity and q is left alone.
 *
 * RoPE.  The pages name RoPE and its theta but not its pairing or precision.
 * Readings: the rotate-half pairing of Qwen3 (dimension i pairs with
 * i + d/2), frequency f_i = theta^(-2i/d) for i in [0, d/2),
 *
 *     x'[i]       = x[i] cos(p f_i) - x[i + d/2] sin(p f_i)
 *     x'[i + d/2] = x[i + d/2] cos(p f_i) + x[i] sin(p f_i)
 *
 * computed in fp64 from the exactly widened bf16 inputs and rounded once to
 * bf16, to nearest with ties to even.
 *
 * Layouts (row-major; bf16 values are passed as their uint16 bit patterns):
 *   q             [num_rows][num_q_heads][head_dim]   (may be NULL)
 *   k_new, v_new  [num_rows][num_kv_heads][head_dim]
 *   new_start     int32 [num_seqs + 1], non-decreasing, new_start[0] >= 0,
 *                 new_start[num_seqs] <= num_rows   (may be NULL)
 *   block_table   int32 [num_seqs][max_blocks]
 *   context_lens  int32 [num_seqs]
 *   k_pool,v_pool [num_pages][page_size][num_kv_heads][head_dim]
 */
#ifndef KV_APPEND_ORACLE_H
#define KV_APPEND_ORACLE_H

#include <stdint.h>

#include "paged_attn_oracle.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Nearest bf16 to x, ties to even (the bit pattern); NaN gives 0x7FC0. */
uint16_t oracle_round_bf16(double x);

/* Rotates one head vector of head_dim (even) fp64 values in place by
 * position pos with base theta, rotate-half pairing. */
void oracle_rope_f64(double *x, int32_t head_dim, double pos, double theta);

/* Checks the append against the shape: new-token counts within the context,
 * rows within num_rows, and every written block inside the table and pool. */
int oracle_kv_append_validate(const oracle_shape *s, int32_t num_rows,
                              const int32_t *new_start, const int32_t *block_table,
                              const int32_t *context_lens);

/* Performs the append (see the top of this file); rope is 0 or 1. */
int oracle_kv_append(const oracle_shape *s, int32_t num_rows, int32_t rope, double theta,
                     uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *new_start, const int32_t *block_table,
                     const int32_t *context_lens, uint16_t *k_pool, uint16_t *v_pool);

#ifdef __cplusplus
}
#endif

#endif
