/*
 * paged_attn_oracle.h -- fp64 CPU oracle for one decode step of paged
 * grouped-query attention.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The HIP library never includes,
 * links or calls it, and it includes nothing of the HIP library.
 *
 * What it computes (the plain definition, with no blocking, partitioning or
 * online rescaling): for every request b and query head h,
 *
 *     G  = num_q_heads / num_kv_heads,   g = floor(h / G)
 *     n  = context_lens[b]
 *     for t in [0, n):  page = block_table[b][t / page_size], slot = t % page_size
 *                       k_t = K[page][slot][g][:],  v_t = V[page][slot][g][:]
 *                       z_t = scale * sum_d q[b][h][d] * k_t[d]
 *     m = max_t z_t,  w_t = exp(z_t - m),  l = sum_t w_t
 *     out[b][h][:] = sum_t w_t v_t / l,      lse[b][h] = m + ln(l)
 *
 * with n == 0 giving out = 0 and lse = -inf.  Sources on the pages:
 *  - the decoder is a Qwen3-0.6B LLM (FunASR vLLM guide, "Supported Models")
 *    with 16 query heads and 8 KV heads and a KV cache ("Fun-ASR-Nano Native
 *    Runtime Design", section "Decoder And Prompt"), so query heads share KV
 *    heads in groups of G = 2;
 *  - the KV cache is paged and allocated on demand (FunASR vLLM guide,
 *    "Why vLLM?" table: PagedAttention, on-demand allocation);
 *  - prefill builds the KV cache of the whole prompt and decode then emits
 *    one token per step (MOSS-TD article, "ASR model basics"), so the single
 *    query of a decode step attends to every cached token with no causal mask.
 * The attention formula itself is the standard scaled dot-product softmax of
 * such a decoder; the pages do not print it.  Readings where the pages are
 * silent: contiguous head grouping g = h / G, natural-log LSE, the context
 * length counts the current token, and bf16 inputs widen exactly to fp64.
 *
 * Layouts (all row-major, element counts):
 *   q            uint16 bf16 bits [num_seqs][num_q_heads][head_dim]
 *   k_pool,v_pool uint16 bf16 bits [num_pages][page_size][num_kv_heads][head_dim]
 *   block_table  int32 [num_seqs][max_blocks]
 *   context_lens int32 [num_seqs]
 *   out          double [num_seqs][num_q_heads][head_dim]
 *   lse          double [num_seqs][num_q_heads]
 */
#ifndef PAGED_ATTN_ORACLE_H
#define PAGED_ATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_blocks;
} oracle_shape;

enum {
    ORACLE_OK = 0,
    ORACLE_EINVAL = 1,     /* bad shape, bad context length or page index */
    ORACLE_ENOMEM = 2
};

/* Checks shape fields and, for every request, that its context fits the
 * block table and that every block it uses names a page of the pool. */
int oracle_validate(const oracle_shape *s, const int32_t *block_table,
                    const int32_t *context_lens);

/* One (request, query head): writes head_dim outputs and one LSE. */
int oracle_attend_one(const oracle_shape *s, const uint16_t *q,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_table, const int32_t *context_lens,
                      double scale, int32_t b, int32_t h,
                      double *out_row, double *lse);

/* Every (request, query head), OpenMP-parallel over the pairs. */
int oracle_paged_attn(const oracle_shape *s, const uint16_t *q,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_table, const int32_t *context_lens,
                      double scale, double *out, double *lse);

/* Threads an OpenMP region of this library would use. */
int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif
