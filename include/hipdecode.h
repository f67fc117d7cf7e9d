/*
 * hipdecode.h -- C ABI of the MI355X (gfx950) paged GQA decode-attention library.
 *
 * One call computes the attention of one decode step for one layer: every
 * request's single new query attends to all tokens of that request's paged KV
 * cache.  This is the step that dominates long-audio transcription (MOSS-TD
 * article, "Time spent: profiling": decode is over 94% of total time for long
 * audio at concurrency 1), over a cache that prefill builds and decode extends
 * one token per step ("ASR model basics"; "Chunked prefill for long audio"),
 * stored in on-demand pages (FunASR vLLM guide, "Why vLLM?": PagedAttention).
 * The decoder is Qwen3-0.6B-shaped (audio.cpp "Fun-ASR-Nano Native Runtime
 * Design", "Decoder And Prompt": 16 query heads over 8 KV heads), so query
 * heads share KV heads in groups of G = num_q_heads / num_kv_heads.
 *
 * For request b, query head h, G = num_q_heads / num_kv_heads, g = h / G,
 * n = context_lens[b], and cached token t in [0, n) stored at
 *     page = block_table[b * max_blocks_per_seq + t / 16], slot = t % 16:
 *     z_t       = scale * dot(q[b][h][:], K[page][slot][g][:])
 *     out[b][h] = sum_t softmax(z)_t * V[page][slot][g][:]
 *     lse[b][h] = ln(sum_t exp(z_t))                 (natural log)
 * n == 0 gives out = 0 and lse = -inf.
 *
 * Layouts (row-major, contiguous; element types in brackets):
 *   q             [num_seqs][num_q_heads][128]               bf16
 *   k_pool,v_pool [num_pages][16][num_kv_heads][128]         bf16
 *   block_table   [num_seqs][max_blocks_per_seq]             int32
 *   context_lens  [num_seqs]                                 int32
 *   out           [num_seqs][num_q_heads][128]               bf16 or fp32 (out_dtype)
 *   lse           [num_seqs][num_q_heads]                    fp32, may be NULL
 *   workspace     hipdecode_workspace_bytes(params) bytes, zero-filled before
 *                 its first use (hipdecode_workspace_init or any zero fill);
 *                 every completed call leaves its counters at zero again.
 *                 The counters lead the workspace (num_seqs * num_kv_heads *
 *                 256 bytes) and the split partials follow them, so calls
 *                 that share a workspace must have the same num_seqs *
 *                 num_kv_heads; zero-fill it again before a call that
 *                 changes that product.
 * q, k_pool, v_pool, out and workspace must be 16-byte aligned; all of them are
 * device memory.  Supported shapes: head_dim 128, page size 16, G in {1, 2, 4}
 * (16-wavefront workgroups for G <= 2 only).
 *
 * Pool placement (performance only).  KV head g's rows sit at byte offset
 * 256 * g of each token row.  On MI355X, rows whose address has bit 8 set
 * were measured to stream more slowly, so with both pools at offsets whose
 * bit 8 agrees the odd heads finish last.  Allocating V at an odd multiple of
 * 256 bytes from K (for instance both pools in one allocation, V starting
 * 256 bytes after K ends) gave every head one pool of each kind: 2-4% faster
 * calls on most of the measured shapes, none slower.
 *
 * Ownership and ordering.  The caller owns every buffer.  The library
 * allocates nothing, keeps no per-call state, never synchronises the host and
 * enqueues its work on `stream` (a hipStream_t; NULL is the null stream), so a
 * call may be captured into a HIP graph.  Calls that share a workspace must be
 * ordered (same stream, or synchronised); `out` and `lse` must not alias any
 * input.
 *
 * Errors.  Argument errors are returned synchronously, before anything is
 * enqueued.  HIPDECODE_ERR_HIP means the launch itself failed.  Faults while
 * the kernel runs surface at the caller's next synchronisation.  Device-side
 * contents are the caller's contract: context_lens[b] <= max_context_len and
 * 0 <= block_table entries < num_pages for the ceil(n/16) blocks a request
 * uses.  The kernel does not read memory outside the pools when that contract
 * is broken (it clamps n to max_context_len and skips page indices outside
 * the pool), but the values it then returns are unspecified.  Nothing aborts
 * and no C++ exception crosses this interface.
 */
#ifndef HIPDECODE_H
#define HIPDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HIPDECODE_ABI_VERSION 1

typedef enum {
    HIPDECODE_OK = 0,
    HIPDECODE_ERR_NULL = 1,        /* a required pointer is NULL */
    HIPDECODE_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
    HIPDECODE_ERR_UNSUPPORTED = 3, /* valid but not built: head_dim, page size, group, dtype */
    HIPDECODE_ERR_ALIGN = 4,       /* a buffer is not 16-byte aligned */
    HIPDECODE_ERR_WORKSPACE = 5,   /* workspace smaller than hipdecode_workspace_bytes */
    HIPDECODE_ERR_SCALE = 6,       /* scale is not finite, or rope_theta not finite and > 0 */
    HIPDECODE_ERR_HIP = 7          /* the HIP runtime refused the launch */
} hipdecode_status;

typedef enum {
    HIPDECODE_BF16 = 0,            /* out rounded to bf16, nearest-even */
    HIPDECODE_F32 = 1
} hipdecode_dtype;

typedef struct {
    int32_t num_seqs;              /* B >= 0; B == 0 is a no-op */
    int32_t num_q_heads;           /* Hq */
    int32_t num_kv_heads;          /* Hkv; Hq % Hkv == 0 */
    int32_t head_dim;              /* must be 128 */
    int32_t page_size;             /* tokens per page; must be 16 */
    int32_t num_pages;             /* P, rows of each pool */
    int32_t max_blocks_per_seq;    /* row stride of block_table, in int32 elements */
    int32_t max_context_len;       /* host upper bound of context_lens[]; sizes the grid */
    int32_t partition_tokens;      /* split-K partition: 0 = planner's choice, else a multiple of 64 */
    int32_t workgroup_waves;       /* wavefronts per workgroup: 0 = planner's choice, else 4 or 16 */
    int32_t schedule;              /* 0 = planner's choice, 1 = split by partition (the only one) */
    int32_t out_dtype;             /* hipdecode_dtype */
    float scale;                   /* applied to q.k, e.g. 1/sqrt(128) */
} hipdecode_params;

/* HIPDECODE_ABI_VERSION of the built library. */
int hipdecode_abi_version(void);

/* Pure host check of the parameter block (no HIP calls): HIPDECODE_OK or the
 * first problem found.  A NULL pointer gives HIPDECODE_ERR_NULL. */
hipdecode_status hipdecode_check_params(const hipdecode_params *params);

/* Tokens per split-K partition that a call with these parameters uses (the
 * planner's choice when partition_tokens is 0); 0 if the parameters are
 * invalid.  Pure host function. */
int32_t hipdecode_partition_tokens(const hipdecode_params *params);

/* Wavefronts per workgroup that a call with these parameters uses (the
 * planner's choice when workgroup_waves is 0); 0 if the parameters are
 * invalid.  Pure host function. */
int32_t hipdecode_workgroup_waves(const hipdecode_params *params);

/* Work schedule that a call with these parameters uses: 1 = split, one
 * workgroup per (request, KV head, partition), the grid mapped onto the
 * real (request, partition) units of a ragged batch inside the kernel; 0 if
 * the parameters are invalid (any schedule but 0 and 1 is).  Pure host
 * function. */
int32_t hipdecode_schedule(const hipdecode_params *params);

/* Bytes of workspace a call with these parameters needs; 0 if they are
 * invalid.  Pure host function. */
size_t hipdecode_workspace_bytes(const hipdecode_params *params);

/* Zero-fills `bytes` bytes of workspace on `stream` with a fill kernel (no
 * hipMemset node, so it is safe under graph capture). */
hipdecode_status hipdecode_workspace_init(void *workspace, size_t bytes, void *stream);

/* One decode step of paged GQA attention (see the top of this file). */
hipdecode_status hipdecode_paged_attn(const hipdecode_params *params,
                                      const void *q,
                                      const void *k_pool,
                                      const void *v_pool,
                                      const int32_t *block_table,
                                      const int32_t *context_lens,
                                      void *out,
                                      float *lse,
                                      void *workspace,
                                      size_t workspace_bytes,
                                      void *stream);

/* ------------------------------------------------------------------------
 * KV-cache append.
 *
 * Before a decode step attends, each request's cache is extended by the token
 * it has just produced; prefill writes a chunk of prompt tokens the same way
 * (MOSS-TD article, "ASR model basics" and "Chunked prefill for long audio";
 * paged cache: FunASR vLLM guide, "Why vLLM?").  The Qwen3 decoder rotates
 * queries and keys by RoPE with theta 1e6 (audio.cpp "Fun-ASR-Nano Native
 * Runtime Design", "Decoder And Prompt"); the pages give no pairing or
 * precision, so this library takes the rotate-half pairing and an exact
 * rotation rounded once.
 *
 * For request b with n_b new tokens and context length c_b (which already
 * counts them), new token j in [0, n_b) is at position p = c_b - n_b + j and
 * comes from row r = new_start[b] + j of the packed inputs (r = b and n_b = 1,
 * or n_b = 0 when c_b == 0, if new_start is NULL).  With
 * page = block_table[b][p / 16] and slot = p % 16:
 *     K[page][slot][g][:] = R_p(k_new[r][g][:])   for every KV head g
 *     V[page][slot][g][:] = v_new[r][g][:]        (bit copy)
 *     q[r][h][:]          = R_p(q[r][h][:])       for every query head h, in place
 * With rope == HIPDECODE_ROPE_NONE, R_p is a bit copy and q is not touched.
 * Otherwise, for i in [0, 64) and f_i = rope_theta^(-i/64):
 *     x'[i]      = x[i] cos(p f_i) - x[i + 64] sin(p f_i)
 *     x'[i + 64] = x[i + 64] cos(p f_i) + x[i] sin(p f_i)
 * evaluated in fp64 from the exactly widened bf16 inputs and rounded once to
 * the nearest bf16, ties to even.  f_i itself is evaluated in fp64 as
 * 2^(-(i/64) log2(rope_theta)), within a few units in the last place of the
 * power, so a rotated value within about 1e-12 (relative) of a midpoint
 * between two bf16 numbers may round to either of them.
 *
 * Layouts (row-major, contiguous):
 *   q             [num_rows][num_q_heads][128]   bf16, may be NULL
 *   k_new, v_new  [num_rows][num_kv_heads][128]  bf16
 *   new_start     [num_seqs + 1]                 int32, may be NULL
 *   block_table, context_lens, k_pool, v_pool as for hipdecode_paged_attn.
 * q, k_new, v_new, k_pool and v_pool must be 16-byte aligned; all are device
 * memory.  Calls are stream-ordered and asynchronous, allocate nothing, and
 * may be captured into a HIP graph.
 *
 * Device-side contract: new_start non-decreasing with new_start[num_seqs] <=
 * num_rows; n_b <= min(c_b, max_new_tokens); the blocks written name pool
 * pages; no two new tokens share a slot; k_new, v_new and q do not overlap
 * the pools.  When it is broken the kernel still neither reads nor writes
 * outside the buffers the sizes describe: a request with n_b > c_b, n_b >
 * max_new_tokens or rows outside [0, num_rows) writes nothing, and a token
 * whose block lies past max_blocks_per_seq or names no pool page is skipped.
 * Overlapping slots or buffers give unspecified contents.
 * ------------------------------------------------------------------------ */

typedef enum {
    HIPDECODE_ROPE_NONE = 0,
    HIPDECODE_ROPE_HALF = 1        /* rotate-half pairing: i with i + head_dim/2 */
} hipdecode_rope;

typedef struct {
    int32_t num_seqs;              /* B >= 0; B == 0 is a no-op */
    int32_t num_q_heads;           /* Hq, heads of q */
    int32_t num_kv_heads;          /* Hkv; Hq % Hkv == 0 */
    int32_t head_dim;              /* must be 128 */
    int32_t page_size;             /* must be 16 */
    int32_t num_pages;             /* P, rows of each pool */
    int32_t max_blocks_per_seq;    /* row stride of block_table, in int32 elements */
    int32_t num_rows;              /* rows of k_new, v_new and q; >= num_seqs if new_start is NULL */
    int32_t max_new_tokens;        /* host upper bound of any n_b; sizes the grid (1 if new_start is NULL) */
    int32_t rope;                  /* hipdecode_rope */
    double rope_theta;             /* RoPE base, e.g. 1e6; finite and > 0 when rope is on */
} hipdecode_append_params;

/* Pure host check of an append parameter block: HIPDECODE_OK or the first
 * problem found. */
hipdecode_status hipdecode_check_append_params(const hipdecode_append_params *params);

/* Appends new tokens' keys and values to the paged cache (see above). */
hipdecode_status hipdecode_kv_append(const hipdecode_append_params *params,
                                     void *q,
                                     const void *k_new,
                                     const void *v_new,
                                     const int32_t *new_start,
                                     const int32_t *block_table,
                                     const int32_t *context_lens,
                                     void *k_pool,
                                     void *v_pool,
                                     void *stream);

/* ------------------------------------------------------------------------
 * Chunked-prefill attention.
 *
 * Prefill builds a long prompt's cache in chunks of query tokens (MOSS-TD
 * article, "Chunked prefill for long audio": 4096-token blocks).  After a
 * chunk's keys and values have been appended (hipdecode_kv_append, with the
 * same row offsets), each chunk token attends causally to the cache up to its
 * own position.  For request b with n_b chunk tokens and context length c_b
 * (which counts them), chunk token j is at position p = c_b - n_b + j, its
 * query is row r = new_start[b] + j, and for every query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)):
 *     z_t      = scale * dot(q[r][h][:], K[page(b,t)][t % 16][g][:])   for t <= p
 *     out[r][h] = sum_{t <= p} softmax(z)_t V[page(b,t)][t % 16][g][:]
 *     lse[r][h] = ln sum_{t <= p} exp(z_t)
 * which is the decode step of hipdecode_paged_attn for a context of p + 1.
 * Rows no request names are not written.
 *
 * Layouts: q [num_rows][num_q_heads][128] bf16; out the same shape in
 * out_dtype; lse [num_rows][num_q_heads] fp32, may be NULL; new_start
 * [num_seqs + 1] int32; the rest as for hipdecode_paged_attn.  q, the pools
 * and out must be 16-byte aligned.  Supported: head_dim 128, page size 16,
 * G = num_q_heads / num_kv_heads in {1, 2, 4}.  No workspace; asynchronous on
 * `stream`, graph-capturable.
 *
 * Scores, softmax weights, the running sums and lse are fp32.  The weighted
 * sum of V runs on the matrix cores in fp16: each weight is rounded to its
 * nearest fp16 (within 2^-11, relative; the weights are kept in fp16's normal
 * range), and V enters exactly (every bf16 value below 2^16 in magnitude has
 * an fp16 form; below 2^-17 it is kept to within 2^-25).  The output is then
 * off by at most 2^-11 times the softmax-weighted mean of |V| over the row's
 * keys, before its own rounding.  V entries of magnitude 2^16 or more are
 * outside the contract.
 *
 * Device-side contract as for the append: new_start non-decreasing, n_b <=
 * min(c_b, max_new_tokens), rows within num_rows, c_b <= 16 *
 * max_blocks_per_seq, blocks in the pool; and |V| < 2^16 for the entries
 * read.  A request that breaks the first conditions writes nothing; pages
 * outside the pool read as page 0, so memory outside the buffers is never
 * touched; V past the range turns into inf in the products of the rows of
 * its step.
 * ------------------------------------------------------------------------ */

typedef struct {
    int32_t num_seqs;              /* B >= 0; B == 0 is a no-op */
    int32_t num_q_heads;           /* Hq */
    int32_t num_kv_heads;          /* Hkv; Hq / Hkv in {1, 2, 4} */
    int32_t head_dim;              /* must be 128 */
    int32_t page_size;             /* must be 16 */
    int32_t num_pages;             /* P, rows of each pool */
    int32_t max_blocks_per_seq;    /* row stride of block_table, >= 1 */
    int32_t num_rows;              /* rows of q, out and lse */
    int32_t max_new_tokens;        /* host upper bound of any n_b; sizes the grid */
    int32_t out_dtype;             /* hipdecode_dtype */
    float scale;                   /* applied to q.k */
} hipdecode_prefill_params;

/* Pure host check of a prefill parameter block. */
hipdecode_status hipdecode_check_prefill_params(const hipdecode_prefill_params *params);

/* Chunked-prefill attention over the paged cache (see above). */
hipdecode_status hipdecode_prefill_attn(const hipdecode_prefill_params *params,
                                        const void *q,
                                        const void *k_pool,
                                        const void *v_pool,
                                        const int32_t *new_start,
                                        const int32_t *block_table,
                                        const int32_t *context_lens,
                                        void *out,
                                        float *lse,
                                        void *stream);

/* ------------------------------------------------------------------------
 * Graph-replayed decode step.
 *
 * Decode runs as captured graphs replayed with the batch padded to fixed
 * bucket sizes, and the host prepares the next step while the GPU still runs
 * the current one (MOSS-TD article, "Autoregressive decoding": decode is
 * replayed as graphs with padded batch buckets, and asynchronous lookahead
 * scheduling never waits on the GPU).  A runner holds one HIP graph per
 * bucket -- 1, 2, 4, ... up to the first power of two >= max_seqs -- each
 * capturing, for layer l = 0 .. num_layers-1 in order,
 *     hipdecode_paged_attn_append  (append one new token per request, RoPE
 *                                   when rope_theta > 0, and attend)
 * over `bucket` rows of the caller's buffers.  A step for num_seqs requests
 * writes their context lengths, and zeros up to the bucket, through a pinned
 * double buffer to `context_lens` with one asynchronous copy, then launches
 * the bucket's graph (captured on first use).  Padding rows have context
 * length 0: they append nothing and their out is 0 and lse -inf.  The host
 * blocks only when the staging half it needs still feeds a copy issued two
 * steps earlier that has not completed.
 *
 * Buffers (the caller owns them; the runner keeps the pointers): per layer l,
 * k_pool[l], v_pool[l] as for hipdecode_paged_attn; q[l] [max_bucket][Hq][128]
 * bf16 (read, not rotated in place); k_new[l], v_new[l]
 * [max_bucket][Hkv][128] bf16; out[l] [max_bucket][Hq][128] in out_dtype;
 * lse[l] [max_bucket][Hq] fp32 (lse itself may be NULL: no LSE);
 * block_table [max_bucket][max_blocks_per_seq] and context_lens [max_bucket]
 * int32, device memory.  The caller updates q, k_new, v_new and block_table
 * between steps with work ordered on the same stream.  The runner allocates
 * an attention workspace with one slice per bucket, two pinned staging
 * buffers, two events, a capture stream and the graphs, and frees them in
 * hipdecode_step_runner_destroy.
 * A runner is used from one thread, its steps on one stream.
 * ------------------------------------------------------------------------ */

typedef struct hipdecode_step_runner hipdecode_step_runner;

typedef struct {
    int32_t num_layers;            /* L >= 1 */
    int32_t max_seqs;              /* largest batch of a step, >= 1 */
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;              /* 128 */
    int32_t page_size;             /* 16 */
    int32_t num_pages;             /* rows of each layer's pools */
    int32_t max_blocks_per_seq;
    int32_t max_context_len;       /* bound of every step's context lengths */
    int32_t out_dtype;             /* hipdecode_dtype */
    float scale;
    double rope_theta;             /* > 0: RoPE on K and q; 0: none */
} hipdecode_step_config;

typedef struct {
    void *const *k_pool;           /* host arrays of num_layers device pointers */
    void *const *v_pool;
    void *const *q;
    const void *const *k_new;
    const void *const *v_new;
    void *const *out;
    float *const *lse;             /* may be NULL */
    int32_t *block_table;          /* device */
    int32_t *context_lens;         /* device */
} hipdecode_step_buffers;

/* Rows of the bucket a step of num_seqs requests runs in (pure host); 0 if
 * num_seqs is not in [1, max_seqs]. */
int32_t hipdecode_step_bucket(int32_t max_seqs, int32_t num_seqs);

/* Checks the configuration and buffers, sizes and zero-fills the workspace;
 * graphs are captured on first use.  *runner is NULL on failure. */
hipdecode_status hipdecode_step_runner_create(const hipdecode_step_config *config,
                                              const hipdecode_step_buffers *buffers,
                                              hipdecode_step_runner **runner);

/* One decode step for num_seqs requests (0 is a no-op) with host context
 * lengths context_lens_host[0 .. num_seqs), enqueued on `stream`.  A length
 * below 0 or above max_context_len gives HIPDECODE_ERR_SHAPE and enqueues
 * nothing. */
hipdecode_status hipdecode_step_runner_step(hipdecode_step_runner *runner, int32_t num_seqs,
                                            const int32_t *context_lens_host, void *stream);

/* Synchronizes the device (steps may still run on the caller's streams),
 * then frees what the runner allocated. */
hipdecode_status hipdecode_step_runner_destroy(hipdecode_step_runner *runner);

/* One decode step of append and attention in a single launch: the same
 * result as hipdecode_kv_append (one new token per request, new_start NULL;
 * RoPE on K and q with rope_theta when rope_theta > 0, none when 0) followed
 * by hipdecode_paged_attn, except that q is read, not rotated in place.  The
 * workgroup that folds a request's last page takes the new token's K and V
 * from k_new/v_new [num_seqs][num_kv_heads][128] (bf16, 16-byte aligned),
 * writes them to their slot and folds them from registers; every workgroup
 * rotates its query heads itself.  A rope_theta that is negative or not
 * finite gives HIPDECODE_ERR_SCALE.  Same buffers, workspace
 * and contract as hipdecode_paged_attn otherwise; the pools are written.  A
 * request whose context_lens[b] exceeds max_context_len (a broken contract)
 * writes nothing to the pools, as hipdecode_kv_append would not; its out and
 * lse are unspecified. */
hipdecode_status hipdecode_paged_attn_append(const hipdecode_params *params,
                                             double rope_theta,
                                             const void *q,
                                             const void *k_new,
                                             const void *v_new,
                                             void *k_pool,
                                             void *v_pool,
                                             const int32_t *block_table,
                                             const int32_t *context_lens,
                                             void *out,
                                             float *lse,
                                             void *workspace,
                                             size_t workspace_bytes,
                                             void *stream);

/* ------------------------------------------------------------------------
 * Allocation-free decode.
 *
 * For callers that cannot allocate device memory at all -- code running under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc --
 * and so cannot provide the workspace hipdecode_paged_attn takes.  Same
 * parameters, buffers, result and contract as hipdecode_paged_attn without
 * `workspace`/`workspace_bytes`: the arrival counters and split partials live
 * in a static device array of HIPDECODE_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.
 *
 * Limits: at most 4096 (request, KV head) pairs (num_seqs * num_kv_heads),
 * and the split partials must fit the rest of the array (16 MiB minus 1 MiB of
 * counters: for example 32 requests up to 67,500 tokens, or 16 at 28,672,
 * fit); a call past either gives HIPDECODE_ERR_WORKSPACE and enqueues
 * nothing.  The first call on a device looks up the array's address there and
 * zero-fills its counter region with a kernel on `stream`; every completed
 * call leaves the counters at zero again.
 *
 * Every call on a GPU shares that GPU's array: calls that may overlap in time
 * on one GPU (different streams without ordering between them, or several
 * host threads) race on it and give unspecified results.  Order them.
 * ------------------------------------------------------------------------ */

#define HIPDECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

hipdecode_status hipdecode_paged_attn_noalloc(const hipdecode_params *params,
                                              const void *q,
                                              const void *k_pool,
                                              const void *v_pool,
                                              const int32_t *block_table,
                                              const int32_t *context_lens,
                                              void *out,
                                              float *lse,
                                              void *stream);

/* ------------------------------------------------------------------------
 * Contract violations met on the device.
 *
 * The kernels never read or write outside the buffers the sizes describe,
 * even when device-side contents break the contract; they clamp or skip
 * instead (see each entry point).  Each time they do, they also set a bit in
 * a flag word of the library, one word per GPU, so that a caller can find out
 * afterwards that a result it holds is unspecified.  Setting a bit costs
 * nothing on the normal path.
 *   HIPDECODE_VIOLATION_CONTEXT: a context length below 0 or above
 *       max_context_len (decode), or past 16 * max_blocks_per_seq tokens
 *       (append, prefill);
 *   HIPDECODE_VIOLATION_PAGE: a block-table entry that a request uses names
 *       no page of the pool;
 *   HIPDECODE_VIOLATION_ROWS: append or prefill: a request with more new
 *       tokens than its context or than max_new_tokens, or rows outside
 *       [0, num_rows) (new_start decreasing included);
 *   HIPDECODE_VIOLATION_VALUE: prefill: a workgroup's weighted sums of V
 *       came out inf or NaN: a V entry of magnitude 2^16 or more, which
 *       fp16 cannot hold, reached its products, or q, K or V held inf or
 *       NaN.
 * ------------------------------------------------------------------------ */

#define HIPDECODE_VIOLATION_CONTEXT 1u
#define HIPDECODE_VIOLATION_PAGE 2u
#define HIPDECODE_VIOLATION_ROWS 4u
#define HIPDECODE_VIOLATION_VALUE 8u

/* Waits for all work on the current device (hipDeviceSynchronize), then
 * stores in *flags the OR of the HIPDECODE_VIOLATION_* bits that kernels of
 * this library have set on it since the previous call, and clears them.  Not
 * for use under graph capture; calls from several host threads, or while
 * another thread launches work on the device, may lose bits. */
hipdecode_status hipdecode_contract_violations(uint32_t *flags);

/* Static English text for a status code; never NULL. */
const char *hipdecode_status_string(hipdecode_status status);

#ifdef __cplusplus
}
#endif

#endif /* HIPDECODE_H */
