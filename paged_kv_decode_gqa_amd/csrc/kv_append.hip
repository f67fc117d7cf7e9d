// kv_append.hip -- writes new tokens' keys and values into their cache pages,
// rotating K (and q, in place) by RoPE when asked; the extern "C" entry points
// hipdecode_check_append_params and hipdecode_kv_append.
//
// Every decode step appends the token each request just produced, and
// prefill appends a chunk of prompt tokens, to the paged cache that attention
// then reads (MOSS-TD article, "ASR model basics"; FunASR vLLM guide, "Why
// vLLM?").  RoPE with theta 1e6 belongs to the Qwen3 decoder (audio.cpp
// "Fun-ASR-Nano Native Runtime Design", "Decoder And Prompt").
//
// One 256-thread workgroup per new token.  The token's 64 rotation angles
// are evaluated once, in fp64, by the first wavefront and shared through LDS;
// every thread then takes items of 16 per head: four dimension pairs of a K
// or q head to rotate, or a 16-byte chunk of V (or of K, without RoPE) to
// copy.  The work is a few KB per token, so the kernel is bound by HBM for
// prefill chunks and by launch latency for one decode token per request.
#include "hipdecode.h"
#include "internal.h"

#include <math.h>

namespace hipdecode {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kHalfDim = kHeadDim / 2;          // rotation pairs per head
constexpr int kPairsPerItem = 4;
constexpr int kItemsPerHead = kHalfDim / kPairsPerItem;   // also the 16-byte chunks of one head's row
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

struct AppendArgs {
    uint16_t *q;
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *new_start;
    const int32_t *block_table;
    const int32_t *context_lens;
    uint16_t *k_pool;
    uint16_t *v_pool;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_blocks;
    int32_t num_rows;
    int32_t max_new;
    double theta;
};

__device__ inline double widen_bf16(uint32_t bits16) { return (double)__uint_as_float(bits16 << 16); }

// Nearest bf16 of an fp64 value, ties to even, by rounding twice: first to
// fp32 towards zero with a sticky last bit ("rounding to odd"), then to bf16
// to nearest even.  fp32 keeps 16 more significand bits than bf16, which is
// more than the two extra bits rounding to odd needs for the second rounding
// to equal a direct one (Boldo and Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", IEEE TC 2008).
__device__ inline uint32_t round_bf16(double x)
{
    if (x != x)
        return 0x7FC0u;
    const float t = __double2float_rz(x);
    uint32_t b = __float_as_uint(t);
    if ((double)t != x)
        b |= 1u;
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

__device__ inline void copy16(const uint16_t *src, uint16_t *dst)
{
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}

// Rotates pairs [4s, 4s+4) of one head: dims 4s.. with dims 64+4s..
__device__ inline void rotate_item(const uint16_t *src, uint16_t *dst, int s, const double (*cs)[2])
{
    const uint2 lo = *reinterpret_cast<const uint2 *>(src + kPairsPerItem * s);
    const uint2 hi = *reinterpret_cast<const uint2 *>(src + kHalfDim + kPairsPerItem * s);
    const uint32_t a[4] = {lo.x & 0xFFFFu, lo.x >> 16, lo.y & 0xFFFFu, lo.y >> 16};
    const uint32_t b[4] = {hi.x & 0xFFFFu, hi.x >> 16, hi.y & 0xFFFFu, hi.y >> 16};
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double c = cs[kPairsPerItem * s + e][0];
        const double sn = cs[kPairsPerItem * s + e][1];
        const double x0 = widen_bf16(a[e]);
        const double x1 = widen_bf16(b[e]);
        ra[e] = round_bf16(x0 * c - x1 * sn);
        rb[e] = round_bf16(x1 * c + x0 * sn);
    }
    *reinterpret_cast<uint2 *>(dst + kPairsPerItem * s) = make_uint2(ra[0] | (ra[1] << 16), ra[2] | (ra[3] << 16));
    *reinterpret_cast<uint2 *>(dst + kHalfDim + kPairsPerItem * s) =
        make_uint2(rb[0] | (rb[1] << 16), rb[2] | (rb[3] << 16));
}

template <bool ROPE, bool HAS_Q>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a)
{
    __shared__ double cs[kHalfDim][2];

    // Everything up to the rotation table is uniform across the workgroup,
    // so the early returns leave no thread waiting at the barrier.
    const int bid = blockIdx.x;
    const int b = bid / a.max_new;
    const int j = bid - b * a.max_new;
    const int ctx = a.context_lens[b];
    int start, n;
    if (a.new_start != nullptr) {
        start = a.new_start[b];
        n = a.new_start[b + 1] - start;
    } else {
        start = b;
        n = ctx > 0 ? 1 : 0;
    }
    // A request that breaks the contract (more new tokens than its context or
    // the host bound, rows outside the inputs) writes nothing at all.
    if (j >= n || n > ctx || n > a.max_new || start < 0 || (int64_t)start + n > a.num_rows)
        return;
    const int pos = ctx - n + j;
    const int blk = pos / kPageSize;
    if (blk >= a.max_blocks)
        return;
    const int page = a.block_table[(size_t)b * a.max_blocks + blk];
    if ((unsigned)page >= (unsigned)a.num_pages)
        return;
    const size_t row = (size_t)start + j;
    const size_t slot = (size_t)page * kPageSize + pos % kPageSize;

    if (ROPE) {
        if (threadIdx.x < kHalfDim) {
            const int i = threadIdx.x;
            const double freq = pow(a.theta, -2.0 * (double)i / (double)kHeadDim);
            double sn, c;
            sincos((double)pos * freq, &sn, &c);
            cs[i][0] = c;
            cs[i][1] = sn;
        }
        __syncthreads();
    }

    const size_t kv_row = (size_t)a.num_kv_heads * kHeadDim;
    const uint16_t *kn = a.k_new + row * kv_row;
    const uint16_t *vn = a.v_new + row * kv_row;
    uint16_t *kd = a.k_pool + slot * kv_row;
    uint16_t *vd = a.v_pool + slot * kv_row;
    const int n_kv = a.num_kv_heads * kItemsPerHead;
    const int n_q = HAS_Q ? a.num_q_heads * kItemsPerHead : 0;
    const int total = 2 * n_kv + n_q;
    for (int it = threadIdx.x; it < total; it += kAppendThreads) {
        if (it < n_kv) {
            if (ROPE) {
                const int h = it / kItemsPerHead;
                rotate_item(kn + h * kHeadDim, kd + h * kHeadDim, it % kItemsPerHead, cs);
            } else {
                copy16(kn + it * 8, kd + it * 8);
            }
        } else if (it < 2 * n_kv) {
            const int c = it - n_kv;
            copy16(vn + c * 8, vd + c * 8);
        } else if (HAS_Q) {
            const int c = it - 2 * n_kv;
            const int h = c / kItemsPerHead;
            uint16_t *qh = a.q + (row * a.num_q_heads + h) * kHeadDim;
            rotate_item(qh, qh, c % kItemsPerHead, cs);
        }
    }
}

hipdecode_status check_append(const hipdecode_append_params *pp)
{
    if (pp == nullptr)
        return HIPDECODE_ERR_NULL;
    const hipdecode_append_params &p = *pp;
    if (p.num_seqs < 0 || p.num_q_heads <= 0 || p.num_kv_heads <= 0 || p.head_dim <= 0 ||
        p.page_size <= 0 || p.num_pages <= 0 || p.max_blocks_per_seq < 0 || p.num_rows < 0 ||
        p.max_new_tokens < 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.num_q_heads % p.num_kv_heads != 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.head_dim != kHeadDim || p.page_size != kPageSize)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.rope != HIPDECODE_ROPE_NONE && p.rope != HIPDECODE_ROPE_HALF)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.rope != HIPDECODE_ROPE_NONE && !(isfinite(p.rope_theta) && p.rope_theta > 0.0))
        return HIPDECODE_ERR_SCALE;
    // rows and heads fit the 32-bit item arithmetic; the grid fits one dimension
    if ((int64_t)p.num_q_heads * kItemsPerHead > (int64_t)1 << 30 ||
        (int64_t)p.num_seqs * (p.max_new_tokens > 0 ? p.max_new_tokens : 1) >= kMaxGrid)
        return HIPDECODE_ERR_SHAPE;
    return HIPDECODE_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace
}  // namespace hipdecode

using namespace hipdecode;

HIPDECODE_API hipdecode_status hipdecode_check_append_params(const hipdecode_append_params *params)
{
    return check_append(params);
}

HIPDECODE_API hipdecode_status hipdecode_kv_append(const hipdecode_append_params *params, void *q,
                                                   const void *k_new, const void *v_new,
                                                   const int32_t *new_start, const int32_t *block_table,
                                                   const int32_t *context_lens, void *k_pool, void *v_pool,
                                                   void *stream)
{
    const hipdecode_status st = check_append(params);
    if (st != HIPDECODE_OK)
        return st;
    const hipdecode_append_params &p = *params;
    if (new_start == nullptr && p.num_rows < p.num_seqs)
        return HIPDECODE_ERR_SHAPE;
    const int32_t max_new = new_start == nullptr ? 1 : p.max_new_tokens;
    if (p.num_seqs == 0 || max_new == 0 || p.num_rows == 0)
        return HIPDECODE_OK;
    if (k_new == nullptr || v_new == nullptr || block_table == nullptr || context_lens == nullptr ||
        k_pool == nullptr || v_pool == nullptr)
        return HIPDECODE_ERR_NULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
        (q != nullptr && !aligned(q, 16)) || !aligned(block_table, 4) || !aligned(context_lens, 4) ||
        (new_start != nullptr && !aligned(new_start, 4)))
        return HIPDECODE_ERR_ALIGN;

    AppendArgs a;
    a.q = static_cast<uint16_t *>(q);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.new_start = new_start;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.k_pool = static_cast<uint16_t *>(k_pool);
    a.v_pool = static_cast<uint16_t *>(v_pool);
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.num_pages = p.num_pages;
    a.max_blocks = p.max_blocks_per_seq;
    a.num_rows = p.num_rows;
    a.max_new = max_new;
    a.theta = p.rope_theta;

    const dim3 grid((unsigned)((int64_t)p.num_seqs * max_new));
    const dim3 block(kAppendThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.rope == HIPDECODE_ROPE_NONE)
        hipLaunchKernelGGL((kv_append_kernel<false, false>), grid, block, 0, s, a);
    else if (q == nullptr)
        hipLaunchKernelGGL((kv_append_kernel<true, false>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((kv_append_kernel<true, true>), grid, block, 0, s, a);
    return hipGetLastError() == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
}
