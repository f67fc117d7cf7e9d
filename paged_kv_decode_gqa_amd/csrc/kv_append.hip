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
// Each new token is handled by one wavefront (four tokens per workgroup) or,
// when there are few tokens, by all four wavefronts of a workgroup; no
// workgroup barrier is used.  Lane l always works on dimension pairs
// [4s, 4s+4) with s = l % 16 (and the pair partner i + 64 of each), so it needs
// only four rotation angles; each wavefront evaluates the token's 64 angles in
// fp64, lane i the angle of pair i, and shares them through its own slice of
// LDS.  The input rows are loaded before the block table and the angles are
// looked at, so those latencies overlap.  A rotated value is computed in fp64
// and rounded once to bf16 (see round_to_odd_f32).  The work is a few KB per
// token: HBM-bound for prefill chunks, latency-bound for one decode token per
// request.
#include "hipdecode.h"
#include "internal.h"
#include "rope_round.h"

#include <math.h>

namespace hipdecode {
namespace {

constexpr int kAppendWaves = 4;                 // wavefronts per workgroup
constexpr int kAppendThreads = 64 * kAppendWaves;
constexpr int kHalfDim = kHeadDim / 2;          // rotation pairs per head
constexpr int kPairsPerItem = 4;
constexpr int kItemsPerHead = kHalfDim / kPairsPerItem;   // also the 16-byte chunks of one head's row
constexpr int kRotPre = 6;    // rotation items loaded ahead per wavefront-token: 8 K heads + 16 q heads
constexpr int kCopyPre = 4;   // 16-byte chunks loaded ahead: V (and K without RoPE) of 8 heads
constexpr int64_t kMaxGrid = (int64_t)1 << 31;
constexpr int64_t kFewTokens = 1024;            // up to this many, four wavefronts share each token

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
    int32_t token_groups;   // workgroups per request: ceil(max_new / tokens per workgroup)
    double log2_theta;      // with RoPE: log2 of its theta
    uint32_t *violations;   // contract-violation flag word of this device
};

using rope::bf16x2_t;
using rope::f32x2_t;
using rope::pack_bf16;

// Every row is read once and written once per call: non-temporal accesses
// stream them past the caches (measured 2.7% faster on a 4,096-token chunk).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint4 load16(const uint16_t *p)
{
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store16(uint16_t *p, uint4 v)
{
    __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4 *>(p));
}
__device__ inline uint2 load8(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ inline void store8(uint16_t *p, uint2 v)
{
    __builtin_nontemporal_store(nt_u32x2{v.x, v.y}, reinterpret_cast<nt_u32x2 *>(p));
}

// Rotates four pairs: element e of lo pairs with element e of hi.
//
// Fast rounding: t = fp32 nearest of the fp64 value y, then bf16 nearest even
// of t.  Every bf16 rounding boundary (a midpoint between bf16 neighbours) is
// an fp32 number and rounding is monotonic, so t lies on the same side of
// each boundary as y unless t is itself a boundary; the two roundings then
// agree with the direct one.  Items where some t is a boundary (low 16 bits
// 0x8000, probability about 2^-16 per value) or NaN take the exact path.
__device__ inline void rotate4(uint2 lo, uint2 hi, const double2 (&cs)[kPairsPerItem], uint2 &out_lo,
                               uint2 &out_hi)
{
    const uint32_t a[4] = {lo.x << 16, lo.x & 0xFFFF0000u, lo.y << 16, lo.y & 0xFFFF0000u};
    const uint32_t b[4] = {hi.x << 16, hi.x & 0xFFFF0000u, hi.y << 16, hi.y & 0xFFFF0000u};
    double y0[4], y1[4];
    float t0[4], t1[4];
    bool unsure = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double x0 = (double)__uint_as_float(a[e]);
        const double x1 = (double)__uint_as_float(b[e]);
        y0[e] = x0 * cs[e].x - x1 * cs[e].y;
        y1[e] = x1 * cs[e].x + x0 * cs[e].y;
        t0[e] = (float)y0[e];
        t1[e] = (float)y1[e];
        unsure |= (__float_as_uint(t0[e]) & 0xFFFFu) == 0x8000u || t0[e] != t0[e];
        unsure |= (__float_as_uint(t1[e]) & 0xFFFFu) == 0x8000u || t1[e] != t1[e];
    }
    if (__builtin_expect(unsure, 0)) {
        out_lo = make_uint2(pack_bf16(y0[0], y0[1]), pack_bf16(y0[2], y0[3]));
        out_hi = make_uint2(pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3]));
        return;
    }
    auto cvt = [](float x, float y) {
        const f32x2_t v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    };
    out_lo = make_uint2(cvt(t0[0], t0[1]), cvt(t0[2], t0[3]));
    out_hi = make_uint2(cvt(t1[0], t1[1]), cvt(t1[2], t1[3]));
}

// WPT: wavefronts per token, 1 or 4.
template <bool ROPE, bool HAS_Q, int WPT>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a)
{
    constexpr int kTokensPerGroup = kAppendWaves / WPT;
    constexpr int kRot = (kRotPre + WPT - 1) / WPT;              // rotation items per lane loaded ahead
    constexpr int kCopies = ((ROPE ? kCopyPre / 2 : kCopyPre) + WPT - 1) / WPT;
    __shared__ double2 angles[kAppendWaves][kHalfDim];   // (cos, sin) of each pair, per wavefront

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wt = w % WPT;                               // this wavefront's share of its token
    const int b = blockIdx.x / a.token_groups;
    const int j = (blockIdx.x - b * a.token_groups) * kTokensPerGroup + w / WPT;
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
    // the host bound, rows outside the inputs) writes nothing at all.  All of
    // this is uniform across the wavefront, and nothing below waits for the
    // other wavefronts, so a wavefront may leave on its own.
    const bool rows_bad = n < 0 || n > max(ctx, 0) || n > a.max_new || start < 0 || (int64_t)start + n > a.num_rows;
    if (j >= n || rows_bad) {
        if (lane == 0 && (rows_bad || ctx < 0))
            report_violation(a.violations, (rows_bad ? HIPDECODE_VIOLATION_ROWS : 0u) |
                                               (ctx < 0 ? HIPDECODE_VIOLATION_CONTEXT : 0u));
        return;
    }
    const int pos = ctx - n + j;
    const size_t row = (size_t)start + j;
    const size_t kv_row = (size_t)a.num_kv_heads * kHeadDim;
    const int kv_items = a.num_kv_heads * kItemsPerHead;
    const int rot_items = (ROPE ? kv_items : 0) + (HAS_Q ? a.num_q_heads * kItemsPerHead : 0);
    const int copy_items = (ROPE ? 0 : kv_items) + kv_items;
    const int s = lane % kItemsPerHead;   // the same for every item of this lane

    // Rotation item it: K head it / 16 (with RoPE), then q heads.  Copy item c:
    // K 16-byte chunk c (without RoPE), then V chunks.
    auto rot_src = [&](int it) -> const uint16_t * {
        if (ROPE && it < kv_items)
            return a.k_new + row * kv_row + (size_t)(it / kItemsPerHead) * kHeadDim;
        return a.q + (row * a.num_q_heads + (it - (ROPE ? kv_items : 0)) / kItemsPerHead) * kHeadDim;
    };
    auto copy_src = [&](int c) -> const uint16_t * {
        if (!ROPE && c < kv_items)
            return a.k_new + row * kv_row + (size_t)c * 8;
        return a.v_new + row * kv_row + (size_t)(c - (ROPE ? 0 : kv_items)) * 8;
    };

    // Item k of this lane is lane + 64 * (wt + WPT * k).  Loads are issued for
    // every preloaded item without branches (indices past the end are clamped
    // to the last item and their results dropped), copy chunks first, so the
    // compiler can count them exactly and the angle evaluation below overlaps
    // them.
    auto item = [&](int k) { return lane + 64 * (wt + WPT * k); };
    uint4 cp[kCopies];
#pragma unroll
    for (int k = 0; k < kCopies; ++k)
        cp[k] = load16(copy_src(min(item(k), copy_items - 1)));
    uint2 lo[kRot], hi[kRot];
    if (ROPE) {
#pragma unroll
        for (int k = 0; k < kRot; ++k) {
            const uint16_t *src = rot_src(min(item(k), rot_items - 1));
            lo[k] = load8(src + kPairsPerItem * s);
            hi[k] = load8(src + kHalfDim + kPairsPerItem * s);
        }
    }

    const int blk = pos / kPageSize;
    if (blk >= a.max_blocks) {
        if (lane == 0)
            report_violation(a.violations, HIPDECODE_VIOLATION_CONTEXT);
        return;
    }
    const int page = a.block_table[(size_t)b * a.max_blocks + blk];
    if ((unsigned)page >= (unsigned)a.num_pages) {
        if (lane == 0)
            report_violation(a.violations, HIPDECODE_VIOLATION_PAGE);
        return;
    }
    const size_t slot = (size_t)page * kPageSize + pos % kPageSize;
    uint16_t *kd = a.k_pool + slot * kv_row;
    uint16_t *vd = a.v_pool + slot * kv_row;
    auto rot_dst = [&](int it) -> uint16_t * {
        if (ROPE && it < kv_items)
            return kd + (it / kItemsPerHead) * kHeadDim;
        return a.q + (row * a.num_q_heads + (it - (ROPE ? kv_items : 0)) / kItemsPerHead) * kHeadDim;
    };
    auto copy_dst = [&](int c) -> uint16_t * {
        if (!ROPE && c < kv_items)
            return kd + c * 8;
        return vd + (c - (ROPE ? 0 : kv_items)) * 8;
    };

    double2 cs[kPairsPerItem];
    if (ROPE) {
        // lane i: the angle of pair i, evaluated in fp64
        angles[w][lane] = rope::angle_of(rope::frequency(a.log2_theta, lane), pos);
        // LDS operations of one wavefront complete in order; this keeps the
        // compiler from moving the reads above the write.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int e = 0; e < kPairsPerItem; ++e)
            cs[e] = angles[w][kPairsPerItem * s + e];
    }

#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
        const int c = item(k);
        if (c < copy_items)
            store16(copy_dst(c), cp[k]);
    }
    for (int c = item(kCopies); c < copy_items; c += 64 * WPT)
        store16(copy_dst(c), load16(copy_src(c)));

    if (ROPE) {
#pragma unroll
        for (int k = 0; k < kRot; ++k) {
            const int it = item(k);
            if (it < rot_items) {
                uint2 ol, oh;
                rotate4(lo[k], hi[k], cs, ol, oh);
                uint16_t *dst = rot_dst(it);
                store8(dst + kPairsPerItem * s, ol);
                store8(dst + kHalfDim + kPairsPerItem * s, oh);
            }
        }
        for (int it = item(kRot); it < rot_items; it += 64 * WPT) {
            const uint16_t *src = rot_src(it);
            uint2 ol, oh;
            rotate4(load8(src + kPairsPerItem * s), load8(src + kHalfDim + kPairsPerItem * s), cs, ol, oh);
            uint16_t *dst = rot_dst(it);
            store8(dst + kPairsPerItem * s, ol);
            store8(dst + kHalfDim + kPairsPerItem * s, oh);
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
        (int64_t)p.num_seqs * (((int64_t)(p.max_new_tokens > 0 ? p.max_new_tokens : 1) + kAppendWaves - 1) /
                               kAppendWaves) >= kMaxGrid)
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
    a.log2_theta = p.rope != HIPDECODE_ROPE_NONE ? log2(p.rope_theta) : 0.0;
    a.violations = violation_word();

    // Few tokens (a decode step): four wavefronts per token, for latency.
    const bool few = (int64_t)p.num_seqs * max_new <= kFewTokens;
    const int tokens_per_group = few ? 1 : kAppendWaves;
    a.token_groups = (max_new + tokens_per_group - 1) / tokens_per_group;
    const dim3 grid((unsigned)((int64_t)p.num_seqs * a.token_groups));
    const dim3 block(kAppendThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the kernel's wavefronts per token must match tokens_per_group above
    const bool rope = p.rope != HIPDECODE_ROPE_NONE;
    const bool has_q = rope && q != nullptr;
    if (few) {
        if (!rope)
            hipLaunchKernelGGL((kv_append_kernel<false, false, kAppendWaves>), grid, block, 0, s, a);
        else if (!has_q)
            hipLaunchKernelGGL((kv_append_kernel<true, false, kAppendWaves>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((kv_append_kernel<true, true, kAppendWaves>), grid, block, 0, s, a);
    } else {
        if (!rope)
            hipLaunchKernelGGL((kv_append_kernel<false, false, 1>), grid, block, 0, s, a);
        else if (!has_q)
            hipLaunchKernelGGL((kv_append_kernel<true, false, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((kv_append_kernel<true, true, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
}
