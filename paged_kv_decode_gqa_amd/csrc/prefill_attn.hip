// prefill_attn.hip -- chunked-prefill attention over the paged KV cache on
// MFMA, and the extern "C" entry points hipdecode_check_prefill_params and
// hipdecode_prefill_attn.
//
// Prefill processes a long prompt in chunks of query tokens over the cache
// (MOSS-TD article, "Chunked prefill for long audio"): after a chunk's keys
// and values have been appended, chunk token j of request b (position
// p = c_b - n_b + j) attends to cached tokens 0 .. p.  Unlike a decode step
// this is a dense contraction (many queries per key), so it runs on the
// matrix cores.
//
// Work decomposition.  One workgroup of eight wavefronts per (request, KV
// head, tile of query tokens).  A wavefront owns 32 query rows -- 32/G chunk
// tokens times the G query heads that share the KV head -- which is one
// 32x32 MFMA tile, so a workgroup holds 256 rows: every K/V byte brought into
// LDS serves 256 rows, which keeps the re-reads of the context (one pass per
// tile) within what the caches deliver.  Keys go by in steps of 64 (four
// pages), staged in LDS and double-buffered -- K row-major, V transposed --
// and used in two halves of 32.
//
// Per step and wavefront, with v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32):
//   S^T[key][row]  = sum_d K[key][d] Q[row][d]        8 MFMAs, A = K, B = Q^T
//   O^T[dim][row] += sum_key V[key][dim] P[row][key]  8 MFMAs, A = V^T, B = P^T
// Lane l of the S^T accumulator holds row l % 32 and keys
// 8(r/4) + 4(l/32) + r%4 for registers r = 0..15, which is exactly how the
// B operand of the second product wants P^T, provided both products agree
// on the order of the key index: V^T is stored in LDS with bits 2 and 3 of
// the key index swapped, so that each lane's eight keys are one contiguous
// 16-byte read.  The softmax is online, in base 2 with scale*log2(e) folded
// in (one FMA and one v_exp_f32 per score); the two lanes (l, l ^ 32) that
// share a row combine their maxima with v_permlane32_swap.  P is rounded to bf16 for the matrix cores; the running
// sum uses the fp32 values.
#include "hipdecode.h"
#include "internal.h"

#include <math.h>

namespace hipdecode {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRowsPerWave = 32;          // one 32x32 MFMA tile of (token, head) rows
constexpr int kKeys = 64;                 // keys per LDS step: four pages, used in two halves of 32
constexpr int kKStride = kHeadDim + 8;    // LDS K row, bf16 elements (16 B of padding)
constexpr int kVStride = kKeys + 8;       // LDS V^T row (one dimension), bf16 elements
constexpr int kDimBlocks = kHeadDim / 32; // O^T is four 32x32 accumulators
constexpr float kNegBig = -1.0e30f;       // running-max start: finite, so no inf - inf
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *new_start;
    const int32_t *block_table;
    const int32_t *context_lens;
    void *out;
    float *lse;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_blocks;
    int32_t num_rows;
    int32_t max_new;
    int32_t tiles;          // query tiles per request
    float scale_log2;       // max(|scale| * log2(e), 2^-100): positive, see the launch
    uint32_t q_sign;        // 0x80008000 when scale < 0: q is negated on load instead
};

// Position of key index t inside an LDS row of V^T: bits 2 and 3 swapped.
__device__ inline int vt_slot(int t) { return (t & ~0xC) | ((t & 4) << 1) | ((t & 8) >> 1); }

__device__ inline float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline f32x16_t zero16()
{
    f32x16_t z;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        z[i] = 0.f;
    return z;
}

__device__ inline uint32_t pack2_bf16(float x, float y)
{
    const f32x2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int G, bool OUT_F32>
__global__ __launch_bounds__(kPfThreads) void prefill_attn_kernel(PrefillArgs a)
{
    constexpr int kTokPerWave = kRowsPerWave / G;
    constexpr int kTileTokens = kPfWaves * kTokPerWave;
    __shared__ __align__(16) uint16_t k_lds[2][kKeys * kKStride];
    __shared__ __align__(16) uint16_t vt_lds[2][kHeadDim * kVStride];

    // KV head fastest, heavier (later) tiles first.
    const int bid = blockIdx.x;
    const int g = bid % a.num_kv_heads;
    const int rest = bid / a.num_kv_heads;
    const int tile = a.tiles - 1 - rest % a.tiles;
    const int b = rest / a.tiles;
    const int ctx = a.context_lens[b];
    const int start = a.new_start[b];
    const int n = a.new_start[b + 1] - start;
    const int t0 = tile * kTileTokens;
    // Uniform across the workgroup: a request that breaks the contract, or a
    // tile past its chunk, does nothing.
    if (n <= 0 || n > ctx || n > a.max_new || start < 0 || (int64_t)start + n > a.num_rows || t0 >= n ||
        (int64_t)ctx > (int64_t)a.max_blocks * kPageSize)
        return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;          // this lane's row in the wavefront's tile
    const int half = lane >> 5;       // which 8 of each 16 along the contracted index
    const int tq = t0 + w * kTokPerWave + j / G;
    const int h = g * G + j % G;
    const bool row_ok = tq < n;
    const int pos = row_ok ? ctx - n + tq : -1;      // -1: every key masked
    const size_t row = (size_t)start + min(tq, n - 1);

    // Q^T operand: dims 16 ks + 8 half .. +7 of this lane's row.  A negative
    // scale is applied as a sign flip of q (exact), so that the scale factor
    // used below is never negative and the row maximum of scale * s is
    // scale times the maximum of s.
    bf16x8_t qop[kHeadDim / 16];
    {
        const uint16_t *qrow = a.q + (row * a.num_q_heads + h) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks) {
            uint4 u = *reinterpret_cast<const uint4 *>(qrow + 16 * ks + 8 * half);
            u.x ^= a.q_sign;
            u.y ^= a.q_sign;
            u.z ^= a.q_sign;
            u.w ^= a.q_sign;
            qop[ks] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    const int tile_last = min(t0 + kTileTokens, n) - 1;
    const int kv_end = ctx - n + tile_last + 1;          // keys [0, kv_end)
    const int nblk = (kv_end + kKeys - 1) / kKeys;
    const int full_blk = (ctx - n + t0 + 1) / kKeys;      // steps with no masked key in any row

    // Staging: for K, thread tid moves dims 8 dc .. 8 dc + 7 of keys 2 tp and
    // 2 tp + 1 (always on one page; 16 consecutive threads read a key's whole
    // row).  For V the key pair varies fastest instead (vp = tid % 32, dims
    // 8 vd .. 8 vd + 7 with vd = tid / 32), so that the transposed 4-byte
    // writes of one wavefront -- 32 key pairs of two dimensions -- fall on 64
    // different LDS banks.  Pipeline: at step kb the K/V loads of step kb + 2
    // are issued, with a page id fetched one step earlier, and the page id of
    // step kb + 3 is fetched; step kb + 1 goes from registers to LDS at the end
    // of step kb.  Keys past kv_end are clamped to the last one (masked).
    const int dc = tid & 15;
    const int tp = tid >> 4;
    const int vp = tid & 31;
    const int vd = tid >> 5;
    const size_t kv_row = (size_t)a.num_kv_heads * kHeadDim;
    const int32_t *table = a.block_table + (size_t)b * a.max_blocks;
    auto first_key = [&](int kb) __attribute__((always_inline)) { return min(kb * kKeys + 2 * tp, kv_end - 1); };
    auto page_of = [&](int kb) __attribute__((always_inline)) {
        const int blk = min(first_key(kb) / kPageSize, a.max_blocks - 1);
        const int page = table[blk];
        return (unsigned)page < (unsigned)a.num_pages ? page : 0;
    };
    auto v_first_key = [&](int kb) __attribute__((always_inline)) { return min(kb * kKeys + 2 * vp, kv_end - 1); };
    auto v_page_of = [&](int kb) __attribute__((always_inline)) {
        const int blk = min(v_first_key(kb) / kPageSize, a.max_blocks - 1);
        const int page = table[blk];
        return (unsigned)page < (unsigned)a.num_pages ? page : 0;
    };
    auto offsets = [&](int key0, int page, int chunk, size_t &o0, size_t &o1) __attribute__((always_inline)) {
        const int key1 = min(key0 + 1, kv_end - 1);
        const size_t base = (size_t)page * kPageSize * kv_row + (size_t)g * kHeadDim + chunk * 8;
        o0 = base + (size_t)(key0 % kPageSize) * kv_row;
        o1 = base + (size_t)(key1 % kPageSize) * kv_row;
    };

    f32x16_t acc[kDimBlocks];
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
        acc[db] = zero16();
    float m_run = kNegBig;
    float l_run = 0.f;

    auto scores = [&](int buf, int hh) __attribute__((always_inline)) {
        // S^T = K Q^T for keys 32 hh .. 32 hh + 31 of this step
        f32x16_t s = zero16();
        const uint16_t *kl = &k_lds[buf][(32 * hh + j) * kKStride + 8 * half];
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks) {
            const bf16x8_t kop = *reinterpret_cast<const bf16x8_t *>(kl + 16 * ks);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s, 0, 0, 0);
        }
        return s;
    };
    auto softmax_pv = [&](int kb, int buf, int hh, f32x16_t s) __attribute__((always_inline)) {

        // Online softmax in base 2 (row j; keys 8(r/4) + 4 half + r%4).  With
        // c = |scale| log2(e) > 0, the row maximum of c s is c max(s) and
        // p = 2^(c s - m) is one FMA and one v_exp_f32 (weights below 2^-126
        // of the row maximum may flush to zero); a masked score is -inf, so
        // its weight is exactly 0.
        if (kb >= full_blk) {  // only steps reaching past the tile's first position
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * kKeys + 32 * hh + 8 * (r / 4) + 4 * half + (r % 4);
                s[r] = key > pos ? -INFINITY : s[r];
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mx = fmaxf(mx, s[r]);
        const float c = a.scale_log2;
        const float m_new = fmaxf(m_run, pair_max(mx) * c);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        uint32_t pp[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m_new));   // masked: 2^-inf = 0
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -m_new));
            psum += p0 + p1;
            pp[r / 2] = pack2_bf16(p0, p1);
        }
        l_run = l_run * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                acc[db] *= alpha;
        }

        // O^T += V^T P^T, two k-steps of 16 keys
        const uint16_t *vl = &vt_lds[buf][j * kVStride + 32 * hh + 8 * half];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const uint4 u = make_uint4(pp[4 * kh], pp[4 * kh + 1], pp[4 * kh + 2], pp[4 * kh + 3]);
            const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, u);
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) {
                const bf16x8_t vop = *reinterpret_cast<const bf16x8_t *>(vl + (32 * db) * kVStride + 16 * kh);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, acc[db], 0, 0, 0);
            }
        }
    };
    // Both halves' scores are issued first: the matrix cores work on the
    // second half's S while the first half's softmax runs on the VALU, and on
    // the first half's P.V while the second softmax runs.  (Staggering the
    // second wavefront of each SIMD by half a step, with a third LDS buffer,
    // measured 12% slower: it takes the kernel to 256 registers.)
    auto compute_step = [&](int kb, int buf) __attribute__((always_inline)) {
        const f32x16_t s0 = scores(buf, 0);
        const f32x16_t s1 = scores(buf, 1);
        softmax_pv(kb, buf, 0, s0);
        softmax_pv(kb, buf, 1, s1);
    };

    // Two register stages, A and B, alternate; the loop is unrolled by two so
    // that every register is named statically.
    uint4 a_k0, a_k1, a_v0, a_v1, b_k0, b_k1, b_v0, b_v1;
#define HIPDECODE_PF_LOAD(P, KB, PAGE, VPAGE)                                   \
    do {                                                                        \
        size_t o0_, o1_;                                                        \
        offsets(first_key(KB), (PAGE), dc, o0_, o1_);                           \
        P##_k0 = *reinterpret_cast<const uint4 *>(a.k_pool + o0_);              \
        P##_k1 = *reinterpret_cast<const uint4 *>(a.k_pool + o1_);              \
        offsets(v_first_key(KB), (VPAGE), vd, o0_, o1_);                        \
        P##_v0 = *reinterpret_cast<const uint4 *>(a.v_pool + o0_);              \
        P##_v1 = *reinterpret_cast<const uint4 *>(a.v_pool + o1_);              \
    } while (0)
#define HIPDECODE_PF_STORE(P, BUF) store_step(P##_k0, P##_k1, P##_v0, P##_v1, (BUF))
    auto store_step = [&](uint4 k0, uint4 k1, uint4 v0, uint4 v1, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<uint4 *>(&k_lds[buf][(2 * tp) * kKStride + dc * 8]) = k0;
        *reinterpret_cast<uint4 *>(&k_lds[buf][(2 * tp + 1) * kKStride + dc * 8]) = k1;
        // V^T: dimensions 8 vd + 2 i and 8 vd + 2 i + 1, keys 2 vp and 2 vp + 1 side by side
        uint16_t *vt = &vt_lds[buf][(vd * 8) * kVStride + vt_slot(2 * vp)];
        const uint32_t x0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t x1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint32_t *>(vt + (2 * i) * kVStride) = (x0[i] & 0xFFFFu) | (x1[i] << 16);
            *reinterpret_cast<uint32_t *>(vt + (2 * i + 1) * kVStride) = (x0[i] >> 16) | (x1[i] & 0xFFFF0000u);
        }
    };

    int page_ahead = 0, vpage_ahead = 0;      // pages of step kb + 2 (K and V mappings)
    HIPDECODE_PF_LOAD(a, 0, page_of(0), v_page_of(0));
    if (nblk > 1)
        HIPDECODE_PF_LOAD(b, 1, page_of(1), v_page_of(1));
    if (nblk > 2) {
        page_ahead = page_of(2);
        vpage_ahead = v_page_of(2);
    }
    HIPDECODE_PF_STORE(a, 0);
    __syncthreads();
    for (int kb = 0; kb < nblk; kb += 2) {
        // step kb: A is free (step kb is in LDS), B holds step kb + 1
        if (kb + 2 < nblk)
            HIPDECODE_PF_LOAD(a, kb + 2, page_ahead, vpage_ahead);
        if (kb + 3 < nblk) {
            page_ahead = page_of(kb + 3);
            vpage_ahead = v_page_of(kb + 3);
        }
        compute_step(kb, 0);
        if (kb + 1 < nblk)
            HIPDECODE_PF_STORE(b, 1);
        __syncthreads();
        if (kb + 1 >= nblk)
            break;
        // step kb + 1: B is free, A holds step kb + 2
        if (kb + 3 < nblk)
            HIPDECODE_PF_LOAD(b, kb + 3, page_ahead, vpage_ahead);
        if (kb + 4 < nblk) {
            page_ahead = page_of(kb + 4);
            vpage_ahead = v_page_of(kb + 4);
        }
        compute_step(kb + 1, 1);
        if (kb + 2 < nblk)
            HIPDECODE_PF_STORE(a, 0);
        __syncthreads();
    }
#undef HIPDECODE_PF_LOAD
#undef HIPDECODE_PF_STORE

    // Rows: out[row][h][dim], dims 32 db + 8 (r/4) + 4 half + r%4.
    const float l_tot = pair_sum(l_run);
    if (!row_ok)
        return;
    const float inv = 1.f / l_tot;
    if (OUT_F32) {
        float *o = static_cast<float *>(a.out) + (row * a.num_q_heads + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                *reinterpret_cast<float4 *>(o + 32 * db + 8 * rr + 4 * half) =
                    make_float4(acc[db][4 * rr] * inv, acc[db][4 * rr + 1] * inv, acc[db][4 * rr + 2] * inv,
                                acc[db][4 * rr + 3] * inv);
    } else {
        uint16_t *o = static_cast<uint16_t *>(a.out) + (row * a.num_q_heads + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                *reinterpret_cast<uint2 *>(o + 32 * db + 8 * rr + 4 * half) =
                    make_uint2(pack2_bf16(acc[db][4 * rr] * inv, acc[db][4 * rr + 1] * inv),
                               pack2_bf16(acc[db][4 * rr + 2] * inv, acc[db][4 * rr + 3] * inv));
    }
    if (a.lse != nullptr && half == 0)
        a.lse[row * a.num_q_heads + h] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
}

hipdecode_status check_prefill(const hipdecode_prefill_params *pp)
{
    if (pp == nullptr)
        return HIPDECODE_ERR_NULL;
    const hipdecode_prefill_params &p = *pp;
    if (p.num_seqs < 0 || p.num_q_heads <= 0 || p.num_kv_heads <= 0 || p.head_dim <= 0 ||
        p.page_size <= 0 || p.num_pages <= 0 || p.max_blocks_per_seq < 1 || p.num_rows < 0 ||
        p.max_new_tokens < 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.num_q_heads % p.num_kv_heads != 0)
        return HIPDECODE_ERR_SHAPE;
    const int group = p.num_q_heads / p.num_kv_heads;
    if (p.head_dim != kHeadDim || p.page_size != kPageSize || (group != 1 && group != 2 && group != 4))
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.out_dtype != HIPDECODE_BF16 && p.out_dtype != HIPDECODE_F32)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (!isfinite(p.scale))
        return HIPDECODE_ERR_SCALE;
    const int64_t tile_tokens = kPfWaves * (kRowsPerWave / group);
    const int64_t tiles = ((int64_t)p.max_new_tokens + tile_tokens - 1) / tile_tokens;
    if ((int64_t)p.num_seqs * tiles * p.num_kv_heads >= kMaxGrid)
        return HIPDECODE_ERR_SHAPE;
    return HIPDECODE_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int G>
hipError_t launch_g(const PrefillArgs &a, unsigned grid, bool out_f32, hipStream_t s)
{
    if (out_f32)
        hipLaunchKernelGGL((prefill_attn_kernel<G, true>), dim3(grid), dim3(kPfThreads), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_attn_kernel<G, false>), dim3(grid), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace hipdecode

using namespace hipdecode;

HIPDECODE_API hipdecode_status hipdecode_check_prefill_params(const hipdecode_prefill_params *params)
{
    return check_prefill(params);
}

HIPDECODE_API hipdecode_status hipdecode_prefill_attn(const hipdecode_prefill_params *params, const void *q,
                                                      const void *k_pool, const void *v_pool,
                                                      const int32_t *new_start, const int32_t *block_table,
                                                      const int32_t *context_lens, void *out, float *lse,
                                                      void *stream)
{
    const hipdecode_status st = check_prefill(params);
    if (st != HIPDECODE_OK)
        return st;
    const hipdecode_prefill_params &p = *params;
    if (p.num_seqs == 0 || p.max_new_tokens == 0 || p.num_rows == 0)
        return HIPDECODE_OK;
    if (q == nullptr || k_pool == nullptr || v_pool == nullptr || new_start == nullptr ||
        block_table == nullptr || context_lens == nullptr || out == nullptr)
        return HIPDECODE_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
        !aligned(new_start, 4) || !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(lse, 4))
        return HIPDECODE_ERR_ALIGN;

    const int group = p.num_q_heads / p.num_kv_heads;
    const int tile_tokens = kPfWaves * (kRowsPerWave / group);
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_pool = static_cast<const uint16_t *>(k_pool);
    a.v_pool = static_cast<const uint16_t *>(v_pool);
    a.new_start = new_start;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    a.lse = lse;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.num_pages = p.num_pages;
    a.max_blocks = p.max_blocks_per_seq;
    a.num_rows = p.num_rows;
    a.max_new = p.max_new_tokens;
    a.tiles = (p.max_new_tokens + tile_tokens - 1) / tile_tokens;
    // c = |scale| log2(e), kept at least 2^-100 so that c * -inf = -inf: for
    // any scale that small every weight 2^(c s - m) is 1.0f anyway (|s| stays
    // far below 2^70), so scale 0 still gives the mean of V and ln(n).
    a.scale_log2 = fmaxf(fabsf(p.scale) * 1.44269504088896340736f, 0x1p-100f);
    a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * a.tiles * p.num_kv_heads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f32 = p.out_dtype == HIPDECODE_F32;
    hipError_t e;
    if (group == 1)
        e = launch_g<1>(a, grid, f32, s);
    else if (group == 2)
        e = launch_g<2>(a, grid, f32, s);
    else
        e = launch_g<4>(a, grid, f32, s);
    return e == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
}
