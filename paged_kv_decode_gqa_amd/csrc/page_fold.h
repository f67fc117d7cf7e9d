// page_fold.h -- device helpers shared by the decode kernels: loading one
// 16-token page of one KV head into registers and folding it into online-
// softmax streams for the G query heads that share the KV head.
//
// Wavefront layout.  A page holds 16 tokens; for one KV head each token is a
// 256-byte row and rows are num_kv_heads*256 bytes apart.  Lane l of a
// wavefront belongs to row-group r = l / 16 and owns dims [8s, 8s+8) with
// s = l % 16; row-group r holds tokens r, r+4, r+8, r+12 of every page.  Each
// 16-byte load of the wavefront therefore reads four whole 256-byte rows.
//
// The four row-groups are independent softmax streams (own running max m and
// sum l, base-2 units), so the page loop needs no communication across
// row-groups; q.k partial sums are combined inside a row-group with four DPP
// steps.  p.v runs in fp32 FMAs on bf16 values widened exactly, so the
// softmax weights are never rounded.
#pragma once

#include "internal.h"

#include <math.h>

namespace hipdecode {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ u32x4 load16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row; every lane of the row receives it.
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp_f32<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_f32<0x141>(x);   // row_half_mirror: the other quad of each 8
    x += dpp_f32<0x140>(x);   // row_mirror: the other 8 of the row
    return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool F32>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v)
{
    if constexpr (F32)
        static_cast<float *>(out)[idx] = v;
    else
        static_cast<__bf16 *>(out)[idx] = static_cast<__bf16>(v);   // nearest, ties to even
}

// One page of one KV head: tokens row + 4t, dims [8s, 8s+8) of this lane.
struct PageRegs {
    u32x4 k[4];
    u32x4 v[4];
};

// A buffer resource for one page: the page's first byte as a wave-uniform
// 64-bit base in scalar registers, and a record limit no lane offset reaches
// (offsets stay inside the 32 KiB page).  Each lane then supplies only a
// 32-bit byte offset, so a pool may be any size.
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped) loads
constexpr int kCachePolicyNt = 2;          // non-temporal: stream through the caches

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_resource(const uint16_t *page)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(page), (short)0, 0x7fffffff, kBufferWord3);
}

// kpage/vpage: the page's first element (wave-uniform); lane_off: this
// lane's byte offset inside the page (head, row-group and dims); tok4: the
// byte distance of four slots.  K/V rows are read once per call:
// non-temporal loads stream them through the caches without displacing
// anything (measured 8-9% faster on MI355X; the scope bits sc0/sc1 on top
// of it measured no different).
__device__ __forceinline__ void load_page(PageRegs &r, const uint16_t *kpage, const uint16_t *vpage,
                                          uint32_t lane_off, uint32_t tok4)
{
    const __amdgpu_buffer_rsrc_t rk = page_resource(kpage);
    const __amdgpu_buffer_rsrc_t rv = page_resource(vpage);
#pragma unroll
    for (int t = 0; t < 4; ++t)
        r.k[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + t * tok4, 0,
                                                                                 kCachePolicyNt));
#pragma unroll
    for (int t = 0; t < 4; ++t)
        r.v[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + t * tok4, 0,
                                                                                 kCachePolicyNt));
}

template <int G>
struct Stream {
    float m[G];       // running max of scores, log2 units (-inf before any token)
    float l[G];       // running sum of 2^(score - m)
    float acc[G][8];  // running sum of 2^(score - m) * v over this lane's 8 dims

    __device__ __forceinline__ void init()
    {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[h][e] = 0.f;
        }
    }
};

// Fold one page into this row-group's stream.  MASK marks a request's last
// page: tokens at or past ctx get weight 0 through selects, so whatever the
// unused slots hold (NaN included) never enters the arithmetic.
template <int G, bool MASK>
__device__ __forceinline__ void fold_page(Stream<G> &st, const PageRegs &r, const u32x4 (&qv)[G],
                                          float scale_log2, int tok_first, int ctx)
{
    float s[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float d = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                d = dot2_bf16(r.k[t][w], qv[h][w], d);
            s[h][t] = row_sum16(d) * scale_log2;
        }

    bool valid[4] = {true, true, true, true};
    if constexpr (MASK) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            valid[t] = tok_first + 4 * t < ctx;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                s[h][t] = valid[t] ? s[h][t] : -INFINITY;
    }

    float p[G][4];
    float alpha[G];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float mx = fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3]));
        const float m_new = fmaxf(st.m[h], mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[h] = exp2_fast(st.m[h] - m_use);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            p[h][t] = exp2_fast(s[h][t] - m_use);
        st.l[h] = fmaf(st.l[h], alpha[h], (p[h][0] + p[h][1]) + (p[h][2] + p[h][3]));
        st.m[h] = m_new;
        rescale |= (alpha[h] != 1.0f);
    }
    // the running max rarely moves after the first pages: rescale only then
    if (__any(rescale)) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                st.acc[h][e] *= alpha[h];
    }

#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float vl[4], vh[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            vl[t] = bf16_lo(r.v[t][w]);
            vh[t] = bf16_hi(r.v[t][w]);
            if constexpr (MASK) {
                vl[t] = valid[t] ? vl[t] : 0.f;
                vh[t] = valid[t] ? vh[t] : 0.f;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float a0 = st.acc[h][2 * w], a1 = st.acc[h][2 * w + 1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a0 = fmaf(p[h][t], vl[t], a0);
                a1 = fmaf(p[h][t], vh[t], a1);
            }
            st.acc[h][2 * w] = a0;
            st.acc[h][2 * w + 1] = a1;
        }
    }
}

// Cross-workgroup data (split partials) is written and read only with
// relaxed device-scope atomics, which the gfx950 memory model keeps coherent
// across the XCDs' L2 caches.  Ordering against the arrival ticket comes from
// waiting for these stores to complete before the ticket increment.  This
// avoids the L2 writeback and invalidate that a device-scope fence issues,
// which would be paid by every workgroup.
__device__ __forceinline__ void coherent_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float coherent_load(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two consecutive floats, 8-byte aligned, as one 64-bit coherent load.
__device__ __forceinline__ uint64_t coherent_load8(const float *p)
{
    return __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Weight of a stream with running max m when merged under the overall max M
// (M_use is M, or 0 when every stream is empty).
__device__ __forceinline__ float merge_weight(float m, float M_use) { return exp2_fast(m - M_use); }

}  // namespace dev
}  // namespace hipdecode
