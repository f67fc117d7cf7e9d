// paged_decode.hip -- gfx950 kernels for one decode step of paged GQA attention.
//
// One workgroup owns one (request b, KV head g, split-K partition) triple and
// serves all G query heads that read KV head g (the 16-query/8-KV grouping of
// the audio.cpp "Decoder And Prompt" section), so every K/V byte of the cache
// is fetched from HBM exactly once per call.  The work is bound by HBM
// bandwidth: per cached token and query head it is 2x128 multiply-adds against
// 256 bytes of K and 256 bytes of V shared by the G heads.
//
// Wavefront layout.  A page holds 16 tokens of one KV head, each a 256-byte
// row, with rows num_kv_heads*256 bytes apart.  The 64 lanes of a wavefront
// form 8 octets; octet o owns tokens o and o+8 of the page and lane s of the
// octet owns dims [8s, 8s+8) and [64+8s, 64+8s+8) of those rows.  Each of the
// four 16-byte loads per lane per tensor (token pair x dim half) therefore
// moves eight whole 128-byte lines.  q.k uses v_dot2c_f32_bf16 on packed bf16
// pairs and is summed across the octet with three DPP steps; p.v runs in fp32
// FMAs so the softmax weights are never rounded to bf16.
//
// Online softmax.  Each octet is an independent softmax stream with its own
// running max m and sum l (base-2 units: scores are pre-multiplied by
// scale*log2(e)), so no cross-octet traffic happens inside the page loop.  At
// the end the 32 streams of the workgroup are merged through LDS with the
// usual (m, l, acc) rule
//     M = max m_i,  L = sum l_i 2^(m_i - M),  A = sum acc_i 2^(m_i - M).
// A request whose context spans several partitions writes its partial
// (M, L, A) to the workspace; the last workgroup of a (request, KV head) to
// arrive, found with an atomic ticket, merges the partials with the same rule,
// writes out = A/L and lse = ln2 * (M + log2 L), and resets the ticket, so a
// call is a single kernel launch.
#include "internal.h"

#include <math.h>

namespace hipdecode {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kStreams = kWaves * 8;   // softmax streams per workgroup (octets)

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

// Sum over the 8 lanes of an aligned octet; every lane of the octet gets it.
__device__ __forceinline__ float octet_sum(float x)
{
    x += dpp_f32<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_f32<0x141>(x);   // row_half_mirror: lane i <- lane 7-i, i.e. the other quad
    return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// dim of acc index i (0..15) for lane s of an octet
__device__ __forceinline__ int acc_dim(int s, int i) { return s * 8 + (i >> 3) * 64 + (i & 7); }

template <bool F32>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v)
{
    if constexpr (F32)
        static_cast<float *>(out)[idx] = v;
    else
        static_cast<__bf16 *>(out)[idx] = static_cast<__bf16>(v);   // round to nearest even
}

struct PageRegs {
    u32x4 k[2][2];   // [token o / o+8][dim half]
    u32x4 v[2][2];
};

__device__ __forceinline__ void load_page(PageRegs &r, const uint16_t *kb, const uint16_t *vb,
                                          size_t page_off, size_t tok8)
{
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            r.k[t][j] = load16(kb + page_off + t * tok8 + j * 64);
            r.v[t][j] = load16(vb + page_off + t * tok8 + j * 64);
        }
}

template <int G>
struct Stream {
    float m[G];
    float l[G];
    float acc[G][16];
};

// Fold one page into the octet's softmax stream.  MASK: tokens at or past ctx
// (only on a request's last page) get weight 0 and their K/V are never used
// arithmetically, so garbage or NaN in unused slots cannot leak in.
template <int G, bool MASK>
__device__ __forceinline__ void consume(Stream<G> &st, const PageRegs &r, const u32x4 (&qv)[G][2],
                                        float scale_log2, int tok_first, int ctx)
{
    float s[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float d = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    d = dot2_bf16(r.k[t][j][w], qv[h][j][w], d);
            s[h][t] = octet_sum(d) * scale_log2;
        }

    bool valid[2] = {true, true};
    if constexpr (MASK) {
        valid[0] = tok_first < ctx;
        valid[1] = tok_first + 8 < ctx;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                s[h][t] = valid[t] ? s[h][t] : -INFINITY;
    }

    float p[G][2];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float m_new = fmaxf(st.m[h], fmaxf(s[h][0], s[h][1]));
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[h] = exp2_fast(st.m[h] - m_use);
        p[h][0] = exp2_fast(s[h][0] - m_use);
        p[h][1] = exp2_fast(s[h][1] - m_use);
        st.l[h] = st.l[h] * alpha[h] + p[h][0] + p[h][1];
        st.m[h] = m_new;
    }

#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = j * 8 + w * 2;
            float v0l = bf16_lo(r.v[0][j][w]), v0h = bf16_hi(r.v[0][j][w]);
            float v1l = bf16_lo(r.v[1][j][w]), v1h = bf16_hi(r.v[1][j][w]);
            if constexpr (MASK) {
                v0l = valid[0] ? v0l : 0.f;
                v0h = valid[0] ? v0h : 0.f;
                v1l = valid[1] ? v1l : 0.f;
                v1h = valid[1] ? v1h : 0.f;
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                st.acc[h][i] = fmaf(p[h][1], v1l, fmaf(p[h][0], v0l, st.acc[h][i] * alpha[h]));
                st.acc[h][i + 1] = fmaf(p[h][1], v1h, fmaf(p[h][0], v0h, st.acc[h][i + 1] * alpha[h]));
            }
        }
}

template <int G, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(DecodeArgs a)
{
    __shared__ float s_acc[kStreams][G][kHeadDim];
    __shared__ float s_m[kStreams][G];
    __shared__ float s_l[kStreams][G];
    __shared__ int s_last;

    // Workgroup -> (b, split, g) with the KV head fastest: consecutive
    // workgroups read the same pages' neighbouring head rows.
    const int Hkv = a.num_kv_heads;
    const int g = blockIdx.x % Hkv;
    const int rest = blockIdx.x / Hkv;
    const int split = rest % a.nsplit_max;
    const int b = rest / a.nsplit_max;
    const int tid = threadIdx.x;

    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context_len ? a.max_context_len : ctx);
    const int n_pages = (ctx + kPageSize - 1) / kPageSize;
    const int nsplit_b = (n_pages + a.partition_pages - 1) / a.partition_pages;
    const size_t row0 = (size_t)b * a.num_q_heads + (size_t)g * G;   // first query row of the group

    if (ctx == 0) {
        if (split == 0) {
            for (int i = tid; i < G * kHeadDim; i += kThreads)
                store_out<OUT_F32>(a.out, row0 * kHeadDim + i, 0.f);
            if (a.lse != nullptr && tid < G)
                a.lse[row0 + tid] = -INFINITY;
        }
        return;
    }
    if (split >= nsplit_b)
        return;

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int oct = lane >> 3;
    const int sub = lane & 7;

    u32x4 qv[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            qv[h][j] = load16(a.q + (row0 + h) * kHeadDim + sub * 8 + j * 64);

    Stream<G> st;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            st.acc[h][i] = 0.f;
    }

    const size_t tok_stride = (size_t)Hkv * kHeadDim;   // elements between slots of a page
    const size_t page_stride = (size_t)kPageSize * tok_stride;
    const size_t lane_off = (size_t)g * kHeadDim + (size_t)oct * tok_stride + (size_t)sub * 8;
    const uint16_t *kb = a.k_pool + lane_off;
    const uint16_t *vb = a.v_pool + lane_off;
    const size_t tok8 = 8 * tok_stride;

    // Pages of this partition, dealt to the wavefronts round-robin; lane i of
    // a wavefront holds the block-table entry of its i-th page.
    const int p_begin = split * a.partition_pages;
    const int p_end = min(p_begin + a.partition_pages, n_pages);
    const int span = p_end - p_begin;
    const int npw = span > wave ? (span - wave + kWaves - 1) / kWaves : 0;
    const int32_t *trow = a.block_table + (size_t)b * a.max_blocks;
    const int my_entry = lane < npw ? trow[p_begin + wave + kWaves * lane] : -1;
    const unsigned num_pages = (unsigned)a.num_pages;

    PageRegs ra, rb;
    auto issue = [&](PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys < num_pages)
            load_page(r, kb, vb, (size_t)phys * page_stride, tok8);
    };
    auto fold = [&](const PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys >= num_pages)
            return;   // outside the pool: skipped, never read
        const int pg = p_begin + wave + kWaves * i;
        if ((pg + 1) * kPageSize <= ctx)
            consume<G, false>(st, r, qv, a.scale_log2, 0, 0);
        else
            consume<G, true>(st, r, qv, a.scale_log2, pg * kPageSize + oct, ctx);
    };

    if (npw > 0)
        issue(ra, 0);
    for (int i = 0; i < npw; i += 2) {
        if (i + 1 < npw)
            issue(rb, i + 1);
        fold(ra, i);
        if (i + 1 >= npw)
            break;
        if (i + 2 < npw)
            issue(ra, i + 2);
        fold(rb, i + 1);
    }

    // ---- merge the workgroup's 32 streams through LDS ----
    const int sid = wave * 8 + oct;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s_acc[sid][h][acc_dim(sub, i)] = st.acc[h][i];
        if (sub == 0) {
            s_m[sid][h] = st.m[h];
            s_l[sid][h] = st.l[h];
        }
    }
    __syncthreads();

    const bool single = (nsplit_b == 1);
    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int h = idx / kHeadDim;
        const int d = idx % kHeadDim;
        float M = -INFINITY;
        for (int s = 0; s < kStreams; ++s)
            M = fmaxf(M, s_m[s][h]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, A = 0.f;
        for (int s = 0; s < kStreams; ++s) {
            const float w = exp2_fast(s_m[s][h] - M_use);
            L = fmaf(s_l[s][h], w, L);
            A = fmaf(s_acc[s][h][d], w, A);
        }
        if (single) {
            store_out<OUT_F32>(a.out, (row0 + h) * kHeadDim + d, A / L);
            if (d == 0 && a.lse != nullptr)
                a.lse[row0 + h] = (M + log2f(L)) * 0.69314718055994530942f;
        } else {
            const size_t pi = (row0 + h) * (size_t)a.nsplit_max + split;
            a.part_acc[pi * kHeadDim + d] = A;
            if (d == 0) {
                a.part_ml[pi * 2 + 0] = M;
                a.part_ml[pi * 2 + 1] = L;
            }
        }
    }
    if (single)
        return;

    // ---- the last partition of (b, g) to finish merges all partials ----
    __threadfence();
    __syncthreads();
    int32_t *ticket = a.counters + (size_t)b * Hkv + g;
    if (tid == 0)
        s_last = (atomicAdd(ticket, 1) == nsplit_b - 1);
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();

    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int h = idx / kHeadDim;
        const int d = idx % kHeadDim;
        const size_t base = (row0 + h) * (size_t)a.nsplit_max;
        float M = -INFINITY;
        for (int i = 0; i < nsplit_b; ++i)
            M = fmaxf(M, __hip_atomic_load(a.part_ml + (base + i) * 2, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, A = 0.f;
        for (int i = 0; i < nsplit_b; ++i) {
            const float mi = __hip_atomic_load(a.part_ml + (base + i) * 2, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            const float li = __hip_atomic_load(a.part_ml + (base + i) * 2 + 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            const float ai = __hip_atomic_load(a.part_acc + (base + i) * kHeadDim + d, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            const float w = exp2_fast(mi - M_use);
            L = fmaf(li, w, L);
            A = fmaf(ai, w, A);
        }
        store_out<OUT_F32>(a.out, (row0 + h) * kHeadDim + d, A / L);
        if (d == 0 && a.lse != nullptr)
            a.lse[row0 + h] = (M + log2f(L)) * 0.69314718055994530942f;
    }
    if (tid == 0)
        atomicExch(ticket, 0);
}

__global__ void zero_fill_kernel(uint8_t *p, size_t bytes)
{
    const size_t n16 = bytes / 16;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        reinterpret_cast<u32x4 *>(p)[i] = u32x4{0u, 0u, 0u, 0u};
    const size_t tail = bytes - n16 * 16;
    if (blockIdx.x == 0 && threadIdx.x < tail)
        p[n16 * 16 + threadIdx.x] = 0;
}

template <int G>
hipError_t launch_g(const DecodeArgs &a, bool out_f32, unsigned grid, hipStream_t stream)
{
    if (out_f32)
        hipLaunchKernelGGL((paged_decode_kernel<G, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((paged_decode_kernel<G, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, int group, bool out_f32, int num_seqs,
                               hipStream_t stream)
{
    const size_t grid = (size_t)num_seqs * (size_t)a.nsplit_max * (size_t)a.num_kv_heads;
    if (grid == 0)
        return hipSuccess;
    switch (group) {
    case 1: return launch_g<1>(a, out_f32, (unsigned)grid, stream);
    case 2: return launch_g<2>(a, out_f32, (unsigned)grid, stream);
    case 4: return launch_g<4>(a, out_f32, (unsigned)grid, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream)
{
    if (bytes == 0)
        return hipSuccess;
    const size_t n16 = bytes / 16 + 1;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<uint8_t *>(p), bytes);
    return hipGetLastError();
}

}  // namespace hipdecode
