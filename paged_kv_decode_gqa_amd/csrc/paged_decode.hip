// paged_decode.hip -- gfx950 kernel for one decode step of paged GQA attention,
// split by (request, KV head, partition of the context).
//
// One workgroup owns one (request b, KV head g, split-K partition) triple and
// serves all G query heads that read KV head g (the 16-query/8-KV grouping of
// the audio.cpp "Decoder And Prompt" section), so every K/V byte of the cache
// is fetched from HBM exactly once per call.  The work is bound by HBM
// bandwidth: per cached token and query head it is 2x128 multiply-adds against
// 256 bytes of K and 256 bytes of V shared by the G heads.  Page-level work is
// in page_fold.h.
//
// The four wavefronts take the partition's pages round-robin, each with one
// page in flight while it folds the previous one; their 16 row-group streams
// are merged through LDS with the rule
//     M = max m_i,  L = sum l_i 2^(m_i - M),  A = sum acc_i 2^(m_i - M).
// A request whose context spans several partitions writes each partition's
// (M, L, A) to the workspace; the last workgroup of a (request, KV head) to
// arrive, found with an atomic ticket, merges the partials with the same rule
// (all threads loading in parallel), writes out = A/L and
// lse = ln2 * (M + log2 L), and resets the ticket, so a call is one launch.
// The partials travel through device-scope atomics (see page_fold.h), not
// through fences, so no workgroup flushes or invalidates the L2.
#include "page_fold.h"

namespace hipdecode {
namespace {

using namespace dev;

constexpr int kRowStreams = kWaves * 4;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Block-wide reductions over kThreads; `red` is kWaves floats of LDS.
__device__ __forceinline__ float block_max(float v, float *red)
{
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = fmaxf(r, red[w]);
    return r;
}

__device__ __forceinline__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r += red[w];
    return r;
}

template <int G, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void paged_decode_kernel(DecodeArgs a)
{
    __shared__ f32x4 s_acc4[kRowStreams * G * kHeadDim / 4];
    __shared__ float s_m[kRowStreams][G];
    __shared__ float s_l[kRowStreams][G];
    __shared__ float s_w[G][kMaxMergeSplits];
    __shared__ float s_red[kWaves];
    __shared__ int s_last;
    float *s_acc = reinterpret_cast<float *>(s_acc4);   // [kRowStreams][G][kHeadDim]

    // Workgroup -> (b, split, g) with the KV head fastest: consecutive
    // workgroups read neighbouring head rows of the same pages.
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
    const int row = lane >> 4;
    const int sub = lane & 15;

    u32x4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h] = load16(a.q + (row0 + h) * kHeadDim + sub * 8);

    Stream<G> st;
    st.init();

    const uint32_t tok_bytes = (uint32_t)Hkv * kHeadDim * 2;   // bytes between slots of a page
    const size_t page_elems = (size_t)kPageSize * Hkv * kHeadDim;
    const uint32_t lane_off = (uint32_t)g * kHeadDim * 2 + (uint32_t)row * tok_bytes + (uint32_t)sub * 16;
    const uint32_t tok4 = 4 * tok_bytes;

    // Full pages of this partition, dealt to the wavefronts round-robin; lane
    // i of a wavefront holds the block-table entry of its i-th page.  A
    // request's last page may be partly filled: it is folded separately,
    // with masking, after the loop.
    const int p_begin = split * a.partition_pages;
    const int p_end = min(p_begin + a.partition_pages, n_pages);
    const bool tail_partial = (p_end == n_pages) && (ctx % kPageSize != 0);
    const int full_end = tail_partial ? p_end - 1 : p_end;
    const int span = full_end - p_begin;
    const int npw = span > wave ? (span - wave + kWaves - 1) / kWaves : 0;
    const int32_t *trow = a.block_table + (size_t)b * a.max_blocks;
    const int my_entry = lane < npw ? trow[p_begin + wave + kWaves * lane] : -1;
    const unsigned num_pages = (unsigned)a.num_pages;

    PageRegs ra, rb;
    auto issue = [&](PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys < num_pages)
            load_page(r, a.k_pool + (size_t)phys * page_elems, a.v_pool + (size_t)phys * page_elems,
                      lane_off, tok4);
    };
    auto fold = [&](const PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys < num_pages)   // a page outside the pool is skipped, never read
            fold_page<G, false>(st, r, qv, a.scale_log2, 0, 0);
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
    if (tail_partial && wave == kWaves - 1) {
        const int phys = trow[full_end];
        if ((unsigned)phys < num_pages) {
            load_page(ra, a.k_pool + (size_t)phys * page_elems, a.v_pool + (size_t)phys * page_elems,
                      lane_off, tok4);
            fold_page<G, true>(st, ra, qv, a.scale_log2, full_end * kPageSize + row, ctx);
        }
    }

    // ---- merge the workgroup's 16 row-group streams through LDS ----
    const int sid = wave * 4 + row;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        f32x4 *dst = s_acc4 + ((sid * G + h) * kHeadDim + sub * 8) / 4;
        dst[0] = f32x4{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
        dst[1] = f32x4{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
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
#pragma unroll
        for (int s = 0; s < kRowStreams; ++s)
            M = fmaxf(M, s_m[s][h]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int s = 0; s < kRowStreams; ++s) {
            const float w = merge_weight(s_m[s][h], M_use);
            L = fmaf(s_l[s][h], w, L);
            A = fmaf(s_acc[(s * G + h) * kHeadDim + d], w, A);
        }
        if (single) {
            store_out<OUT_F32>(a.out, (row0 + h) * kHeadDim + d, A / L);
            if (d == 0 && a.lse != nullptr)
                a.lse[row0 + h] = (M + log2f(L)) * kLn2;
        } else {
            const size_t pi = (row0 + h) * (size_t)a.nsplit_max + split;
            coherent_store(a.part_acc + pi * kHeadDim + d, A);
            if (d == 0) {
                coherent_store(a.part_ml + pi * 2 + 0, M);
                coherent_store(a.part_ml + pi * 2 + 1, L);
            }
        }
    }
    if (single)
        return;

    // ---- the last partition of (b, g) to finish merges all partials ----
    // every wavefront's partial stores have completed before the ticket moves
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int32_t *ticket = a.counters + (size_t)b * Hkv + g;
    if (tid == 0)
        s_last = (__hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  nsplit_b - 1);
    __syncthreads();
    if (!s_last)
        return;

    const size_t nsm = (size_t)a.nsplit_max;
    float Mh[G], Lh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float *ml = a.part_ml + (row0 + h) * nsm * 2;
        float mx = -INFINITY;
        for (int i = tid; i < nsplit_b; i += kThreads)
            mx = fmaxf(mx, coherent_load(ml + 2 * i));
        Mh[h] = block_max(mx, s_red);
        const float M_use = (Mh[h] == -INFINITY) ? 0.f : Mh[h];
        float ls = 0.f;
        for (int i = tid; i < nsplit_b; i += kThreads) {
            const float w = merge_weight(coherent_load(ml + 2 * i), M_use);
            s_w[h][i] = w;
            ls = fmaf(coherent_load(ml + 2 * i + 1), w, ls);
        }
        Lh[h] = block_sum(ls, s_red);
    }
    __syncthreads();

    // every thread owns 4 dims of one head and a 1/kSets share of the partials
    constexpr int kChunks = G * kHeadDim / 4;
    constexpr int kSets = kThreads / kChunks;
    const int chunk = tid % kChunks;
    const int set = tid / kChunks;
    const int h = chunk / (kHeadDim / 4);
    const int c = chunk % (kHeadDim / 4);
    const float *acc_h = a.part_acc + (row0 + h) * nsm * kHeadDim + 4 * c;
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int i = set; i < nsplit_b; i += kSets)
        A += s_w[h][i] * coherent_load4(acc_h + (size_t)i * kHeadDim);
    s_acc4[set * kChunks + chunk] = A;
    __syncthreads();
    if (set == 0) {
#pragma unroll
        for (int s = 1; s < kSets; ++s)
            A += s_acc4[s * kChunks + chunk];
        float hl = Lh[0];
#pragma unroll
        for (int hh = 1; hh < G; ++hh)
            hl = (hh == h) ? Lh[hh] : hl;
        const size_t o = (row0 + h) * kHeadDim + 4 * c;
        store_out<OUT_F32>(a.out, o + 0, A[0] / hl);
        store_out<OUT_F32>(a.out, o + 1, A[1] / hl);
        store_out<OUT_F32>(a.out, o + 2, A[2] / hl);
        store_out<OUT_F32>(a.out, o + 3, A[3] / hl);
        if (c == 0 && a.lse != nullptr) {
            float hm = Mh[0];
#pragma unroll
            for (int hh = 1; hh < G; ++hh)
                hm = (hh == h) ? Mh[hh] : hm;
            a.lse[row0 + h] = (hm + log2f(hl)) * kLn2;
        }
    }
    if (tid == 0)
        __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
