// paged_decode.hip -- gfx950 kernels for one decode step of paged GQA attention.
//
// Every workgroup serves all G query heads that read one KV head (the
// 16-query/8-KV grouping of the audio.cpp "Decoder And Prompt" section), so
// each K/V byte of the cache is fetched from HBM once per call.  The work is
// bound by HBM bandwidth: per cached token and query head it is 2x128
// multiply-adds against 256 bytes of K and 256 bytes of V shared by the G
// heads.  Page-level work is in page_fold.h.
//
// One workgroup per (request b, KV head g, partition of the context).  The
// grid is sized by the host's max_context_len.  In a ragged batch the
// workgroups map onto the real (request, partition) units in order, so the
// slots past the last one, not slots scattered through the grid, are the
// ones that exit at once.
//
// Inside a workgroup the wavefronts take pages round-robin, each with one page
// in flight while it folds the previous one; their streams are merged with
//     M = max m_i,  L = sum l_i 2^(m_i - M),  A = sum acc_i 2^(m_i - M).
// A (request, KV head) covered by one workgroup writes out = A/L and
// lse = ln2 * (M + log2 L) directly.  Otherwise each workgroup writes its
// partial (M, L, A) to the workspace and the last one to arrive, found with an
// atomic ticket, merges them with the same rule and resets the ticket, so a
// call is one launch.  Partials travel through device-scope atomics (see
// page_fold.h), not fences, so no workgroup flushes or invalidates the L2.
#include "page_fold.h"
#include "rope_round.h"

namespace hipdecode {
namespace {

using namespace dev;

constexpr int kRegPartials = 8;   // final merge: partial sums per thread loaded up front

// Reductions over a wavefront: four DPP steps inside each row of 16 lanes
// (as row_sum16 does), then the four rows' results through v_readlane, so no
// step waits on an LDS-based lane shuffle.
__device__ __forceinline__ float row_max16(float x)
{
    x = fmaxf(x, dpp_f32<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f32<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f32<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp_f32<0x140>(x));   // row_mirror
    return x;
}

__device__ __forceinline__ float lane_value(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = row_max16(v);
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = row_sum16(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// The values of x in the two lanes of each pair (l, l ^ O), O = 16 or 32,
// handed to both of them in the same order: `lo` from the member with the
// bit clear, `hi` from the other (v_permlane16_swap / v_permlane32_swap).
template <int O>
__device__ __forceinline__ void pair_values(float x, float &lo, float &hi)
{
    const uint32_t u = __float_as_uint(x);
    if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
    } else {
        static_assert(O == 32, "pairs 16 or 32 lanes apart");
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
    }
}

// Merge the two streams of each lane pair (l, l ^ O); both lanes end with the
// same merged stream.
template <int G, int O>
__device__ __forceinline__ void merge_pairs(Stream<G> &st)
{
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m_lo, m_hi, l_lo, l_hi;
        pair_values<O>(st.m[h], m_lo, m_hi);
        pair_values<O>(st.l[h], l_lo, l_hi);
        const float M = fmaxf(m_lo, m_hi);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float w_lo = merge_weight(m_lo, M_use);
        const float w_hi = merge_weight(m_hi, M_use);
        st.l[h] = fmaf(l_lo, w_lo, l_hi * w_hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a_lo, a_hi;
            pair_values<O>(st.acc[h][e], a_lo, a_hi);
            st.acc[h][e] = fmaf(a_lo, w_lo, a_hi * w_hi);
        }
        st.m[h] = M;
    }
}

// Merge the four row-group streams of a wavefront (lanes l, l^16, l^32, l^48
// hold the same dims) so that every row-group ends with the wavefront's total.
template <int G>
__device__ __forceinline__ void merge_row_groups(Stream<G> &st)
{
    merge_pairs<G, 16>(st);
    merge_pairs<G, 32>(st);
}

// LDS shared by both kernels.
template <int G, int WAVES>
struct Smem {
    static constexpr int kThreadsWG = 64 * WAVES;
    static constexpr int kChunks = G * kHeadDim / 4;   // float4 chunks of G heads
    static constexpr int kSets = kThreadsWG / kChunks;  // final merge: partial subsets
    static constexpr int kScratch4 =
        (WAVES * G * kHeadDim / 4 > kThreadsWG) ? WAVES * G * kHeadDim / 4 : kThreadsWG;
    f32x4 acc4[kScratch4];          // [WAVES][G][kHeadDim] floats, or final-merge scratch
    float m[WAVES][G];
    float l[WAVES][G];
    float w[G][kMaxMergeSplits];    // final merge: partial maxima, then weights
    float lw[G][kMaxMergeSplits];   // final merge: partial sums
    float head_m[G];
    float head_l[G];
    int last;
};

// Per-lane coordinates inside a workgroup.
struct Lane {
    int tid, lane, wave, row, sub;
    __device__ __forceinline__ Lane()
    {
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        row = lane >> 4;
        sub = lane & 15;
    }
};

template <int G>
__device__ __forceinline__ void load_q(u32x4 (&qv)[G], const DecodeArgs &a, size_t row0, int sub)
{
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h] = load16(a.q + (row0 + h) * kHeadDim + sub * 8);
}

// Fold pages [p_begin, p_end) (at most 64 per wavefront) of KV head g of a
// request with ctx tokens and n_pages pages into this wavefront's stream.
// entry: the block-table entry of page p_begin + wave + WAVES * lane, or
// anything for lanes past the range.  A partly filled last page of the
// request is folded by the last wavefront, with masking, after the others.
// FUSED: the request's last page always goes that way, and its new token
// (slot (ctx - 1) % 16, row b of k_new/v_new) is taken from k_new/v_new --
// K rotated with `angles` when RoPE is on -- written to the pool and folded
// from registers; no other workgroup reads that page.  With append_new false
// (a context length past the host bound, so ctx was clamped and slot ctx - 1
// holds a real cached token) nothing is written and the page is folded as
// the pool holds it.
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

template <int G, int WAVES, bool FUSED = false, class Hook = NoHook>
__device__ __forceinline__ void fold_range(Stream<G> &st, const DecodeArgs &a, const u32x4 (&qv)[G],
                                           const int32_t *trow, int g, int p_begin, int p_end,
                                           int n_pages, int ctx, int entry, const Lane &ln, int b = 0,
                                           const double2 *angles = nullptr, Hook before_fold = Hook(),
                                           bool append_new = true)
{
    const uint32_t tok_bytes = (uint32_t)a.num_kv_heads * kHeadDim * 2;   // bytes between slots
    const size_t page_elems = (size_t)kPageSize * a.num_kv_heads * kHeadDim;
    const uint32_t lane_off = (uint32_t)g * kHeadDim * 2 + (uint32_t)ln.row * tok_bytes + (uint32_t)ln.sub * 16;
    const uint32_t tok4 = 4 * tok_bytes;

    const bool tail_partial = (p_end == n_pages) && (FUSED || ctx % kPageSize != 0);
    const int full_end = tail_partial ? p_end - 1 : p_end;
    const int span = full_end - p_begin;
    const int npw = span > ln.wave ? (span - ln.wave + WAVES - 1) / WAVES : 0;
    const int my_entry = ln.lane < npw ? entry : -1;
    const unsigned num_pages = (unsigned)a.num_pages;

    // The steady-state loop issues its loads unconditionally so that the
    // compiler's wait counts stay exact and page i+1 really is in flight while
    // page i is folded; the last one or two pages are peeled off after it.  A
    // page id outside the pool is fetched as page 0 (which exists whenever
    // any context is non-empty) and never folded.
    PageRegs ra, rb;
    auto issue = [&](PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        const int safe = (unsigned)phys < num_pages ? phys : 0;
        load_page(r, a.k_pool + (size_t)safe * page_elems, a.v_pool + (size_t)safe * page_elems, lane_off, tok4);
    };
    auto fold = [&](const PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys < num_pages)   // a page outside the pool is never folded
            fold_page<G, false>(st, r, qv, a.scale_log2, 0, 0);
    };

    // before_fold runs in every wavefront once the first page is in flight
    // (the fused kernel rotates q there); it may hold a workgroup barrier.
    if (npw > 0)
        issue(ra, 0);
    before_fold();
    if (npw > 0) {
        int i = 0;
        for (; i + 2 < npw; i += 2) {
            issue(rb, i + 1);
            fold(ra, i);
            issue(ra, i + 2);
            fold(rb, i + 1);
        }
        if (i + 1 < npw) {
            issue(rb, i + 1);
            fold(ra, i);
            fold(rb, i + 1);
        } else {
            fold(ra, i);
        }
    }
    if (tail_partial && ln.wave == WAVES - 1) {
        const int phys = trow[full_end];
        if ((unsigned)phys < num_pages) {
            load_page(ra, a.k_pool + (size_t)phys * page_elems, a.v_pool + (size_t)phys * page_elems,
                      lane_off, tok4);
            if constexpr (FUSED) {
                const int slot = (ctx - 1) % kPageSize;
                if (append_new && ln.row == (slot & 3)) {   // the 16 lanes holding the new token, in register slot / 4
                    const size_t nrow = ((size_t)b * a.num_kv_heads + g) * kHeadDim;
                    u32x4 kn = load16(a.k_new + nrow + ln.sub * 8);
                    const u32x4 vn = load16(a.v_new + nrow + ln.sub * 8);
                    if (angles != nullptr) {
                        const u32x4 kp = load16(a.k_new + nrow + (ln.sub ^ 8) * 8);
                        const int base = 8 * (ln.sub & 7);
                        const uint4 r = rope::rotate8(make_uint4(kn.x, kn.y, kn.z, kn.w),
                                                      make_uint4(kp.x, kp.y, kp.z, kp.w), ln.sub >= 8,
                                                      [&](int e) { return angles[base + e]; });
                        kn = u32x4{r.x, r.y, r.z, r.w};
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (t == (slot >> 2)) {
                            ra.k[t] = kn;
                            ra.v[t] = vn;
                        }
                    }
                    const size_t off = (size_t)phys * page_elems * 2 + lane_off + (size_t)(slot >> 2) * tok4;
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(a.k_pool_w) + off) = kn;
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(a.v_pool_w) + off) = vn;
                }
            }
            fold_page<G, true>(st, ra, qv, a.scale_log2, full_end * kPageSize + ln.row, ctx);
        }
    }
}

// Row-groups inside each wavefront, then the wavefronts' totals into LDS.
// The caller syncs the workgroup afterwards.
template <int G, int WAVES>
__device__ __forceinline__ void publish_streams(Stream<G> &st, Smem<G, WAVES> &sm, const Lane &ln)
{
    merge_row_groups<G>(st);
    if (ln.row == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            f32x4 *dst = sm.acc4 + ((ln.wave * G + h) * kHeadDim + ln.sub * 8) / 4;
            dst[0] = f32x4{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
            dst[1] = f32x4{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
            if (ln.sub == 0) {
                sm.m[ln.wave][h] = st.m[h];
                sm.l[ln.wave][h] = st.l[h];
            }
        }
    }
}

// Combine the workgroup's wavefronts for query head h, dim d: (M, L, A).
template <int G, int WAVES>
__device__ __forceinline__ void combine_waves(const Smem<G, WAVES> &sm, int h, int d, float &M, float &L,
                                              float &A)
{
    const float *s_acc = reinterpret_cast<const float *>(sm.acc4);
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        M = fmaxf(M, sm.m[w][h]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    L = 0.f;
    A = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const float wt = merge_weight(sm.m[w][h], M_use);
        L = fmaf(sm.l[w][h], wt, L);
        A = fmaf(s_acc[(w * G + h) * kHeadDim + d], wt, A);
    }
}

// Write the workgroup's result for G query heads: final output when one
// workgroup covers the (request, KV head), else a partial at partial index
// part_index(h).  The caller syncs before and after.
template <int G, int WAVES, bool OUT_F32, class PartIndex>
__device__ __forceinline__ void emit(const DecodeArgs &a, const Smem<G, WAVES> &sm, size_t row0, bool final,
                                     PartIndex part_index, const Lane &ln)
{
    for (int idx = ln.tid; idx < G * kHeadDim; idx += Smem<G, WAVES>::kThreadsWG) {
        const int h = idx / kHeadDim;
        const int d = idx % kHeadDim;
        float M, L, A;
        combine_waves<G, WAVES>(sm, h, d, M, L, A);
        if (final) {
            store_out<OUT_F32>(a.out, (row0 + h) * kHeadDim + d, A / L);
            if (d == 0 && a.lse != nullptr)
                a.lse[row0 + h] = (M + log2f(L)) * kLn2;
        } else {
            const size_t pi = part_index(h);
            coherent_store(a.part_acc + pi * kHeadDim + d, A);
            if (d == 0) {
                coherent_store(a.part_ml + pi * 2 + 0, M);
                coherent_store(a.part_ml + pi * 2 + 1, L);
            }
        }
    }
}

// After emitting a partial: take the ticket of (request, KV head); true in the
// last of `count` workgroups to arrive.  Uniform across the workgroup.
template <int G, int WAVES>
__device__ __forceinline__ bool arrive(int32_t *ticket, int count, Smem<G, WAVES> &sm, const Lane &ln,
                                       int inc = 1)
{
    // every wavefront's partial stores have completed before the ticket moves
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ln.tid == 0)
        sm.last = (__hip_atomic_fetch_add(ticket, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc == count);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(sm.last) != 0;
}

// An empty partial (no tokens): weight 0 in any merge.
template <int G, int WAVES>
__device__ __forceinline__ void emit_empty(const DecodeArgs &a, size_t part_base, const Lane &ln)
{
    for (int idx = ln.tid; idx < G * kHeadDim; idx += Smem<G, WAVES>::kThreadsWG) {
        const size_t pi = part_base + idx / kHeadDim;
        coherent_store(a.part_acc + pi * kHeadDim + idx % kHeadDim, 0.f);
        if (idx % kHeadDim == 0) {
            coherent_store(a.part_ml + pi * 2 + 0, -INFINITY);
            coherent_store(a.part_ml + pi * 2 + 1, 0.f);
        }
    }
}

// Merge `count` partials of G query heads (partial i of head h at index
// part_index(i, h)), write out and lse, and reset the ticket.
template <int G, int WAVES, bool OUT_F32, class PartIndex>
__device__ __forceinline__ void merge_partials(const DecodeArgs &a, Smem<G, WAVES> &sm, size_t row0, int count,
                                               PartIndex part_index, int32_t *ticket, const Lane &ln)
{
    using S = Smem<G, WAVES>;
    // Every thread owns 4 dims of one head and a 1/kSets share of the
    // partials.  Its first kRegPartials partial sums and the (m, l) pair of
    // partial tid are loaded in one batch, without branches (indices past the
    // end are clamped and their values dropped), so the merge waits on
    // memory once; (m, l) pairs past the first kThreadsWG follow in a loop.
    const int chunk = ln.tid % S::kChunks;
    const int set = ln.tid / S::kChunks;
    const int h = chunk / (kHeadDim / 4);
    const int c = chunk % (kHeadDim / 4);
    const int n_ml = G * count;
    const int idx0 = min(ln.tid, n_ml - 1);
    const int hh0 = idx0 / count;
    const uint64_t ml0 = coherent_load8(a.part_ml + part_index(idx0 - hh0 * count, hh0) * 2);
    f32x4 pre[kRegPartials];
#pragma unroll
    for (int r = 0; r < kRegPartials; ++r) {
        const int i = min(set + r * S::kSets, count - 1);
        pre[r] = coherent_load4(a.part_acc + part_index(i, h) * kHeadDim + 4 * c);
    }
    if (ln.tid < n_ml) {
        sm.w[hh0][idx0 - hh0 * count] = __uint_as_float((uint32_t)ml0);
        sm.lw[hh0][idx0 - hh0 * count] = __uint_as_float((uint32_t)(ml0 >> 32));
    }
    for (int idx = ln.tid + S::kThreadsWG; idx < n_ml; idx += S::kThreadsWG) {
        const int hh = idx / count;
        const int i = idx - hh * count;
        const uint64_t ml = coherent_load8(a.part_ml + part_index(i, hh) * 2);
        sm.w[hh][i] = __uint_as_float((uint32_t)ml);
        sm.lw[hh][i] = __uint_as_float((uint32_t)(ml >> 32));
    }
    __syncthreads();
    // wavefront hw turns head hw's maxima into weights and sums L
    if (ln.wave < G) {
        const int hw = ln.wave;
        float mx = -INFINITY;
        for (int i = ln.lane; i < count; i += 64)
            mx = fmaxf(mx, sm.w[hw][i]);
        mx = wave_max(mx);
        const float M_use = (mx == -INFINITY) ? 0.f : mx;
        float ls = 0.f;
        for (int i = ln.lane; i < count; i += 64) {
            const float w = merge_weight(sm.w[hw][i], M_use);
            sm.w[hw][i] = w;
            ls = fmaf(sm.lw[hw][i], w, ls);
        }
        ls = wave_sum(ls);
        if (ln.lane == 0) {
            sm.head_m[hw] = mx;
            sm.head_l[hw] = ls;
        }
    }
    __syncthreads();

    f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kRegPartials; ++r) {
        const int i = set + r * S::kSets;
        if (i < count)
            A += sm.w[h][i] * pre[r];
    }
#pragma unroll 8
    for (int i = set + kRegPartials * S::kSets; i < count; i += S::kSets)
        A += sm.w[h][i] * coherent_load4(a.part_acc + part_index(i, h) * kHeadDim + 4 * c);
    sm.acc4[set * S::kChunks + chunk] = A;
    __syncthreads();
    if (set == 0) {
#pragma unroll
        for (int s = 1; s < S::kSets; ++s)
            A += sm.acc4[s * S::kChunks + chunk];
        const float hl = sm.head_l[h];
        const size_t o = (row0 + h) * kHeadDim + 4 * c;
        store_out<OUT_F32>(a.out, o + 0, A[0] / hl);
        store_out<OUT_F32>(a.out, o + 1, A[1] / hl);
        store_out<OUT_F32>(a.out, o + 2, A[2] / hl);
        store_out<OUT_F32>(a.out, o + 3, A[3] / hl);
        if (c == 0 && a.lse != nullptr)
            a.lse[row0 + h] = (sm.head_m[h] + log2f(hl)) * kLn2;
    }
    if (ln.tid == 0)
        __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool OUT_F32>
__device__ __forceinline__ void write_empty(const DecodeArgs &a, size_t row0, int rows, int tid, int nthreads)
{
    for (int i = tid; i < rows * kHeadDim; i += nthreads)
        store_out<OUT_F32>(a.out, row0 * kHeadDim + i, 0.f);
    if (a.lse != nullptr)
        for (int i = tid; i < rows; i += nthreads)
            a.lse[row0 + i] = -INFINITY;
}

__device__ __forceinline__ int clamp_ctx(int ctx, int max_ctx)
{
    return ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
}

// Inclusive prefix sum over the 64 lanes of a wavefront: four DPP row shifts
// sum inside each row of 16 lanes, then the rows' totals (read into scalar
// registers) are added to the rows after them.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The work list.  The grid has a slot for every partition
// the longest context could need, but a ragged batch has far fewer real
// (request, partition) units.  Unit u is the u-th real unit in request order,
// partitions ascending; an empty request counts one unit, which writes its
// empty output.  Slots past the last real unit get b = -1 and exit, so every
// workgroup the dispatcher places early carries work.
struct RealUnit {
    int b, split, ctx;
    bool over;   // the request's context length exceeds the host bound (ctx is clamped)
};

__device__ __forceinline__ RealUnit real_unit(const DecodeArgs &a, int u)
{
    const int lane = (int)(threadIdx.x & 63);
    const int span = kPageSize * a.partition_pages;
    RealUnit r{-1, 0, 0, false};
    int carry = 0;
    for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
        const int j = c0 + lane;
        const int raw = j < a.num_seqs ? a.context_lens[j] : 0;
        const int cj = clamp_ctx(raw, a.max_context_len);
        const int nj = j < a.num_seqs ? max(1, (cj + span - 1) / span) : 0;
        const int incl = wave_inclusive_scan(nj, lane);
        const int excl = incl - nj;
        const unsigned long long hit = __ballot(u >= carry + excl && u < carry + incl);
        if (hit != 0ull) {
            const int l = __builtin_amdgcn_readfirstlane(__ffsll(hit) - 1);
            r.b = c0 + l;
            r.split = u - carry - __builtin_amdgcn_readlane(excl, l);
            r.ctx = __builtin_amdgcn_readlane(cj, l);
            r.over = __builtin_amdgcn_readlane(raw, l) > a.max_context_len;
            break;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    return r;
}

// ---------------------------------------------------------------------------
// workgroup = (real unit, KV head), KV head fastest so consecutive
// workgroups read neighbouring head rows of the same pages (the heads are
// XOR-ed by dispatch round below).  A
// single request, or a batch with one partition per request, maps the grid
// directly (unit = request * nsplit_max + partition; units past a request's
// partition count exit); any other batch goes through real_unit().
// ---------------------------------------------------------------------------
template <int G, int WAVES, bool OUT_F32, bool FUSED>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4)))
void paged_decode_kernel(DecodeArgs a)
{
    __shared__ Smem<G, WAVES> sm;
    const Lane ln;
    const int Hkv = a.num_kv_heads;
    const int rest = blockIdx.x / Hkv;
    // The dispatcher hands out workgroups in rounds of one per CU (256 on
    // MI355X), so one CU holds workgroups r * 256 + i of successive rounds r.
    // XOR-ing the KV head with the round gives each CU rows of several heads,
    // whose addresses differ in bits 8-10 of the token row; measured 1.4%
    // faster at 16 x 28,672 tokens and 1.8% at the 32-request mix, unchanged
    // when the grid is a single round.  The XOR value is taken from the first
    // workgroup of the unit's Hkv consecutive ones, and acts within groups of
    // head_mix heads (a power of two dividing Hkv), so every unit still maps
    // its Hkv workgroups onto its Hkv heads one to one.
    const int round = (int)(((unsigned)rest * (unsigned)Hkv) >> 8);
    const int g = (int)(blockIdx.x % Hkv) ^ (round & (a.head_mix - 1));
    const int pp = a.partition_pages;
    // Unit `rest` in the full grid: request rest / nsplit_max, partition rest % nsplit_max.
    const int b_full = rest / a.nsplit_max;
    const int split_full = rest % a.nsplit_max;

    // Issued before the context length arrives: lane i of each wavefront
    // fetches the table entry of its i-th page of this partition, bounded by
    // the table row (entries past the request's pages are never used).
    const int spec_idx = split_full * pp + ln.wave + WAVES * ln.lane;
    const int spec_full = (spec_idx < a.max_blocks && ln.lane * WAVES < pp)
                              ? a.block_table[(size_t)b_full * a.max_blocks + spec_idx] : -1;

    int b, split, ctx, spec_entry;
    [[maybe_unused]] bool over;   // context length past the host bound: the fused kernel appends nothing
    if (a.num_seqs == 1 || a.nsplit_max == 1) {
        // Every unit of the full grid up to a request's partition count is real.
        b = b_full;
        split = split_full;
        const int raw = a.context_lens[b];
        ctx = clamp_ctx(raw, a.max_context_len);
        over = raw > a.max_context_len;
        spec_entry = spec_full;
        const int nsplit_b = (ctx + kPageSize * pp - 1) / (kPageSize * pp);
        if (ctx == 0 ? split != 0 : split >= nsplit_b)
            return;
    } else {
        const RealUnit u = real_unit(a, rest);
        const int span = kPageSize * pp;
        if (u.b < 0 || u.split < 0 || u.split >= max(1, (u.ctx + span - 1) / span))
            return;   // past the last real unit
        b = u.b;
        split = u.split;
        ctx = u.ctx;
        over = u.over;
        spec_entry = spec_full;
        if (b != b_full || split != split_full) {   // ragged batch: fetch this partition's entries
            const int idx = split * pp + ln.wave + WAVES * ln.lane;
            spec_entry = (idx < a.max_blocks && ln.lane * WAVES < pp)
                             ? a.block_table[(size_t)b * a.max_blocks + idx] : -1;
        }
    }
    const int32_t *trow = a.block_table + (size_t)b * a.max_blocks;
    const int p_begin = split * pp;
    const int n_pages = (ctx + kPageSize - 1) / kPageSize;
    const int nsplit_b = (n_pages + pp - 1) / pp;
    const size_t row0 = (size_t)b * a.num_q_heads + (size_t)g * G;   // first query row of the group

    if (ctx == 0) {
        write_empty<OUT_F32>(a, row0, G, ln.tid, 64 * WAVES);
        return;
    }

    u32x4 qv[G];
    load_q<G>(qv, a, row0, ln.sub);
    // Fused: RoPE of this lane's 8 dimensions of its G query heads at position
    // ctx - 1.  The partner dimensions are loaded here, before the first page;
    // the 64 angles (first wavefront, through LDS) and the rotation run while
    // that page is in flight.
    __shared__ double2 angles[FUSED ? rope::kHalf : 1];
    const bool rope_on = FUSED && a.rope_theta > 0.0;
    u32x4 qp[G];
    if constexpr (FUSED) {
        if (rope_on) {
#pragma unroll
            for (int h = 0; h < G; ++h)
                qp[h] = load16(a.q + (row0 + h) * kHeadDim + (ln.sub ^ 8) * 8);
        }
    }
    auto rotate_q = [&]() __attribute__((always_inline)) {
        if constexpr (FUSED) {
            if (rope_on) {
                if (ln.wave == 0)
                    angles[ln.lane] = rope::angle(a.rope_theta, ctx - 1, ln.lane);
                __syncthreads();
                const int base = 8 * (ln.sub & 7);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint4 r = rope::rotate8(make_uint4(qv[h].x, qv[h].y, qv[h].z, qv[h].w),
                                                  make_uint4(qp[h].x, qp[h].y, qp[h].z, qp[h].w), ln.sub >= 8,
                                                  [&](int e) { return angles[base + e]; });
                    qv[h] = u32x4{r.x, r.y, r.z, r.w};
                }
            }
        }
    };
    Stream<G> st;
    st.init();
    if constexpr (FUSED)
        fold_range<G, WAVES, FUSED>(st, a, qv, trow, g, p_begin, min(p_begin + a.partition_pages, n_pages),
                                    n_pages, ctx, spec_entry, ln, b, rope_on ? angles : nullptr, rotate_q, !over);
    else
        fold_range<G, WAVES, FUSED>(st, a, qv, trow, g, p_begin, min(p_begin + a.partition_pages, n_pages),
                                    n_pages, ctx, spec_entry, ln, b);
    publish_streams<G, WAVES>(st, sm, ln);
    __syncthreads();

    const size_t nsm = (size_t)a.nsplit_max;
    const bool single = (nsplit_b == 1);
    emit<G, WAVES, OUT_F32>(a, sm, row0, single, [&](int h) { return (row0 + h) * nsm + split; }, ln);
    if (single)
        return;
    int32_t *ticket = a.counters + ((size_t)b * Hkv + g) * kCounterStride;
    if (!arrive<G, WAVES>(ticket, nsplit_b, sm, ln))
        return;
    merge_partials<G, WAVES, OUT_F32>(a, sm, row0, nsplit_b,
                                      [&](int i, int h) { return (row0 + h) * nsm + i; }, ticket, ln);
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

template <int G, int WAVES>
hipError_t launch_split(const DecodeArgs &a, bool out_f32, unsigned grid, hipStream_t stream, bool fused)
{
    const dim3 block(64 * WAVES);
    if (fused && out_f32)
        hipLaunchKernelGGL((paged_decode_kernel<G, WAVES, true, true>), dim3(grid), block, 0, stream, a);
    else if (fused)
        hipLaunchKernelGGL((paged_decode_kernel<G, WAVES, false, true>), dim3(grid), block, 0, stream, a);
    else if (out_f32)
        hipLaunchKernelGGL((paged_decode_kernel<G, WAVES, true, false>), dim3(grid), block, 0, stream, a);
    else
        hipLaunchKernelGGL((paged_decode_kernel<G, WAVES, false, false>), dim3(grid), block, 0, stream, a);
    return hipGetLastError();
}

template <int G>
hipError_t launch_g(const DecodeArgs &a, int waves, bool out_f32, hipStream_t stream, bool fused)
{
    const unsigned grid = (unsigned)((size_t)a.num_seqs * a.nsplit_max * a.num_kv_heads);
    if constexpr (G <= 2) {   // G = 4 at 16 wavefronts would not fit 128 VGPRs without spilling
        if (waves == 16)
            return launch_split<G, 16>(a, out_f32, grid, stream, fused);
    }
    return waves == 4 ? launch_split<G, 4>(a, out_f32, grid, stream, fused) : hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, int group, int waves, bool out_f32, hipStream_t stream,
                               bool fused)
{
    if (a.num_seqs == 0)
        return hipSuccess;
    switch (group) {
    case 1: return launch_g<1>(a, waves, out_f32, stream, fused);
    case 2: return launch_g<2>(a, waves, out_f32, stream, fused);
    case 4: return launch_g<4>(a, waves, out_f32, stream, fused);
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
