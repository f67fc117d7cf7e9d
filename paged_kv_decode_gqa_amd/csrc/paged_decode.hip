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
// workgroups map onto the real (request, partition) units, full partitions
// first, so the slots past the last one, not slots scattered through the
// grid, are the ones that exit at once.
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

// LDS of the decode kernel.  With four wavefronts the 16 row-group streams
// go to LDS as they are and are merged there in one step; sixteen
// wavefronts first merge their row-groups in registers, so LDS holds one
// stream per wavefront.  The final merge uses acc as scratch when several
// threads share a dim.
template <int G, int WAVES>
struct Smem {
    static constexpr int kThreadsWG = 64 * WAVES;
    static constexpr int kRowGroups = WAVES == 4 ? 4 : 1;   // streams per wavefront kept apart
    static constexpr int kStreams = WAVES * kRowGroups;
    static_assert(kStreams <= 64, "one stream per lane when weighing them");
    float acc[kStreams][G][kHeadDim];   // unnormalised sums of V per stream
    float m[kStreams][G];
    float l[kStreams][G];
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

// RoPE of the 8 dims [8 sub, 8 sub + 8) of a head that all four row-groups
// of a wavefront hold alike (q, or the new token's K), given the partner
// dims: row-group r rotates word r (dims 8 sub + 2r and 8 sub + 2r + 1) and
// three lane swaps hand every row-group all four words.  cs(e): the angles
// of pair 8 (sub % 8) + e.  Called with every lane of the wavefront active.
template <typename CS>
__device__ __forceinline__ u32x4 rotate_shared(u32x4 own, u32x4 partner, bool second_half, int row, CS cs)
{
    const uint32_t o = row == 0 ? own.x : row == 1 ? own.y : row == 2 ? own.z : own.w;
    const uint32_t p = row == 0 ? partner.x : row == 1 ? partner.y : row == 2 ? partner.z : partner.w;
    const uint32_t mine = rope::rotate2(o, p, second_half, cs(2 * row), cs(2 * row + 1));
    float w_even, w_odd, w0, w1, w2, w3;
    pair_values<16>(__uint_as_float(mine), w_even, w_odd);   // words of rows r & 2 and (r & 2) | 1
    pair_values<32>(w_even, w0, w2);
    pair_values<32>(w_odd, w1, w3);
    return u32x4{__float_as_uint(w0), __float_as_uint(w1), __float_as_uint(w2), __float_as_uint(w3)};
}

// Fold pages [p_begin, p_end) (at most 64 per wavefront) of KV head g of a
// request with ctx tokens and n_pages pages into this wavefront's stream.
// entry: the block-table entry of page p_begin + wave + WAVES * lane, or
// anything for lanes past the range.  Full pages go round-robin over the
// wavefronts; a partly filled last page of the request goes to the wavefront
// next in turn, as the last page of its pipeline, and is folded with masking.
// FUSED: the request's last page always goes that way, and its new token
// (slot (ctx - 1) % 16, row b of k_new/v_new, loaded together with the page)
// is taken from k_new/v_new -- K rotated with `angles` when RoPE is on --
// written to the pool and folded from registers; no other workgroup reads
// that page.  With append_new false (a context length past the host bound,
// so ctx was clamped and slot ctx - 1 holds a real cached token) nothing is
// written and the page is folded as the pool holds it.  Returns
// HIPDECODE_VIOLATION_PAGE if a page id the range uses lies outside the pool
// (that page was skipped), else 0.
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

template <int G, int WAVES, bool FUSED = false, class Hook = NoHook>
__device__ __forceinline__ uint32_t fold_range(Stream<G> &st, const DecodeArgs &a, const u32x4 (&qv)[G],
                                           int g, int p_begin, int p_end, int n_pages, int ctx, int entry,
                                           const Lane &ln, int b = 0, const double2 *angles = nullptr,
                                           Hook before_fold = Hook(), bool append_new = true)
{
    const uint32_t tok_bytes = (uint32_t)a.num_kv_heads * kHeadDim * 2;   // bytes between slots
    const size_t page_elems = (size_t)kPageSize * a.num_kv_heads * kHeadDim;
    const uint32_t lane_off = (uint32_t)g * kHeadDim * 2 + (uint32_t)ln.row * tok_bytes + (uint32_t)ln.sub * 16;
    const uint32_t tok4 = 4 * tok_bytes;

    const bool tail_partial = (p_end == n_pages) && (FUSED || ctx % kPageSize != 0);
    const int full_end = tail_partial ? p_end - 1 : p_end;
    const int span = full_end - p_begin;
    const int npw = span > ln.wave ? (span - ln.wave + WAVES - 1) / WAVES : 0;
    // The last page, at relative index span, is page span / WAVES of
    // wavefront span % WAVES, which has exactly that many full pages.
    const bool my_tail = tail_partial && ln.wave == span % WAVES;
    const int n = npw + (my_tail ? 1 : 0);
    const int my_entry = ln.lane < n ? entry : -1;
    const unsigned num_pages = (unsigned)a.num_pages;

    // FUSED: the 16 lanes that hold the new token (register slot / 4) take
    // its K and V, and K's partner dims for RoPE, loaded before the first
    // page; once before_fold has the angles they rotate K, write the token to
    // the pool and park it in LDS, from where the fold of the last page takes
    // it.  Every lane loads (the request's row exists whenever ctx > 0), with
    // no branch, so that the compiler's wait for the table entry before the
    // first page counts these loads and does not wait for them.
    [[maybe_unused]] const int slot = (ctx - 1) % kPageSize;
    [[maybe_unused]] const bool new_lanes = FUSED && my_tail && append_new && ln.row == (slot & 3);
    __shared__ u32x4 new_tok[FUSED ? 2 : 1][FUSED ? 16 : 1];
    [[maybe_unused]] u32x4 kn, vn, kp;
    if constexpr (FUSED) {
        const size_t nrow = ((size_t)b * a.num_kv_heads + g) * kHeadDim;
        kn = load16(a.k_new + nrow + ln.sub * 8);
        vn = load16(a.v_new + nrow + ln.sub * 8);
        kp = load16(a.k_new + nrow + (ln.sub ^ 8) * 8);
    }

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
    auto fold_full = [&](const PageRegs &r, int i) {
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys < num_pages)   // a page outside the pool is never folded
            fold_page<G, false>(st, r, qv, a.scale_log2, 0, 0);
    };
    // The wavefront's last page: the request's partly filled last page when
    // this wavefront holds it, else a full one.
    auto fold_last = [&](PageRegs &r, int i) {
        if (!my_tail) {
            fold_full(r, i);
            return;
        }
        const int phys = __builtin_amdgcn_readlane(my_entry, i);
        if ((unsigned)phys >= num_pages)
            return;
        if constexpr (FUSED) {
            if (new_lanes) {
                const u32x4 k_tok = new_tok[0][ln.sub];
                const u32x4 v_tok = new_tok[1][ln.sub];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (t == (slot >> 2)) {
                        r.k[t] = k_tok;
                        r.v[t] = v_tok;
                    }
                }
            }
        }
        fold_page<G, true>(st, r, qv, a.scale_log2, full_end * kPageSize + ln.row, ctx);
    };

    // before_fold runs in every wavefront once the first page is in flight
    // (the fused kernel rotates q there); it may hold a workgroup barrier.
    // The fused kernel issues that page even in a wavefront with no pages (it
    // fetches page 0 and folds nothing): with the load under a branch, the
    // compiler's wait for q inside before_fold would also wait for the page.
    if (FUSED || n > 0)
        issue(ra, 0);
    before_fold();
    if constexpr (FUSED) {
        if (my_tail && angles != nullptr) {   // the whole wavefront: rotate_shared swaps lanes
            const int base = 8 * (ln.sub & 7);
            kn = rotate_shared(kn, kp, ln.sub >= 8, ln.row, [&](int e) { return angles[base + e]; });
        }
        if (new_lanes) {
            const int phys = __builtin_amdgcn_readlane(my_entry, npw);
            if ((unsigned)phys < num_pages) {
                const size_t off = (size_t)phys * page_elems * 2 + lane_off + (size_t)(slot >> 2) * tok4;
                *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(a.k_pool_w) + off) = kn;
                *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(a.v_pool_w) + off) = vn;
            }
            new_tok[0][ln.sub] = kn;
            new_tok[1][ln.sub] = vn;
        }
    }
    if (n > 0) {
        int i = 0;
        for (; i + 2 < n; i += 2) {
            issue(rb, i + 1);
            fold_full(ra, i);
            issue(ra, i + 2);
            fold_full(rb, i + 1);
        }
        if (i + 1 < n) {
            issue(rb, i + 1);
            fold_full(ra, i);
            fold_last(rb, i + 1);
        } else {
            fold_last(ra, i);
        }
    }
    // pages outside the pool were skipped above
    return __ballot(ln.lane < n && (unsigned)entry >= num_pages) != 0ull ? HIPDECODE_VIOLATION_PAGE : 0u;
}

// The workgroup's streams into LDS (row-groups merged first only with
// sixteen wavefronts).  The caller syncs the workgroup afterwards.
template <int G, int WAVES>
__device__ __forceinline__ void publish_streams(Stream<G> &st, Smem<G, WAVES> &sm, const Lane &ln)
{
    using S = Smem<G, WAVES>;
    if constexpr (S::kRowGroups == 1)
        merge_row_groups<G>(st);
    if (S::kRowGroups == 4 || ln.row == 0) {
        const int s = ln.wave * S::kRowGroups + (S::kRowGroups == 4 ? ln.row : 0);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(&sm.acc[s][h][ln.sub * 8]);
            dst[0] = f32x4{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
            dst[1] = f32x4{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
            if (ln.sub == 0) {
                sm.m[s][h] = st.m[h];
                sm.l[s][h] = st.l[h];
            }
        }
    }
}

// Max and sum over the first N lanes of a wavefront, handed to every lane
// (lanes past N must hold -inf and 0).
template <int N>
__device__ __forceinline__ float lanes_max(float x)
{
    if constexpr (N <= 16)
        return lane_value(row_max16(x), 0);
    else
        return wave_max(x);
}

template <int N>
__device__ __forceinline__ float lanes_sum(float x)
{
    if constexpr (N <= 16)
        return lane_value(row_sum16(x), 0);
    else
        return wave_sum(x);
}

// Write the workgroup's result for G query heads: final output when one
// workgroup covers the (request, KV head), else a partial at partial index
// part_index(h).  Each thread takes dims of one head at a time (uniform
// across its wavefront); lane j weighs stream j, so the streams' weights
// reach the sums as scalars.  The caller syncs before and after.
template <int G, int WAVES, bool OUT_F32, class PartIndex>
__device__ __forceinline__ void emit(const DecodeArgs &a, const Smem<G, WAVES> &sm, size_t row0, bool final,
                                     PartIndex part_index, const Lane &ln)
{
    using S = Smem<G, WAVES>;
    constexpr int NS = S::kStreams;
    for (int idx = ln.tid; idx < G * kHeadDim; idx += S::kThreadsWG) {
        const int h = __builtin_amdgcn_readfirstlane(idx / kHeadDim);
        const int d = idx % kHeadDim;
        // The streams' sums for this dim, read before the weights are formed
        // so that the LDS reads overlap that work rather than each other's.
        float sums[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
            sums[s] = sm.acc[s][h][d];
        const float ms = ln.lane < NS ? sm.m[ln.lane][h] : -INFINITY;
        const float ls = ln.lane < NS ? sm.l[ln.lane][h] : 0.f;
        const float M = lanes_max<NS>(ms);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float w = merge_weight(ms, M_use);   // 0 past the streams
        const float L = lanes_sum<NS>(ls * w);
        // four independent chains, so the FMAs do not wait on one another
        constexpr int kChains = NS >= 4 ? 4 : NS;
        float part[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            part[c] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            part[s % kChains] = fmaf(lane_value(w, s), sums[s], part[s % kChains]);
        float A = part[0];
#pragma unroll
        for (int c = 1; c < kChains; ++c)
            A += part[c];
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

// K consecutive floats (K = 1 or 2) of a partial, coherently.
template <int K>
__device__ __forceinline__ void load_dims(float (&v)[K], const float *p)
{
    if constexpr (K == 1) {
        v[0] = coherent_load(p);
    } else {
        static_assert(K == 2, "one or two dims per thread");
        const uint64_t u = coherent_load8(p);
        v[0] = __uint_as_float((uint32_t)u);
        v[1] = __uint_as_float((uint32_t)(u >> 32));
    }
}

// The final merge of `count` partials of G query heads (partial i of head h
// at index part_index(i, h)).  Thread t owns K dims of one head; when the
// workgroup has more threads than dims, the threads of a dim split the
// partials into S sets and add their sums through LDS at the end.  Every
// wavefront finds its head's maximum and sum itself, lane j weighing
// partials j, j + 64, ... (one round of 64 at a time), so the weights reach
// the sums as scalars and no workgroup barrier separates the loads from the
// sums.  A thread's first PRE partials are loaded in one batch right after
// the (m, l) pairs; the rest go in batches of NB, each batch's loads issued
// before any of them is used, so that each batch costs one memory round trip.
template <int G, int WAVES, int PRE, bool OUT_F32, class PartIndex>
__device__ __forceinline__ void merge_partials_pre(const DecodeArgs &a, Smem<G, WAVES> &sm, size_t row0,
                                                   int count, PartIndex part_index, const Lane &ln)
{
    constexpr int D = G * kHeadDim;
    constexpr int NT = 64 * WAVES;
    constexpr int K = D > NT ? D / NT : 1;          // dims per thread
    constexpr int S = NT > D ? NT / D : 1;          // sets of partials
    constexpr int TPS = D / K;                      // threads per set
    constexpr int NB = 32 / K;                      // partials per batch after the first
    constexpr int kRounds = kMaxMergeSplits / 64;   // rounds of 64 (m, l) pairs at most
    static_assert(K <= 2 && TPS % 64 == 0, "whole wavefronts per set and head");
    const int t = ln.tid % TPS;
    const int set = __builtin_amdgcn_readfirstlane(ln.tid / TPS);
    const int h = __builtin_amdgcn_readfirstlane(t * K / kHeadDim);
    const int d = (t * K) % kHeadDim;
    const float *acc_base = a.part_acc + d;
    auto acc_ptr = [&](int i) { return acc_base + part_index(i, h) * kHeadDim; };
    auto ml_of = [&](int i) { return coherent_load8(a.part_ml + part_index(min(i, count - 1), h) * 2); };
    float A[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        A[k] = 0.f;
    // partials [i_begin, i_end) of this set, i = set (mod S), weights w of the round starting at c0
    auto add_batches = [&](int i_begin, int i_end, float w, int c0) {
        for (int i0 = i_begin; i0 < i_end; i0 += NB * S) {
            float v[NB][K];
#pragma unroll
            for (int r = 0; r < NB; ++r)
                load_dims<K>(v[r], acc_ptr(min(i0 + r * S, count - 1)));
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const int i = i0 + r * S;
                if (i < i_end) {
                    const float wi = lane_value(w, i - c0);
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        A[k] = fmaf(wi, v[r][k], A[k]);
                }
            }
        }
    };

    // round 0: (m, l) of partial `lane`, then this set's first PRE partials
    const uint64_t ml0 = ml_of(ln.lane);
    float pre[PRE][K];
#pragma unroll
    for (int r = 0; r < PRE; ++r)
        load_dims<K>(pre[r], acc_ptr(min(set + r * S, count - 1)));
    const float m0 = ln.lane < count ? __uint_as_float((uint32_t)ml0) : -INFINITY;
    const float l0 = ln.lane < count ? __uint_as_float((uint32_t)(ml0 >> 32)) : 0.f;
    float mx = m0;
    if (count > 64) {
        // the maxima of the later rounds, in one batch (indices past the end clamped, values dropped)
        uint64_t mlr[kRounds - 1];
#pragma unroll
        for (int c = 1; c < kRounds; ++c)
            mlr[c - 1] = ml_of(64 * c + ln.lane);
#pragma unroll
        for (int c = 1; c < kRounds; ++c)
            if (64 * c + ln.lane < count)
                mx = fmaxf(mx, __uint_as_float((uint32_t)mlr[c - 1]));
    }
    const float M = wave_max(mx);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float w0 = merge_weight(m0, M_use);
    float lsum = l0 * w0;
    const int n0 = min(count, 64);
    // four independent chains over the prefetched partials, so the FMAs do
    // not wait on one another
    float chain[4][K];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < K; ++k)
            chain[c][k] = 0.f;
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        const int i = set + r * S;
        if (i < n0) {
            const float wi = lane_value(w0, i);
#pragma unroll
            for (int k = 0; k < K; ++k)
                chain[r % 4][k] = fmaf(wi, pre[r][k], chain[r % 4][k]);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        A[k] += (chain[0][k] + chain[1][k]) + (chain[2][k] + chain[3][k]);
    add_batches(set + PRE * S, n0, w0, 0);
    for (int c0 = 64; c0 < count; c0 += 64) {   // the later rounds of 64 partials
        const int j = c0 + ln.lane;
        const uint64_t ml = ml_of(j);
        const float wj = j < count ? merge_weight(__uint_as_float((uint32_t)ml), M_use) : 0.f;
        lsum = fmaf(j < count ? __uint_as_float((uint32_t)(ml >> 32)) : 0.f, wj, lsum);
        add_batches(c0 + (set - c0 % S + S) % S, min(count, c0 + 64), wj, c0);
    }
    const float L = wave_sum(lsum);
    if constexpr (S > 1) {
        float *scratch = &sm.acc[0][0][0];
#pragma unroll
        for (int k = 0; k < K; ++k)
            scratch[set * D + t * K + k] = A[k];
        __syncthreads();
        if (set != 0)
            return;
#pragma unroll
        for (int s = 1; s < S; ++s)
#pragma unroll
            for (int k = 0; k < K; ++k)
                A[k] += scratch[s * D + t * K + k];
    }
    const size_t o = (row0 + h) * kHeadDim + d;
#pragma unroll
    for (int k = 0; k < K; ++k)
        store_out<OUT_F32>(a.out, o + k, A[k] / L);
    if (d == 0 && a.lse != nullptr)
        a.lse[row0 + h] = (M + log2f(L)) * kLn2;
}

// The final merge, with as many partials loaded up front as a set needs
// (8 or 32), and the ticket reset for the next call.
template <int G, int WAVES, bool OUT_F32, class PartIndex>
__device__ __forceinline__ void merge_partials(const DecodeArgs &a, Smem<G, WAVES> &sm, size_t row0, int count,
                                               PartIndex part_index, int32_t *ticket, const Lane &ln)
{
    constexpr int D = G * kHeadDim;
    constexpr int S = 64 * WAVES > D ? 64 * WAVES / D : 1;
    if (count <= 8 * S)
        merge_partials_pre<G, WAVES, 8, OUT_F32>(a, sm, row0, count, part_index, ln);
    else
        merge_partials_pre<G, WAVES, 32, OUT_F32>(a, sm, row0, count, part_index, ln);
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

// The work list.  The grid has a slot for every partition the longest
// context could need, but a ragged batch has far fewer real (request,
// partition) units.  Unit u is the u-th real unit: first every full
// partition, in request order, partitions ascending; then each request's
// partly filled last partition, in request order (an empty request counts
// one such unit, which writes its empty output).  Slots past the last real
// unit get b = -1 and exit, so every workgroup the dispatcher places early
// carries work, and the short units come last: the workgroups resident on a
// CU run close to one after another in dispatch order, so the last ones set
// the tail of the call.
struct RealUnit {
    int b, split, ctx;
    bool over;   // the request's context length exceeds the host bound (ctx is clamped)
    bool bad;    // the request's context length is negative or exceeds the host bound
};

__device__ __forceinline__ RealUnit real_unit(const DecodeArgs &a, int u)
{
    const int lane = (int)(threadIdx.x & 63);
    const int span = kPageSize * a.partition_pages;
    RealUnit r{-1, 0, 0, false, false};
    for (int pass = 0; pass < 2; ++pass) {   // 0: full partitions, 1: partly filled last ones
        int carry = 0;
        for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
            const int j = c0 + lane;
            const int raw = j < a.num_seqs ? a.context_lens[j] : 0;
            const int cj = clamp_ctx(raw, a.max_context_len);
            const int nj = j >= a.num_seqs ? 0 : pass == 0 ? cj / span : ((cj == 0 || cj % span != 0) ? 1 : 0);
            const int incl = wave_inclusive_scan(nj, lane);
            const int excl = incl - nj;
            const unsigned long long hit = __ballot(u >= carry + excl && u < carry + incl);
            if (hit != 0ull) {
                const int l = __builtin_amdgcn_readfirstlane(__ffsll(hit) - 1);
                r.b = c0 + l;
                r.ctx = __builtin_amdgcn_readlane(cj, l);
                r.split = pass == 0 ? u - carry - __builtin_amdgcn_readlane(excl, l) : r.ctx / span;
                const int raw_l = __builtin_amdgcn_readlane(raw, l);
                r.over = raw_l > a.max_context_len;
                r.bad = raw_l < 0 || r.over;
                return r;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        u -= carry;
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
// Four wavefronts per SIMD fit in 128 VGPRs for G <= 2; G = 4 holds twice the
// softmax state and runs two per SIMD (about 172 VGPRs) rather than spill.
template <int G, int WAVES, bool OUT_F32, bool FUSED>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(G == 4 ? 2 : 4)))
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
    // Contract violations met here, reported once no load of the call is in
    // flight, so that the branch leaves the waits on the main path alone.
    uint32_t viol = 0;
    if (a.num_seqs == 1 || a.nsplit_max == 1) {
        // Every unit of the full grid up to a request's partition count is real.
        b = b_full;
        split = split_full;
        const int raw = a.context_lens[b];
        ctx = clamp_ctx(raw, a.max_context_len);
        over = raw > a.max_context_len;
        if (split == 0 && (raw < 0 || over))
            viol = HIPDECODE_VIOLATION_CONTEXT;
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
        if (split == 0 && u.bad)
            viol = HIPDECODE_VIOLATION_CONTEXT;
        spec_entry = spec_full;
        if (b != b_full || split != split_full) {   // ragged batch: fetch this partition's entries
            const int idx = split * pp + ln.wave + WAVES * ln.lane;
            spec_entry = (idx < a.max_blocks && ln.lane * WAVES < pp)
                             ? a.block_table[(size_t)b * a.max_blocks + idx] : -1;
        }
    }
    const int p_begin = split * pp;
    const int n_pages = (ctx + kPageSize - 1) / kPageSize;
    const int nsplit_b = (n_pages + pp - 1) / pp;
    const size_t row0 = (size_t)b * a.num_q_heads + (size_t)g * G;   // first query row of the group

    if (ctx == 0) {
        write_empty<OUT_F32>(a, row0, G, ln.tid, 64 * WAVES);
        if (viol != 0 && ln.tid == 0)
            report_violation(a.violations, viol);
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
    // Loaded with RoPE off too: loads under a branch leave the compiler's
    // wait for the table entry, which the first page needs, counting too few
    // loads after it, so that wait would also hold for q.
    u32x4 qp[G];
    if constexpr (FUSED) {
#pragma unroll
        for (int h = 0; h < G; ++h)
            qp[h] = load16(a.q + (row0 + h) * kHeadDim + (ln.sub ^ 8) * 8);
    }
    auto rotate_q = [&]() __attribute__((always_inline)) {
        if constexpr (FUSED) {
            if (rope_on) {
                if (ln.wave == 0)
                    angles[ln.lane] = rope::angle_of(rope::frequency(a.rope_log2_theta, ln.lane), ctx - 1);
                __syncthreads();
                const int base = 8 * (ln.sub & 7);
#pragma unroll
                for (int h = 0; h < G; ++h)
                    qv[h] = rotate_shared(qv[h], qp[h], ln.sub >= 8, ln.row, [&](int e) { return angles[base + e]; });
            }
        }
    };
    Stream<G> st;
    st.init();
    if constexpr (FUSED)
        viol |= fold_range<G, WAVES, FUSED>(st, a, qv, g, p_begin, min(p_begin + a.partition_pages, n_pages),
                                            n_pages, ctx, spec_entry, ln, b, rope_on ? angles : nullptr, rotate_q,
                                            !over);
    else
        viol |= fold_range<G, WAVES, FUSED>(st, a, qv, g, p_begin, min(p_begin + a.partition_pages, n_pages),
                                            n_pages, ctx, spec_entry, ln, b);
    if (viol != 0 && ln.lane == 0)
        report_violation(a.violations, viol);
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
