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
// head, pair of half-tiles of query tokens).  A wavefront owns 32 query rows
// -- 32/G chunk tokens times the G query heads that share the KV head --
// which is one 32x32 MFMA tile, so a workgroup holds 256 rows: every K/V byte
// brought into LDS serves up to 256 rows, which keeps the re-reads of the
// context (one pass per workgroup) within what the caches deliver.  Causal
// attention gives late chunk tokens more keys than early ones, so wavefronts
// 0-3 take an early half-tile and wavefronts 4-7 the matching late one.
// Past the early rows' last key their wavefronts write them out and each
// takes half of every remaining step of a late wavefront's rows, with a
// softmax state of its own that is merged through LDS at the end.  Keys go
// by in steps of 64 (four
// pages), copied straight from the pools into a three-stage LDS ring
// (global_load_lds, two steps ahead), both K and V row-major, and used in two
// halves of 32.  Before a step's barrier each wavefront rewrites the V rows
// it copied as fp16, in place.
//
// Per 32-key half and wavefront, with 32x32x16 MFMAs (A 32x16, B 16x32):
//   S^T[key][row]  = sum_d K[key][d] Q[row][d]        8 MFMAs (bf16), A = K, B = Q^T
//   O^T[dim][row] += sum_key V[key][dim] P[row][key]  8 MFMAs (fp16), A = V^T, B = P^T
// Lane l of the S^T accumulator holds row l % 32 and keys
// 8(r/4) + 4(l/32) + r%4 for registers r = 0..15, which is exactly how the
// B operand of the second product wants P^T, provided both products agree
// on the order of the key index: the V^T operand is read with transposing
// LDS reads (ds_read_b64_tr_b16) that take those same keys.  The softmax is
// online, in base 2 with scale*log2(e) folded in (one FMA and one v_exp_f32
// per score), against a running maximum that moves only when the weights
// grow large; the two lanes (l, l ^ 32) that share a row combine their
// maxima and sums with v_permlane32_swap.  P.V runs in fp16: each weight is
// rounded to the nearest fp16 (2^-11 relative, four times finer than bf16)
// for the matrix cores, while the running sum adds up the fp32 weights, and
// V is widened to fp16 in LDS by the wavefront that copied it (exact for
// |V| < 2^16; larger values are reported as a contract violation).
#include "hipdecode.h"
#include "internal.h"

#include <math.h>
#include <type_traits>

namespace hipdecode {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRowsPerWave = 32;          // one 32x32 MFMA tile of (token, head) rows
constexpr int kKeys = 64;                 // keys per step: four pages, used in two halves of 32
constexpr int kRowBytes = kHeadDim * 2;   // one K or V row in LDS: 16 chunks of 16 bytes
constexpr int kStepBytes = kKeys * kRowBytes;
constexpr int kStages = 3;                // LDS stages: the copy runs two steps ahead
constexpr int kDimBlocks = kHeadDim / 32; // O^T is four 32x32 accumulators
constexpr float kNegBig = -1.0e30f;       // running-max start: finite, so no inf - inf
constexpr float kPsumMax = 32768.0f;      // a half's weights summing past this move the running max
constexpr float kWeightBias = 4.0f;       // weights carry a factor 2^4: the running max sits 4 below the row max
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
    int32_t pairs;          // workgroups (pairs of half-tiles) per request and KV head
    float scale_log2;       // max(|scale| * log2(e), 2^-100): positive, see the launch
    uint32_t q_sign;        // 0x80008000 when scale < 0: q is negated on load instead
    uint32_t *violations;   // contract-violation flag word of this device
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// LDS rows are stored with their 16-byte chunks permuted: chunk c of step
// row r sits at position c ^ swz(r), with a different permutation for K and
// for V to suit their reads.  K is read 16 bytes per lane, one chunk of rows
// j = 0..31: swz_k(r) = r mod 16 puts sixteen consecutive rows' chunk in
// sixteen different positions.  V is read with transposing 8-byte reads, in
// which 32 lanes touch chunks 4 db .. 4 db + 3 of four consecutive rows:
// swz_v spreads those 16 (row, chunk) pairs over all 16 positions.  Either
// way no two lanes of one LDS cycle meet in a bank, for 64 banks (256 bytes a
// cycle) as for 32.
__device__ inline int swz_k(int r) { return r & 15; }
__device__ inline int swz_v(int r) { return ((r & 3) << 2) | (r & 2); }

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

// Two fp32 values to packed fp16, each rounded to nearest even (one
// v_cvt_pk_f16_f32).
__device__ inline uint32_t pack2_f16(float x, float y)
{
    const f32x2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}


// Wait until at most N of this wavefront's vector-memory loads are
// outstanding (the copies into LDS count among them).
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);   // expcnt and lgkmcnt left at their maxima
}

// Workgroup barrier for the LDS stages.  A plain s_barrier: every wavefront
// has already waited for its own copies (wait_vm) and consumed its LDS reads,
// and a fence here would make the compiler wait for all loads, including the
// copies still running for later steps.  The memory clobber keeps LDS accesses
// on their side of it.
__device__ inline void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The same barrier after this wavefront's own LDS writes have completed, so
// that the other wavefronts read them once past it.
__device__ inline void stage_barrier_after_writes()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy 16 bytes per lane from global memory (uniform base + 32-bit lane
// offset) straight into LDS: lane i lands at byte lds_addr + 16 i.  Written
// out here, rather than through the compiler's builtin, because the compiler
// then waits for every such copy before any LDS read, which would leave no
// copy in flight behind the compute; the waits are wait_vm() calls instead.
__device__ inline void copy_to_lds(const uint8_t *base, uint32_t off, const lds_u8_t *dst)
{
    const uint32_t lds_addr = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

// A wave-uniform 4-byte load through the scalar cache, waited for at once.
// Its wait (lgkmcnt) is independent of the copies into LDS (vmcnt), which a
// vector load of the same value would have to wait behind.
__device__ inline int scalar_load(const int32_t *p)
{
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

template <int G, bool OUT_F32>
__global__ __launch_bounds__(kPfThreads) void prefill_attn_kernel(PrefillArgs a)
{
    constexpr int kTokPerWave = kRowsPerWave / G;
    constexpr int kHalfWaves = kPfWaves / 2;
    constexpr int kHalfTokens = kHalfWaves * kTokPerWave;   // chunk tokens of one half-tile
    __shared__ __align__(16) uint8_t k_lds[kStages][kStepBytes];
    __shared__ __align__(16) uint8_t v_lds[kStages][kStepBytes];

    // KV head fastest.  Workgroup `pair` of a request takes two half-tiles of
    // its chunk: half-tile `pair` (wavefronts 0-3) and half-tile
    // halves - 1 - pair (wavefronts 4-7), an early and a late stretch of the
    // chunk, so that every workgroup has about the same number of keys to
    // attend over.  With an odd number of half-tiles the middle one comes
    // alone and wavefronts 4-7 of its workgroup hold no rows.
    const int bid = blockIdx.x;
    const int g = bid % a.num_kv_heads;
    const int rest = bid / a.num_kv_heads;
    const int pair = rest % a.pairs;
    const int b = rest / a.pairs;
    const int ctx = a.context_lens[b];
    const int start = a.new_start[b];
    const int n = a.new_start[b + 1] - start;
    // Uniform across the workgroup: a request that breaks the contract, or a
    // pair past its chunk, does nothing.
    const bool rows_bad = n < 0 || n > max(ctx, 0) || n > a.max_new || start < 0 || (int64_t)start + n > a.num_rows;
    const bool ctx_bad = ctx < 0 || (int64_t)ctx > (int64_t)a.max_blocks * kPageSize;
    if (n <= 0 || rows_bad || ctx_bad) {
        if (threadIdx.x == 0 && (rows_bad || ctx_bad))
            report_violation(a.violations, (rows_bad ? HIPDECODE_VIOLATION_ROWS : 0u) |
                                               (ctx_bad ? HIPDECODE_VIOLATION_CONTEXT : 0u));
        return;
    }
    const int halves = (n + kHalfTokens - 1) / kHalfTokens;
    if (pair >= (halves + 1) / 2)
        return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;          // this lane's row in the wavefront's tile
    const int half = lane >> 5;       // which 8 of each 16 along the contracted index
    const bool upper = w >= kHalfWaves;
    const int half_tile = upper ? halves - 1 - pair : pair;
    const bool wave_live = !(upper && half_tile == pair);   // uniform
    const int tw0 = half_tile * kHalfTokens + (w % kHalfWaves) * kTokPerWave;   // this wavefront's first token
    int tq = tw0 + j / G;
    const int h = g * G + j % G;
    bool row_ok = wave_live && tq < n;
    int pos = row_ok ? ctx - n + tq : -1;      // -1: every key masked
    size_t row = (size_t)start + min(tq, n - 1);

    // Q^T operand: dims 16 ks + 8 half .. +7 of this lane's row.  A negative
    // scale is applied as a sign flip of q (exact), so that the scale factor
    // used below is never negative and the row maximum of scale * s is
    // scale times the maximum of s.
    bf16x8_t qop[kHeadDim / 16];
    auto load_q = [&]() __attribute__((always_inline)) {
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
    };
    load_q();

    const int last_tok = min((halves - pair) * kHalfTokens, n) - 1;   // the workgroup's last chunk token
    const int kv_end = ctx - n + last_tok + 1;           // keys [0, kv_end)
    const int nblk = (kv_end + kKeys - 1) / kKeys;
    // Step bounds, uniform across the workgroup.  Steps before e1 mask no key
    // of any row (wavefront 0 holds the first token); the early half-tile
    // attends to keys of steps before e2; the late half-tile, if any, masks
    // no key before e3 and attends up to the last step.
    const bool has_upper = halves - 1 - pair != pair;
    const int e1 = (ctx - n + pair * kHalfTokens + 1) / kKeys;
    const int e2 = (ctx - n + min((pair + 1) * kHalfTokens, n) - 1) / kKeys + 1;
    const int e3 = has_upper ? (ctx - n + (halves - 1 - pair) * kHalfTokens + 1) / kKeys : 0;

    // Copies into LDS.  Wavefront w moves step rows 8w .. 8w + 7 of K and of
    // V -- eight consecutive keys, so one page -- as two 1 KiB copies of four
    // rows each (global_load_lds: lane i lands at byte 16 i of the copy).
    // Lane i takes row 4k + i / 16 of the pair and fetches the chunk whose
    // permuted position is i % 16.  Keys past kv_end are fetched as key
    // kv_end - 1, so masked keys still hold finite values (their weight is an
    // exact 0, and 0 times a finite V is 0).
    const int drow = lane >> 4;
    const uint32_t kv_row_bytes = (uint32_t)a.num_kv_heads * kRowBytes;
    const size_t page_bytes = (size_t)kPageSize * kv_row_bytes;
    const uint8_t *k_bytes = reinterpret_cast<const uint8_t *>(a.k_pool) + (size_t)g * kRowBytes;
    const uint8_t *v_bytes = reinterpret_cast<const uint8_t *>(a.v_pool) + (size_t)g * kRowBytes;
    uint32_t k_chunk[2], v_chunk[2], k_full[2], v_full[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = 8 * w + 4 * k + drow;
        k_chunk[k] = (uint32_t)(((lane & 15) ^ swz_k(r)) * 16);
        v_chunk[k] = (uint32_t)(((lane & 15) ^ swz_v(r)) * 16);
        // a step with all eight keys in range: the key's slot is r mod 16
        k_full[k] = (uint32_t)(r % kPageSize) * kv_row_bytes + k_chunk[k];
        v_full[k] = (uint32_t)(r % kPageSize) * kv_row_bytes + v_chunk[k];
    }
    const int32_t *table = a.block_table + (size_t)b * a.max_blocks;
    auto issue = [&](int kb, int stage) __attribute__((always_inline)) {
        const int key_w = kb * kKeys + 8 * w;                // first of this wavefront's eight keys
        const int pidx = min(key_w, kv_end - 1) / kPageSize;
        const int raw_page = scalar_load(table + pidx);
        const int page = (unsigned)raw_page < (unsigned)a.num_pages ? raw_page : 0;
        const size_t pbase = (size_t)page * page_bytes;
        const bool full = key_w + 8 <= kv_end;   // uniform
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t ko = k_full[k], vo = v_full[k];
            if (!full) {
                const uint32_t row_off = (uint32_t)(min(key_w + 4 * k + drow, kv_end - 1) % kPageSize) * kv_row_bytes;
                ko = row_off + k_chunk[k];
                vo = row_off + v_chunk[k];
            }
            const int r0 = 8 * w + 4 * k;
            copy_to_lds(k_bytes + pbase, ko, (const lds_u8_t *)&k_lds[stage][r0 * kRowBytes]);
            copy_to_lds(v_bytes + pbase, vo, (const lds_u8_t *)&v_lds[stage][r0 * kRowBytes]);
        }
    };

    // LDS read offsets inside a stage.  K operand of S^T: row 32 hh + j,
    // chunk 2 ks + half.  V^T operand of O^T (two transposing 8-byte reads per
    // MFMA): in the 16-lane group q = lane / 16, lane i reads row
    // 4 (q / 2) + i / 4 (plus 16 kh + 8 e + 32 hh) at dims 32 db + 16 (q % 2) +
    // 4 (i % 4); the read hands lane i the four rows' values of dim
    // 32 db + 16 (q % 2) + i, which is the A layout (row = dim, k = key).
    uint32_t k_off[kHeadDim / 16];
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks)
        k_off[ks] = (uint32_t)(j * kRowBytes + ((2 * ks + half) ^ swz_k(j)) * 16);
    uint32_t v_off[kDimBlocks];
    {
        const int q = lane >> 4;
        const int i = lane & 15;
        const int vr = 4 * (q >> 1) + (i >> 2);
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db)
            v_off[db] = (uint32_t)(vr * kRowBytes + ((4 * db + 2 * (q & 1) + ((i & 3) >> 1)) ^ swz_v(vr)) * 16 +
                                   8 * (i & 1));
    }

    f32x16_t acc[kDimBlocks];
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
        acc[db] = zero16();
    float m_run = kNegBig;
    float l_run = 0.f;

    auto scores = [&](int stage, int hh) __attribute__((always_inline)) {
        // S^T = K Q^T for keys 32 hh .. 32 hh + 31 of this step
        const uint8_t *kl = &k_lds[stage][32 * hh * kRowBytes];
        bf16x8_t kop[kHeadDim / 16];
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks)
            kop[ks] = *reinterpret_cast<const bf16x8_t *>(kl + k_off[ks]);
        f32x16_t s = zero16();
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], s, 0, 0, 0);
        return s;
    };
    // The softmax weights of one 32-key half, and their fp16 forms.
    struct Half {
        float pw[16];      // 2^(c s - m) per key of this lane
        float psum;        // their sum
        uint32_t pp[8];    // fp16 forms, packed pairs (keys in the S^T accumulator's order)
    };
    // Online softmax in base 2 (row j; keys 8(r/4) + 4 half + r%4).  With
    // c = |scale| log2(e) > 0, the row maximum of c s is c max(s) and
    // p = 2^(c s - m) is one FMA and one v_exp_f32 (weights below 2^-126 of
    // the row maximum may flush to zero); a masked score is -inf, so its
    // weight is exactly 0.
    //
    // The running max m is not brought up to date on every half.  weights()
    // computes p = 2^(c s - m) against the m in hand, with no branch; only
    // when some lane's half sums past kPsumMax -- a row maximum well above m,
    // or m still at its start value on a row's first half -- does settle()
    // find the row maxima, move m to 4 below the largest (kWeightBias), rescale
    // l and the accumulators, and recompute the weights.  Every weight is
    // then 2^4 times its value against the row maximum; out and lse share the
    // reference m, so the factor cancels in both.
    //
    // Each weight goes to the matrix cores as its nearest fp16, within 2^-11
    // of it (relative), while l_run adds up the fp32 weights, so out is off
    // by at most 2^-11 times the weighted mean of |V| over the row's keys.  A
    // half's fp32 weights sum to at most 2^15 once settled, so none rounds
    // to an fp16 inf.  With the factor 2^4, weights down to 2^-18 of the row
    // maximum stay normal fp16 numbers; smaller ones keep an absolute error
    // under 2^-29 of it, against l >= 2^4 of it.
    auto pack = [&](Half &w) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            w.pp[r / 2] = pack2_f16(w.pw[r], w.pw[r + 1]);
    };
    auto exps = [&](Half &w, const f32x16_t &s, float m) __attribute__((always_inline)) {
        const float c = a.scale_log2;
        w.psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            w.pw[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m));   // masked: 2^-inf = 0
            w.pw[r + 1] = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -m));
            w.psum += w.pw[r] + w.pw[r + 1];
        }
    };
    auto weights = [&](auto masked, int kb, int hh, f32x16_t &s, Half &w) __attribute__((always_inline)) {
        if constexpr (decltype(masked)::value) {  // only steps reaching past the tile's first position
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * kKeys + 32 * hh + 8 * (r / 4) + 4 * half + (r % 4);
                s[r] = key > pos ? -INFINITY : s[r];
            }
        }
        exps(w, s, m_run);
        pack(w);
    };
    auto settle = [&](const f32x16_t &s, Half &w) __attribute__((always_inline)) {
        if (__any(!(w.psum <= kPsumMax))) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[r]);
            const float m_new = fmaxf(m_run, pair_max(mx) * a.scale_log2 - kWeightBias);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                acc[db] *= alpha;
            exps(w, s, m_new);
            pack(w);
        }
        l_run += w.psum;
    };
    // V^T operands of one half: O^T += V^T P^T in two k-steps of 16 keys.
    // P^T: lane l holds keys 16 kh + 4 half + e and 16 kh + 8 + 4 half + e
    // (e < 4) of the half, in the S^T accumulator's own order; the V^T reads
    // take the same keys.
    auto read_vt = [&](int stage, int hh, i16x8_t (&vv)[2][kDimBlocks]) __attribute__((always_inline)) {
        const lds_u8_t *vl = (const lds_u8_t *)&v_lds[stage][32 * hh * kRowBytes];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) {
                const lds_u8_t *p = vl + 16 * kh * kRowBytes + v_off[db];
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p + 8 * kRowBytes));
                vv[kh][db] = i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    };
    auto pv = [&](const i16x8_t (&vv)[2][kDimBlocks], const Half &w) __attribute__((always_inline)) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const f16x8_t pop = __builtin_bit_cast(
                f16x8_t, make_uint4(w.pp[4 * kh], w.pp[4 * kh + 1], w.pp[4 * kh + 2], w.pp[4 * kh + 3]));
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) {
                const f16x8_t vop = __builtin_bit_cast(f16x8_t, vv[kh][db]);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pop, acc[db], 0, 0, 0);
            }
        }
    };
    // One half alone (the late rows' steps, each wavefront on one half).
    auto softmax_pv = [&](auto masked, int kb, int stage, int hh, f32x16_t s) __attribute__((always_inline)) {
        Half w;
        weights(masked, kb, hh, s, w);
        settle(s, w);
        i16x8_t vv[2][kDimBlocks];
        read_vt(stage, hh, vv);
        __builtin_amdgcn_sched_barrier(0);
        pv(vv, w);
    };
    // Both halves: the scores of both are issued first, so the matrix cores
    // work on the second half's S while the first half's weights are formed;
    // the second half's weights and their fp16 forms (branch-free) are formed
    // beside the first half's P.V products, whose V^T operands, and the second
    // half's, are read before them; only then can the second half's rare
    // rescale (which needs the first half's products in the accumulators)
    // run, followed by its P.V.
    auto compute_step = [&](auto masked, int kb, int stage) __attribute__((always_inline)) {
        // all sixteen K operands of the step are read before the first MFMA
        bf16x8_t k0[kHeadDim / 16], k1[kHeadDim / 16];
        const uint8_t *kl0 = &k_lds[stage][0];
        const uint8_t *kl1 = &k_lds[stage][32 * kRowBytes];
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks) {
            k0[ks] = *reinterpret_cast<const bf16x8_t *>(kl0 + k_off[ks]);
            k1[ks] = *reinterpret_cast<const bf16x8_t *>(kl1 + k_off[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16_t s0 = zero16(), s1 = zero16();
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks)
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0[ks], qop[ks], s0, 0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks)
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[ks], qop[ks], s1, 0, 0, 0);
        Half w0, w1;
        weights(masked, kb, 0, s0, w0);
        settle(s0, w0);
        i16x8_t vv0[2][kDimBlocks], vv1[2][kDimBlocks];
        read_vt(stage, 0, vv0);
        read_vt(stage, 1, vv1);
        __builtin_amdgcn_sched_barrier(0);
        pv(vv0, w0);
        weights(masked, kb, 1, s1, w1);
        settle(s1, w1);
        pv(vv1, w1);
    };

    // V rows to fp16, in place in LDS: this wavefront's eight rows of a step
    // (the ones it copied: bytes 2048 w .. 2048 w + 2047 of the stage), 32
    // bytes per lane.  A bf16 value has 8 significant bits, so its fp16 form
    // is exact for 2^-17 <= |v| < 2^16; below that the fp16 subnormals keep it
    // to within 2^-25.  A value of 2^16 or more becomes inf, which makes
    // every product sum of the step's rows inf or NaN (0 * inf is NaN for
    // masked keys); write_rows finds that, once per wavefront.
    auto widen_v = [&](int stg) __attribute__((always_inline)) {
        uint4 *p = reinterpret_cast<uint4 *>(&v_lds[stg][8 * w * kRowBytes]) + lane;
        uint4 x[2] = {p[0], p[64]};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t *u = reinterpret_cast<uint32_t *>(&x[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(u[e] << 16);
                const float hi = __uint_as_float(u[e] & 0xFFFF0000u);
                u[e] = pack2_f16(lo, hi);
            }
        }
        p[0] = x[0];
        p[64] = x[1];
    };

    // Pipeline: step kb + 2 is copied into LDS while step kb is computed.
    // Per step each wavefront issues four copies; before the barrier of step
    // kb it waits until only step kb + 1's four may still be in flight.
    issue(0, 0);
    if (nblk > 1)
        issue(1, 1);
    // Page ids outside the pool are read as page 0 above; they are found here
    // once, from the workgroup's table entries, while the first copies fly,
    // and reported at the end.
    bool bad_page;
    {
        const int npages = (kv_end + kPageSize - 1) / kPageSize;
        bool bad = false;
        for (int i = tid; i < npages; i += kPfThreads)
            bad |= (unsigned)table[i] >= (unsigned)a.num_pages;
        bad_page = __ballot(bad) != 0ull;
    }
    wait_vm<0>();   // q and the first copies: nothing older than a step's copies stays in flight in the loop
    int stage = 0;
    auto sync_step = [&](int kb) __attribute__((always_inline)) {
        if (kb + 1 < nblk)
            wait_vm<4>();
        else
            wait_vm<0>();
        widen_v(stage);
        stage_barrier_after_writes();
        if (kb + 2 < nblk)
            issue(kb + 2, stage == 0 ? 2 : stage - 1);
    };
    // Four stretches of steps, each with one form of the step: every
    // wavefront unmasked; the early half-tile's causal edge (all masked; the
    // mask changes nothing for the late rows there); then the late rows alone,
    // each step split between their wavefront and a helper (below), unmasked
    // and then, over their causal edge, masked.  A wavefront with nothing to
    // do in a stretch still copies its share and meets the barriers.
    int kb = 0;
    for (const int end = min(e1, nblk); kb < end; ++kb) {
        sync_step(kb);
        if (wave_live)
            compute_step(std::false_type{}, kb, stage);
        stage = stage == kStages - 1 ? 0 : stage + 1;
    }
    for (const int end = min(e2, nblk); kb < end; ++kb) {
        sync_step(kb);
        if (wave_live)
            compute_step(std::true_type{}, kb, stage);
        stage = stage == kStages - 1 ? 0 : stage + 1;
    }
    // Rows: out[row][h][dim], dims 32 db + 8 (r/4) + 4 half + r%4.
    // A non-finite product sum: a V entry past fp16's range (or inf or NaN
    // among q, K and V) reached this wavefront's products.  The sums stay far
    // below fp32's range otherwise, so their total is finite exactly when
    // each is.
    bool nonfinite = false;
    auto write_rows = [&]() __attribute__((always_inline)) {
        {
            float t = 0.f;
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    t += acc[db][r];
            nonfinite |= !(fabsf(t) <= 3.0e38f);
        }
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
    };

    // The early rows are done.  Their wavefronts write them and then help the
    // late wavefront of the same position (w + 4): from here each of the two
    // takes one 32-key half of every step for the late rows -- the late
    // wavefront the first half, its helper the second -- with a softmax state
    // of its own, and the two states are merged at the end.
    const int tw0_late = (halves - 1 - pair) * kHalfTokens + (w % kHalfWaves) * kTokPerWave;
    const bool late_rows = has_upper && tw0_late < n;   // uniform
    if (!upper) {
        write_rows();
        if (late_rows) {
            tq = tw0_late + j / G;
            row_ok = tq < n;
            pos = row_ok ? ctx - n + tq : -1;
            row = (size_t)start + min(tq, n - 1);
            load_q();
            wait_vm<0>();   // q, and with it the copies issued before it
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                acc[db] = zero16();
            m_run = kNegBig;
            l_run = 0.f;
        }
    }
    const int my_half = upper ? 0 : 1;
    for (const int end = min(e3, nblk); kb < end; ++kb) {
        sync_step(kb);
        if (late_rows) {
            const f32x16_t sc = scores(stage, my_half);
            softmax_pv(std::false_type{}, kb, stage, my_half, sc);
        }
        stage = stage == kStages - 1 ? 0 : stage + 1;
    }
    for (; kb < nblk; ++kb) {
        sync_step(kb);
        if (late_rows) {
            const f32x16_t sc = scores(stage, my_half);
            softmax_pv(std::true_type{}, kb, stage, my_half, sc);
        }
        stage = stage == kStages - 1 ? 0 : stage + 1;
    }

    if (has_upper) {
        // Merge each helper's state into its late wavefront's, through the
        // LDS stages (no step reads them any more): 64 lanes x (64 sums,
        // running max, running sum) floats per helper, lane-major.
        __syncthreads();
        float *xch = reinterpret_cast<float *>((w % kHalfWaves) < 2 ? &k_lds[0][0] : &v_lds[0][0]) +
                     (w % 2) * (kDimBlocks * 16 + 2) * 64;
        if (!upper && late_rows) {
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    xch[(db * 16 + r) * 64 + lane] = acc[db][r];
            xch[(kDimBlocks * 16) * 64 + lane] = m_run;
            xch[(kDimBlocks * 16 + 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (upper && late_rows) {
            const float m_h = xch[(kDimBlocks * 16) * 64 + lane];
            const float l_h = xch[(kDimBlocks * 16 + 1) * 64 + lane];
            const float m_new = fmaxf(m_run, m_h);
            const float a_u = __builtin_amdgcn_exp2f(m_run - m_new);
            const float a_h = __builtin_amdgcn_exp2f(m_h - m_new);
            l_run = l_run * a_u + l_h * a_h;
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[db][r] = acc[db][r] * a_u + xch[(db * 16 + r) * 64 + lane] * a_h;
            m_run = m_new;
        }
    }
    if (upper)
        write_rows();
    const bool big_v = __any(nonfinite);
    if ((bad_page || big_v) && lane == 0)
        report_violation(a.violations,
                         (bad_page ? HIPDECODE_VIOLATION_PAGE : 0u) | (big_v ? HIPDECODE_VIOLATION_VALUE : 0u));
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
    const int64_t half_tokens = (kPfWaves / 2) * (kRowsPerWave / group);
    const int64_t pairs = (((int64_t)p.max_new_tokens + half_tokens - 1) / half_tokens + 1) / 2;
    if ((int64_t)p.num_seqs * pairs * p.num_kv_heads >= kMaxGrid)
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
    const int half_tokens = (kPfWaves / 2) * (kRowsPerWave / group);
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
    a.pairs = ((p.max_new_tokens + half_tokens - 1) / half_tokens + 1) / 2;   // workgroups per (request, KV head)
    // c = |scale| log2(e), kept at least 2^-100 so that c * -inf = -inf: for
    // any scale that small every weight 2^(c s - m) is 1.0f anyway (|s| stays
    // far below 2^70), so scale 0 still gives the mean of V and ln(n).
    a.scale_log2 = fmaxf(fabsf(p.scale) * 1.44269504088896340736f, 0x1p-100f);
    a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
    a.violations = violation_word();
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * a.pairs * p.num_kv_heads);
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
