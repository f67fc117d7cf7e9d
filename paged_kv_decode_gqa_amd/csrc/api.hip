// api.hip -- the extern "C" interface declared in include/hipdecode.h:
// parameter checks, the split-K planner, the workspace layout and the launch.
#include "hipdecode.h"
#include "internal.h"

#include <math.h>

#include <atomic>
#include <mutex>

namespace hipdecode {
namespace {

constexpr int64_t kTargetWorkgroupsMany = 1024;   // 4-wave workgroups resident at once (4 per CU)
constexpr int64_t kTargetWorkgroupsFew = 256;     // one per CU, for a few long requests
constexpr int64_t kFewPairs = 32;                 // (request, KV head) pairs counted as few
constexpr int64_t kSingleSplitMax = 2048;         // contexts up to this long are not split at all
constexpr int64_t kBalancedPartition = 2048;      // partition when the target would exceed kMaxPartition
constexpr int64_t kShortPartitionMaxSplits = 8;   // 64-token partitions only for contexts of at most this many

// hipdecode_paged_attn_noalloc: its static scratch and the fixed region of
// arrival counters at the start of it (4096 (request, KV head) pairs).
constexpr size_t kNoallocBytes = HIPDECODE_NOALLOC_SCRATCH_BYTES;
constexpr size_t kNoallocCounterBytes = (size_t)4096 * kCounterStride * sizeof(int32_t);
static_assert(kNoallocBytes % 256 == 0 && kNoallocCounterBytes < kNoallocBytes, "scratch layout");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One schedule: split by partition (a ragged batch maps the grid onto its
// real (request, partition) units inside the kernel).
int32_t plan_schedule(const hipdecode_params &) { return kScheduleSplit; }

// 4-wave workgroups unless 16 are asked for.
int32_t plan_waves(const hipdecode_params &p) { return p.workgroup_waves > 0 ? p.workgroup_waves : 4; }

// Partition size, in multiples of 64 tokens, at most 4096 and at most
// kMaxMergeSplits partials per request.  Short contexts of many requests are
// not split (one request at 512 tokens measured 7.4 us with 64-token
// partitions against 8.5 us unsplit; sixteen at 200-420 tokens were fastest
// unsplit).  A few requests get about one workgroup per CU (fewer, larger partitions
// merge faster, and a CU holding two workgroups would finish last); larger
// batches get about four per CU.  64-token partitions are kept for contexts
// of at most eight of them; a longer context gets at least 128 tokens per
// partition (one request at 1024 tokens: 6.31 us against 6.65 us; two at 768:
// 6.96 against 7.25), since a wavefront then folds two pages instead of one
// and half as many partials are merged.  A batch that would want partitions
// past the maximum has work to spare and gets smaller ones, which even out
// requests of very different lengths.
int32_t plan_partition(const hipdecode_params &p)
{
    if (p.partition_tokens > 0)
        return p.partition_tokens;
    const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
    if (pairs <= 0 || p.max_context_len <= 0)
        return 256;
    const bool few = pairs <= kFewPairs;
    if (p.max_context_len <= kSingleSplitMax && !few)
        return (int32_t)(ceil_div(p.max_context_len, kMinPartition) * kMinPartition);
    const int64_t target = few ? kTargetWorkgroupsFew : kTargetWorkgroupsMany;
    const int64_t want_splits = target / pairs > 0 ? target / pairs : 1;
    int64_t part = ceil_div(p.max_context_len, want_splits);
    const int64_t floor_part = ceil_div(p.max_context_len, kMaxMergeSplits);
    if (part < floor_part)
        part = floor_part;
    part = ceil_div(part, kMinPartition) * kMinPartition;
    if (part == kMinPartition && p.max_context_len > kShortPartitionMaxSplits * kMinPartition)
        part = 2 * kMinPartition;
    if (part > kMaxPartition)
        part = kBalancedPartition;
    return (int32_t)part;
}

int32_t nsplit_max_of(const hipdecode_params &p, int32_t part)
{
    const int64_t n = ceil_div(p.max_context_len, part);
    return n < 1 ? 1 : (int32_t)n;
}

size_t counter_bytes(const hipdecode_params &p)
{
    return (size_t)p.num_seqs * (size_t)p.num_kv_heads * kCounterStride * sizeof(int32_t);
}

// counter_region: bytes reserved for the arrival counters at the start; the
// caller-workspace layout reserves exactly what the call needs, the static
// scratch of the allocation-free entry point a fixed region (so every call
// finds its counters where the previous calls left them at zero).
WorkspaceLayout layout_with(const hipdecode_params &p, size_t counter_region)
{
    WorkspaceLayout w;
    w.counters = 0;
    // one 256-byte line per counter: the tickets of different KV heads never
    // meet on one line (measured 4% at the 32-request mix, 14% at 1 x 3.5k)
    w.part_ml = align256(counter_region);
    const int32_t nsplit = nsplit_max_of(p, plan_partition(p));
    if (nsplit <= 1) {
        w.part_acc = w.part_ml;
        w.total = w.part_ml;   // a single partition per request needs only the counters
        return w;
    }
    const size_t partials = (size_t)p.num_seqs * (size_t)p.num_q_heads * (size_t)nsplit;
    w.part_acc = w.part_ml + align256(partials * 2 * sizeof(float));
    w.total = w.part_acc + partials * kHeadDim * sizeof(float);
    return w;
}

WorkspaceLayout layout_of(const hipdecode_params &p) { return layout_with(p, counter_bytes(p)); }

hipdecode_status check(const hipdecode_params *pp)
{
    if (pp == nullptr)
        return HIPDECODE_ERR_NULL;
    const hipdecode_params &p = *pp;
    if (p.num_seqs < 0 || p.num_q_heads <= 0 || p.num_kv_heads <= 0 || p.num_pages < 0 ||
        p.max_blocks_per_seq < 0 || p.max_context_len < 0 || p.partition_tokens < 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.num_q_heads % p.num_kv_heads != 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.head_dim <= 0 || p.page_size <= 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.head_dim != kHeadDim || p.page_size != kPageSize)
        return HIPDECODE_ERR_UNSUPPORTED;
    const int group = p.num_q_heads / p.num_kv_heads;
    if (group != 1 && group != 2 && group != 4)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.out_dtype != HIPDECODE_BF16 && p.out_dtype != HIPDECODE_F32)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (!isfinite(p.scale))
        return HIPDECODE_ERR_SCALE;
    if ((int64_t)p.max_context_len > (int64_t)p.max_blocks_per_seq * kPageSize)
        return HIPDECODE_ERR_SHAPE;
    if (p.num_seqs > 0 && p.max_context_len > 0 && p.num_pages == 0)
        return HIPDECODE_ERR_SHAPE;
    if (p.partition_tokens != 0 &&
        (p.partition_tokens % kMinPartition != 0 || p.partition_tokens > kMaxPartition))
        return HIPDECODE_ERR_SHAPE;
    if (p.workgroup_waves != 0 && p.workgroup_waves != 4 && p.workgroup_waves != 16)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.workgroup_waves == 16 && group > 2)
        return HIPDECODE_ERR_UNSUPPORTED;
    if (p.schedule < 0 || p.schedule > kScheduleSplit)
        return HIPDECODE_ERR_UNSUPPORTED;
    // index arithmetic inside the kernel: rows of q/out and the grid stay in 31 bits
    const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
    if (rows * kHeadDim > INT32_MAX)
        return HIPDECODE_ERR_SHAPE;
    const int32_t nsplit = nsplit_max_of(p, plan_partition(p));
    if (nsplit > kMaxMergeSplits)
        return HIPDECODE_ERR_SHAPE;
    const int64_t grid = (int64_t)p.num_seqs * p.num_kv_heads * nsplit;
    if (grid > INT32_MAX)
        return HIPDECODE_ERR_SHAPE;
    return HIPDECODE_OK;
}

}  // namespace
}  // namespace hipdecode

using namespace hipdecode;

HIPDECODE_API int hipdecode_abi_version(void) { return HIPDECODE_ABI_VERSION; }

HIPDECODE_API hipdecode_status hipdecode_check_params(const hipdecode_params *params)
{
    return check(params);
}

HIPDECODE_API int32_t hipdecode_partition_tokens(const hipdecode_params *params)
{
    if (check(params) != HIPDECODE_OK)
        return 0;
    return plan_partition(*params);
}

HIPDECODE_API int32_t hipdecode_workgroup_waves(const hipdecode_params *params)
{
    if (check(params) != HIPDECODE_OK)
        return 0;
    return plan_waves(*params);
}

HIPDECODE_API int32_t hipdecode_schedule(const hipdecode_params *params)
{
    if (check(params) != HIPDECODE_OK)
        return 0;
    return plan_schedule(*params);
}

HIPDECODE_API size_t hipdecode_workspace_bytes(const hipdecode_params *params)
{
    if (check(params) != HIPDECODE_OK)
        return 0;
    return layout_of(*params).total;
}

HIPDECODE_API hipdecode_status hipdecode_workspace_init(void *workspace, size_t bytes, void *stream)
{
    if (bytes == 0)
        return HIPDECODE_OK;
    if (workspace == nullptr)
        return HIPDECODE_ERR_NULL;
    if (!aligned16(workspace))
        return HIPDECODE_ERR_ALIGN;
    return launch_zero_fill(workspace, bytes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? HIPDECODE_OK
               : HIPDECODE_ERR_HIP;
}

namespace hipdecode {
namespace {

// Pointer and argument checks of a decode call, before anything is enqueued.
hipdecode_status check_call(const hipdecode_params *params, const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_table, const int32_t *context_lens, void *out, float *lse,
                            void *workspace, bool fused, const void *k_new, const void *v_new, double rope_theta)
{
    const hipdecode_status st = check(params);
    if (st != HIPDECODE_OK)
        return st;
    const hipdecode_params &p = *params;
    if (fused && (!(rope_theta >= 0.0) || !isfinite(rope_theta)))
        return HIPDECODE_ERR_SCALE;
    if (p.num_seqs == 0)
        return HIPDECODE_OK;
    if (q == nullptr || out == nullptr || context_lens == nullptr || block_table == nullptr ||
        workspace == nullptr)
        return HIPDECODE_ERR_NULL;
    if (p.max_context_len > 0 && (k_pool == nullptr || v_pool == nullptr))
        return HIPDECODE_ERR_NULL;
    if (fused && p.max_context_len > 0 && (k_new == nullptr || v_new == nullptr))
        return HIPDECODE_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) ||
        (k_pool != nullptr && !aligned16(k_pool)) || (v_pool != nullptr && !aligned16(v_pool)) ||
        (k_new != nullptr && !aligned16(k_new)) || (v_new != nullptr && !aligned16(v_new)) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u) != 0)
        return HIPDECODE_ERR_ALIGN;
    return HIPDECODE_OK;
}

// The body of the decode entry points; `fused` also appends each request's
// new token (k_new/v_new, RoPE with rope_theta when > 0) inside the kernel;
// `scratch_mode`: `workspace` is the static scratch of the allocation-free
// entry point.
hipdecode_status run_decode(const hipdecode_params *params, const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_table, const int32_t *context_lens, void *out, float *lse,
                            void *workspace, size_t workspace_bytes, void *stream, bool fused,
                            const void *k_new, const void *v_new, double rope_theta, bool scratch_mode = false)
{
    const hipdecode_status st = check_call(params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace,
                                           fused, k_new, v_new, rope_theta);
    if (st != HIPDECODE_OK || params->num_seqs == 0)
        return st;
    const hipdecode_params &p = *params;
    WorkspaceLayout w;
    if (scratch_mode) {
        // the allocation-free entry point: `workspace` is this device's static
        // scratch, counters in a fixed region at its start
        if (counter_bytes(p) > kNoallocCounterBytes)
            return HIPDECODE_ERR_WORKSPACE;
        w = layout_with(p, kNoallocCounterBytes);
    } else {
        w = layout_of(p);
    }
    if (workspace_bytes < w.total)
        return HIPDECODE_ERR_WORKSPACE;

    const int32_t part = plan_partition(p);
    const int32_t nsplit = nsplit_max_of(p, part);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    DecodeArgs a;
    a.num_seqs = p.num_seqs;
    a.q = static_cast<const uint16_t *>(q);
    a.k_pool = static_cast<const uint16_t *>(k_pool);
    a.v_pool = static_cast<const uint16_t *>(v_pool);
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    a.lse = lse;
    a.counters = reinterpret_cast<int32_t *>(ws + w.counters);
    a.part_ml = reinterpret_cast<float *>(ws + w.part_ml);
    a.part_acc = reinterpret_cast<float *>(ws + w.part_acc);
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.num_pages = p.num_pages;
    a.max_blocks = p.max_blocks_per_seq;
    a.max_context_len = p.max_context_len;
    a.partition_pages = part / kPageSize;
    a.nsplit_max = nsplit;
    a.head_mix = p.num_kv_heads % 8 == 0 ? 8 : p.num_kv_heads % 4 == 0 ? 4 : p.num_kv_heads % 2 == 0 ? 2 : 1;
    a.scale_log2 = p.scale * 1.44269504088896340736f;
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.k_pool_w = fused ? static_cast<uint16_t *>(const_cast<void *>(k_pool)) : nullptr;
    a.v_pool_w = fused ? static_cast<uint16_t *>(const_cast<void *>(v_pool)) : nullptr;
    a.rope_theta = fused ? rope_theta : 0.0;
    a.rope_log2_theta = a.rope_theta > 0.0 ? log2(a.rope_theta) : 0.0;
    a.violations = violation_word();

    const hipError_t e = launch_paged_decode(a, p.num_q_heads / p.num_kv_heads, plan_waves(p),
                                             p.out_dtype == HIPDECODE_F32, static_cast<hipStream_t>(stream), fused);
    return e == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
}

}  // namespace
}  // namespace hipdecode

HIPDECODE_API hipdecode_status hipdecode_paged_attn(const hipdecode_params *params, const void *q,
                                                    const void *k_pool, const void *v_pool,
                                                    const int32_t *block_table,
                                                    const int32_t *context_lens, void *out,
                                                    float *lse, void *workspace,
                                                    size_t workspace_bytes, void *stream)
{
    return run_decode(params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace, workspace_bytes,
                      stream, false, nullptr, nullptr, 0.0);
}

HIPDECODE_API hipdecode_status hipdecode_paged_attn_append(const hipdecode_params *params, double rope_theta,
                                                           const void *q, const void *k_new, const void *v_new,
                                                           void *k_pool, void *v_pool,
                                                           const int32_t *block_table,
                                                           const int32_t *context_lens, void *out, float *lse,
                                                           void *workspace, size_t workspace_bytes, void *stream)
{
    return run_decode(params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace, workspace_bytes,
                      stream, true, k_new, v_new, rope_theta);
}

// ---------------------------------------------------------------------------
// Allocation-free decode.  The workspace of hipdecode_paged_attn (arrival
// counters and split partials) lives in this file-scope device array instead
// of caller memory.  Each device holds its own copy, for the life of the
// process.  Host code never passes the array's name to a kernel: its address
// on the current device comes from hipGetSymbolAddress, once per device, and
// only that pointer is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[hipdecode::kNoallocBytes];

namespace hipdecode {
namespace {

constexpr int kNoallocMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kNoallocMaxDevices];   // per device: the address of `scratch`, once looked up

// The current device's scratch address; on the first call for a device the
// counter region is zero-filled on `stream` (static storage starts at zero
// as well; every completed call leaves its counters at zero again).
hipdecode_status scratch_of_current_device(hipStream_t stream, void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices)
        return HIPDECODE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return HIPDECODE_ERR_HIP;
        if (launch_zero_fill(p, kNoallocCounterBytes, stream) != hipSuccess)
            return HIPDECODE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return HIPDECODE_OK;
}

}  // namespace
}  // namespace hipdecode

HIPDECODE_API hipdecode_status hipdecode_paged_attn_noalloc(const hipdecode_params *params, const void *q,
                                                            const void *k_pool, const void *v_pool,
                                                            const int32_t *block_table,
                                                            const int32_t *context_lens, void *out, float *lse,
                                                            void *stream)
{
    // every argument check happens before the scratch is looked up or cleared;
    // a non-null stand-in passes the workspace pointer check
    const hipdecode_status st = check_call(params, q, k_pool, v_pool, block_table, context_lens, out, lse,
                                           reinterpret_cast<void *>(uintptr_t{256}), false, nullptr, nullptr, 0.0);
    if (st != HIPDECODE_OK || params->num_seqs == 0)
        return st;
    if (counter_bytes(*params) > kNoallocCounterBytes ||
        layout_with(*params, kNoallocCounterBytes).total > kNoallocBytes)
        return HIPDECODE_ERR_WORKSPACE;
    void *ws = nullptr;
    const hipdecode_status sst = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
    if (sst != HIPDECODE_OK)
        return sst;
    return run_decode(params, q, k_pool, v_pool, block_table, context_lens, out, lse, ws, kNoallocBytes, stream,
                      false, nullptr, nullptr, 0.0, true);
}

// ---------------------------------------------------------------------------
// Contract violations.  One flag word per device, in this file-scope device
// array; host code uses only the address hipGetSymbolAddress gives for the
// current device, looked up once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t violation_flags[64];

namespace hipdecode {
namespace {

std::mutex g_violation_mutex;
std::atomic<uint32_t *> g_violation_ptr[kNoallocMaxDevices];

}  // namespace

uint32_t *violation_word()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices)
        return nullptr;
    uint32_t *w = g_violation_ptr[dev].load(std::memory_order_acquire);
    if (w != nullptr)
        return w;
    std::lock_guard<std::mutex> lock(g_violation_mutex);
    w = g_violation_ptr[dev].load(std::memory_order_relaxed);
    if (w == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(violation_flags)) != hipSuccess || p == nullptr)
            return nullptr;
        w = static_cast<uint32_t *>(p);
        g_violation_ptr[dev].store(w, std::memory_order_release);
    }
    return w;
}

}  // namespace hipdecode

HIPDECODE_API hipdecode_status hipdecode_contract_violations(uint32_t *flags)
{
    if (flags == nullptr)
        return HIPDECODE_ERR_NULL;
    uint32_t *w = violation_word();
    if (w == nullptr)
        return HIPDECODE_ERR_HIP;
    const uint32_t zero = 0;
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(flags, w, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(w, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess)
        return HIPDECODE_ERR_HIP;
    return HIPDECODE_OK;
}

HIPDECODE_API const char *hipdecode_status_string(hipdecode_status status)
{
    switch (status) {
    case HIPDECODE_OK: return "ok";
    case HIPDECODE_ERR_NULL: return "a required pointer is NULL";
    case HIPDECODE_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case HIPDECODE_ERR_UNSUPPORTED: return "unsupported head_dim, page size, group size or dtype";
    case HIPDECODE_ERR_ALIGN: return "a buffer is not suitably aligned";
    case HIPDECODE_ERR_WORKSPACE: return "workspace smaller than hipdecode_workspace_bytes()";
    case HIPDECODE_ERR_SCALE: return "scale is not finite, or rope_theta is not finite and positive";
    case HIPDECODE_ERR_HIP: return "the HIP runtime refused the launch";
    }
    return "unknown status";
}
