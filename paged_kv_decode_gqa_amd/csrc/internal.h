// internal.h -- declarations shared by the host API and the kernel translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hipdecode.h"

// Exported entry points of the C ABI; everything else has hidden visibility.
#define HIPDECODE_API extern "C" __attribute__((visibility("default")))

namespace hipdecode {

constexpr int kHeadDim = 128;   // dims per head; a K or V row is 256 bytes
constexpr int kPageSize = 16;   // tokens per page
constexpr int kMinPartition = 64;     // split-K partitions are multiples of this many tokens
constexpr int kMaxPartition = 4096;   // at most 256 pages, so at most 64 per wavefront: one table entry per lane
constexpr int kMaxMergeSplits = 1024; // partitions per request: bounds the partials one workgroup merges
constexpr int kCounterStride = 64;   // int32 per arrival counter: each on its own 256-byte line
constexpr int kScheduleSplit = 1;

// Byte offsets inside the caller's workspace.  Partials are indexed
// [B][Hq][nsplit].
struct WorkspaceLayout {
    size_t counters;   // int32 [B][Hkv][kCounterStride]: arrivals per (request, KV head) in element 0; zero between calls
    size_t part_ml;    // fp32  [partials][2]: (running max, running sum) in log2 units
    size_t part_acc;   // fp32  [partials][128]: unnormalised weighted sums of V
    size_t total;
};

struct DecodeArgs {
    int32_t num_seqs;
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *block_table;
    const int32_t *context_lens;
    void *out;
    float *lse;
    int32_t *counters;
    float *part_ml;
    float *part_acc;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_blocks;
    int32_t max_context_len;
    int32_t partition_pages;
    int32_t nsplit_max;          // partitions of the longest context
    int32_t head_mix;            // largest power of two <= 8 dividing num_kv_heads: KV heads XOR-ed by dispatch round
    float scale_log2;   // scale * log2(e): scores are kept in base-2 units
    // Fused append (hipdecode_paged_attn_append) only: each request's new
    // token, written to its slot and folded from registers, and RoPE.
    const uint16_t *k_new;   // [B][Hkv][128]
    const uint16_t *v_new;   // [B][Hkv][128]
    uint16_t *k_pool_w;      // the pools, writable
    uint16_t *v_pool_w;
    double rope_theta;       // > 0: q and the new key are rotated at position ctx - 1
    double rope_log2_theta;  // log2(rope_theta) when rope_theta > 0
    uint32_t *violations;    // contract-violation flag word of this device
};

// The contract-violation flag word of the current device (the
// HIPDECODE_VIOLATION_* bits), looked up once per device; nullptr if the
// runtime cannot name it.
uint32_t *violation_word();

// Sets a contract-violation bit: a device-scope atomic OR through the vector
// memory path, taken only where a kernel has already found the contract
// broken.
__device__ __forceinline__ void report_violation(uint32_t *word, uint32_t bit)
{
    if (word != nullptr)
        __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// waves: 4 or 16 wavefronts per workgroup; fused: the kernel that also
// appends each request's new token
hipError_t launch_paged_decode(const DecodeArgs &a, int group, int waves, bool out_f32, hipStream_t stream,
                               bool fused = false);
hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream);

}  // namespace hipdecode
