// internal.h -- declarations shared by the host API and the kernel translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hipdecode {

constexpr int kHeadDim = 128;   // dims per head; a K or V row is 256 bytes
constexpr int kPageSize = 16;   // tokens per page
constexpr int kWaves = 4;       // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMinPartition = 64;     // split-K partitions are multiples of this many tokens
constexpr int kMaxPartition = 4096;   // at most 256 pages: 64 per wavefront, one table entry per lane
constexpr int kMaxMergeSplits = 1024; // partitions per request the final merge can weigh in LDS

// Byte offsets inside the caller's workspace.
struct WorkspaceLayout {
    size_t counters;   // int32 [B][Hkv]: arrivals per (request, KV head); zero between calls
    size_t part_ml;    // fp32  [B][Hq][nsplit][2]: (running max, running sum) in log2 units
    size_t part_acc;   // fp32  [B][Hq][nsplit][128]: unnormalised weighted sums of V
    size_t total;
};

struct DecodeArgs {
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
    int32_t nsplit_max;
    float scale_log2;   // scale * log2(e): scores are kept in base-2 units
};

hipError_t launch_paged_decode(const DecodeArgs &a, int group, bool out_f32, int num_seqs,
                               hipStream_t stream);
hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream);

}  // namespace hipdecode
