// step_runner.hip -- graph-replayed decode step: the extern "C" entry points
// hipdecode_step_bucket and hipdecode_step_runner_{create,step,destroy}.
//
// Decode steps are replayed as captured graphs with the batch padded to a
// fixed bucket size, and the host prepares step t+1 while the GPU runs step t
// (MOSS-TD article, "Autoregressive decoding").  One graph per power-of-two
// bucket holds, layer after layer, the fused KV append and paged attention
// (hipdecode_paged_attn_append, one launch per layer) of that bucket's rows;
// it is captured from this library's own entry point on a private stream the
// first time the bucket is used.  The per-step input the
// graphs read -- the context lengths -- goes through two pinned host buffers
// used in turn, each released by an event recorded after its copy.
#include "hipdecode.h"
#include "internal.h"

#include <math.h>
#include <new>
#include <string.h>

struct hipdecode_step_runner {
    hipdecode_step_config cfg;
    int32_t max_bucket;
    int32_t num_buckets;
    // per-layer device pointers (copies of the caller's arrays)
    void **k_pool;
    void **v_pool;
    void **q;
    const void **k_new;
    const void **v_new;
    void **out;
    float **lse;
    int32_t *block_table;
    int32_t *context_lens;
    // owned resources
    void *workspace;              // one slice per bucket, at ws_offset[log2(bucket)]
    size_t workspace_bytes;
    size_t ws_offset[33];         // slice k spans [ws_offset[k], ws_offset[k + 1])
    int32_t *staging[2];          // pinned, max_bucket int32 each
    hipEvent_t staged[2];         // recorded after the copy out of staging[i]
    bool staged_pending[2];
    hipStream_t capture;
    hipGraphExec_t graphs[32];    // by log2(bucket)
    uint64_t steps;
};

namespace hipdecode {
namespace {

int32_t bucket_of(int32_t max_seqs, int32_t n)
{
    if (max_seqs < 1 || n < 1 || n > max_seqs)
        return 0;
    int32_t b = 1;
    while (b < n)
        b <<= 1;
    return b;
}

int32_t log2_of(int32_t b)
{
    int32_t k = 0;
    while ((1 << k) < b)
        ++k;
    return k;
}

hipdecode_params attn_params(const hipdecode_step_config &c, int32_t rows)
{
    hipdecode_params p;
    memset(&p, 0, sizeof p);
    p.num_seqs = rows;
    p.num_q_heads = c.num_q_heads;
    p.num_kv_heads = c.num_kv_heads;
    p.head_dim = c.head_dim;
    p.page_size = c.page_size;
    p.num_pages = c.num_pages;
    p.max_blocks_per_seq = c.max_blocks_per_seq;
    p.max_context_len = c.max_context_len;
    p.out_dtype = c.out_dtype;
    p.scale = c.scale;
    return p;
}

hipdecode_append_params append_params(const hipdecode_step_config &c, int32_t rows)
{
    hipdecode_append_params p;
    memset(&p, 0, sizeof p);
    p.num_seqs = rows;
    p.num_q_heads = c.num_q_heads;
    p.num_kv_heads = c.num_kv_heads;
    p.head_dim = c.head_dim;
    p.page_size = c.page_size;
    p.num_pages = c.num_pages;
    p.max_blocks_per_seq = c.max_blocks_per_seq;
    p.num_rows = rows;
    p.max_new_tokens = 1;
    p.rope = c.rope_theta > 0.0 ? HIPDECODE_ROPE_HALF : HIPDECODE_ROPE_NONE;
    p.rope_theta = c.rope_theta > 0.0 ? c.rope_theta : 1.0;
    return p;
}

hipdecode_status check_config(const hipdecode_step_config *c, const hipdecode_step_buffers *b)
{
    if (c == nullptr || b == nullptr)
        return HIPDECODE_ERR_NULL;
    if (c->num_layers < 1 || c->max_seqs < 1 || c->max_seqs > (1 << 24))
        return HIPDECODE_ERR_SHAPE;
    if (!(c->rope_theta >= 0.0) || !isfinite(c->rope_theta))
        return HIPDECODE_ERR_SCALE;
    const int32_t max_bucket = bucket_of(c->max_seqs, c->max_seqs);
    hipdecode_params p = attn_params(*c, max_bucket);
    hipdecode_status st = hipdecode_check_params(&p);
    if (st != HIPDECODE_OK)
        return st;
    hipdecode_append_params ap = append_params(*c, max_bucket);
    st = hipdecode_check_append_params(&ap);
    if (st != HIPDECODE_OK)
        return st;
    if (b->k_pool == nullptr || b->v_pool == nullptr || b->q == nullptr || b->k_new == nullptr ||
        b->v_new == nullptr || b->out == nullptr || b->block_table == nullptr || b->context_lens == nullptr)
        return HIPDECODE_ERR_NULL;
    for (int32_t l = 0; l < c->num_layers; ++l)
        if (b->k_pool[l] == nullptr || b->v_pool[l] == nullptr || b->q[l] == nullptr || b->k_new[l] == nullptr ||
            b->v_new[l] == nullptr || b->out[l] == nullptr)
            return HIPDECODE_ERR_NULL;
    return HIPDECODE_OK;
}

void release(hipdecode_step_runner *r)
{
    for (int i = 0; i < 32; ++i)
        if (r->graphs[i] != nullptr)
            (void)hipGraphExecDestroy(r->graphs[i]);
    for (int i = 0; i < 2; ++i) {
        if (r->staged[i] != nullptr)
            (void)hipEventDestroy(r->staged[i]);
        if (r->staging[i] != nullptr)
            (void)hipHostFree(r->staging[i]);
    }
    if (r->capture != nullptr)
        (void)hipStreamDestroy(r->capture);
    if (r->workspace != nullptr)
        (void)hipFree(r->workspace);
    delete[] r->k_pool;
    delete[] r->v_pool;
    delete[] r->q;
    delete[] r->k_new;
    delete[] r->v_new;
    delete[] r->out;
    delete[] r->lse;
    delete r;
}

// Captures every layer's fused append and attention for `bucket` rows.
hipdecode_status capture(hipdecode_step_runner *r, int32_t bucket, hipGraphExec_t *exec)
{
    const hipdecode_params p = attn_params(r->cfg, bucket);
    const int32_t k = log2_of(bucket);
    void *ws = static_cast<uint8_t *>(r->workspace) + r->ws_offset[k];
    const size_t ws_bytes = r->ws_offset[k + 1] - r->ws_offset[k];
    if (hipStreamBeginCapture(r->capture, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return HIPDECODE_ERR_HIP;
    hipdecode_status st = HIPDECODE_OK;
    for (int32_t l = 0; l < r->cfg.num_layers && st == HIPDECODE_OK; ++l)
        st = hipdecode_paged_attn_append(&p, r->cfg.rope_theta, r->q[l], r->k_new[l], r->v_new[l], r->k_pool[l],
                                         r->v_pool[l], r->block_table, r->context_lens, r->out[l],
                                         r->lse != nullptr ? r->lse[l] : nullptr, ws, ws_bytes, r->capture);
    hipGraph_t graph = nullptr;
    const hipError_t end = hipStreamEndCapture(r->capture, &graph);
    if (st != HIPDECODE_OK || end != hipSuccess || graph == nullptr) {
        if (graph != nullptr)
            (void)hipGraphDestroy(graph);
        return st != HIPDECODE_OK ? st : HIPDECODE_ERR_HIP;
    }
    const hipError_t inst = hipGraphInstantiate(exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    return inst == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
}

}  // namespace
}  // namespace hipdecode

using namespace hipdecode;

HIPDECODE_API int32_t hipdecode_step_bucket(int32_t max_seqs, int32_t num_seqs)
{
    return bucket_of(max_seqs, num_seqs);
}

HIPDECODE_API hipdecode_status hipdecode_step_runner_create(const hipdecode_step_config *config,
                                                            const hipdecode_step_buffers *buffers,
                                                            hipdecode_step_runner **runner)
{
    if (runner == nullptr)
        return HIPDECODE_ERR_NULL;
    *runner = nullptr;
    const hipdecode_status st = check_config(config, buffers);
    if (st != HIPDECODE_OK)
        return st;
    hipdecode_step_runner *r = new (std::nothrow) hipdecode_step_runner();
    if (r == nullptr)
        return HIPDECODE_ERR_HIP;
    r->cfg = *config;
    r->max_bucket = bucket_of(config->max_seqs, config->max_seqs);
    r->num_buckets = log2_of(r->max_bucket) + 1;
    const int32_t L = config->num_layers;
    r->k_pool = new (std::nothrow) void *[L];
    r->v_pool = new (std::nothrow) void *[L];
    r->q = new (std::nothrow) void *[L];
    r->k_new = new (std::nothrow) const void *[L];
    r->v_new = new (std::nothrow) const void *[L];
    r->out = new (std::nothrow) void *[L];
    r->lse = buffers->lse != nullptr ? new (std::nothrow) float *[L] : nullptr;
    if (!r->k_pool || !r->v_pool || !r->q || !r->k_new || !r->v_new || !r->out || (buffers->lse && !r->lse)) {
        release(r);
        return HIPDECODE_ERR_HIP;
    }
    for (int32_t l = 0; l < L; ++l) {
        r->k_pool[l] = buffers->k_pool[l];
        r->v_pool[l] = buffers->v_pool[l];
        r->q[l] = buffers->q[l];
        r->k_new[l] = buffers->k_new[l];
        r->v_new[l] = buffers->v_new[l];
        r->out[l] = buffers->out[l];
        if (r->lse != nullptr)
            r->lse[l] = buffers->lse[l];
    }
    r->block_table = buffers->block_table;
    r->context_lens = buffers->context_lens;

    // One slice of the workspace per bucket.  A workspace keeps its arrival
    // counters at zero between calls only for calls of one layout (the
    // counters lead it, sized by the batch), so buckets must not share one:
    // a smaller bucket's partials would land on a larger one's counters.
    size_t ws = 0;
    for (int32_t k = 0; k < r->num_buckets; ++k) {
        const hipdecode_params p = attn_params(r->cfg, (int32_t)1 << k);
        const size_t need = hipdecode_workspace_bytes(&p);
        r->ws_offset[k] = ws;
        ws += (need < 256 ? 256 : need + 255) & ~(size_t)255;
    }
    r->ws_offset[r->num_buckets] = ws;
    r->workspace_bytes = ws;
    bool ok = hipStreamCreateWithFlags(&r->capture, hipStreamNonBlocking) == hipSuccess &&
              hipMalloc(&r->workspace, r->workspace_bytes) == hipSuccess;
    for (int i = 0; i < 2 && ok; ++i)
        ok = hipHostMalloc(reinterpret_cast<void **>(&r->staging[i]), (size_t)r->max_bucket * sizeof(int32_t),
                           hipHostMallocDefault) == hipSuccess &&
             hipEventCreateWithFlags(&r->staged[i], hipEventDisableTiming) == hipSuccess;
    ok = ok && hipdecode_workspace_init(r->workspace, r->workspace_bytes, r->capture) == HIPDECODE_OK &&
         hipStreamSynchronize(r->capture) == hipSuccess;
    if (!ok) {
        release(r);
        return HIPDECODE_ERR_HIP;
    }
    *runner = r;
    return HIPDECODE_OK;
}

HIPDECODE_API hipdecode_status hipdecode_step_runner_step(hipdecode_step_runner *r, int32_t num_seqs,
                                                          const int32_t *context_lens_host, void *stream)
{
    if (r == nullptr)
        return HIPDECODE_ERR_NULL;
    if (num_seqs == 0)
        return HIPDECODE_OK;
    const int32_t bucket = bucket_of(r->cfg.max_seqs, num_seqs);
    if (bucket == 0)
        return HIPDECODE_ERR_SHAPE;
    if (context_lens_host == nullptr)
        return HIPDECODE_ERR_NULL;
    // the graphs were sized for max_context_len: a longer context would be
    // clamped by the kernel and its new token written over a cached one
    for (int32_t k = 0; k < num_seqs; ++k)
        if (context_lens_host[k] < 0 || context_lens_host[k] > r->cfg.max_context_len)
            return HIPDECODE_ERR_SHAPE;
    hipGraphExec_t &exec = r->graphs[log2_of(bucket)];
    if (exec == nullptr) {
        const hipdecode_status st = capture(r, bucket, &exec);
        if (st != HIPDECODE_OK) {
            exec = nullptr;
            return st;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int i = (int)(r->steps & 1);
    // the copy issued from this half two steps ago must be done before it is refilled
    if (r->staged_pending[i] && hipEventSynchronize(r->staged[i]) != hipSuccess)
        return HIPDECODE_ERR_HIP;
    int32_t *h = r->staging[i];
    memcpy(h, context_lens_host, (size_t)num_seqs * sizeof(int32_t));
    for (int32_t k = num_seqs; k < bucket; ++k)
        h[k] = 0;
    if (hipMemcpyAsync(r->context_lens, h, (size_t)bucket * sizeof(int32_t), hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipEventRecord(r->staged[i], s) != hipSuccess)
        return HIPDECODE_ERR_HIP;
    r->staged_pending[i] = true;
    if (hipGraphLaunch(exec, s) != hipSuccess)
        return HIPDECODE_ERR_HIP;
    ++r->steps;
    return HIPDECODE_OK;
}

HIPDECODE_API hipdecode_status hipdecode_step_runner_destroy(hipdecode_step_runner *r)
{
    if (r == nullptr)
        return HIPDECODE_ERR_NULL;
    // graphs launched on the caller's streams may still run: let the device
    // finish before the workspace and the graphs go away
    const hipdecode_status st = hipDeviceSynchronize() == hipSuccess ? HIPDECODE_OK : HIPDECODE_ERR_HIP;
    release(r);
    return st;
}
