// decode_graph.hip -- the decode step of the attention core, eager or replayed
// from HIP graphs captured per batch bucket.
//
// "nano-vllm code walkthrough", "Misc implementation details" (graphs in the
// decode stage): every decode shape is fixed except the number of sequences,
// so one graph is captured per batch size of a ladder (1, 2, 4, 8, 16, ...)
// over static buffers, and a step runs the smallest captured size that holds
// the batch.  "3.3 Model skeleton and core operators", section 7.1: rows
// padded up to the captured size carry slot id -1, so the cache scatter skips
// them; their context length is 0, so decode reads no key for them.
//
// One step = pkv_qk_norm_rope_store over the step's qkv rows (q', and k' / v
// into their cache slots) followed by pkv_attn_decode_paged, run as one split
// kernel that does both (decode_step_run) and the merge.  The graph for
// bucket n is exactly the eager step at batch n, captured once; a replay for
// a batch b < n first marks rows [b, n) as padding with one small kernel,
// unless the caller keeps those rows padded itself (PKV_DECODE_CALLER_PADS),
// as the pages' runner does when it fills its static buffers.
#include <new>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace {

using pkv::set_error;

// Rows [b0, b1) become padding: slot id -1 (no cache write), context length 0.
__global__ void __launch_bounds__(256) pad_rows_kernel(int32_t* __restrict__ slot_mapping,
                                                       int32_t* __restrict__ context_lens, int32_t b0, int32_t b1) {
    const int32_t i = b0 + (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < b1) {
        slot_mapping[i] = -1;
        context_lens[i] = 0;
    }
}

int step(const pkv_decode_step_desc& d, int32_t batch, hipStream_t stream) {
    return pkv::decode_step_run(d, batch, stream);
}

int check_desc(const pkv_decode_step_desc* d) {
    if (!d) return set_error(PKV_ERR_INVALID_ARG, "decode step: desc is NULL");
    if (d->max_batch <= 0) return set_error(PKV_ERR_INVALID_ARG, "decode step: max_batch must be > 0");
    if (!d->qkv || !d->q_out || !d->o || !d->slot_mapping || !d->context_lens)
        return set_error(PKV_ERR_INVALID_ARG, "decode step: a required buffer is NULL");
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim != 128)
        return set_error(PKV_ERR_UNSUPPORTED, "decode step: heads must be positive and head_dim 128");
    const int64_t width = (int64_t)(d->num_q_heads + 2 * d->num_kv_heads) * d->head_dim;
    if (d->qkv_row_stride < width)
        return set_error(PKV_ERR_INVALID_ARG, "decode step: qkv_row_stride %lld < (Hq + 2 Hkv) * head_dim = %lld",
                     (long long)d->qkv_row_stride, (long long)width);
    if (d->flags & ~PKV_DECODE_CALLER_PADS)
        return set_error(PKV_ERR_INVALID_ARG, "decode step: unknown flags 0x%x", (unsigned)d->flags);
    if (d->num_blocks <= 0 || d->block_size != 256)
        return set_error(PKV_ERR_INVALID_ARG, "decode step: needs num_blocks > 0 and block_size 256");
    const size_t need = pkv_decode_step_workspace_bytes(d->max_batch, d->num_q_heads, d->num_kv_heads,
                                                        d->head_dim, d->max_blocks_per_seq, d->block_size);
    if (need == 0) return set_error(PKV_ERR_INVALID_ARG, "decode step: invalid sizes");
    if (!d->workspace || d->workspace_bytes < need)
        return set_error(PKV_ERR_WORKSPACE, "decode step: workspace of %zu bytes needed for max_batch %d, %zu given",
                     need, d->max_batch, d->workspace ? d->workspace_bytes : (size_t)0);
    return PKV_OK;
}

}  // namespace

struct pkv_decode_graph_s {
    pkv_decode_step_desc desc;
    int32_t num_buckets;
    int32_t buckets[PKV_DECODE_GRAPH_MAX_BUCKETS];
    hipGraph_t graph[PKV_DECODE_GRAPH_MAX_BUCKETS];
    hipGraphExec_t exec[PKV_DECODE_GRAPH_MAX_BUCKETS];
};

extern "C" {

size_t pkv_decode_step_workspace_bytes(int32_t max_batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size) {
    if (max_batch <= 0) return 0;
    // The split length depends on the batch only while it has fewer than ~1400 split
    // items; from 4096 sequences on it is fixed and the workspace grows with the
    // batch, so its largest value is at max_batch.
    size_t best = 0;
    const int32_t last = max_batch < 4096 ? max_batch : 4096;
    for (int32_t b = 1; b <= last; ++b) {
        const size_t w = pkv_attn_decode_workspace_bytes(b, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                                         block_size);
        if (w == 0) return 0;
        if (w > best) best = w;
    }
    if (max_batch > last) {
        const size_t w = pkv_attn_decode_workspace_bytes(max_batch, num_q_heads, num_kv_heads, head_dim,
                                                         max_blocks_per_seq, block_size);
        if (w == 0) return 0;
        if (w > best) best = w;
    }
    return best;
}

int pkv_decode_step(const pkv_decode_step_desc* desc, int32_t batch, void* stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (batch < 0 || batch > desc->max_batch)
        return set_error(PKV_ERR_INVALID_ARG, "pkv_decode_step: batch %d outside [0, max_batch %d]", batch,
                     desc->max_batch);
    if (batch == 0) return PKV_OK;
    return step(*desc, batch, (hipStream_t)stream);
}

int pkv_decode_graph_create(const pkv_decode_step_desc* desc, const int32_t* buckets, int32_t num_buckets,
                            pkv_decode_graph* out) {
    if (!out) return set_error(PKV_ERR_INVALID_ARG, "pkv_decode_graph_create: out is NULL");
    *out = nullptr;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!buckets || num_buckets <= 0 || num_buckets > PKV_DECODE_GRAPH_MAX_BUCKETS)
        return set_error(PKV_ERR_INVALID_ARG, "pkv_decode_graph_create: 1..%d buckets required",
                     PKV_DECODE_GRAPH_MAX_BUCKETS);
    for (int i = 0; i < num_buckets; ++i) {
        if (buckets[i] <= 0 || buckets[i] > desc->max_batch || (i > 0 && buckets[i] <= buckets[i - 1]))
            return set_error(PKV_ERR_INVALID_ARG,
                         "pkv_decode_graph_create: buckets must increase strictly within [1, max_batch %d]",
                         desc->max_batch);
    }
    pkv_decode_graph g = new (std::nothrow) pkv_decode_graph_s();
    if (!g) return set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_create: out of host memory");
    g->desc = *desc;
    g->num_buckets = 0;
    hipStream_t cap = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete g;
        return set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_create: stream: %s", hipGetErrorString(e));
    }
    for (int i = 0; i < num_buckets; ++i) {
        e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            rc = set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_create: begin capture: %s", hipGetErrorString(e));
            break;
        }
        const int src = step(g->desc, buckets[i], cap);
        hipGraph_t graph = nullptr;
        e = hipStreamEndCapture(cap, &graph);
        if (src != PKV_OK || e != hipSuccess || !graph) {
            if (graph) (void)hipGraphDestroy(graph);
            rc = src != PKV_OK ? src
                               : set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_create: end capture: %s",
                                       hipGetErrorString(e));
            break;
        }
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiateWithFlags(&exec, graph, 0);
        if (e != hipSuccess) {
            (void)hipGraphDestroy(graph);
            rc = set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_create: instantiate: %s", hipGetErrorString(e));
            break;
        }
        g->buckets[i] = buckets[i];
        g->graph[i] = graph;
        g->exec[i] = exec;
        g->num_buckets = i + 1;
    }
    (void)hipStreamDestroy(cap);
    if (rc != PKV_OK) {
        pkv_decode_graph_destroy(g);
        return rc;
    }
    *out = g;
    return PKV_OK;
}

int32_t pkv_decode_graph_bucket(pkv_decode_graph g, int32_t batch) {
    if (!g || batch <= 0) return -1;
    for (int i = 0; i < g->num_buckets; ++i)
        if (g->buckets[i] >= batch) return g->buckets[i];
    return -1;
}

int pkv_decode_graph_launch(pkv_decode_graph g, int32_t batch, void* stream) {
    if (!g) return set_error(PKV_ERR_INVALID_ARG, "pkv_decode_graph_launch: graph is NULL");
    if (batch == 0) return PKV_OK;
    int i = 0;
    while (i < g->num_buckets && g->buckets[i] < batch) ++i;
    if (batch < 0 || i == g->num_buckets)
        return set_error(PKV_ERR_INVALID_ARG, "pkv_decode_graph_launch: batch %d outside [0, largest bucket %d]", batch,
                     g->buckets[g->num_buckets - 1]);
    const int32_t n = g->buckets[i];
    hipStream_t s = (hipStream_t)stream;
    if (n > batch && !(g->desc.flags & PKV_DECODE_CALLER_PADS)) {
        const unsigned blocks = (unsigned)((n - batch + 255) / 256);
        hipLaunchKernelGGL(pad_rows_kernel, dim3(blocks), dim3(256), 0, s, g->desc.slot_mapping,
                           g->desc.context_lens, batch, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_launch: pad: %s", hipGetErrorString(e));
    }
    const hipError_t e = hipGraphLaunch(g->exec[i], s);
    if (e != hipSuccess) return set_error(PKV_ERR_LAUNCH, "pkv_decode_graph_launch: %s", hipGetErrorString(e));
    return PKV_OK;
}

void pkv_decode_graph_destroy(pkv_decode_graph g) {
    if (!g) return;
    for (int i = 0; i < g->num_buckets; ++i) {
        (void)hipGraphExecDestroy(g->exec[i]);
        (void)hipGraphDestroy(g->graph[i]);
    }
    delete g;
}

}  // extern "C"
