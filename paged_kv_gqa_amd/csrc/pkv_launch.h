// pkv_launch.h -- host-side launchers (internal C++ interface between the
// validating C entry points and the kernel translation units).  Arguments
// reaching these functions have been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Sets the thread-local message pkv_last_error() returns; returns code.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

hipError_t launch_rope_cache_build(float* table, int32_t max_pos, int32_t rot_dim, double theta,
                                   hipStream_t stream);

hipError_t launch_qk_norm_rope(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                               void* q_out, void* k_out, const int64_t* positions, int32_t n_tokens,
                               int32_t hq, int32_t hkv, const void* gq, const void* gk, float eps,
                               const float* table, int32_t max_pos, hipStream_t stream);

hipError_t launch_qk_norm_rope_store(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                                     const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache,
                                     void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                                     const int64_t* positions, int32_t n_tokens, int32_t hq, int32_t hkv,
                                     const void* gq, const void* gk, float eps, const float* table, int32_t max_pos,
                                     hipStream_t stream);

hipError_t launch_store_kvcache(const void* key, int64_t key_row_stride, const void* value,
                                int64_t value_row_stride, void* k_cache, void* v_cache, int64_t num_slots,
                                const int32_t* slot_mapping, int32_t n_tokens, int64_t row_bytes,
                                int32_t elem_bytes, hipStream_t stream);

hipError_t launch_add_rms_norm(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                               int32_t n_tokens, int32_t hidden, float eps, hipStream_t stream);

hipError_t launch_silu_and_mul(const void* x, int64_t x_row_stride, void* out, int64_t out_row_stride,
                               int32_t n_tokens, int32_t inter, hipStream_t stream);

hipError_t launch_sample_gumbel(const void* logits, int64_t row_stride, int32_t logits_f32,
                                const float* temperatures, const float* noise, int64_t noise_row_stride,
                                uint64_t seed, uint64_t offset, int64_t* tokens, int32_t num_rows, int32_t vocab,
                                hipStream_t stream);

struct PrefillArgs {
    const void* q;
    int64_t q_row_stride;
    const void* k;
    int64_t k_row_stride;
    const void* v;
    int64_t v_row_stride;
    void* o;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int32_t num_seqs;
    int32_t total_q;
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;
    int32_t hq;
    int32_t hkv;
    float scale_log2;            // softmax_scale * log2(e)
    const int32_t* block_table;  // NULL: contiguous K/V
    int32_t max_blocks;
    int64_t num_blocks;
    void* workspace;             // key-split partial sums (NULL: no split)
    size_t workspace_bytes;
};
hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t stream);
// Workspace the call's key split uses (0: the call does not split).
size_t prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t hq, int32_t hkv);

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* o;
    const int32_t* context_lens;
    const int32_t* block_table;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t hq;
    int32_t hkv;
    int64_t num_blocks;
    float scale_log2;
    void* workspace;
};
// The decode step's own inputs when QK-Norm + RoPE + scatter run inside the
// split kernel (launch_decode_step): the step's raw q | k | v rows, their
// positions and cache slots, the norm weights and the RoPE table.
struct StepArgs {
    const uint16_t* qkv;         // bf16 rows: q (hq heads) | k (hkv) | v (hkv)
    int64_t qkv_stride;          // elements
    const int64_t* positions;
    const int32_t* slot_mapping;
    const uint16_t* q_norm_weight;
    const uint16_t* k_norm_weight;
    float eps;
    const float* table;          // fp32 [max_pos][128]: cos half, sin half
    int32_t max_pos;
    uint16_t* q_out;             // q' of the step
    uint16_t* k_cache;           // the caches, written at the new tokens' slots
    uint16_t* v_cache;
    int64_t num_slots;
};
// Length of one split-K work item in 16-key chunks.
int decode_split_chunks(int32_t num_seqs, int32_t hkv, int32_t max_blocks);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t max_blocks);
hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream);
// One decode step: q' and the new tokens' k' / v computed inside the split kernel
// (a.q unused), then the same merge as launch_attn_decode.
hipError_t launch_decode_step(const DecodeArgs& a, const StepArgs& st, hipStream_t stream);
// The checked decode step (pkv_decode_step and the graph captures): status code,
// message set on failure.
int decode_step_run(const pkv_decode_step_desc& d, int32_t batch, hipStream_t stream);
// Size of the fixed device array pkv_attn_decode_paged_noalloc uses as its workspace.
constexpr size_t kDecodeScratchBytes = size_t(96) << 20;
// Its device address on the current device (looked up once per device).
hipError_t decode_scratch(void** ptr);

}  // namespace pkv
