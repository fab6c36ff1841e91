// api.hip -- the extern "C" entry points declared in include/pkv.h.
//
// Every entry point validates its scalar arguments and pointers on the host,
// turning the asserts the pages place in front of the store_kvcache kernel
// ("3.3 Model skeleton and core operators", section 7.1; "Nano-vLLM 源码解读
// #17 注意力层", section 5.1: contiguous head_dim, contiguous heads, one slot =
// D contiguous elements, one slot id per token) and the head divisibility the
// attention layer relies on into status codes, before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>

#include "pkv.h"
#include "pkv_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return PKV_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

#define PKV_REQUIRE(cond, code, ...) \
    do {                             \
        if (!(cond)) return fail((code), __VA_ARGS__); \
    } while (0)

int check_heads(const char* fn, int32_t hq, int32_t hkv, int32_t head_dim) {
    PKV_REQUIRE(hq > 0 && hkv > 0, PKV_ERR_INVALID_ARG, "%s: head counts must be positive (Hq=%d, Hkv=%d)", fn, hq,
                hkv);
    PKV_REQUIRE(hq % hkv == 0, PKV_ERR_INVALID_ARG, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn, hq,
                hkv);
    PKV_REQUIRE(head_dim == 128, PKV_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (only 128)", fn, head_dim);
    return PKV_OK;
}

}  // namespace

namespace pkv {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return g_err; }

int pkv_version(void) { return (1 << 16) | 0; }

int pkv_rope_cache_build(float* cos_sin_cache, int32_t max_position, int32_t rotary_dim, double theta,
                         void* stream) {
    const char* fn = "pkv_rope_cache_build";
    PKV_REQUIRE(cos_sin_cache, PKV_ERR_INVALID_ARG, "%s: cos_sin_cache is NULL", fn);
    PKV_REQUIRE(max_position > 0, PKV_ERR_INVALID_ARG, "%s: max_position must be > 0 (got %d)", fn, max_position);
    PKV_REQUIRE(rotary_dim == 128, PKV_ERR_UNSUPPORTED, "%s: rotary_dim %d unsupported (only 128 = head_dim)", fn,
                rotary_dim);
    PKV_REQUIRE(theta > 0.0, PKV_ERR_INVALID_ARG, "%s: theta must be > 0", fn);
    return launched(pkv::launch_rope_cache_build(cos_sin_cache, max_position, rotary_dim, theta, (hipStream_t)stream),
                    fn);
}

int pkv_qk_norm_rope(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride, void* q_out,
                     void* k_out, const int64_t* positions, int32_t n_tokens, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, const void* q_norm_weight, const void* k_norm_weight,
                     float eps, const float* cos_sin_cache, int32_t max_position, void* stream) {
    const char* fn = "pkv_qk_norm_rope";
    int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim);
    if (rc) return rc;
    PKV_REQUIRE(n_tokens >= 0, PKV_ERR_INVALID_ARG, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
    if (n_tokens == 0) return ok();
    PKV_REQUIRE(q && k && q_out && k_out && positions && q_norm_weight && k_norm_weight && cos_sin_cache,
                PKV_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    const int64_t qw = (int64_t)num_q_heads * head_dim, kw = (int64_t)num_kv_heads * head_dim;
    PKV_REQUIRE(q_row_stride >= qw, PKV_ERR_INVALID_ARG, "%s: q_row_stride %lld < num_q_heads*head_dim %lld", fn,
                (long long)q_row_stride, (long long)qw);
    PKV_REQUIRE(k_row_stride >= kw, PKV_ERR_INVALID_ARG, "%s: k_row_stride %lld < num_kv_heads*head_dim %lld", fn,
                (long long)k_row_stride, (long long)kw);
    PKV_REQUIRE(q_row_stride % 8 == 0 && k_row_stride % 8 == 0, PKV_ERR_INVALID_ARG,
                "%s: row strides must be multiples of 8 elements (16-byte rows)", fn);
    PKV_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)q_out | (uintptr_t)k_out | (uintptr_t)q_norm_weight |
                 (uintptr_t)k_norm_weight | (uintptr_t)cos_sin_cache) % 16 == 0,
                PKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    PKV_REQUIRE(max_position > 0, PKV_ERR_INVALID_ARG, "%s: max_position must be > 0", fn);
    PKV_REQUIRE(eps >= 0.f, PKV_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    // In place is allowed only as an exact alias of a contiguous input.
    PKV_REQUIRE(q_out != q || q_row_stride == qw, PKV_ERR_INVALID_ARG,
                "%s: in-place q needs q_row_stride == num_q_heads*head_dim", fn);
    PKV_REQUIRE(k_out != k || k_row_stride == kw, PKV_ERR_INVALID_ARG,
                "%s: in-place k needs k_row_stride == num_kv_heads*head_dim", fn);
    return launched(pkv::launch_qk_norm_rope(q, q_row_stride, k, k_row_stride, q_out, k_out, positions, n_tokens,
                                             num_q_heads, num_kv_heads, q_norm_weight, k_norm_weight, eps,
                                             cos_sin_cache, max_position, (hipStream_t)stream),
                    fn);
}

namespace {
// Checks of pkv_qk_norm_rope_store (also run by the decode step, which fuses it).
int norm_store_check(const char* fn, const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                     const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache, void* v_cache,
                     int64_t num_slots, const int32_t* slot_mapping, const int64_t* positions, int32_t n_tokens,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, const void* q_norm_weight,
                     const void* k_norm_weight, float eps, const float* cos_sin_cache, int32_t max_position) {
    int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim);
    if (rc) return rc;
    PKV_REQUIRE(n_tokens >= 0, PKV_ERR_INVALID_ARG, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
    PKV_REQUIRE(num_slots >= 0, PKV_ERR_INVALID_ARG, "%s: num_slots must be >= 0", fn);
    if (n_tokens == 0) return PKV_OK;
    PKV_REQUIRE(q && k && v && q_out && k_cache && v_cache && slot_mapping && positions && q_norm_weight &&
                    k_norm_weight && cos_sin_cache,
                PKV_ERR_INVALID_ARG, "%s: a required pointer is NULL (only k_out may be NULL)", fn);
    const int64_t qw = (int64_t)num_q_heads * head_dim, kw = (int64_t)num_kv_heads * head_dim;
    PKV_REQUIRE(q_row_stride >= qw, PKV_ERR_INVALID_ARG, "%s: q_row_stride %lld < num_q_heads*head_dim %lld", fn,
                (long long)q_row_stride, (long long)qw);
    PKV_REQUIRE(k_row_stride >= kw && v_row_stride >= kw, PKV_ERR_INVALID_ARG,
                "%s: k/v row strides (%lld, %lld) must be >= num_kv_heads*head_dim %lld", fn,
                (long long)k_row_stride, (long long)v_row_stride, (long long)kw);
    PKV_REQUIRE(q_row_stride % 8 == 0 && k_row_stride % 8 == 0 && v_row_stride % 8 == 0, PKV_ERR_INVALID_ARG,
                "%s: row strides must be multiples of 8 elements (16-byte rows)", fn);
    PKV_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)q_out | (uintptr_t)k_out |
                 (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)q_norm_weight | (uintptr_t)k_norm_weight |
                 (uintptr_t)cos_sin_cache) % 16 == 0,
                PKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    PKV_REQUIRE(max_position > 0, PKV_ERR_INVALID_ARG, "%s: max_position must be > 0", fn);
    PKV_REQUIRE(eps >= 0.f, PKV_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    PKV_REQUIRE(k_cache != v_cache, PKV_ERR_INVALID_ARG, "%s: k_cache and v_cache must be distinct", fn);
    PKV_REQUIRE(q_out != q || q_row_stride == qw, PKV_ERR_INVALID_ARG,
                "%s: in-place q needs q_row_stride == num_q_heads*head_dim", fn);
    PKV_REQUIRE(!k_out || k_out != k || k_row_stride == kw, PKV_ERR_INVALID_ARG,
                "%s: in-place k needs k_row_stride == num_kv_heads*head_dim", fn);
    return PKV_OK;
}
}  // namespace

int pkv_qk_norm_rope_store(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                           const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache,
                           void* v_cache, int64_t num_slots, const int32_t* slot_mapping, const int64_t* positions,
                           int32_t n_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           const void* q_norm_weight, const void* k_norm_weight, float eps,
                           const float* cos_sin_cache, int32_t max_position, void* stream) {
    const char* fn = "pkv_qk_norm_rope_store";
    const int rc = norm_store_check(fn, q, q_row_stride, k, k_row_stride, v, v_row_stride, q_out, k_out, k_cache,
                                    v_cache, num_slots, slot_mapping, positions, n_tokens, num_q_heads, num_kv_heads,
                                    head_dim, q_norm_weight, k_norm_weight, eps, cos_sin_cache, max_position);
    if (rc) return rc;
    if (n_tokens == 0) return ok();
    return launched(pkv::launch_qk_norm_rope_store(q, q_row_stride, k, k_row_stride, v, v_row_stride, q_out, k_out,
                                                   k_cache, v_cache, num_slots, slot_mapping, positions, n_tokens,
                                                   num_q_heads, num_kv_heads, q_norm_weight, k_norm_weight, eps,
                                                   cos_sin_cache, max_position, (hipStream_t)stream),
                    fn);
}

int pkv_store_kvcache(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                      void* k_cache, void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                      int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes, void* stream) {
    const char* fn = "pkv_store_kvcache";
    PKV_REQUIRE(n_tokens >= 0, PKV_ERR_INVALID_ARG, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
    PKV_REQUIRE(num_kv_heads > 0 && head_dim > 0, PKV_ERR_INVALID_ARG, "%s: num_kv_heads and head_dim must be > 0",
                fn);
    PKV_REQUIRE(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4, PKV_ERR_INVALID_ARG,
                "%s: elem_bytes must be 1, 2 or 4 (got %d)", fn, elem_bytes);
    const int64_t D = (int64_t)num_kv_heads * head_dim;
    PKV_REQUIRE(key_row_stride >= D && value_row_stride >= D, PKV_ERR_INVALID_ARG,
                "%s: row strides (%lld, %lld) must be >= D = num_kv_heads*head_dim = %lld", fn,
                (long long)key_row_stride, (long long)value_row_stride, (long long)D);
    PKV_REQUIRE(num_slots >= 0, PKV_ERR_INVALID_ARG, "%s: num_slots must be >= 0", fn);
    if (n_tokens == 0) return ok();
    PKV_REQUIRE(key && value && k_cache && v_cache && slot_mapping, PKV_ERR_INVALID_ARG,
                "%s: a required pointer is NULL", fn);
    PKV_REQUIRE(k_cache != v_cache, PKV_ERR_INVALID_ARG, "%s: k_cache and v_cache must be distinct", fn);
    return launched(pkv::launch_store_kvcache(key, key_row_stride, value, value_row_stride, k_cache, v_cache,
                                              num_slots, slot_mapping, n_tokens, D * elem_bytes, elem_bytes,
                                              (hipStream_t)stream),
                    fn);
}

int pkv_attn_prefill_varlen(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                            const void* v, int64_t v_row_stride, void* o, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            float softmax_scale, int32_t causal, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks, void* workspace,
                            size_t workspace_bytes, void* stream) {
    const char* fn = "pkv_attn_prefill_varlen";
    int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim);
    if (rc) return rc;
    PKV_REQUIRE(causal == 1, PKV_ERR_UNSUPPORTED, "%s: only causal attention is built (causal=%d)", fn, causal);
    const int G = num_q_heads / num_kv_heads;
    PKV_REQUIRE(G == 1 || G == 2 || G % 4 == 0, PKV_ERR_UNSUPPORTED,
                "%s: GQA group %d unsupported (1, 2 or a multiple of 4)", fn, G);
    PKV_REQUIRE(num_seqs >= 0 && total_q >= 0 && max_seqlen_q >= 0 && max_seqlen_k >= 0, PKV_ERR_INVALID_ARG,
                "%s: sizes must be >= 0", fn);
    PKV_REQUIRE(max_seqlen_q <= max_seqlen_k || num_seqs == 0, PKV_ERR_INVALID_ARG,
                "%s: max_seqlen_q %d > max_seqlen_k %d (every sequence needs Lk >= Lq)", fn, max_seqlen_q,
                max_seqlen_k);
    if (num_seqs == 0 || total_q == 0) return ok();
    PKV_REQUIRE(q && k && v && o && cu_seqlens_q && cu_seqlens_k, PKV_ERR_INVALID_ARG,
                "%s: a required pointer is NULL", fn);
    PKV_REQUIRE(softmax_scale > 0.f, PKV_ERR_INVALID_ARG, "%s: softmax_scale must be > 0", fn);
    const int64_t qw = (int64_t)num_q_heads * head_dim, kw = (int64_t)num_kv_heads * head_dim;
    PKV_REQUIRE(q_row_stride >= qw, PKV_ERR_INVALID_ARG, "%s: q_row_stride %lld < num_q_heads*head_dim", fn,
                (long long)q_row_stride);
    PKV_REQUIRE(k_row_stride >= kw && v_row_stride >= kw, PKV_ERR_INVALID_ARG,
                "%s: k/v row strides must be >= num_kv_heads*head_dim", fn);
    PKV_REQUIRE(q_row_stride % 8 == 0 && k_row_stride % 8 == 0 && v_row_stride % 8 == 0, PKV_ERR_INVALID_ARG,
                "%s: row strides must be multiples of 8 elements", fn);
    PKV_REQUIRE(k_row_stride <= (int64_t)1 << 24 && v_row_stride <= (int64_t)1 << 24, PKV_ERR_INVALID_ARG,
                "%s: k/v row strides must be at most 2^24 elements", fn);
    {
        // o must not overlap q: rows flagged by the fast pass are recomputed from q.
        const uintptr_t q0 = (uintptr_t)q, q1 = q0 + (uintptr_t)(((int64_t)(total_q - 1) * q_row_stride + qw) * 2);
        const uintptr_t o0 = (uintptr_t)o, o1 = o0 + (uintptr_t)((int64_t)total_q * qw * 2);
        PKV_REQUIRE(o1 <= q0 || q1 <= o0, PKV_ERR_INVALID_ARG, "%s: o must not overlap q", fn);
    }
    PKV_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) % 16 == 0, PKV_ERR_INVALID_ARG,
                "%s: tensors must be 16-byte aligned", fn);
    if (workspace && workspace_bytes) {
        PKV_REQUIRE((uintptr_t)workspace % 256 == 0, PKV_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned",
                    fn);
        // the split writes partial sums while q and the keys are read and o written;
        // it uses at most the first 512 MiB (pkv_attn_prefill_workspace_bytes)
        const size_t used = workspace_bytes < (size_t(512) << 20) ? workspace_bytes : (size_t(512) << 20);
        const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + used;
        PKV_REQUIRE(w1 > w0, PKV_ERR_WORKSPACE, "%s: workspace range wraps the address space", fn);
        const uintptr_t q0 = (uintptr_t)q, q1 = q0 + (uintptr_t)(((int64_t)(total_q - 1) * q_row_stride + qw) * 2);
        const uintptr_t o0 = (uintptr_t)o, o1 = o0 + (uintptr_t)((int64_t)total_q * qw * 2);
        PKV_REQUIRE((w1 <= q0 || q1 <= w0) && (w1 <= o0 || o1 <= w0), PKV_ERR_WORKSPACE,
                    "%s: workspace must not overlap q or o", fn);
        if (block_table && num_blocks > 0) {
            // the caches' extent is known here (num_blocks slots of block_size rows)
            const uintptr_t cache_bytes = (uintptr_t)num_blocks * (uintptr_t)block_size * (uintptr_t)kw * 2;
            const uintptr_t k0 = (uintptr_t)k, v0 = (uintptr_t)v;
            PKV_REQUIRE((w1 <= k0 || k0 + cache_bytes <= w0) && (w1 <= v0 || v0 + cache_bytes <= w0),
                        PKV_ERR_WORKSPACE, "%s: workspace must not overlap the caches", fn);
        }
    }
    if (block_table) {
        PKV_REQUIRE(block_size == 256, PKV_ERR_UNSUPPORTED, "%s: block_size %d unsupported (only 256)", fn,
                    block_size);
        PKV_REQUIRE(max_blocks_per_seq > 0, PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", fn);
        PKV_REQUIRE(num_blocks > 0, PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
        PKV_REQUIRE(k_row_stride == kw && v_row_stride == kw, PKV_ERR_INVALID_ARG,
                    "%s: with a block table k/v are caches; row strides must equal num_kv_heads*head_dim", fn);
        PKV_REQUIRE(k != v, PKV_ERR_INVALID_ARG, "%s: k_cache and v_cache must be distinct", fn);
        PKV_REQUIRE((int64_t)max_seqlen_k <= (int64_t)max_blocks_per_seq * block_size, PKV_ERR_INVALID_ARG,
                    "%s: max_seqlen_k %d exceeds the block table's capacity", fn, max_seqlen_k);
    }
    pkv::PrefillArgs a;
    a.q = q;
    a.q_row_stride = q_row_stride;
    a.k = k;
    a.k_row_stride = k_row_stride;
    a.v = v;
    a.v_row_stride = v_row_stride;
    a.o = o;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.block_table = block_table;
    a.max_blocks = block_table ? max_blocks_per_seq : 0;
    a.num_blocks = block_table ? num_blocks : 0;
    a.workspace = workspace;
    a.workspace_bytes = workspace ? workspace_bytes : 0;
    return launched(pkv::launch_attn_prefill(a, (hipStream_t)stream), fn);
}

size_t pkv_attn_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                        int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim) {
    if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < max_seqlen_q || num_q_heads <= 0 ||
        num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim != 128)
        return 0;
    return pkv::prefill_workspace_bytes(num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads);
}

size_t pkv_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim != 128 ||
        max_blocks_per_seq <= 0 || block_size != 256)
        return 0;
    if (num_seqs == 0) return 256;
    return pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq);
}

namespace {
// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

// The decode workspace (written by the split kernel while q and the caches are read,
// then read by the merge while o is written) must not share bytes with them.
int decode_workspace_check(const char* fn, const void* ws, size_t need, const void* q, const void* o,
                           const void* k_cache, const void* v_cache, int32_t rows, int32_t num_q_heads,
                           int32_t num_kv_heads, int64_t num_blocks) {
    const size_t qo = (size_t)rows * num_q_heads * 128 * 2;
    const size_t cache = (size_t)num_blocks * 256 * num_kv_heads * 128 * 2;
    PKV_REQUIRE(!overlaps(ws, need, q, qo) && !overlaps(ws, need, o, qo) && !overlaps(ws, need, k_cache, cache) &&
                    !overlaps(ws, need, v_cache, cache),
                PKV_ERR_WORKSPACE, "%s: workspace must not overlap q, o or the caches", fn);
    return PKV_OK;
}

// Checks shared by the two decode entry points; on success fills `a` (workspace unset).
int decode_args(const char* fn, const void* q, const void* k_cache, const void* v_cache, void* o,
                const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                float softmax_scale, pkv::DecodeArgs& a) {
    int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim);
    if (rc) return rc;
    const int G = num_q_heads / num_kv_heads;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, PKV_ERR_UNSUPPORTED,
                "%s: GQA group %d unsupported (1, 2, 4, 8 or 16)", fn, G);
    PKV_REQUIRE(block_size == 256, PKV_ERR_UNSUPPORTED, "%s: block_size %d unsupported (only 256)", fn, block_size);
    PKV_REQUIRE(num_seqs >= 0, PKV_ERR_INVALID_ARG, "%s: num_seqs must be >= 0", fn);
    PKV_REQUIRE(max_blocks_per_seq > 0, PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", fn);
    if (num_seqs == 0) return PKV_OK;
    PKV_REQUIRE(pkv_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                                block_size) > 0,
                PKV_ERR_UNSUPPORTED, "%s: %d sequences of up to %d blocks exceed the launch grid", fn, num_seqs,
                max_blocks_per_seq);
    PKV_REQUIRE(q && k_cache && v_cache && o && context_lens && block_table, PKV_ERR_INVALID_ARG,
                "%s: a required pointer is NULL", fn);
    PKV_REQUIRE(k_cache != v_cache, PKV_ERR_INVALID_ARG, "%s: k_cache and v_cache must be distinct", fn);
    PKV_REQUIRE(num_blocks > 0, PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
    PKV_REQUIRE(softmax_scale > 0.f, PKV_ERR_INVALID_ARG, "%s: softmax_scale must be > 0", fn);
    PKV_REQUIRE(((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)o) % 16 == 0,
                PKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.o = o;
    a.context_lens = context_lens;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.num_blocks = num_blocks;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.workspace = nullptr;
    return PKV_OK;
}
}  // namespace

int pkv_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o,
                          const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks_per_seq,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, float softmax_scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const char* fn = "pkv_attn_decode_paged";
    pkv::DecodeArgs a;
    int rc = decode_args(fn, q, k_cache, v_cache, o, context_lens, block_table, max_blocks_per_seq, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, a);
    if (rc) return rc;
    if (num_seqs == 0) return ok();
    const size_t need = pkv_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                        max_blocks_per_seq, block_size);
    PKV_REQUIRE(workspace != nullptr && workspace_bytes >= need, PKV_ERR_WORKSPACE,
                "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
    PKV_REQUIRE((uintptr_t)workspace % 256 == 0, PKV_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    rc = decode_workspace_check(fn, workspace, need, q, o, k_cache, v_cache, num_seqs, num_q_heads, num_kv_heads,
                                num_blocks);
    if (rc) return rc;
    a.workspace = workspace;
    return launched(pkv::launch_attn_decode(a, (hipStream_t)stream), fn);
}

extern "C++" {
namespace pkv {
// One decode step (pkv_decode_step and its graphs): the checks of
// pkv_qk_norm_rope_store and pkv_attn_decode_paged on the step's buffers, then one
// split kernel that also applies QK-Norm + RoPE to the step's q rows and stores its
// k' / v rows, and the merge.  The results are those of calling the two entry
// points in turn, bit for bit, when each row's slot is its key ctx - 1 (as the
// engine's slot mapping has it); a slot elsewhere is still written, but that
// row's attention then reads whatever its cache row holds.
int decode_step_run(const pkv_decode_step_desc& d, int32_t batch, hipStream_t stream) {
    const int64_t k0 = (int64_t)d.num_q_heads * d.head_dim, v0 = k0 + (int64_t)d.num_kv_heads * d.head_dim;
    const uint16_t* qkv = (const uint16_t*)d.qkv;
    int rc = norm_store_check("pkv_decode_step", qkv, d.qkv_row_stride, qkv + k0, d.qkv_row_stride, qkv + v0,
                              d.qkv_row_stride, d.q_out, nullptr, d.k_cache, d.v_cache, d.num_blocks * d.block_size,
                              d.slot_mapping, d.positions, batch, d.num_q_heads, d.num_kv_heads, d.head_dim,
                              d.q_norm_weight, d.k_norm_weight, d.eps, d.cos_sin_cache, d.max_position);
    if (rc) return rc;
    pkv::DecodeArgs a;
    rc = decode_args("pkv_decode_step", d.q_out, d.k_cache, d.v_cache, d.o, d.context_lens, d.block_table,
                     d.max_blocks_per_seq, batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.block_size,
                     d.num_blocks, d.softmax_scale, a);
    if (rc) return rc;
    if (batch == 0) return ok();
    const size_t need = pkv_attn_decode_workspace_bytes(batch, d.num_q_heads, d.num_kv_heads, d.head_dim,
                                                        d.max_blocks_per_seq, d.block_size);
    PKV_REQUIRE(d.workspace != nullptr && d.workspace_bytes >= need, PKV_ERR_WORKSPACE,
                "pkv_decode_step: workspace of %zu bytes needed, %zu given", need,
                d.workspace ? d.workspace_bytes : (size_t)0);
    PKV_REQUIRE((uintptr_t)d.workspace % 256 == 0, PKV_ERR_WORKSPACE, "pkv_decode_step: workspace must be 256-byte aligned");
    rc = decode_workspace_check("pkv_decode_step", d.workspace, need, d.q_out, d.o, d.k_cache, d.v_cache, batch,
                                d.num_q_heads, d.num_kv_heads, d.num_blocks);
    if (rc) return rc;
    PKV_REQUIRE(!overlaps(d.workspace, need, d.qkv, (size_t)batch * d.qkv_row_stride * 2), PKV_ERR_WORKSPACE,
                "pkv_decode_step: workspace must not overlap qkv");
    a.workspace = d.workspace;
    pkv::StepArgs sa;
    sa.qkv = qkv;
    sa.qkv_stride = d.qkv_row_stride;
    sa.positions = d.positions;
    sa.slot_mapping = d.slot_mapping;
    sa.q_norm_weight = (const uint16_t*)d.q_norm_weight;
    sa.k_norm_weight = (const uint16_t*)d.k_norm_weight;
    sa.eps = d.eps;
    sa.table = d.cos_sin_cache;
    sa.max_pos = d.max_position;
    sa.q_out = (uint16_t*)d.q_out;
    sa.k_cache = (uint16_t*)d.k_cache;
    sa.v_cache = (uint16_t*)d.v_cache;
    sa.num_slots = d.num_blocks * d.block_size;
    return launched(pkv::launch_decode_step(a, sa, stream), "pkv_decode_step");
}
}  // namespace pkv
}  // extern "C++"

int pkv_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                  const int32_t* context_lens, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  float softmax_scale, void* stream) {
    const char* fn = "pkv_attn_decode_paged_noalloc";
    pkv::DecodeArgs a;
    int rc = decode_args(fn, q, k_cache, v_cache, o, context_lens, block_table, max_blocks_per_seq, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, a);
    if (rc) return rc;
    if (num_seqs == 0) return ok();
    const size_t need = pkv_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                        max_blocks_per_seq, block_size);
    PKV_REQUIRE(need <= pkv::kDecodeScratchBytes, PKV_ERR_WORKSPACE,
                "%s: this batch needs %zu bytes of split-K workspace, more than the %zu of the library's fixed "
                "device array; call pkv_attn_decode_paged with a workspace instead",
                fn, need, pkv::kDecodeScratchBytes);
    void* ws = nullptr;
    hipError_t e = pkv::decode_scratch(&ws);
    if (e != hipSuccess)
        return fail(PKV_ERR_LAUNCH, "%s: device address of the fixed workspace: %s", fn, hipGetErrorString(e));
    a.workspace = ws;
    return launched(pkv::launch_attn_decode(a, (hipStream_t)stream), fn);
}

int pkv_add_rms_norm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                     int32_t n_tokens, int32_t hidden, float eps, void* stream) {
    const char* fn = "pkv_add_rms_norm";
    PKV_REQUIRE(n_tokens >= 0, PKV_ERR_INVALID_ARG, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
    PKV_REQUIRE(hidden > 0 && hidden % 8 == 0, PKV_ERR_INVALID_ARG, "%s: hidden %d must be a positive multiple of 8",
                fn, hidden);
    PKV_REQUIRE(hidden <= 8 * 256 * 8, PKV_ERR_UNSUPPORTED, "%s: hidden %d above the built maximum 16384", fn, hidden);
    PKV_REQUIRE(eps >= 0.f, PKV_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    if (n_tokens == 0) return ok();
    PKV_REQUIRE(x && weight && y, PKV_ERR_INVALID_ARG, "%s: x, weight and y are required", fn);
    PKV_REQUIRE((residual == nullptr) == (residual_out == nullptr), PKV_ERR_INVALID_ARG,
                "%s: residual and residual_out are given together or not at all", fn);
    PKV_REQUIRE(!residual_out || residual_out != y, PKV_ERR_INVALID_ARG, "%s: y and residual_out must differ", fn);
    PKV_REQUIRE(((uintptr_t)x | (uintptr_t)residual | (uintptr_t)weight | (uintptr_t)y | (uintptr_t)residual_out) %
                        16 == 0,
                PKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    return launched(pkv::launch_add_rms_norm(x, residual, weight, y, residual_out, n_tokens, hidden, eps,
                                             (hipStream_t)stream),
                    fn);
}

int pkv_silu_and_mul(const void* x, int64_t x_row_stride, void* out, int64_t out_row_stride, int32_t n_tokens,
                     int32_t intermediate, void* stream) {
    const char* fn = "pkv_silu_and_mul";
    PKV_REQUIRE(n_tokens >= 0, PKV_ERR_INVALID_ARG, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
    PKV_REQUIRE(intermediate > 0 && intermediate % 8 == 0, PKV_ERR_INVALID_ARG,
                "%s: intermediate %d must be a positive multiple of 8", fn, intermediate);
    PKV_REQUIRE(x_row_stride >= 2 * (int64_t)intermediate && out_row_stride >= intermediate, PKV_ERR_INVALID_ARG,
                "%s: row strides (%lld, %lld) shorter than the rows", fn, (long long)x_row_stride,
                (long long)out_row_stride);
    PKV_REQUIRE(x_row_stride % 8 == 0 && out_row_stride % 8 == 0, PKV_ERR_INVALID_ARG,
                "%s: row strides must be multiples of 8 elements", fn);
    if (n_tokens == 0) return ok();
    PKV_REQUIRE(x && out, PKV_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    PKV_REQUIRE(((uintptr_t)x | (uintptr_t)out) % 16 == 0, PKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned",
                fn);
    return launched(pkv::launch_silu_and_mul(x, x_row_stride, out, out_row_stride, n_tokens, intermediate,
                                             (hipStream_t)stream),
                    fn);
}

int pkv_sample_gumbel(const void* logits, int64_t logits_row_stride, int32_t logits_dtype, const float* temperatures,
                      const float* noise, int64_t noise_row_stride, uint64_t seed, uint64_t offset, int64_t* tokens,
                      int32_t num_rows, int32_t vocab, void* stream) {
    const char* fn = "pkv_sample_gumbel";
    PKV_REQUIRE(logits_dtype == PKV_DTYPE_BF16 || logits_dtype == PKV_DTYPE_F32, PKV_ERR_UNSUPPORTED,
                "%s: logits_dtype %d unsupported (bf16 or fp32)", fn, logits_dtype);
    PKV_REQUIRE(num_rows >= 0 && vocab > 0, PKV_ERR_INVALID_ARG, "%s: num_rows must be >= 0 and vocab > 0", fn);
    PKV_REQUIRE(logits_row_stride >= vocab, PKV_ERR_INVALID_ARG, "%s: logits_row_stride %lld < vocab %d", fn,
                (long long)logits_row_stride, vocab);
    const int64_t align_elems = logits_dtype == PKV_DTYPE_BF16 ? 8 : 4;
    PKV_REQUIRE(logits_row_stride % align_elems == 0, PKV_ERR_INVALID_ARG,
                "%s: logits_row_stride must be a multiple of %lld elements (16-byte rows)", fn,
                (long long)align_elems);
    if (noise)
        PKV_REQUIRE(noise_row_stride >= vocab && noise_row_stride % 4 == 0, PKV_ERR_INVALID_ARG,
                    "%s: noise_row_stride must be >= vocab and a multiple of 4", fn);
    if (num_rows == 0) return ok();
    PKV_REQUIRE(logits && temperatures && tokens, PKV_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    PKV_REQUIRE(((uintptr_t)logits | (uintptr_t)noise) % 16 == 0, PKV_ERR_INVALID_ARG,
                "%s: logits and noise must be 16-byte aligned", fn);
    PKV_REQUIRE((uintptr_t)tokens % 8 == 0, PKV_ERR_INVALID_ARG, "%s: tokens must be 8-byte aligned", fn);
    return launched(pkv::launch_sample_gumbel(logits, logits_row_stride, logits_dtype == PKV_DTYPE_F32, temperatures,
                                              noise, noise_row_stride, seed, offset, tokens, num_rows, vocab,
                                              (hipStream_t)stream),
                    fn);
}

}  // extern "C"
