// store_kvcache.hip -- scatter of K/V rows into the paged KV cache (gfx950).
//
// "3.3 Model skeleton and core operators", section 7.1 and "Nano-vLLM 源码解读
// #17 注意力层", section 5.1: each token's K row and V row (D = Hkv * head_dim
// contiguous elements) go to cache row slot_mapping[t]; slot -1 marks a
// padding token that writes nothing.  The cache is a flat array of slots of D
// elements (k_cache.stride(1) == D).
//
// Design: the pages launch one program per token.  Here a workgroup of 256
// lanes moves one or several whole tokens; every lane moves 16-byte chunks, so
// a 2 KiB row is one fully coalesced 128-lane sweep for K and another for V,
// and the token and piece of a lane come from the block shape, not from an
// index division.  Byte offsets are
// 64-bit (a slot index times 2 KiB passes 4 GiB in large pools).  Slots
// outside [0, num_slots) are skipped like -1, so bad metadata can never write
// outside the cache.  The copy is bit for bit (dtype-agnostic).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Block shape (tx, ty): ty tokens per workgroup, tx lanes per token walking its
// 2 * chunks 16-byte pieces (K pieces, then V pieces); no index division.
template <typename Chunk>
__global__ void __launch_bounds__(256) store_kvcache_kernel(
    const char* __restrict__ key, int64_t key_row_bytes, const char* __restrict__ value, int64_t value_row_bytes,
    char* __restrict__ k_cache, char* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, int32_t n_tokens, int64_t row_bytes) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.y + threadIdx.y;
    if (t >= n_tokens) return;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;  // -1: padding token
    const int32_t chunks = (int32_t)(row_bytes / (int64_t)sizeof(Chunk));
    const Chunk* ks = reinterpret_cast<const Chunk*>(key + t * key_row_bytes);
    const Chunk* vs = reinterpret_cast<const Chunk*>(value + t * value_row_bytes);
    Chunk* kd = reinterpret_cast<Chunk*>(k_cache + slot * row_bytes);
    Chunk* vd = reinterpret_cast<Chunk*>(v_cache + slot * row_bytes);
    for (int32_t c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
        if (c < chunks) kd[c] = ks[c];
        else vd[c - chunks] = vs[c - chunks];
    }
}

hipError_t launch_store_kvcache(const void* key, int64_t key_row_stride, const void* value,
                                int64_t value_row_stride, void* k_cache, void* v_cache, int64_t num_slots,
                                const int32_t* slot_mapping, int32_t n_tokens, int64_t row_bytes,
                                int32_t elem_bytes, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    const int64_t kb = key_row_stride * elem_bytes, vb = value_row_stride * elem_bytes;
    auto aligned = [&](int64_t a) {
        return (((uintptr_t)key | (uintptr_t)value | (uintptr_t)k_cache | (uintptr_t)v_cache) % a == 0) &&
               kb % a == 0 && vb % a == 0 && row_bytes % a == 0;
    };
    auto go = [&](auto chunk_tag) -> hipError_t {
        using Chunk = decltype(chunk_tag);
        const int64_t per_token = 2 * (row_bytes / (int64_t)sizeof(Chunk));
        if (per_token > 0x7FFFFFFF) return hipErrorInvalidValue;
        // lanes per token: the token's pieces rounded up to a wave, at most 256
        int tx = (int)(per_token >= 256 ? 256 : ((per_token + 63) / 64) * 64);
        const int ty = 256 / tx;
        const int64_t blocks = ((int64_t)n_tokens + ty - 1) / ty;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(store_kvcache_kernel<Chunk>, dim3((unsigned)blocks), dim3(tx, ty), 0, stream,
                           (const char*)key, kb, (const char*)value, vb, (char*)k_cache, (char*)v_cache,
                           num_slots, slot_mapping, n_tokens, row_bytes);
        return hipGetLastError();
    };
    if (aligned(16)) return go(u32x4{});
    if (aligned(4)) return go(uint32_t{});
    return go(uint8_t{});
}

}  // namespace pkv
