// rope.hip -- RoPE cos/sin table and the fused QK-Norm + RoPE kernel (gfx950).
//
// "3.3 Model skeleton and core operators", section 2 (RMSNorm in fp32 with eps
// inside the root), section 3 (table built once at init: cos half then sin
// half; rotation of the pair (i, i + d/2); Q and K only), section 8 (QK-Norm
// applied per head on [token, head, head_dim] views, then RoPE).
// "Nano-vLLM 源码解读 #17 注意力层", section 4 (QK-Norm over head_dim,
// V untouched).  "同一个 Qwen3，两种写法", section 3.5 (one fp32 table of
// max_position rows looked up by position).
//
// Design: the two elementwise steps the pages compile separately are fused
// into one pass.  Each (token, head) vector of 128 bf16 is owned by 16 lanes,
// 8 elements (one 16-byte load) per lane.  The sum of squares is a 16-lane
// butterfly; the rotation partner of elements [8s, 8s+8) lives in lane s ^ 8,
// fetched with a cross-lane shuffle.  Math is fp32 throughout and the result
// is rounded to bf16 once.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// One thread per (position, frequency): inv_f = fp32(theta^(-2i/r)), the
// angle is the fp32 product fp32(p) * inv_f, and cos/sin of that fp32 angle
// are evaluated in double and rounded to fp32.
__global__ void __launch_bounds__(256) rope_cache_kernel(float* __restrict__ table, int32_t max_pos,
                                                         int32_t rot_dim, double theta) {
    const int half = rot_dim >> 1;
    const int64_t n = (int64_t)max_pos * half;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p = (int32_t)(e / half);
        const int i = (int)(e - (int64_t)p * half);
        const float inv = (float)pow(theta, -(2.0 * (double)i) / (double)rot_dim);
        const float ang = (float)p * inv;  // one IEEE fp32 multiply
        float* row = table + (int64_t)p * rot_dim;
        row[i] = (float)cos((double)ang);
        row[half + i] = (float)sin((double)ang);
    }
}

hipError_t launch_rope_cache_build(float* table, int32_t max_pos, int32_t rot_dim, double theta,
                                   hipStream_t stream) {
    const int64_t n = (int64_t)max_pos * (rot_dim / 2);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, max_pos, rot_dim,
                       theta);
    return hipGetLastError();
}

// QK-Norm + RoPE of one 128-element head vector held by a 16-lane group, 8
// elements per lane (x = this lane's 16-byte chunk, may be zero for dead
// groups).  All 16 lanes of the group must call it together: the sum of
// squares and the rotation partner cross lanes.  Returns this lane's 8 output
// elements packed as bf16 (one RNE rounding of the fp32 result).
__device__ __forceinline__ u32x4 norm_rope_chunk(u32x4 xo, const uint16_t* __restrict__ g, float eps,
                                                 const float* __restrict__ table_row, int sub) {
    u32x4 xp;
#pragma unroll
    for (int w = 0; w < 4; ++w) xp[w] = __shfl_xor(xo[w], 8, 16);
    const u32x4 go = ldg128(g + sub * 8);
    const u32x4 gp = ldg128(g + (sub ^ 8) * 8);

    float xa[8], xb[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        xa[2 * w] = bf16lo(xo[w]);
        xa[2 * w + 1] = bf16hi(xo[w]);
        xb[2 * w] = bf16lo(xp[w]);
        xb[2 * w + 1] = bf16hi(xp[w]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xa[e] * xa[e];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 16);
    const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);

    const float* cs = table_row + (sub & 7) * 8;
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + 64);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 68);
    const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // Lanes 0..7 hold x1 (first half): y1 = x1 c - x2 s.  Lanes 8..15 hold x2: y2 = x2 c + x1 s.
    const float sgn = sub < 8 ? -1.0f : 1.0f;
    u32x4 res;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float out[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const int e = 2 * w + hlf;
            const float ga = hlf ? bf16hi(go[w]) : bf16lo(go[w]);
            const float gb = hlf ? bf16hi(gp[w]) : bf16lo(gp[w]);
            const float ya = xa[e] * r * ga;
            const float yb = xb[e] * r * gb;
            out[hlf] = ya * cv[e] + sgn * (yb * sv[e]);
        }
        res[w] = pack_bf16x2(out[0], out[1]);
    }
    return res;
}

__device__ __forceinline__ const float* rope_row(const float* table, const int64_t* positions, int64_t t, bool live,
                                                 int32_t max_pos) {
    int64_t pos = live ? positions[t] : 0;
    pos = pos < 0 ? 0 : (pos >= max_pos ? (int64_t)max_pos - 1 : pos);
    return table + pos * kHeadDim;
}

// 16 lanes per (token, head) item; 16 items per 256-thread block.
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(
    const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,  // may alias the outputs
    uint16_t* q_out, uint16_t* k_out, const int64_t* __restrict__ positions, int32_t n_tokens, int32_t hq,
    int32_t hkv, const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk, float eps,
    const float* __restrict__ table, int32_t max_pos) {
    const int heads = hq + hkv;
    const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    const int64_t n_items = (int64_t)n_tokens * heads;
    // Items past the end still take part in the shuffles (all 16 lanes of a
    // group share the same item, so a whole group is either in or out).
    const bool live = item < n_items;
    const int64_t it = live ? item : 0;
    const int64_t t = it / heads;
    const int h = (int)(it - t * heads);
    const bool is_q = h < hq;
    const uint16_t* src = is_q ? q + t * q_row_stride + (int64_t)h * kHeadDim
                               : k + t * k_row_stride + (int64_t)(h - hq) * kHeadDim;
    uint16_t* dst = is_q ? q_out + (t * hq + h) * kHeadDim : k_out + (t * hkv + (h - hq)) * kHeadDim;

    const u32x4 xo = live ? ldg128(src + sub * 8) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 res = norm_rope_chunk(xo, is_q ? gq : gk, eps, rope_row(table, positions, t, live, max_pos), sub);
    if (live) stg128(dst + sub * 8, res);
}

// QK-Norm + RoPE fused with the cache scatter.  Per token the items are the
// Hq query heads, the Hkv key heads and the Hkv value heads (16 lanes each).
// Query heads go to q_out; rotated key heads go straight to k_cache row
// slot_mapping[t] (and to k_out when it is given); value heads are copied to
// v_cache row slot_mapping[t].  A slot outside [0, num_slots) (the padding
// id -1 included) writes no cache row.
__global__ void __launch_bounds__(256) qk_norm_rope_store_kernel(
    const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,
    const uint16_t* __restrict__ v, int64_t v_row_stride, uint16_t* q_out, uint16_t* k_out,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, const int64_t* __restrict__ positions, int32_t n_tokens, int32_t hq,
    int32_t hkv, const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk, float eps,
    const float* __restrict__ table, int32_t max_pos) {
    const int heads = hq + 2 * hkv;
    const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    const bool live = item < (int64_t)n_tokens * heads;
    const int64_t it = live ? item : 0;
    const int64_t t = it / heads;
    const int h = (int)(it - t * heads);
    const int64_t D = (int64_t)hkv * kHeadDim;
    const int64_t slot = live ? (int64_t)slot_mapping[t] : -1;
    const bool to_cache = slot >= 0 && slot < num_slots;

    if (h >= hq + hkv) {  // value head: plain copy into the cache (the whole group takes this branch)
        const int hv = h - hq - hkv;
        if (to_cache)
            stg128(v_cache + slot * D + (int64_t)hv * kHeadDim + sub * 8,
                   ldg128(v + t * v_row_stride + (int64_t)hv * kHeadDim + sub * 8));
        return;
    }
    const bool is_q = h < hq;
    const uint16_t* src = is_q ? q + t * q_row_stride + (int64_t)h * kHeadDim
                               : k + t * k_row_stride + (int64_t)(h - hq) * kHeadDim;
    const u32x4 xo = live ? ldg128(src + sub * 8) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 res = norm_rope_chunk(xo, is_q ? gq : gk, eps, rope_row(table, positions, t, live, max_pos), sub);
    if (!live) return;
    if (is_q) {
        stg128(q_out + (t * hq + h) * kHeadDim + sub * 8, res);
    } else {
        const int hk = h - hq;
        if (k_out) stg128(k_out + (t * hkv + hk) * kHeadDim + sub * 8, res);
        if (to_cache) stg128(k_cache + slot * D + (int64_t)hk * kHeadDim + sub * 8, res);
    }
}

hipError_t launch_qk_norm_rope(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                               void* q_out, void* k_out, const int64_t* positions, int32_t n_tokens,
                               int32_t hq, int32_t hkv, const void* gq, const void* gk, float eps,
                               const float* table, int32_t max_pos, hipStream_t stream) {
    const int64_t items = (int64_t)n_tokens * (hq + hkv);
    if (items == 0) return hipSuccess;
    const int64_t blocks = (items + 15) / 16;
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)q, q_row_stride, (const uint16_t*)k, k_row_stride, (uint16_t*)q_out,
                       (uint16_t*)k_out, positions, n_tokens, hq, hkv, (const uint16_t*)gq, (const uint16_t*)gk,
                       eps, table, max_pos);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope_store(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                                     const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache,
                                     void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                                     const int64_t* positions, int32_t n_tokens, int32_t hq, int32_t hkv,
                                     const void* gq, const void* gk, float eps, const float* table, int32_t max_pos,
                                     hipStream_t stream) {
    const int64_t items = (int64_t)n_tokens * (hq + 2 * hkv);
    if (items == 0) return hipSuccess;
    const int64_t blocks = (items + 15) / 16;
    hipLaunchKernelGGL(qk_norm_rope_store_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)q,
                       q_row_stride, (const uint16_t*)k, k_row_stride, (const uint16_t*)v, v_row_stride,
                       (uint16_t*)q_out, (uint16_t*)k_out, (uint16_t*)k_cache, (uint16_t*)v_cache, num_slots,
                       slot_mapping, positions, n_tokens, hq, hkv, (const uint16_t*)gq, (const uint16_t*)gk, eps,
                       table, max_pos);
    return hipGetLastError();
}

}  // namespace pkv
