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
// into one pass.  A wave owns one token (or, for short batches, a chunk of its
// heads); each (token, head) vector of 128 bf16 is owned by one 16-lane group,
// 8 elements (one 16-byte load) per lane, and the four groups of the wave walk
// the heads.  The cos/sin row and the norm weights are loaded once per wave,
// not once per head.  The sum
// of squares is a 16-lane butterfly; the rotation partner of elements
// [8s, 8s+8) lives in lane s ^ 8, fetched with a cross-lane shuffle.  Math is
// fp32 throughout and the result is rounded to bf16 once.  The q/k/v rows are
// read, and k'/v written into the cache, with non-temporal accesses (each byte
// is touched once); the table rows and weights, which every token reads, go
// through the caches as usual.  The fused pass writes q' through the caches
// too (32768 tokens at 32/8 heads: 146 -> 131 us; streaming q' as well: 149 us).
// The unfused pass streams q' and k' (its outputs' dirty lines otherwise slow the
// store_kvcache that follows: 114 + 66 us against 118 + 47 us for the pair).
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
// elements per lane (xo = this lane's 16-byte chunk, zero for dead groups).
// go / gp are this lane's and its rotation partner's 8 weights, cv / sv the
// cos and sin of this lane's 8 frequencies.  All 16 lanes of the group must
// call it together: the sum of squares and the rotation partner cross lanes.
// Returns this lane's 8 outputs packed as bf16 (one RNE rounding of the fp32
// result).
__device__ __forceinline__ u32x4 norm_rope_apply(u32x4 xo, u32x4 go, u32x4 gp, float eps, const float* cv,
                                                 const float* sv, int sub) {
    u32x4 xp;
#pragma unroll
    for (int w = 0; w < 4; ++w) xp[w] = __shfl_xor(xo[w], 8, 16);
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

// One token's table row, clamped position.
__device__ __forceinline__ const float* rope_row(const float* table, const int64_t* positions, int64_t t,
                                                 int32_t max_pos) {
    int64_t pos = positions[t];
    pos = pos < 0 ? 0 : (pos >= max_pos ? (int64_t)max_pos - 1 : pos);
    return table + pos * kHeadDim;
}

__device__ __forceinline__ void load_cos_sin(const float* __restrict__ row, int sub, float* cv, float* sv) {
    const float* cs = row + (sub & 7) * 8;
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + 64);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 68);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cv[i] = c0[i];
        cv[4 + i] = c1[i];
        sv[i] = s0[i];
        sv[4 + i] = s1[i];
    }
}

// A wave owns one token, or for short batches one chunk of a token's heads
// (hpw heads, a multiple of 4; the heads are numbered q, then k, then v).  Its
// four 16-lane groups take the chunk's heads in turn (head lo+g, lo+g+4, ...),
// kChunk heads per group loaded before any is stored, so several loads are in
// flight even when the outputs alias the inputs.  The table row and the
// weights are loaded once per wave.
constexpr int kChunk = 4;

template <typename LoadF, typename StoreF>
__device__ __forceinline__ void norm_rope_heads(int lo, int hi, int grp, int sub, u32x4 go, u32x4 gp, float eps,
                                                const float* cv, const float* sv, LoadF load, StoreF store) {
    for (int h0 = lo; h0 < hi; h0 += 4 * kChunk) {
        u32x4 x[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int h = h0 + 4 * c + grp;
            x[c] = h < hi ? load(h) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int h = h0 + 4 * c + grp;
            if (h0 + 4 * c >= hi) break;               // no group of the wave has this head (uniform)
            const u32x4 res = norm_rope_apply(x[c], go, gp, eps, cv, sv, sub);
            if (h < hi) store(h, res);
        }
    }
}

// 4 waves per 256-thread block; wave w handles token w / chunks, heads
// [hpw * (w % chunks), hpw * (w % chunks + 1)) of the token's hq + hkv heads.
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(
    const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,  // may alias the outputs
    uint16_t* q_out, uint16_t* k_out, const int64_t* __restrict__ positions, int32_t n_tokens, int32_t hq,
    int32_t hkv, const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk, float eps,
    const float* __restrict__ table, int32_t max_pos, int32_t hpw, int32_t chunks) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = w / chunks;
    if (t >= n_tokens) return;                       // the whole wave leaves together
    const int lo = hpw * (int)(w - t * chunks), hi = lo + hpw;
    const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
    float cv[8], sv[8];
    load_cos_sin(rope_row(table, positions, t, max_pos), sub, cv, sv);
    if (lo < hq) {
        const uint16_t* qt = q + t * q_row_stride + sub * 8;
        uint16_t* qo = q_out + t * hq * kHeadDim + sub * 8;
        norm_rope_heads(lo, min(hi, hq), grp, sub, ldg128(gq + sub * 8), ldg128(gq + (sub ^ 8) * 8), eps, cv, sv,
                        [&](int h) { return ldg128_stream(qt + (int64_t)h * kHeadDim); },
                        [&](int h, u32x4 r) { stg128_stream(qo + (int64_t)h * kHeadDim, r); });
    }
    if (hi > hq) {
        const uint16_t* kt = k + t * k_row_stride + sub * 8;
        uint16_t* ko = k_out + t * hkv * kHeadDim + sub * 8;
        norm_rope_heads(max(lo, hq) - hq, min(hi, hq + hkv) - hq, grp, sub, ldg128(gk + sub * 8),
                        ldg128(gk + (sub ^ 8) * 8), eps, cv, sv,
                        [&](int h) { return ldg128_stream(kt + (int64_t)h * kHeadDim); },
                        [&](int h, u32x4 r) { stg128_stream(ko + (int64_t)h * kHeadDim, r); });
    }
}

// QK-Norm + RoPE fused with the cache scatter; wave layout as above over the
// token's hq + 2 hkv heads.  Query heads go to q_out; rotated key heads go
// straight to k_cache row slot_mapping[t] (and to k_out when it is given);
// value heads are copied to v_cache row slot_mapping[t].  A slot outside
// [0, num_slots) (the padding id -1 included) writes no cache row.
__global__ void __launch_bounds__(256) qk_norm_rope_store_kernel(
    const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,
    const uint16_t* __restrict__ v, int64_t v_row_stride, uint16_t* q_out, uint16_t* k_out,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, const int64_t* __restrict__ positions, int32_t n_tokens, int32_t hq,
    int32_t hkv, const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk, float eps,
    const float* __restrict__ table, int32_t max_pos, int32_t hpw, int32_t chunks) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = w / chunks;
    if (t >= n_tokens) return;
    const int lo = hpw * (int)(w - t * chunks), hi = lo + hpw;
    const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
    const int64_t D = (int64_t)hkv * kHeadDim;
    const int64_t slot = (int64_t)slot_mapping[t];
    const bool to_cache = slot >= 0 && slot < num_slots;
    uint16_t* kc = to_cache ? k_cache + slot * D + sub * 8 : nullptr;

    // value heads: plain copies into the cache row
    const int vlo = max(lo, hq + hkv) - hq - hkv, vhi = min(hi, hq + 2 * hkv) - hq - hkv;
    if (to_cache && vlo < vhi) {
        const uint16_t* vt = v + t * v_row_stride + sub * 8;
        uint16_t* vc = v_cache + slot * D + sub * 8;
        for (int h0 = vlo; h0 < vhi; h0 += 4 * kChunk) {
            u32x4 x[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int h = h0 + 4 * c + grp;
                if (h < vhi) x[c] = ldg128_stream(vt + (int64_t)h * kHeadDim);
            }
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int h = h0 + 4 * c + grp;
                if (h < vhi) stg128_stream(vc + (int64_t)h * kHeadDim, x[c]);
            }
        }
    }
    if (lo >= hq + hkv) return;
    float cv[8], sv[8];
    load_cos_sin(rope_row(table, positions, t, max_pos), sub, cv, sv);
    if (lo < hq) {
        const uint16_t* qt = q + t * q_row_stride + sub * 8;
        uint16_t* qo = q_out + t * hq * kHeadDim + sub * 8;
        norm_rope_heads(lo, min(hi, hq), grp, sub, ldg128(gq + sub * 8), ldg128(gq + (sub ^ 8) * 8), eps, cv, sv,
                        [&](int h) { return ldg128_stream(qt + (int64_t)h * kHeadDim); },
                        [&](int h, u32x4 r) { stg128(qo + (int64_t)h * kHeadDim, r); });
    }
    if (hi > hq) {
        const uint16_t* kt = k + t * k_row_stride + sub * 8;
        uint16_t* ko = k_out ? k_out + t * hkv * kHeadDim + sub * 8 : nullptr;
        norm_rope_heads(max(lo, hq) - hq, min(hi, hq + hkv) - hq, grp, sub, ldg128(gk + sub * 8),
                        ldg128(gk + (sub ^ 8) * 8), eps, cv, sv,
                        [&](int h) { return ldg128_stream(kt + (int64_t)h * kHeadDim); },
                        [&](int h, u32x4 r) {
                            if (ko) stg128(ko + (int64_t)h * kHeadDim, r);
                            if (kc) stg128_stream(kc + (int64_t)h * kHeadDim, r);
                        });
    }
}

// Heads per wave: all of a token's heads once there are enough tokens to fill
// the device (2048 waves, 8 per CU); fewer tokens split each token's heads
// into chunks (a multiple of 4, at least 4) so the launch still has ~2048 waves.
static void heads_per_wave(int64_t n_tokens, int heads, int32_t& hpw, int32_t& chunks) {
    const int64_t target = 2048;
    int64_t want = (heads * n_tokens + target - 1) / target;   // heads per wave for ~target waves
    want = (want + 3) / 4 * 4;
    if (want < 4) want = 4;
    if (want > heads) want = (heads + 3) / 4 * 4;
    hpw = (int32_t)want;
    chunks = (heads + hpw - 1) / hpw;
}

hipError_t launch_qk_norm_rope(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                               void* q_out, void* k_out, const int64_t* positions, int32_t n_tokens,
                               int32_t hq, int32_t hkv, const void* gq, const void* gk, float eps,
                               const float* table, int32_t max_pos, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    int32_t hpw, chunks;
    heads_per_wave(n_tokens, hq + hkv, hpw, chunks);
    const int64_t blocks = ((int64_t)n_tokens * chunks + 3) / 4;
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)q, q_row_stride, (const uint16_t*)k, k_row_stride, (uint16_t*)q_out,
                       (uint16_t*)k_out, positions, n_tokens, hq, hkv, (const uint16_t*)gq, (const uint16_t*)gk,
                       eps, table, max_pos, hpw, chunks);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope_store(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                                     const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache,
                                     void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                                     const int64_t* positions, int32_t n_tokens, int32_t hq, int32_t hkv,
                                     const void* gq, const void* gk, float eps, const float* table, int32_t max_pos,
                                     hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    int32_t hpw, chunks;
    heads_per_wave(n_tokens, hq + 2 * hkv, hpw, chunks);
    const int64_t blocks = ((int64_t)n_tokens * chunks + 3) / 4;
    hipLaunchKernelGGL(qk_norm_rope_store_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)q,
                       q_row_stride, (const uint16_t*)k, k_row_stride, (const uint16_t*)v, v_row_stride,
                       (uint16_t*)q_out, (uint16_t*)k_out, (uint16_t*)k_cache, (uint16_t*)v_cache, num_slots,
                       slot_mapping, positions, n_tokens, hq, hkv, (const uint16_t*)gq, (const uint16_t*)gk, eps,
                       table, max_pos, hpw, chunks);
    return hipGetLastError();
}

}  // namespace pkv
