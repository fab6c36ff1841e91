// sublayer.hip -- the elementwise steps around the attention core (gfx950):
// residual add + RMSNorm, SiluAndMul, and the Gumbel-max sampler.
//
// "3.3 Model skeleton and core operators", section 2 (RMSNorm with the
// residual folded in: fp32 add, the sum rounded to bf16 is the new residual,
// the fp32 sum is normalised, rounded to bf16, then multiplied by gamma in
// bf16), section 4 (SiluAndMul: front half gate, back half up) and section 9
// (sampler: logits / temperature, softmax, divide by Exp(1) noise clamped at
// 1e-10, argmax).  "同一个 Qwen3，两种写法", section 3.6: the fused add + norm
// moves 32 KiB per 4096-wide bf16 token (read x, residual; write y, residual).
//
// Add + RMSNorm and SiluAndMul are HBM-streaming kernels: 16-byte vector loads
// and stores, fp32 math in registers, one pass over memory.  The sampler also
// reads each logit once, but with its noise drawn in the kernel (Philox4x32-10:
// twenty 32x32->64-bit products per four tokens, two logarithms per token) it
// is bound by vector-ALU issue, not by memory: each row is split over several
// workgroups so the chip holds enough waves to keep the ALUs busy, and the
// partial winners meet through a 64-bit atomic maximum on the row's output slot.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

// ---------------------------------------------------------------------------
// residual add + RMSNorm
// ---------------------------------------------------------------------------
// A row of `hidden` elements is covered by `lpr` lanes (64, 128 or 256; 256 /
// lpr rows per 256-thread block), each owning up to NC chunks of 8 elements
// strided by lpr chunks.  The row's sum of squares: a wave butterfly, then the
// row's waves combine through LDS in wave order (deterministic).  x, residual and
// both outputs stream through the caches (non-temporal: 192 -> 181 us on
// [32768, 4096]); gamma, which every row reads, is cached as usual.
template <int NC>
__global__ void __launch_bounds__(256) add_rms_norm_kernel(const uint16_t* x, const uint16_t* residual,
                                                           const uint16_t* __restrict__ gamma, uint16_t* y,
                                                           uint16_t* residual_out, int32_t n_tokens, int32_t hidden,
                                                           int32_t lpr, float eps) {
    __shared__ float s_part[4];
    const int tid = threadIdx.x;
    const int rpb = 256 / lpr;
    const int lr = tid / lpr, li = tid - lr * lpr;
    const int64_t row = (int64_t)blockIdx.x * rpb + lr;
    const bool live = row < n_tokens;
    const int chunks = hidden >> 3;
    const int64_t base = row * hidden;

    float s[NC][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = li + k * lpr;
        const bool ok = live && c < chunks;
        const u32x4 xv = ok ? ldg128_stream(x + base + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        if (residual) {
            const u32x4 rv = ok ? ldg128_stream(residual + base + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // fp32 add of the two bf16 values (exact inputs, one IEEE rounding)
                s[k][2 * w] = bf16lo(xv[w]) + bf16lo(rv[w]);
                s[k][2 * w + 1] = bf16hi(xv[w]) + bf16hi(rv[w]);
            }
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                s[k][2 * w] = bf16lo(xv[w]);
                s[k][2 * w + 1] = bf16hi(xv[w]);
            }
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(s[k][e], s[k][e], part);
        ss += part;
        if (ok && residual_out) {
            u32x4 ro;
#pragma unroll
            for (int w = 0; w < 4; ++w) ro[w] = pack_bf16x2(s[k][2 * w], s[k][2 * w + 1]);
            stg128_stream(residual_out + base + 8 * c, ro);
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    const int wpr = lpr >> 6;
    float tot = 0.f;
    for (int j = 0; j < wpr; ++j) tot += s_part[lr * wpr + j];
    const float r = 1.0f / sqrtf(tot / (float)hidden + eps);
    if (!live) return;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = li + k * lpr;
        if (c >= chunks) break;
        const u32x4 gv = ldg128(gamma + 8 * c);
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // normalised value rounded to bf16, then the bf16 product with gamma
            const float n0 = bf16lo(pack_bf16x2(s[k][2 * w] * r, 0.f));
            const float n1 = bf16lo(pack_bf16x2(s[k][2 * w + 1] * r, 0.f));
            out[w] = pack_bf16x2(n0 * bf16lo(gv[w]), n1 * bf16hi(gv[w]));
        }
        stg128_stream(y + base + 8 * c, out);
    }
}

// ---------------------------------------------------------------------------
// SiluAndMul
// ---------------------------------------------------------------------------
// One lane per 8 output elements: the gate chunk and the up chunk of the same
// columns, silu(g) * u in fp32, one rounding.  A lane loads two chunks' gate and
// up halves before computing either, and rows stream through the caches with
// non-temporal loads and stores (together 7% faster on [32768, 2 x 12288]; the
// non-temporal accesses alone, or the paired loads alone, gain under 1.5%).
__device__ __forceinline__ u32x4 silu_mul8(u32x4 gv, u32x4 uv) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float g0 = bf16lo(gv[w]), g1 = bf16hi(gv[w]);
        const float a0 = g0 / (1.0f + __expf(-g0)) * bf16lo(uv[w]);
        const float a1 = g1 / (1.0f + __expf(-g1)) * bf16hi(uv[w]);
        o[w] = pack_bf16x2(a0, a1);
    }
    return o;
}

__global__ void __launch_bounds__(256) silu_and_mul_kernel(const uint16_t* __restrict__ x, int64_t x_row_stride,
                                                           uint16_t* __restrict__ out, int64_t out_row_stride,
                                                           int32_t n_tokens, int32_t inter) {
    const int cpr = inter >> 3;   // 8-element chunks per row
    for (int64_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
        const uint16_t* row = x + t * x_row_stride;
        uint16_t* orow = out + t * out_row_stride;
        const int step = (int)blockDim.x;
        int c = threadIdx.x;
        for (; c + step < cpr; c += 2 * step) {
            const u32x4 gv0 = ldg128_stream(row + 8 * c), uv0 = ldg128_stream(row + inter + 8 * c);
            const u32x4 gv1 = ldg128_stream(row + 8 * (c + step)), uv1 = ldg128_stream(row + inter + 8 * (c + step));
            stg128_stream(orow + 8 * c, silu_mul8(gv0, uv0));
            stg128_stream(orow + 8 * (c + step), silu_mul8(gv1, uv1));
        }
        if (c < cpr) stg128_stream(orow + 8 * c, silu_mul8(ldg128_stream(row + 8 * c), ldg128_stream(row + inter + 8 * c)));
    }
}

// ---------------------------------------------------------------------------
// Gumbel-max sampler
// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC 2011): 10 rounds of two 32x32->64-bit
// products mixed with the counter and key; the key advances by the Weyl
// constants between rounds.
struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // hi ^ counter ^ key in one gfx950 three-input bitwise op (truth table 0x96 =
        // a ^ b ^ c); the compiler does not form it from two XORs (sampler 38 -> 34 us)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// Exp(1) noise by inversion of the uniform (k + 1) / 2^24 on (0, 1] made from
// the top 24 bits of a draw; returns log2 of the noise clamped at 1e-10.
__device__ __forceinline__ float log2_noise_from_bits(uint32_t bits) {
    const float u = (float)((bits >> 8) + 1u) * 0x1p-24f;
    const float E = fmaxf(-__builtin_amdgcn_logf(u) * 0.69314718055994531f, 1e-10f);
    return __builtin_amdgcn_logf(E);
}

// Score of a token in log2 units: log2(p_i / E_i) up to a per-row constant,
//   = (l_i / T) * log2(e) - log2(E_i).
// The row's softmax normaliser is common to every token, so the argmax needs
// neither the max nor the sum.  Ties keep the lower index.
template <bool F32>
__device__ __forceinline__ void load8(const void* row, int64_t c8, float (&l)[8]) {
    if (F32) {
        const float* p = (const float*)row + 8 * c8;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            l[e] = a[e];
            l[4 + e] = b[e];
        }
    } else {
        const u32x4 v = ldg128((const uint16_t*)row + 8 * c8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            l[2 * w] = bf16lo(v[w]);
            l[2 * w + 1] = bf16hi(v[w]);
        }
    }
}

constexpr int kSampThreads = 256;

// A (score, index) pair as one unsigned 64-bit key whose unsigned order is the
// argmax order with ties to the lower index: the score's bits made monotone in
// the high word, the index complemented in the low word.  0 means "nothing
// taken" (every score NaN); no real pair maps to it.
__device__ __forceinline__ unsigned long long sample_key(float s, int32_t i) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)m << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
}

// Each row is split over `parts` workgroups; each reduces its share to one key
// and folds it into tokens[b] (cleared to 0 by sample_clear_kernel) with a 64-bit
// atomicMax; sample_finish_kernel turns the key back into the token index.
template <bool F32>
__global__ void __launch_bounds__(kSampThreads) sample_gumbel_kernel(
    const void* __restrict__ logits, int64_t row_stride, const float* __restrict__ temperatures,
    const float* __restrict__ noise, int64_t noise_row_stride, uint32_t k0, uint32_t k1, uint32_t off_lo,
    uint32_t off_hi, unsigned long long* __restrict__ keys, int32_t vocab, int32_t parts) {
    __shared__ unsigned long long s_k[kSampThreads / 64];
    const int b = blockIdx.x / parts, part = blockIdx.x - b * parts, tid = threadIdx.x;
    const float T = fmaxf(temperatures[b], 1e-10f);
    const float mul = 1.4426950408889634f / T;  // log2(e) / T
    const char* row = (const char*)logits + (int64_t)b * row_stride * (F32 ? 4 : 2);
    const float* nrow = noise ? noise + (int64_t)b * noise_row_stride : nullptr;
    // This lane's indices only grow, so a strict > keeps the lowest index among equal scores.
    float best_s = -INFINITY;
    int32_t best_i = 0x7FFFFFFF;
    const int64_t n8 = vocab >> 3;
    const int64_t per = (n8 + parts - 1) / parts;
    const int64_t c0 = part * per, c1 = c0 + per < n8 ? c0 + per : n8;
    for (int64_t c = c0 + tid; c < c1; c += kSampThreads) {
        float l[8];
        load8<F32>(row, c, l);
        float ln[8];
        if (nrow) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(nrow + 8 * c);
            const f32x4 bq = *reinterpret_cast<const f32x4*>(nrow + 8 * c + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ln[e] = __builtin_amdgcn_logf(fmaxf(a[e], 1e-10f));
                ln[4 + e] = __builtin_amdgcn_logf(fmaxf(bq[e], 1e-10f));
            }
        } else {
            const uint32_t q = (uint32_t)(2 * c);  // Philox counter word 0: column / 4
            const Philox4 r0 = philox4x32_10(q, (uint32_t)b, off_lo, off_hi, k0, k1);
            const Philox4 r1 = philox4x32_10(q + 1, (uint32_t)b, off_lo, off_hi, k0, k1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ln[e] = log2_noise_from_bits(r0.v[e]);
                ln[4 + e] = log2_noise_from_bits(r1.v[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sc = l[e] * mul - ln[e];
            const bool win = sc > best_s;
            best_s = win ? sc : best_s;
            best_i = win ? (int32_t)(8 * c + e) : best_i;
        }
    }
    // tail of a vocab that is not a multiple of 8 (last part only)
    if (part == parts - 1) {
        for (int32_t i = (int32_t)(n8 << 3) + tid; i < vocab; i += kSampThreads) {
            const float l = F32 ? ((const float*)row)[i] : bf16lo(((const uint16_t*)row)[i]);
            float ln;
            if (nrow) {
                ln = __builtin_amdgcn_logf(fmaxf(nrow[i], 1e-10f));
            } else {
                const Philox4 r = philox4x32_10((uint32_t)(i >> 2), (uint32_t)b, off_lo, off_hi, k0, k1);
                ln = log2_noise_from_bits(r.v[i & 3]);
            }
            const float sc = l * mul - ln;
            const bool win = sc > best_s;
            best_s = win ? sc : best_s;
            best_i = win ? i : best_i;
        }
    }
    unsigned long long key = best_i == 0x7FFFFFFF ? 0ull : sample_key(best_s, best_i);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long k2 = __shfl_xor(key, o, 64);
        key = k2 > key ? k2 : key;
    }
    if ((tid & 63) == 0) s_k[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
        unsigned long long r = s_k[0];
        for (int w = 1; w < kSampThreads / 64; ++w) r = s_k[w] > r ? s_k[w] : r;
        if (r != 0ull) atomicMax(keys + b, r);
    }
}

__global__ void sample_clear_kernel(unsigned long long* __restrict__ keys, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) keys[i] = 0ull;
}

// key -> token index; a row whose every score was NaN (key 0) gets token 0
__global__ void sample_finish_kernel(unsigned long long* __restrict__ keys, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const unsigned long long k = keys[i];
        const int64_t tok = k == 0ull ? 0 : (int64_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        reinterpret_cast<int64_t*>(keys)[i] = tok;
    }
}

}  // namespace

hipError_t launch_add_rms_norm(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                               int32_t n_tokens, int32_t hidden, float eps, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    const int chunks = hidden / 8;
    const int lpr = chunks <= 64 ? 64 : (chunks <= 128 ? 128 : 256);
    const int nc = (chunks + lpr - 1) / lpr;
    const int rpb = 256 / lpr;
    const unsigned blocks = (unsigned)(((int64_t)n_tokens + rpb - 1) / rpb);
#define PKV_RMS_CASE(N)                                                                                            \
    case N:                                                                                                        \
        hipLaunchKernelGGL(add_rms_norm_kernel<N>, dim3(blocks), dim3(256), 0, stream, (const uint16_t*)x,        \
                           (const uint16_t*)residual, (const uint16_t*)gamma, (uint16_t*)y, (uint16_t*)residual_out, \
                           n_tokens, hidden, lpr, eps);                                                            \
        break;
    switch (nc) {
        PKV_RMS_CASE(1)
        PKV_RMS_CASE(2)
        PKV_RMS_CASE(3)
        PKV_RMS_CASE(4)
        PKV_RMS_CASE(5)
        PKV_RMS_CASE(6)
        PKV_RMS_CASE(7)
        PKV_RMS_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef PKV_RMS_CASE
    return hipGetLastError();
}

hipError_t launch_silu_and_mul(const void* x, int64_t x_row_stride, void* out, int64_t out_row_stride,
                               int32_t n_tokens, int32_t inter, hipStream_t stream) {
    if ((int64_t)n_tokens * (inter / 8) == 0) return hipSuccess;
    // one workgroup per row at a time, rows strided over the grid
    const int64_t blocks = n_tokens < 16384 ? n_tokens : 16384;
    hipLaunchKernelGGL(silu_and_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)x,
                       x_row_stride, (uint16_t*)out, out_row_stride, n_tokens, inter);
    return hipGetLastError();
}

hipError_t launch_sample_gumbel(const void* logits, int64_t row_stride, int32_t logits_f32,
                                const float* temperatures, const float* noise, int64_t noise_row_stride,
                                uint64_t seed, uint64_t offset, int64_t* tokens, int32_t num_rows, int32_t vocab,
                                hipStream_t stream) {
    if (num_rows == 0) return hipSuccess;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint32_t o0 = (uint32_t)offset, o1 = (uint32_t)(offset >> 32);
    // Enough workgroups to fill the chip (about 2048), at least 16 chunks of 8 per lane pass.
    const int64_t n8 = vocab >> 3;
    int64_t parts = (2048 + num_rows - 1) / num_rows;
    const int64_t max_parts = n8 / (16 * kSampThreads) > 1 ? n8 / (16 * kSampThreads) : 1;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    const int64_t grid = (int64_t)num_rows * parts;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(tokens);
    const unsigned nb = (unsigned)((num_rows + 255) / 256);
    hipLaunchKernelGGL(sample_clear_kernel, dim3(nb), dim3(256), 0, stream, keys, num_rows);
    if (logits_f32)
        hipLaunchKernelGGL(sample_gumbel_kernel<true>, dim3((unsigned)grid), dim3(kSampThreads), 0, stream, logits,
                           row_stride, temperatures, noise, noise_row_stride, k0, k1, o0, o1, keys, vocab,
                           (int32_t)parts);
    else
        hipLaunchKernelGGL(sample_gumbel_kernel<false>, dim3((unsigned)grid), dim3(kSampThreads), 0, stream, logits,
                           row_stride, temperatures, noise, noise_row_stride, k0, k1, o0, o1, keys, vocab,
                           (int32_t)parts);
    hipLaunchKernelGGL(sample_finish_kernel, dim3(nb), dim3(256), 0, stream, keys, num_rows);
    return hipGetLastError();
}

}  // namespace pkv
