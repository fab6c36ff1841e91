// attn_decode.hip -- single-token paged decode attention (gfx950).
//
// "3.3 Model skeleton and core operators", section 7.2 and "nano-vllm code
// walkthrough", "Decode Stage": one new query per sequence attends the first
// context_lens[b] keys of its paged cache, read through block_table; q head h
// uses kv head h / (Hq/Hkv) ("Nano-vLLM 源码解读 #17 注意力层", section 3).
// The softmax is the exact online form of the same page's section 5.2: partial
// results (m, l, O) over pieces of the context are merged by rescaling with
// exp(m_old - m_new).
//
// Design (HBM-bound: every K/V byte of the context is read once):
//   * Split-K: a workgroup owns (sequence b, kv head g, split s) and walks
//     `split_blocks` consecutive logical 256-token blocks.  One block-table
//     lookup per block; K/V rows of head g are 256 contiguous bytes, rows
//     Hkv*256 bytes apart.
//   * The whole GQA group of q heads is served by the one K/V read.
//   * QK^T on MFMA (v_mfma_f32_16x16x32_bf16): A = 16 keys x 32 dims straight
//     from global memory, B = the group's q vectors (columns >= G are zero).
//   * Softmax over the 256 keys of a block in LDS, online across blocks.
//   * PV on the vector ALU: each lane owns 8 dims of 16 keys; its 16-byte V
//     loads are fully coalesced 256-byte rows.
//   * Keys at or past the context length, and keys of a block id outside the
//     pool, are masked before the exponential and their V rows are replaced by
//     zeros, so nothing outside the context can reach the output.
//   * Partials (m, l, O) go to a caller-owned fp32 workspace; a second kernel
//     merges the splits of each (b, h) in split order (deterministic).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {
constexpr int kDecThreads = 256;
constexpr int kMaxSplitBlocks = 16;
constexpr int kTargetItems = 4096;

struct Workspace {
    float* part_o;   // [B][Hq][S][128]
    float* part_ml;  // [B][Hq][S][2]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Workspace carve(void* base, int32_t B, int32_t hq, int32_t max_splits) {
    Workspace w;
    const size_t o_bytes = align256((size_t)B * hq * max_splits * kHeadDim * sizeof(float));
    w.part_o = (float*)base;
    w.part_ml = (float*)((char*)base + o_bytes);
    return w;
}
}  // namespace

int decode_split_blocks(int32_t num_seqs, int32_t hkv, int32_t max_blocks) {
    int sb = kMaxSplitBlocks;
    while (sb > 1) {
        const int64_t items = (int64_t)num_seqs * hkv * ((max_blocks + sb - 1) / sb);
        if (items >= kTargetItems) break;
        sb >>= 1;
    }
    return sb;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t max_blocks) {
    const int sb = decode_split_blocks(num_seqs, hkv, max_blocks);
    const int64_t ms = (max_blocks + sb - 1) / sb;
    const size_t o_bytes = align256((size_t)num_seqs * hq * ms * kHeadDim * sizeof(float));
    const size_t ml_bytes = align256((size_t)num_seqs * hq * ms * 2 * sizeof(float));
    return o_bytes + ml_bytes;
}

template <int G>
__global__ void __launch_bounds__(kDecThreads, 2) decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t hq, int32_t hkv, int64_t num_blocks, float scale_log2, int32_t split_blocks, int32_t max_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
    static_assert(G >= 1 && G <= 16, "GQA group must fit the 16 MFMA columns");
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + kBlockSize - 1) / kBlockSize;
    const int blk0 = s * split_blocks;
    if (blk0 >= nblk) return;
    const int blk1 = min(blk0 + split_blocks, nblk);

    __shared__ float s_p[kBlockSize][G];          // scores, then probabilities, of one block
    __shared__ float s_red[4][G];                  // per-wave reduction slots
    __shared__ float s_o[16][kHeadDim + 4];        // final cross-key-group reduction

    const int64_t row = (int64_t)hkv * kHeadDim;  // elements between consecutive cache rows

    // B operand: q of head g*G + col, dims 8*(lane/16) + 32*st .. +7, zero for col >= G.
    const int col = lane & 15;
    bf16x8 qb[4];
    {
        const bool on = col < G;
        const uint16_t* qr = q + ((int64_t)b * hq + (int64_t)g * G + (on ? col : 0)) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 w = on ? ldg128(qr + 32 * st) : u32x4{0u, 0u, 0u, 0u};
            qb[st] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // PV ownership: dims 8*sub .. +7 of keys kg + 16*i.
    const int sub = tid & 15, kg = tid >> 4;
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    float m_run[G], l_part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_part[h] = 0.f;
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        const int32_t phys_raw = block_table[(int64_t)b * max_blocks + blk];
        const bool valid = phys_raw >= 0 && (int64_t)phys_raw < num_blocks;
        const int64_t phys = valid ? phys_raw : 0;
        const int nkeys = valid ? min(kBlockSize, ctx - blk * kBlockSize) : 0;
        const uint16_t* kb = k_cache + phys * kBlockSize * row + (int64_t)g * kHeadDim;
        const uint16_t* vb = v_cache + phys * kBlockSize * row + (int64_t)g * kHeadDim;

        // Issue the V loads of this block first: they do not depend on the softmax.
        u32x4 vreg[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) vreg[i] = ldg128_stream(vb + (int64_t)(kg + 16 * i) * row + 8 * sub);

        // QK^T: wave w scores keys 64w .. 64w+63 as 4 tiles of 16.
        u32x4 kreg[4][4];
#pragma unroll
        for (int tl = 0; tl < 4; ++tl)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kreg[tl][st] = ldg128_stream(kb + (int64_t)(64 * wave + 16 * tl + (lane & 15)) * row +
                                             8 * (lane >> 4) + 32 * st);
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[tl][st]), qb[st], c, 0, 0,
                                                            0);
            // c[r] = score of key 64w + 16tl + 4*(lane/16) + r for column lane%16.
            if (col < G) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = 64 * wave + 16 * tl + 4 * (lane >> 4) + r;
                    s_p[key][col] = key < nkeys ? c[r] * scale_log2 : -INFINITY;
                }
            }
        }
        __syncthreads();

        // Block max per head (thread tid owns key tid), then the new running max.
        float sv[G], bm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sv[h] = s_p[tid][h];
            bm[h] = wave_max(sv[h]);
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) s_red[wave][h] = bm[h];
        }
        __syncthreads();
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mb = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
            const float mn = fmaxf(m_run[h], mb);
            const float ref = mn == -INFINITY ? 0.f : mn;  // all keys masked so far: keep zeros
            alpha[h] = exp2f(m_run[h] - ref);
            const float p = exp2f(sv[h] - ref);
            l_part[h] = l_part[h] * alpha[h] + p;
            s_p[tid][h] = p;
            m_run[h] = mn;
        }
        __syncthreads();

        // PV: acc[h][e] = alpha * acc + sum over owned keys of p * v.
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kg + 16 * i;
            const u32x4 w = key < nkeys ? vreg[i] : u32x4{0u, 0u, 0u, 0u};
            float vv[8];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                vv[2 * x] = bf16lo(w[x]);
                vv[2 * x + 1] = bf16hi(w[x]);
            }
            float p[G];
#pragma unroll
            for (int h = 0; h < G; ++h) p[h] = s_p[key][h];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p[h], vv[e], acc[h][e]);
        }
        __syncthreads();  // s_p is rewritten by the next block
    }

    // Merge the 16 key groups of every head and write the split's partials.
    const int64_t bh0 = (int64_t)b * hq + (int64_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float lw = wave_sum(l_part[h]);
        if (lane == 0) s_red[wave][h] = lw;
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[kg][8 * sub + e] = acc[h][e];
        __syncthreads();
        if (tid < kHeadDim) {
            float o = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) o += s_o[j][tid];
            part_o[((bh0 + h) * max_splits + s) * kHeadDim + tid] = o;
        }
        if (tid == 0) {
            float* ml = part_ml + ((bh0 + h) * max_splits + s) * 2;
            ml[0] = m_run[h];
            ml[1] = (s_red[0][h] + s_red[1][h]) + (s_red[2][h] + s_red[3][h]);
        }
        __syncthreads();
    }
}

// One workgroup of 128 threads per (b, h): merge the splits in order.
__global__ void __launch_bounds__(128) decode_combine_kernel(const int32_t* __restrict__ context_lens,
                                                             int32_t max_blocks, int32_t hq, int32_t split_blocks,
                                                             int32_t max_splits, const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             uint16_t* __restrict__ o) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + kBlockSize - 1) / kBlockSize;
    const int ns = (nblk + split_blocks - 1) / split_blocks;
    const int64_t bh = (int64_t)b * hq + h;
    const float* ml = part_ml + bh * max_splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    const float ref = M == -INFINITY ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = exp2f(ml[2 * s] - ref);
        L = fmaf(ml[2 * s + 1], w, L);
        acc = fmaf(part_o[(bh * max_splits + s) * kHeadDim + d], w, acc);
    }
    const float r = L > 0.f ? acc / L : 0.f;
    o[bh * kHeadDim + d] = __builtin_bit_cast(uint16_t, (bf16)r);
}

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    const int G = a.hq / a.hkv;
    const int sb = decode_split_blocks(a.num_seqs, a.hkv, a.max_blocks);
    const int ms = (a.max_blocks + sb - 1) / sb;
    Workspace w = carve(a.workspace, a.num_seqs, a.hq, ms);
    dim3 grid(ms, a.hkv, a.num_seqs);
#define PKV_DECODE_CASE(GG)                                                                                       \
    case GG:                                                                                                      \
        hipLaunchKernelGGL(decode_split_kernel<GG>, grid, dim3(kDecThreads), 0, stream, (const uint16_t*)a.q,     \
                           (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.context_lens, a.block_table, \
                           a.max_blocks, a.hq, a.hkv, a.num_blocks, a.scale_log2, sb, ms, w.part_o, w.part_ml);   \
        break;
    switch (G) {
        PKV_DECODE_CASE(1)
        PKV_DECODE_CASE(2)
        PKV_DECODE_CASE(4)
        PKV_DECODE_CASE(8)
        PKV_DECODE_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef PKV_DECODE_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.hq, a.num_seqs), dim3(kHeadDim), 0, stream, a.context_lens,
                       a.max_blocks, a.hq, sb, ms, w.part_o, w.part_ml, (uint16_t*)a.o);
    return hipGetLastError();
}

}  // namespace pkv
