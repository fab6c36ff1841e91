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
//   * Split-K: a workgroup owns (sequence b, kv head g, split s) and covers
//     `split_blocks` consecutive logical 256-token blocks; the whole GQA group
//     of q heads is served by one read of K/V.
//   * Inside the workgroup each of the 4 waves streams its own 16-key slice
//     of every 64-key quarter block and keeps its own online-softmax state, so
//     the main loop has no workgroup barrier at all.  Loads run ahead in a
//     ring of registers, so a wave keeps several 8 KB chunks of K/V in flight
//     while it computes.
//   * QK^T on MFMA (v_mfma_f32_16x16x32_bf16): A = 16 keys x 32 dims straight
//     from global memory, B = the group's q vectors (columns >= G are zero).
//   * The running max is rescaled lazily: the reference max only moves when a
//     chunk's max exceeds it by more than 2^8 (the weights stay <= 256 in
//     fp32), so the common chunk needs no cross-lane max exchange.  The result
//     is exact: numerator and denominator share the reference.
//   * Probabilities reach the PV lanes through a wave-private LDS slot; PV runs
//     on the vector ALU with each lane owning 8 dims of 4 keys (fully
//     coalesced 256-byte V rows).
//   * Keys at or past the context length and keys of a block id outside the
//     pool are masked before the exponential and their V rows replaced by
//     zeros, so nothing outside the context can reach the output.
//   * The 4 waves merge once at the end; the split's (m, l, O) go to a
//     caller-owned fp32 workspace and a second kernel merges the splits of
//     each (b, h) in split order (deterministic).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {
constexpr int kDecThreads = 256;
#ifndef PKV_DECODE_SPLIT
#define PKV_DECODE_SPLIT 4
#endif
constexpr int kMaxSplitBlocks = PKV_DECODE_SPLIT;   // blocks per split-K work item (at most)
constexpr int kTargetItems = 4096;
constexpr float kLazyMax = 8.0f;   // log2 headroom of the lazy reference max
// Tuning (measured on MI355X, Qwen3-8B decode workload): a ring of 3 chunks of 16
// keys per wave at 2 waves/SIMD, 4-block splits, launched split-index-slowest.
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 3
#endif
#ifndef PKV_DECODE_OCC
#define PKV_DECODE_OCC 2
#endif
#ifndef PKV_DECODE_CHUNK
#define PKV_DECODE_CHUNK 16
#endif
constexpr int kDepth = PKV_DECODE_DEPTH;   // register ring: chunks in flight + the one computed
constexpr int kCK = PKV_DECODE_CHUNK;      // keys per wave per chunk (16 or 32)
constexpr int kTiles = kCK / 16;           // 16-key MFMA tiles per chunk
constexpr int kRounds = kBlockSize / (4 * kCK);  // chunks per 256-token block per wave
constexpr int kOcc = PKV_DECODE_OCC;       // waves per SIMD the register budget is sized for

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

struct Chunk {
    u32x4 k[kTiles][4];   // MFMA A operand: key 16*t + lane%16, dims 8*(lane/16) + 32*st
    u32x4 v[kCK / 4];     // PV: key lane/16 + 4*i, dims 8*(lane%16)
};
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
__global__ void __launch_bounds__(kDecThreads, kOcc) decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t hq, int32_t hkv, int64_t num_blocks, float scale_log2, int32_t split_blocks, int32_t max_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
    static_assert(G >= 1 && G <= 16, "GQA group must fit the 16 MFMA columns");
    // Split index slowest: every sequence's first splits are dispatched before any
    // later split, so the empty workgroups past short contexts trail the real work.
    const int g = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + kBlockSize - 1) / kBlockSize;
    const int blk0 = s * split_blocks;
    if (blk0 >= nblk) return;
    const int nb = min(split_blocks, nblk - blk0);   // blocks of this split (<= 16)
    const int nchunks = nb * kRounds;                // chunks of 4*kCK keys; this wave owns kCK of each

    __shared__ float s_p[4][kCK][G];                 // per-wave probabilities of one chunk
    __shared__ float s_m[4][G], s_l[4][G];           // per-wave final max / sum
    __shared__ float s_o[4][G][kHeadDim];            // per-wave final numerators

    const int64_t row = (int64_t)hkv * kHeadDim;    // elements between consecutive cache rows

    // Block ids of this split, one per lane (lanes >= nb hold -1).
    int my_blk = -1;
    if (lane < nb) {
        const int32_t id = block_table[(int64_t)b * max_blocks + blk0 + lane];
        my_blk = (id >= 0 && (int64_t)id < num_blocks) ? id : -1;
    }

    // B operand: q of head g*G + col, dims 8*(lane/16) + 32*st .. +7, zero for col >= G.
    const int col = lane & 15, grp = lane >> 4;
    bf16x8 qb[4];
    {
        const bool on = col < G;
        const uint16_t* qr = q + ((int64_t)b * hq + (int64_t)g * G + (on ? col : 0)) * kHeadDim + 8 * grp;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 w = on ? ldg128(qr + 32 * st) : u32x4{0u, 0u, 0u, 0u};
            qb[st] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Chunk j covers keys kCK*(4*(j%kRounds) + wave) .. +kCK-1 of block blk0 + j/kRounds.
    auto block_of = [&](int j) { return __builtin_amdgcn_readlane(my_blk, j / kRounds); };
    auto chunk_row0 = [&](int j) { return kCK * (4 * (j % kRounds) + wave); };
    auto load = [&](Chunk& c, int j) {
        const int id = block_of(j);
        const int64_t phys = id < 0 ? 0 : id;
        const int64_t r0 = phys * kBlockSize + chunk_row0(j);   // first cache row of the chunk
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const uint16_t* kp = k_cache + (r0 + 16 * t + col) * row + (int64_t)g * kHeadDim + 8 * grp;
#pragma unroll
            for (int st = 0; st < 4; ++st)
                c.k[t][st] = ldg128(kp + 32 * st);
        }
        __builtin_amdgcn_sched_barrier(0);   // K before V: the scores wait only for K
        const uint16_t* vp = v_cache + (r0 + grp) * row + (int64_t)g * kHeadDim + 8 * col;
#pragma unroll
        for (int i = 0; i < kCK / 4; ++i)
            c.v[i] = ldg128(vp + (int64_t)(4 * i) * row);
    };

    float m_head[G];                  // lazy reference max per head (wave-uniform)
#pragma unroll
    for (int h = 0; h < G; ++h) m_head[h] = -INFINITY;
    float l_run = 0.f;                // lanes col < G: running sum of their keys' weights
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    auto compute = [&](const Chunk& c, int j) {
        const int key0 = (blk0 + j / kRounds) * kBlockSize + chunk_row0(j);
        const int id = block_of(j);
        // ---- scores: tile t holds 16 keys x 16 columns
        float sv[kTiles][4];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c.k[t][st]), qb[st], sc, 0, 0,
                                                             0);
            // sc[r] = score of key key0 + 16t + 4*grp + r for column col
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * t + 4 * grp + r;
                sv[t][r] = (id >= 0 && key < ctx) ? sc[r] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, sv[t][r]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // ---- lazy reference: a head's reference moves only when this chunk's max
        // exceeds it by more than 2^kLazyMax.  Branch-free: the per-head maxima are
        // read into wave-uniform registers and alpha is 1 when nothing moves.
        float ref = 0.f, my_alpha = 1.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), h));
            const float mold = m_head[h];
            const float mn = (mh > mold + kLazyMax) ? mh : mold;
            const float alpha = mold == -INFINITY ? 0.f : exp2f(mold - mn);
            m_head[h] = mn;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            if (col == h) {
                my_alpha = alpha;
                ref = mn == -INFINITY ? 0.f : mn;
            }
        }
        l_run *= my_alpha;
        if (col < G) {
#pragma unroll
            for (int t = 0; t < kTiles; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = exp2f(sv[t][r] - ref);
                    l_run += p;
                    s_p[wave][16 * t + 4 * grp + r][col] = p;
                }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- PV: this lane owns dims 8*col .. +7 of keys grp + 4*i
#pragma unroll
        for (int i = 0; i < kCK / 4; ++i) {
            const int kl = grp + 4 * i;
            const bool live = id >= 0 && (key0 + kl) < ctx;
            const u32x4 w = live ? c.v[i] : u32x4{0u, 0u, 0u, 0u};
            float vv[8];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                vv[2 * x] = bf16lo(w[x]);
                vv[2 * x + 1] = bf16hi(w[x]);
            }
            float p[G];
#pragma unroll
            for (int h = 0; h < G; ++h) p[h] = s_p[wave][kl][h];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p[h], vv[e], acc[h][e]);
        }
        __builtin_amdgcn_wave_barrier();   // s_p is rewritten by the next chunk
    };

    // ---- main loop: kDepth - 1 chunks in flight while one is computed.  Every
    // prefetch is issued unconditionally (past the end it re-reads the last
    // chunk, an L2 hit), so the number of loads in flight is the same on every
    // path and each wait covers exactly the chunk about to be used.
    Chunk ring[kDepth];
    // The trip count is padded to a multiple of the ring depth; padded chunks
    // map to block slots >= nb whose id is -1, so all their keys are masked.
    const int ntrip = (nchunks + kDepth - 1) / kDepth * kDepth;
#pragma unroll
    for (int u = 0; u < kDepth - 1; ++u) load(ring[u], min(u, nchunks - 1));
    for (int j0 = 0; j0 < ntrip; j0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int j = j0 + u;
            load(ring[(u + kDepth - 1) % kDepth], min(j + kDepth - 1, nchunks - 1));
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this chunk's math
            compute(ring[u], j);
        }
    }

    // ---- merge the 4 waves: per head (m, l, O)
    float lsum = l_run;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (lane < G) {
        float mh = m_head[0];
#pragma unroll
        for (int h = 1; h < G; ++h) mh = (lane == h) ? m_head[h] : mh;
        s_m[wave][lane] = mh;
        s_l[wave][lane] = lsum;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[h][e];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[h][e] = v;
        }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_o[wave][h][8 * col + e] = acc[h][e];
    }
    __syncthreads();
    const int64_t bh0 = (int64_t)b * hq + (int64_t)g * G;
    for (int x = tid; x < G * kHeadDim; x += kDecThreads) {
        const int h = x / kHeadDim, d = x % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
        const float ref = M == -INFINITY ? 0.f : M;
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = exp2f(s_m[w][h] - ref);
            o = fmaf(s_o[w][h][d], f, o);
            L = fmaf(s_l[w][h], f, L);
        }
        part_o[((bh0 + h) * max_splits + s) * kHeadDim + d] = o;
        if (d == 0) {
            float* ml = part_ml + ((bh0 + h) * max_splits + s) * 2;
            ml[0] = M;
            ml[1] = L;
        }
    }
}

// One workgroup of 128 threads per (b, h): merge the splits in order.  The
// splits are taken 128 at a time: their (m, l) pairs are loaded by the whole
// workgroup at once and their weights exp2(m_s - M) staged in LDS, then each
// thread (one output dim) sums its column of partial outputs with the loads
// unrolled, so a long context (many splits) costs a few memory latencies, not
// one per split.  The sums run over s in increasing order, as a serial merge.
__global__ void __launch_bounds__(128) decode_combine_kernel(const int32_t* __restrict__ context_lens,
                                                             int32_t max_blocks, int32_t hq, int32_t split_blocks,
                                                             int32_t max_splits, const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             uint16_t* __restrict__ o) {
    __shared__ float s_w[128];
    __shared__ float s_l[128];
    __shared__ float s_red[2];
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + kBlockSize - 1) / kBlockSize;
    const int ns = (nblk + split_blocks - 1) / split_blocks;
    const int64_t bh = (int64_t)b * hq + h;
    const float* ml = part_ml + bh * max_splits * 2;
    const float* po = part_o + bh * max_splits * kHeadDim + d;

    float M = -INFINITY;
    for (int s = d; s < ns; s += 128) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    if ((d & 63) == 0) s_red[d >> 6] = M;
    __syncthreads();
    M = fmaxf(s_red[0], s_red[1]);
    const float ref = M == -INFINITY ? 0.f : M;

    float L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 128) {
        const int n = ns - s0 < 128 ? ns - s0 : 128;
        if (d < n) {
            s_w[d] = exp2f(ml[2 * (s0 + d)] - ref);
            s_l[d] = ml[2 * (s0 + d) + 1];
        }
        __syncthreads();
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            const float w = s_w[i];
            L = fmaf(s_l[i], w, L);
            acc = fmaf(po[(int64_t)(s0 + i) * kHeadDim], w, acc);
        }
        __syncthreads();
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
    dim3 grid(a.hkv, a.num_seqs, ms);
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
