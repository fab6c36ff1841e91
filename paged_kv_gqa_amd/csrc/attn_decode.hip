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
//   * Split-K: a workgroup owns (sequence b, a group of 4 kv heads, split s)
//     and covers up to 8 consecutive logical 256-token blocks (down to 64 keys
//     for short contexts at small batches).  Each of its 4
//     waves owns one kv head and streams the whole split for it, so the waves
//     read adjacent 256-byte pieces of every 2 KiB cache row (1 KiB per key
//     and workgroup), each wave keeps its own online-softmax state and there
//     is no barrier and no cross-wave merge.  The whole GQA group of q heads
//     of a kv head is served by one read of its K/V.
//   * A one-workgroup kernel first sorts the split items by size (counting
//     sort), and workgroups take them largest first: with contexts of very
//     different lengths the last workgroups to start are the smallest, so the
//     tail stays short.  A grid that fits the chip at once skips the sort.
//   * Loads run one 16-key chunk ahead in a register ring.  V is read with
//     non-temporal loads: each V load instruction consumes whole cache lines
//     that nothing reads again, so keeping them only displaces other lines.  K
//     goes through the caches as usual: a K line is consumed by two load
//     instructions (dims 0-63 and 64-127 of a row), and streaming it made the
//     second miss.  8B batch 1782 -> 1634 us, 0.6B batch 197 -> 179 us (both
//     streamed: 1718 and 182 us), outputs unchanged.
//   * Both products on MFMA.  Scores: v_mfma_f32_16x16x32_bf16 with A = 16 keys
//     x 32 dims straight from global memory and B = the group's q vectors
//     (columns >= G are zero); a lane then holds 4 keys of one head column.
//     That layout is already the B operand of P V on v_mfma_f32_16x16x16_bf16,
//     so the probabilities never leave registers; the A operand V^T comes from
//     the chunk's V rows staged in a wave-private LDS tile and read back with
//     the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//   * Every softmax statistic is lane-local (a lane's column is one head).  The
//     running max is rescaled lazily: the reference only moves when a chunk's
//     max exceeds it by more than 2^8 (the weights stay <= 256 in fp32).  The
//     result is exact: numerator and denominator share the reference.
//   * Keys at or past the context length and keys of a block id outside the
//     pool are masked before the exponential and their V rows replaced by
//     zeros, so nothing outside the context can reach the output.
//   * Each wave writes its split's (m, l, O) to a caller-owned fp32 workspace
//     and a second kernel merges the splits of each (b, h) in split order
//     (deterministic).
//   * The decode step (launch_decode_step) runs QK-Norm + RoPE + scatter inside
//     the split kernel: each workgroup normalises and rotates its own q rows,
//     and the one holding a row's last chunk computes the new token's k' and v,
//     stores them at the row's slot and patches them into that chunk.
#include <mutex>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {
constexpr int kDecThreads = 256;
// Tuning (measured on MI355X, Qwen3-8B and 0.6B decode workloads): splits of up
// to 8 blocks, shortened one block at a time while the batch would have fewer
// than ~1400 split items, then halved to 8 and 4 chunks of 16 keys while the grid
// fits the chip at once and no sequence gets more than 128 splits; a ring of 2 chunks of 16 keys per wave, 2
// waves per SIMD.  Longer splits amortise each workgroup's pipeline fill; deeper
// rings did not pay, not even at a batch of one, where a workgroup's time is its
// chain of chunks (each chunk's V staging, scores, softmax and P V wait on one
// another), which shorter splits cut instead.
#ifndef PKV_DECODE_SPLIT
#define PKV_DECODE_SPLIT 8
#endif
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2
#endif
#ifndef PKV_DECODE_OCC
#define PKV_DECODE_OCC 2
#endif
constexpr int kMaxSplitBlocks = PKV_DECODE_SPLIT;   // blocks per split-K work item (at most)
#ifndef PKV_DECODE_TARGET
#define PKV_DECODE_TARGET 1400
#endif
constexpr int kTargetItems = PKV_DECODE_TARGET;
constexpr float kLazyMax = 8.0f;   // log2 headroom of the lazy reference max
constexpr int kDepth = PKV_DECODE_DEPTH;   // register ring: chunks in flight + the one computed
constexpr int kCK = 16;                    // keys per wave per chunk (one 16-key MFMA tile)
constexpr int kOcc = PKV_DECODE_OCC;       // waves per SIMD the register budget is sized for
#ifndef PKV_DECODE_MIN_CHUNKS
#define PKV_DECODE_MIN_CHUNKS 4
#endif
constexpr int kMinSplitChunks = PKV_DECODE_MIN_CHUNKS;   // shortest split (16-key chunks)
#ifndef PKV_DECODE_MAX_SPLITS
#define PKV_DECODE_MAX_SPLITS 128
#endif
constexpr int kMaxSplits = PKV_DECODE_MAX_SPLITS;        // splits per sequence the sub-block lengths allow
constexpr int kResidentItems = 512;                      // split workgroups the chip holds at once (2 per CU)
constexpr int64_t kMaxGridYZ = 65535;                    // largest y / z extent of a launch grid

struct Workspace {
    float* part_o;   // [B][Hq][S][128]
    float* part_ml;  // [B][Hq][S][2]
    int32_t* work;   // [S][B] split items b * S + s, largest first (dispatch order)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Workspace carve(void* base, int32_t B, int32_t hq, int32_t max_splits) {
    Workspace w;
    const size_t o_bytes = align256((size_t)B * hq * max_splits * kHeadDim * sizeof(float));
    const size_t ml_bytes = align256((size_t)B * hq * max_splits * 2 * sizeof(float));
    w.part_o = (float*)base;
    w.part_ml = (float*)((char*)base + o_bytes);
    w.work = (int32_t*)((char*)base + o_bytes + ml_bytes);
    return w;
}

typedef short short4_t __attribute__((ext_vector_type(4)));
struct Chunk {
    u32x4 k[4];           // score A operand: key lane%16, dims 8*(lane/16) + 32*st
    u32x4 v[kCK / 4];     // V rows: key lane/16 + 4*i, dims 8*(lane%16) (staged through LDS)
};
}  // namespace

// Split length in 16-key chunks: whole blocks (8 down to 1) while the batch would
// have fewer than kTargetItems split items; then halved (8, 4 chunks) while the
// halved grid still fits the chip at once and no sequence gets more than
// kMaxSplits splits for the merge to add -- short contexts at small batches, where
// one workgroup's chain of chunks sets the time.
int decode_split_chunks(int32_t num_seqs, int32_t hkv, int32_t max_blocks) {
    constexpr int kCPB = kBlockSize / kCK;
    const int64_t max_chunks = (int64_t)max_blocks * kCPB;
    auto items = [&](int sc) { return (int64_t)num_seqs * ((hkv + 3) / 4) * ((max_chunks + sc - 1) / sc); };
    int sc = kMaxSplitBlocks * kCPB;
    while (sc > kCPB && items(sc) < kTargetItems) sc -= kCPB;
    while (sc > kMinSplitChunks && items(sc) < kTargetItems && items(sc / 2) <= kResidentItems &&
           (max_chunks + sc / 2 - 1) / (sc / 2) <= kMaxSplits)
        sc /= 2;
    return sc;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t max_blocks) {
    const int sc = decode_split_chunks(num_seqs, hkv, max_blocks);
    const int64_t ms = ((int64_t)max_blocks * (kBlockSize / kCK) + sc - 1) / sc;
    // the split grid is (kv head groups, num_seqs, ms): its y and z extents are at most 65535
    if (num_seqs > kMaxGridYZ || ms > kMaxGridYZ) return 0;
    const unsigned __int128 rows = (unsigned __int128)num_seqs * (unsigned)hq * (uint64_t)ms;
    if (rows * (kHeadDim + 2) * sizeof(float) > ((unsigned __int128)1 << 48)) return 0;   // beyond any device
    const size_t o_bytes = align256((size_t)rows * kHeadDim * sizeof(float));
    const size_t ml_bytes = align256((size_t)rows * 2 * sizeof(float));
    const size_t work_bytes = align256((size_t)num_seqs * ms * sizeof(int32_t));
    return o_bytes + ml_bytes + work_bytes;
}

// QK-Norm + RoPE of one 128-element head vector held by the four lanes of a
// column (lanes col + 16 grp, grp = 0..3) in the decode split kernel's operand
// layout: x[st] holds dims 8 grp + 32 st .. +7, so the rotation partner of piece
// st (dims +-64) is piece st ^ 2 of the same lane.  The arithmetic is that of the
// standalone QK-Norm + RoPE kernel (rope.hip, norm_rope_apply), in the same order:
// the per-piece sums of squares are combined along the same tree as its 16-lane
// butterfly (its lane grp + 4 st; partners xor 8, 4, 2, 1 are here pieces st ^ 2,
// st ^ 1 and lanes xor 32, xor 16), so the results are bit-identical.
__device__ __forceinline__ void norm_rope_cols(const u32x4 (&x)[4], const uint16_t* __restrict__ gamma,
                                               const float* __restrict__ trow, float eps, int grp, u32x4 (&out)[4]) {
    float xa[4][8];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            xa[st][2 * w] = bf16lo(x[st][w]);
            xa[st][2 * w + 1] = bf16hi(x[st][w]);
        }
    float ssp[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += xa[st][e] * xa[st][e];
        ssp[st] = ss;
    }
    float t[4], u[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) t[st] = ssp[st] + ssp[st ^ 2];
#pragma unroll
    for (int st = 0; st < 4; ++st) u[st] = t[st] + t[st ^ 1];
    float ss = u[0];
    ss += __shfl_xor(ss, 32, 64);
    ss += __shfl_xor(ss, 16, 64);
    const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const float* cs = trow + 8 * grp + 32 * (st & 1);
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + 64);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 68);
        float cv[8], sv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cv[i] = c0[i];
            cv[4 + i] = c1[i];
            sv[i] = s0[i];
            sv[4 + i] = s1[i];
        }
        const u32x4 go = ldg128(gamma + 8 * grp + 32 * st);
        const u32x4 gp = ldg128(gamma + 8 * grp + 32 * (st ^ 2));
        // The sign as a register value, as in the standalone kernel (where it depends
        // on the lane): a constant here would let the compiler fold it and fuse the
        // other product into the add, which rounds differently.
        float sgn;
        asm("v_mov_b32 %0, %1" : "=v"(sgn) : "v"(st < 2 ? -1.0f : 1.0f));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float o2[2];
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const int e = 2 * w + hlf;
                const float ga = hlf ? bf16hi(go[w]) : bf16lo(go[w]);
                const float gb = hlf ? bf16hi(gp[w]) : bf16lo(gp[w]);
                const float ya = xa[st][e] * r * ga;
                const float yb = xa[st ^ 2][e] * r * gb;
                o2[hlf] = ya * cv[e] + sgn * (yb * sv[e]);
            }
            out[st][w] = pack_bf16x2(o2[0], o2[1]);
        }
    }
}

template <int G, bool kStep>
__global__ void __launch_bounds__(kDecThreads, kOcc) decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t hq, int32_t hkv, int64_t num_blocks, float scale_log2, int32_t split_chunks, int32_t max_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml, const int32_t* __restrict__ work, StepArgs sa) {
    static_assert(G >= 1 && G <= 16, "GQA group must fit the 16 MFMA columns");
    // Dispatch order: split items by decreasing size (full splits first), so the
    // smallest pieces of work come last and the tail stays short.  Without an
    // order (a grid small enough to run all at once) the item is the grid position.
    const int item = work ? work[(int64_t)blockIdx.z * gridDim.y + blockIdx.y]
                          : (int)blockIdx.y * max_splits + (int)blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Each wave owns one kv head of a group of 4 (the 4 waves read adjacent 256-byte
    // pieces of every 2 KiB cache row) and streams the whole split for it.
    const int g = 4 * blockIdx.x + wave, b = item / max_splits, s = item - b * max_splits;
    if (g >= hkv) return;

    // The split covers the context's 16-key chunks c0 .. c0 + nchunks - 1, all for
    // this wave; they lie in blocks blk0 .. blk0 + nb - 1.  The table entries the
    // split can touch follow from s alone, so they are loaded beside the context
    // length instead of after it (one memory round trip less before the first K/V).
    constexpr int kCPB = kBlockSize / kCK;           // chunks per block
    const int c0 = s * split_chunks;
    const int blk0 = c0 / kCPB;
    int raw_blk = -1;
    if (lane < (split_chunks + kCPB - 1) / kCPB + 1 && blk0 + lane < max_blocks)
        raw_blk = block_table[(int64_t)b * max_blocks + blk0 + lane];
    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nchk = (ctx + kCK - 1) / kCK;
    // In a step, split 0 of every row also writes the row's q' (and, with an empty
    // context, stores the new token), so it runs even when it has no keys.
    if (c0 >= nchk && !(kStep && s == 0)) return;
    const int nchunks = c0 < nchk ? min(split_chunks, nchk - c0) : 0;
    const int nb = nchunks > 0 ? (c0 + nchunks - 1) / kCPB - blk0 + 1 : 0;

    constexpr int kVPitch = kHeadDim * 2 + 32;       // bytes per V row in LDS (conflict-free transposed reads)
    __shared__ __attribute__((aligned(16))) unsigned char s_v[4][kCK * kVPitch];   // per-wave V tile

    const int64_t row = (int64_t)hkv * kHeadDim;    // elements between consecutive cache rows

    // Block ids of this split, one per lane (lanes >= nb hold -1).
    const int my_blk = (lane < nb && raw_blk >= 0 && (int64_t)raw_blk < num_blocks) ? raw_blk : -1;

    // Lane (col, grp): col = head column of both products, grp = 4-key group.
    const int col = lane & 15, grp = lane >> 4;
    // B operand of the scores: q of head g*G + col, dims 8*grp + 32*st .. +7, zero for col >= G.
    bf16x8 qb[4];
    // Step: the new token's k' (pieces as q's, for lanes col == its chunk row) and v
    // (this lane's 8 dims), patched into the chunk that holds key ctx - 1.
    u32x4 kn[4], vn = {0u, 0u, 0u, 0u};
    bool inject = false;
    if (kStep) {
        const bool on = col < G;
        const uint16_t* row_in = sa.qkv + (int64_t)b * sa.qkv_stride;
        int64_t pos = sa.positions[b];
        pos = pos < 0 ? 0 : (pos >= sa.max_pos ? (int64_t)sa.max_pos - 1 : pos);
        const float* trow = sa.table + pos * kHeadDim;
        u32x4 x[4], qn[4];
        const uint16_t* qr = row_in + ((int64_t)g * G + (on ? col : 0)) * kHeadDim + 8 * grp;
#pragma unroll
        for (int st = 0; st < 4; ++st) x[st] = ldg128(qr + 32 * st);
        norm_rope_cols(x, sa.q_norm_weight, trow, sa.eps, grp, qn);
#pragma unroll
        for (int st = 0; st < 4; ++st) qb[st] = __builtin_bit_cast(bf16x8, on ? qn[st] : u32x4{0u, 0u, 0u, 0u});
        if (s == 0 && on) {
            uint16_t* qo = sa.q_out + ((int64_t)b * hq + (int64_t)g * G + col) * kHeadDim + 8 * grp;
#pragma unroll
            for (int st = 0; st < 4; ++st) stg128(qo + 32 * st, qn[st]);
        }
        // The split holding the context's last chunk (split 0 when the context is
        // empty) owns the new token: k' and v to its cache slot, and into its chunk.
        if ((nchunks > 0 && c0 + nchunks == nchk) || (nchk == 0 && s == 0)) {
            const uint16_t* kr = row_in + ((int64_t)hq + g) * kHeadDim + 8 * grp;
#pragma unroll
            for (int st = 0; st < 4; ++st) x[st] = ldg128(kr + 32 * st);
            norm_rope_cols(x, sa.k_norm_weight, trow, sa.eps, grp, kn);
            vn = ldg128(row_in + ((int64_t)hq + hkv + g) * kHeadDim + 8 * col);
            const int64_t slot = sa.slot_mapping[b];
            if (slot >= 0 && slot < sa.num_slots) {
                const int64_t rowel = (int64_t)hkv * kHeadDim;
                if (col == 0) {
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        stg128(sa.k_cache + slot * rowel + (int64_t)g * kHeadDim + 8 * grp + 32 * st, kn[st]);
                }
                if (grp == 0) stg128(sa.v_cache + slot * rowel + (int64_t)g * kHeadDim + 8 * col, vn);
                // key ctx - 1 is that slot's row (the engine writes each new token at
                // the end of its context): take it from registers, not from memory
                // this step is writing
                if (nchunks > 0) {
                    const int kl = ctx - 1;
                    const int32_t id = block_table[(int64_t)b * max_blocks + kl / kBlockSize];
                    inject = id >= 0 && (int64_t)id < num_blocks &&
                             (int64_t)id * kBlockSize + kl % kBlockSize == slot;
                }
            }
        }
        if (nchunks == 0) return;
    } else {
        const bool on = col < G;
        const uint16_t* qr = q + ((int64_t)b * hq + (int64_t)g * G + (on ? col : 0)) * kHeadDim + 8 * grp;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 w = on ? ldg128(qr + 32 * st) : u32x4{0u, 0u, 0u, 0u};
            qb[st] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Chunk j of the split is the context's chunk c0 + j: keys 16*((c0+j)%16) .. +15
    // of block slot (c0+j)/16 - blk0.  Chunks j >= nchunks (the trip count's padding)
    // are masked whole.
    auto block_of = [&](int j) { return __builtin_amdgcn_readlane(my_blk, (c0 + j) / kCPB - blk0); };
    auto chunk_row0 = [&](int j) { return kCK * ((c0 + j) % kCPB); };
    auto load = [&](Chunk& c, int j) {
        const int id = block_of(j);
        const int64_t phys = id < 0 ? 0 : id;
        const int64_t r0 = phys * kBlockSize + chunk_row0(j);   // first cache row of the chunk
        // K as the A operand: key col, dims 8*grp + 32*st
        const uint16_t* kp = k_cache + (r0 + col) * row + (int64_t)g * kHeadDim + 8 * grp;
#pragma unroll
        for (int st = 0; st < 4; ++st) c.k[st] = ldg128(kp + 32 * st);
        __builtin_amdgcn_sched_barrier(0);   // K before V: the scores wait only for K
        // V rows: key grp + 4*i, dims 8*col .. +7 (staged through LDS for the transposed read)
        const uint16_t* vp = v_cache + (r0 + grp) * row + (int64_t)g * kHeadDim + 8 * col;
#pragma unroll
        for (int i = 0; i < kCK / 4; ++i) c.v[i] = ldg128_stream(vp + (int64_t)(4 * i) * row);
    };

    float m_ref = -INFINITY;          // lazy reference max of column col (log2 units)
    float l_run = 0.f;                // this lane's share of column col's sum
    f32x4 acc[8];                     // O^T tile d: dims 16d + 4*grp + r, column col
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    unsigned char* vt = s_v[wave];
    typedef __attribute__((address_space(3))) bf16x4* lds4_t;

    auto compute = [&](const Chunk& c, int j) {
        const int key0 = (c0 + j) * kCK;
        const int id = j < nchunks ? block_of(j) : -1;
        // ---- V rows into this wave's LDS tile; keys outside the context become zeros
#pragma unroll
        for (int i = 0; i < kCK / 4; ++i) {
            const bool live = id >= 0 && (key0 + grp + 4 * i) < ctx;
            *reinterpret_cast<u32x4*>(vt + (grp + 4 * i) * kVPitch + 16 * col) =
                live ? c.v[i] : u32x4{0u, 0u, 0u, 0u};
        }
        // ---- scores S[key][col] on MFMA: lane holds keys 4*grp + r of column col
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c.k[st]), qb[st], sc, 0, 0, 0);
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * grp + r;
            sv[r] = (id >= 0 && key < ctx) ? sc[r] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // ---- lazy reference, lane-local (every lane of a column holds the same max)
        const float mn = (mx > m_ref + kLazyMax) ? mx : m_ref;
        const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - mn);
        m_ref = mn;
        const float ref = mn == -INFINITY ? 0.f : mn;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = exp2f(sv[r] - ref);
        // B operand of P V: keys 4*grp + r of column col -- the score layout itself.
        // The row sum adds the same bf16-rounded weights P V uses (dot2 with (1, 1)),
        // so numerator and denominator agree.
        const bf16x4 pb = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
        const float psum = __builtin_amdgcn_fdot2_f32_bf16(
            __builtin_shufflevector(pb, pb, 2, 3), ones,
            __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones, 0.f, false), false);
        l_run = fmaf(l_run, alpha, psum);
        // ---- O^T += V^T P on MFMA; V^T tiles by transposing LDS reads: lane j of the
        // 16-lane group grp addresses key 4*grp + j/4, dims 16d + 4*(j%4) and receives
        // dim 16d + j across those 4 keys.
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds4_t)(vt + (4 * grp + (col >> 2)) * kVPitch + 2 * (16 * d + 4 * (col & 3))));
            acc[d] *= alpha;
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, va),
                                                                __builtin_bit_cast(short4_t, pb), acc[d], 0, 0, 0);
        }
    };

    // ---- main loop: kDepth - 1 chunks in flight while one is computed.  Every
    // prefetch is issued unconditionally (past the end it re-reads the last
    // chunk, an L2 hit), so the number of loads in flight is the same on every
    // path and each wait covers exactly the chunk about to be used.
    Chunk ring[kDepth];
    // The trip count is padded to a multiple of the ring depth; padded chunks are
    // masked whole (their loads re-read the last chunk).
    const int ntrip = (nchunks + kDepth - 1) / kDepth * kDepth;
#pragma unroll
    for (int u = 0; u < kDepth - 1; ++u) load(ring[u], min(u, nchunks - 1));
    for (int j0 = 0; j0 < ntrip; j0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int j = j0 + u;
            load(ring[(u + kDepth - 1) % kDepth], min(j + kDepth - 1, nchunks - 1));
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this chunk's math
            if (kStep && inject && j == nchunks - 1) {
                // the new token is row (ctx - 1) % 16 of this chunk: K is the A operand
                // (key = lane % 16), V rows are key grp + 4 i
                const int rr = (ctx - 1) % kCK;
                if (col == rr) {
#pragma unroll
                    for (int st = 0; st < 4; ++st) ring[u].k[st] = kn[st];
                }
#pragma unroll
                for (int i = 0; i < kCK / 4; ++i)
                    if (grp == rr % 4 && i == rr / 4) ring[u].v[i] = vn;
            }
            compute(ring[u], j);
        }
    }

    // ---- this wave's (m, l, O) for its G heads go straight to the workspace
    float lsum = l_run;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (col < G) {
        const int64_t bh = (int64_t)b * hq + (int64_t)g * G + col;
        float* po = part_o + (bh * max_splits + s) * kHeadDim;
#pragma unroll
        for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4*>(po + 16 * d + 4 * grp) = acc[d];
        if (grp == 0) {
            float* ml = part_ml + (bh * max_splits + s) * 2;
            ml[0] = m_ref;
            ml[1] = lsum;
        }
    }
}

// Dispatch order of the split items (b, s): a counting sort by the number of
// blocks the item covers, largest first, empty items last (one workgroup).
// Items are entered split-major, so within a size class the first splits of
// all sequences come first and the reads of a prefix that several sequences
// share fall close together in time.  The order only schedules work: every
// result is the same.
__global__ void __launch_bounds__(1024) decode_order_kernel(const int32_t* __restrict__ context_lens,
                                                            int32_t max_blocks, int32_t num_seqs, int32_t split_chunks,
                                                            int32_t max_splits, int32_t* __restrict__ work) {
    __shared__ int32_t s_bin[kMaxSplitBlocks * (kBlockSize / kCK) + 1];
    const int tid = threadIdx.x;
    const int cap = max_blocks * kBlockSize;
    const int n_items = num_seqs * max_splits;
    auto key = [&](int it) {   // split_chunks - (chunks of the item): 0 = full
        const int b = it / max_splits, s = it - b * max_splits;
        int ctx = context_lens[b];
        ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
        const int nc = (ctx + kCK - 1) / kCK - s * split_chunks;
        return split_chunks - (nc < 0 ? 0 : (nc > split_chunks ? split_chunks : nc));
    };
    if (tid <= split_chunks) s_bin[tid] = 0;
    __syncthreads();
    for (int it = tid; it < n_items; it += 1024) atomicAdd(&s_bin[key(it)], 1);
    __syncthreads();
    if (tid == 0) {   // exclusive prefix over the bins
        int run = 0;
        for (int i = 0; i <= split_chunks; ++i) {
            const int c = s_bin[i];
            s_bin[i] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int j = tid; j < n_items; j += 1024) {
        const int s = j / num_seqs, b = j - s * num_seqs;
        const int it = b * max_splits + s;
        work[atomicAdd(&s_bin[key(it)], 1)] = it;
    }
}

// Merge of the splits of each (b, h), in split order: one wave per (b, h), four
// per workgroup, each lane owning two output dims.  The (m, l) pairs are read
// with uniform addresses (every lane the same split), the partial outputs as
// 512 contiguous bytes per split, four splits' loads in flight at a time.
// The partial outputs are read once: non-temporal loads (small batches 0.5-3%
// faster; streaming the split kernel's partial stores as well was slower).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 ldg_f2_stream(const float* p) {
    const f32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p));
    return make_float2(v[0], v[1]);
}
constexpr int kCombineWaves = 4;
#ifndef PKV_COMBINE_IN_FLIGHT
#define PKV_COMBINE_IN_FLIGHT 4
#endif
constexpr int kCombineInFlight = PKV_COMBINE_IN_FLIGHT;   // splits whose loads are in flight together
__global__ void __launch_bounds__(64 * kCombineWaves) decode_combine_kernel(
    const int32_t* __restrict__ context_lens, int32_t max_blocks, int32_t hq, int32_t split_chunks,
    int32_t max_splits, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    uint16_t* __restrict__ o) {
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * kCombineWaves + (threadIdx.x >> 6), b = blockIdx.y;
    if (h >= hq) return;
    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int ns = ((ctx + kCK - 1) / kCK + split_chunks - 1) / split_chunks;
    const int64_t bh = (int64_t)b * hq + h;
    const float* ml = part_ml + bh * max_splits * 2;
    const float* po = part_o + bh * max_splits * kHeadDim + 2 * lane;

    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    const float ref = M == -INFINITY ? 0.f : M;

    float L = 0.f;
    float acc0 = 0.f, acc1 = 0.f;
    int s = 0;
    for (; s + kCombineInFlight <= ns; s += kCombineInFlight) {
        float2 p[kCombineInFlight];
        float m[kCombineInFlight], l[kCombineInFlight];
#pragma unroll
        for (int i = 0; i < kCombineInFlight; ++i) {
            p[i] = ldg_f2_stream(po + (int64_t)(s + i) * kHeadDim);
            m[i] = ml[2 * (s + i)];
            l[i] = ml[2 * (s + i) + 1];
        }
#pragma unroll
        for (int i = 0; i < kCombineInFlight; ++i) {
            const float w = exp2f(m[i] - ref);
            L = fmaf(l[i], w, L);
            acc0 = fmaf(p[i].x, w, acc0);
            acc1 = fmaf(p[i].y, w, acc1);
        }
    }
    for (; s < ns; ++s) {
        const float2 p = ldg_f2_stream(po + (int64_t)s * kHeadDim);
        const float w = exp2f(ml[2 * s] - ref);
        L = fmaf(ml[2 * s + 1], w, L);
        acc0 = fmaf(p.x, w, acc0);
        acc1 = fmaf(p.y, w, acc1);
    }
    const float r0 = L > 0.f ? acc0 / L : 0.f, r1 = L > 0.f ? acc1 / L : 0.f;
    *reinterpret_cast<uint32_t*>(o + bh * kHeadDim + 2 * lane) = pack_bf16x2(r0, r1);
}

// Merge for many splits per (b, h) (a long context at a batch of one or two):
// one workgroup per (b, h), wave w adding splits w, w + 4, ..., eight splits'
// loads in flight, against the common reference max; the four waves' sums are
// then added in wave order (deterministic).
constexpr int kWideMergeSplits = 32;   // above this many splits per sequence, the wide merge
__global__ void __launch_bounds__(256) decode_combine_wide_kernel(
    const int32_t* __restrict__ context_lens, int32_t max_blocks, int32_t hq, int32_t split_chunks,
    int32_t max_splits, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    uint16_t* __restrict__ o) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x, b = blockIdx.y;
    __shared__ float s_m[4];
    __shared__ float s_acc[4][3][64];
    int ctx = context_lens[b];
    const int cap = max_blocks * kBlockSize;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int ns = ((ctx + kCK - 1) / kCK + split_chunks - 1) / split_chunks;
    const int64_t bh = (int64_t)b * hq + h;
    const float* ml = part_ml + bh * max_splits * 2;
    const float* po = part_o + bh * max_splits * kHeadDim + 2 * lane;

    float M = -INFINITY;
    for (int s = wave + 4 * lane; s < ns; s += 256) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    if (lane == 0) s_m[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    const float ref = M == -INFINITY ? 0.f : M;

    constexpr int kF = 8;
    float L = 0.f, acc0 = 0.f, acc1 = 0.f;
    int s = wave;
    for (; s + 4 * (kF - 1) < ns; s += 4 * kF) {
        float2 p[kF];
        float m[kF], l[kF];
#pragma unroll
        for (int i = 0; i < kF; ++i) {
            p[i] = ldg_f2_stream(po + (int64_t)(s + 4 * i) * kHeadDim);
            m[i] = ml[2 * (s + 4 * i)];
            l[i] = ml[2 * (s + 4 * i) + 1];
        }
#pragma unroll
        for (int i = 0; i < kF; ++i) {
            const float w = exp2f(m[i] - ref);
            L = fmaf(l[i], w, L);
            acc0 = fmaf(p[i].x, w, acc0);
            acc1 = fmaf(p[i].y, w, acc1);
        }
    }
    for (; s < ns; s += 4) {
        const float2 p = ldg_f2_stream(po + (int64_t)s * kHeadDim);
        const float w = exp2f(ml[2 * s] - ref);
        L = fmaf(ml[2 * s + 1], w, L);
        acc0 = fmaf(p.x, w, acc0);
        acc1 = fmaf(p.y, w, acc1);
    }
    s_acc[wave][0][lane] = L;
    s_acc[wave][1][lane] = acc0;
    s_acc[wave][2][lane] = acc1;
    __syncthreads();
    if (wave != 0) return;
    float Lt = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        Lt += s_acc[w][0][lane];
        a0 += s_acc[w][1][lane];
        a1 += s_acc[w][2][lane];
    }
    const float r0 = Lt > 0.f ? a0 / Lt : 0.f, r1 = Lt > 0.f ? a1 / Lt : 0.f;
    *reinterpret_cast<uint32_t*>(o + bh * kHeadDim + 2 * lane) = pack_bf16x2(r0, r1);
}

// ---- split-K workspace in a fixed device array, for pkv_attn_decode_paged_noalloc.
// Callers that cannot allocate (code under graph capture, tight serving loops)
// get the partials (m, l, O) and the dispatch order here instead of in a
// workspace they pass.  One copy per GPU, held until the process ends; every
// call on a GPU uses the same bytes, so calls that overlap on one GPU race.
// Nothing in it needs clearing between calls: the order kernel writes the whole
// dispatch list, and the merge reads only the splits the split kernel wrote in
// the same call.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device, looked up once per device
// (the host-side name of the array is not a device address).
hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || (uintptr_t)p % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

namespace {
template <bool kStep>
hipError_t launch_decode_impl(const DecodeArgs& a, const StepArgs& sa, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    const int G = a.hq / a.hkv;
    const int sc = decode_split_chunks(a.num_seqs, a.hkv, a.max_blocks);
    const int ms = (a.max_blocks * (kBlockSize / kCK) + sc - 1) / sc;
    Workspace w = carve(a.workspace, a.num_seqs, a.hq, ms);
    dim3 grid((a.hkv + 3) / 4, a.num_seqs, ms);
    // The size-ordered dispatch pays when workgroups queue for the chip; when the
    // whole grid fits at once (two split workgroups per CU, 256 CUs) the order kernel
    // is skipped: one launch less on short, small-batch steps.
    const bool ordered = (int64_t)grid.x * grid.y * grid.z > kResidentItems;
    if (ordered)
        hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens, a.max_blocks,
                           a.num_seqs, sc, ms, w.work);
    const int32_t* work = ordered ? w.work : nullptr;
#define PKV_DECODE_CASE(GG)                                                                                       \
    case GG:                                                                                                      \
        hipLaunchKernelGGL((decode_split_kernel<GG, kStep>), grid, dim3(kDecThreads), 0, stream,                  \
                           (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache,          \
                           a.context_lens, a.block_table, a.max_blocks, a.hq, a.hkv, a.num_blocks, a.scale_log2, \
                           sc, ms, w.part_o, w.part_ml, work, sa);                                                \
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
    if (ms > kWideMergeSplits)
        hipLaunchKernelGGL(decode_combine_wide_kernel, dim3(a.hq, a.num_seqs), dim3(256), 0, stream, a.context_lens,
                           a.max_blocks, a.hq, sc, ms, w.part_o, w.part_ml, (uint16_t*)a.o);
    else
        hipLaunchKernelGGL(decode_combine_kernel, dim3((a.hq + kCombineWaves - 1) / kCombineWaves, a.num_seqs),
                           dim3(64 * kCombineWaves), 0, stream, a.context_lens,
                           a.max_blocks, a.hq, sc, ms, w.part_o, w.part_ml, (uint16_t*)a.o);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream) {
    return launch_decode_impl<false>(a, StepArgs{}, stream);
}

hipError_t launch_decode_step(const DecodeArgs& a, const StepArgs& st, hipStream_t stream) {
    return launch_decode_impl<true>(a, st, stream);
}

}  // namespace pkv
