// attn_prefill.hip -- varlen causal GQA prefill attention on MFMA (gfx950).
//
// What is computed: "3.3 Model skeleton and core operators", section 7.2, and
// "nano-vllm code walkthrough", "Prefill stage": packed sequences delimited by
// cu_seqlens, causal inside each sequence and nothing across sequences (the
// block-diagonal mask of "同一个 Qwen3，两种写法" section 3.2, never built).
// With a block table the keys come from the paged cache ("case 2", prefix hit
// or a later chunk): query i of a sequence sits at absolute position
// Lk - Lq + i.  q head h reads kv head h / (Hq/Hkv) ("Nano-vLLM 源码解读 #17
// 注意力层", section 3).  The softmax is that of the same page's section 5.2,
// in base 2 with the scale folded into the exponent.
//
// Design for CDNA4:
//   * Transposed products keep every softmax statistic lane-local:
//       S^T[key][q] = K . Q^T    and    O^T[d][q] += V^T . P^T
//     on v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane
//     owns one column (one query row), so the row max, the rescale of O and
//     the sum stay in registers; only the max needs one swap with the lane 32
//     away.  The S^T accumulator is, after exp2 and bf16 packing, already the
//     B operand of the PV product.
//   * A workgroup owns one kv head and the query heads of its GQA group that
//     share it; each wave computes 32 query rows of one head.  For batches of
//     long sequences (mean query length >= 2048), and for prefix hits of 1024+
//     queries on average with 4 heads a workgroup, the workgroup has 8 waves
//     (4 heads x 64 positions, or 2 x 128) and 128-key tiles, so each K/V tile
//     staged in LDS feeds 256 query rows; otherwise 4 waves and 64-key tiles
//     (more, smaller workgroups).  K and V are both kept row-major in LDS; the
//     PV product needs V transposed, which the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16) delivers: lane j of a 16-lane group addresses key
//     j/4, dims 4*(j%4) of a 4-key x 16-dim tile and receives its own dim
//     across the 4 keys.
//   * Double-buffered LDS, one barrier per tile.  Tiles (128 keys with 8
//     waves, 64 with 4) never straddle a 256-token block, so the paged loader
//     does one block-table lookup per tile.  The fast pass copies each tile
//     straight from global memory into LDS (global_load_lds_dwordx4, for the
//     next tile while this one is computed: K right after the barrier, V after
//     the QK^T phase):
//     no staging registers and no LDS store instructions; rows are unpadded
//     with 16-byte slots XOR-swizzled per row so the operand reads stay
//     conflict-free.  The exact pass stages tiles through registers into padded
//     rows (16-byte copies; rows past the last key clamped, V zeroed there).
//   * Softmax in two passes.  The fast pass (one kernel) takes exp2 of each
//     score times softmax_scale * log2(e) (fp32) against a fixed reference of
//     0: no row max and no rescale; per score a multiply, an exp2 and halves
//     of a bf16 pack and of the row-sum dot2 (the exact pass adds the max and
//     an fma against it).  The reference cancels in
//     O / l and floating point is scale-invariant away from its range limits,
//     so the weights are the online softmax's up to fp32 rounding while a
//     row's weights stay far from overflow and underflow; a wave whose rows
//     leave l in [2^-64, 2^64] (or whose O is not finite) writes a marker
//     instead of its results.  The exact pass (a second, persistent kernel)
//     recomputes only flagged work items with an online running max that
//     moves only when a row grows by more than 2^8.  A call with nothing
//     flagged costs one short launch whose workgroups read one word and exit;
//     batches under 2e10 FLOP run the exact pass alone in one launch.
//   * Causal tile skipping: a wave stops at the tile holding its last visible
//     key; only tiles that cross the diagonal (or the sequence end) are masked.
//   * Work order: longest query blocks first inside each (sequence, kv head);
//     each such unit runs on one XCD (its K/V stays in that L2) and the units
//     are dealt round-robin over the 8 XCDs (cut into 2-block chunks when there
//     are fewer than 8), so unequal or few sequences balance.  A small batch
//     takes an XCD's units together, heaviest blocks of all of them first.
//   * Key split: when a call's query blocks do not fill the CU slots and keys
//     run long (later chunks over a long cached context), the fast pass cuts
//     each long block's key tiles into 2-4 chunks run by separate workgroups.
//     The fixed reference makes their O and row sums simply add; a merge kernel
//     adds them in chunk order (fp32, from the caller's workspace) and finishes
//     as the fast pass does.
#include <algorithm>
#include <atomic>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {
typedef __attribute__((address_space(3))) bf16x4* lds_ptr_t;
typedef __attribute__((address_space(3))) unsigned char lds_byte;
constexpr int kRowsPerWave = 32;
constexpr int kKPitch = kHeadDim * 2 + 16;  // bytes per K row in LDS (row-major)
constexpr int kVPitch = kHeadDim * 2 + 64;  // bytes per V row in LDS (row-major, read transposed)
constexpr float kLazyLog2 = 8.0f;           // the lazy reference max moves when a row grows by > 2^8
// Keys per tile: 128 for the 8-wave workgroup (one per CU; LDS for two K+V tile
// pairs: 64 KB each unpadded in the fast pass, 74 KB padded in the exact pass),
// 64 for 4 waves (two workgroups per CU).  A tile never straddles a 256-token
// block.
template <int NW>
constexpr int kTileKeys = NW == 8 ? 128 : 64;
// Left by the fast pass in the first output element of a wave whose rows need
// the exact pass: a signalling-NaN pattern, which no arithmetic result converted
// to bf16 can have (those NaNs are quiet).
constexpr uint16_t kFixupMarker = 0x7F81;
constexpr bf16x2 kOnes2 = {(bf16)1.0f, (bf16)1.0f};
// Key split: every chunk of a split work item holds at least this many tiles.
constexpr int kSplitMinChunkTiles = 8;
// Floats one wave leaves per chunk of a split item: its 64 O^T accumulators per
// lane (entry 64 * r + lane) and its partial row sum per lane.
constexpr int kPartFloats = 64 * 64 + 64;
constexpr size_t kSplitMaxBytes = size_t(512) << 20;
constexpr int kWindowUnits = 8;                      // units per XCD dealt as one window, at most
constexpr int64_t kWindowBytes = int64_t(8) << 20;    // their K/V, at most
}  // namespace

// Chunks of a work item of n_tiles key tiles when the call splits items into up to
// nc chunks: 1 (no split) below 2 * kSplitMinChunkTiles tiles.
__host__ __device__ inline int item_chunks(int n_tiles, int nc) {
    return nc > 1 && n_tiles >= 2 * kSplitMinChunkTiles ? min(nc, n_tiles / kSplitMinChunkTiles) : 1;
}

// Highest call number (see launch_attn_prefill) whose fast pass flagged a work
// item; raised with a device-scope atomic, never lowered.  The exact pass of a
// call scans for markers only when this is at least its own number.
__device__ unsigned long long g_prefill_flagged_call = 0;

// End of a wave's 32 query rows of one head: lane holds O^T[d][qi] for
// d = 32dt + 8(r/4) + 4*h32 + r%4 and its part of the row sum.  kCheck (fast
// pass): did every live row stay inside the fast pass's range?  l in [2^-64, 2^64]
// bounds every weight and keeps the row clear of underflow; a finite sum of this
// lane's O entries means no product overflowed.  If not, the wave leaves
// kFixupMarker in its first output element instead of its results, and the exact
// pass recomputes the whole work item.  Otherwise: normalise and store.
template <bool kCheck>
__device__ __forceinline__ void prefill_finish(const PrefillArgs& a, uint64_t call, int cq0, int Lq, int wp0,
                                               int head, bool wave_live, const f32x16 (&oacc)[4], float l_part) {
    const int lane = __lane_id();
    const float l = l_part + __shfl_xor(l_part, 32, 64);
    if (kCheck) {
        float osum = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) osum += oacc[dt][r];
        const bool row_bad = wave_live && !(l >= 0x1p-64f && l <= 0x1p64f && osum - osum == 0.f);
        if (__any(row_bad)) {
            if (lane == 0) {
                *((uint16_t*)a.o + ((int64_t)(cq0 + wp0) * a.hq + head) * kHeadDim) = kFixupMarker;
                atomicMax(&g_prefill_flagged_call, (unsigned long long)call);
            }
            return;
        }
    }
    const int qi = wp0 + (lane & 31), h32 = lane >> 5;
    if (!wave_live || qi >= Lq) return;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int orow = cq0 + qi;
    if (orow >= a.total_q) return;
    uint16_t* op = (uint16_t*)a.o + ((int64_t)orow * a.hq + head) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * h32;
            u32x2 w;
            w[0] = pack_bf16x2(oacc[dt][4 * r4] * inv, oacc[dt][4 * r4 + 1] * inv);
            w[1] = pack_bf16x2(oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv);
            *reinterpret_cast<u32x2*>(op + d) = w;
        }
}

// One work item: query block mb of (sequence b, kv head g, head group hg), with
// NW waves (4 or 8; two waves per SIMD either way: two workgroups of 4 per CU,
// or one of 8).  kExact selects the pass (see the tile loop below).  k_lds3 /
// v_lds3 are the workgroup's tile buffers.
template <int GW, bool PAGED, int NW, bool kExact>
__device__ __forceinline__ void prefill_block(const PrefillArgs& a, int32_t m_blocks, int32_t head_groups,
                                              int32_t work, lds_byte* k_lds3, lds_byte* v_lds3, uint64_t call,
                                              int c = 0, int nc = 1, float* part = nullptr) {
    constexpr int kThreads = 64 * NW;
    constexpr int kKT = kTileKeys<NW>;
    constexpr int kKH = kKT / 32;                       // 32-key blocks per tile
    // The fast pass copies tiles straight from global memory into LDS
    // (global_load_lds_dwordx4: a wave-instruction fills 1 KB of consecutive LDS),
    // so its rows are unpadded and XOR-swizzled in 16-byte slots instead.
    constexpr bool kDma = !kExact;
    constexpr int kKP = kDma ? kHeadDim * 2 : kKPitch;
    constexpr int kVP = kDma ? kHeadDim * 2 : kVPitch;
    constexpr int kKTileBytes = kKT * kKP;
    constexpr int kVTileBytes = kKT * kVP;
    constexpr int kLoadRows = kThreads / 16;            // tile rows one sweep of 16-byte pieces covers
    constexpr int kLoadIters = kKT / kLoadRows;         // sweeps per tile
    constexpr int kPosSub = NW / GW;                    // position sub-blocks per workgroup
    constexpr int kBM = kRowsPerWave * kPosSub;         // query positions per workgroup
    unsigned char* k_lds = (unsigned char*)k_lds3;
    unsigned char* v_lds = (unsigned char*)v_lds3;

    // work = ((b * hkv + g) * head_groups + hg) * m_blocks + (m_blocks - 1 - mb)
    const int mb = m_blocks - 1 - (work % m_blocks);
    int rest = work / m_blocks;
    const int hg = rest % head_groups;
    rest /= head_groups;
    const int g = rest % a.hkv;
    const int b = rest / a.hkv;

    const int cq0 = a.cu_q[b], cq1 = a.cu_q[b + 1];
    const int ck0 = a.cu_k[b], ck1 = a.cu_k[b + 1];
    const int Lq = cq1 - cq0, Lk = ck1 - ck0;
    const int p0 = mb * kBM;
    if (p0 >= Lq || Lk < Lq || Lq <= 0) return;
    if (cq0 < 0 || cq1 > a.total_q || ck0 < 0) return;   // metadata outside the q/o rows: nothing is touched
    const int off = Lk - Lq;                            // absolute position of query 0
    const int G = a.hq / a.hkv;
    if (kExact && call != 0) {
        // Recompute this work item only if one of its waves left the marker.
        bool flagged = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int row = p0 + kRowsPerWave * (w / GW);
            const int hd = g * G + hg * GW + (w % GW);
            if (row < Lq)
                flagged |= *((const uint16_t*)a.o + ((int64_t)(cq0 + row) * a.hq + hd) * kHeadDim) == kFixupMarker;
        }
        if (!flagged) return;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int head = g * G + hg * GW + (wave % GW);
    const int wp0 = p0 + kRowsPerWave * (wave / GW);    // first query (sequence-relative) of this wave
    const int wq_last = min(wp0 + kRowsPerWave, Lq) - 1;
    const bool wave_live = wp0 < Lq;

    // Keys any wave of this workgroup can see: 0 .. off + min(p0 + kBM, Lq) - 1.
    const int wg_keys = off + min(p0 + kBM, Lq);
    const int n_tiles = (wg_keys + kKT - 1) / kKT;
    const int wave_keys = wave_live ? off + wq_last + 1 : 0;
    const int wave_tiles = (wave_keys + kKT - 1) / kKT;
    // Key split (fast pass only): chunk c of the item's nc_item chunks covers key
    // tiles [t_begin, t_end); a split item leaves partial sums in `part`.
    const int nc_item = kExact ? 1 : item_chunks(n_tiles, nc);
    if (c >= nc_item) return;
    const int t_begin = c * n_tiles / nc_item, t_end = (c + 1) * n_tiles / nc_item;
    const bool split = nc_item > 1;

    // ---- Q^T as the B operand: lane owns query row l%32, dims 8*(l/32) + 16*st .. +7.
    // Q stays as given (bf16): its products with K are exact in the fp32
    // accumulator, and the scale is applied to each score in fp32.  (Rounding
    // Q * scale back to bf16 instead would move every score by up to 2^-9 of the
    // sum of |q_i k_i| -- an error that grows with the score.)
    const int qi = wp0 + (lane & 31);
    const int q_row = cq0 + min(qi, Lq - 1);
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)min(q_row, a.total_q - 1) * a.q_row_stride +
                         (int64_t)head * kHeadDim + 8 * (lane >> 5);
    bf16x8 qreg[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) qreg[st] = __builtin_bit_cast(bf16x8, ldg128(qp + 16 * st));
    const int qpos = off + qi;                          // absolute position of this lane's query

    // ---- tile loaders.  Row strides are at most 2^24 elements (checked by the
    // caller), so offsets inside one tile fit in 32 bits: a per-tile base plus a
    // 32-bit lane offset.
    // Exact pass (through registers): thread tid moves 16-byte piece tid%16 of rows
    // tid/16 + kLoadRows*i (i < kLoadIters) of the K and V tiles.  Row offsets are
    // loop-invariant; every load is issued on every path (rows past the last key are
    // clamped onto it), so the compiler's wait counts stay exact.
    const int64_t krs = a.k_row_stride, vrs = a.v_row_stride;
    const int32_t krs32 = (int32_t)krs, vrs32 = (int32_t)vrs;
    const uint16_t* kbase = (const uint16_t*)a.k + (int64_t)g * kHeadDim;
    const uint16_t* vbase = (const uint16_t*)a.v + (int64_t)g * kHeadDim;
    const int32_t* bt = PAGED ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
    const int lrow = tid >> 4, piece = tid & 15;
    int32_t koff[kLoadIters], voff[kLoadIters];
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i) {
        koff[i] = (lrow + kLoadRows * i) * krs32 + piece * 8;
        voff[i] = (lrow + kLoadRows * i) * vrs32 + piece * 8;
    }
    // First cache/array row of tile t and whether its block id is usable (tiles
    // never straddle a 256-token block).
    auto tile_row0 = [&](int t, bool& ok) -> int64_t {
        const int j0 = t * kKT;
        if (PAGED) {
            const int bi = j0 / kBlockSize;
            const int32_t blk = bi < a.max_blocks ? bt[bi] : -1;
            ok = blk >= 0 && (int64_t)blk < a.num_blocks;
            return ok ? (int64_t)blk * kBlockSize + (j0 % kBlockSize) : 0;
        } else {
            ok = true;
            return (int64_t)ck0 + j0;
        }
    };
    // Fast pass: block id of tile t (0 when K/V are contiguous), loaded one iteration
    // before it is needed, and the tile's first row from it.
    // The load takes a clamped index plus an opaque per-lane zero, so the compiler
    // keeps the value in a vector register and does not wait for it until blk_of
    // (next iteration, after the barrier's wait) moves it to a scalar and applies
    // the table bound.
    int32_t lane_zero;
    asm("v_mov_b32 %0, 0" : "=v"(lane_zero));
    auto load_blk = [&](int t) -> int32_t {
        if (!PAGED) return 0;
        return bt[min(t * kKT / kBlockSize, a.max_blocks - 1) + lane_zero];
    };
    auto blk_of = [&](int t, int32_t raw) -> int32_t {
        return t * kKT / kBlockSize < a.max_blocks ? __builtin_amdgcn_readfirstlane(raw) : -1;
    };
    auto row0_of = [&](int t, int32_t blk, bool& ok) -> int64_t {
        if (PAGED) {
            ok = blk >= 0 && (int64_t)blk < a.num_blocks;
            return ok ? (int64_t)blk * kBlockSize + (t * kKT) % kBlockSize : 0;
        }
        ok = true;
        return (int64_t)ck0 + t * kKT;
    };
    u32x4 kst[kLoadIters], vst[kLoadIters];
    auto load_tile = [&](int t) {
        bool ok;
        const int64_t r0 = tile_row0(t, ok);
        const int last = Lk - 1 - t * kKT;              // last valid row of this tile (>= 0)
        const uint16_t* kp = kbase + r0 * krs;
        const uint16_t* vp = vbase + r0 * vrs;
        if (ok && last >= kKT - 1) {
#pragma unroll
            for (int i = 0; i < kLoadIters; ++i) kst[i] = ldg128(kp + koff[i]);
#pragma unroll
            for (int i = 0; i < kLoadIters; ++i) vst[i] = ldg128(vp + voff[i]);
        } else {
            // partial or unusable tile: clamp rows onto valid memory, zero V at store time
#pragma unroll
            for (int i = 0; i < kLoadIters; ++i) {
                const int row = ok ? min(lrow + kLoadRows * i, last) : 0;
                kst[i] = ldg128(kp + (row * krs32 + piece * 8));
            }
#pragma unroll
            for (int i = 0; i < kLoadIters; ++i) {
                const int row = ok ? min(lrow + kLoadRows * i, last) : 0;
                vst[i] = ldg128(vp + (row * vrs32 + piece * 8));
            }
        }
    };
    auto store_tile = [&](int t, unsigned char* kb, unsigned char* vb) {
        bool ok;
        (void)tile_row0(t, ok);
        const int last = Lk - 1 - t * kKT;
        if (!ok || last < kKT - 1) {
            // V rows of keys past the end (or of an unusable block) become zeros, so
            // whatever those cache slots hold cannot reach the output through P V.
#pragma unroll
            for (int i = 0; i < kLoadIters; ++i)
                if (!ok || lrow + kLoadRows * i > last) vst[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kLoadIters; ++i) {
            *reinterpret_cast<u32x4*>(kb + (lrow + kLoadRows * i) * kKPitch + piece * 16) = kst[i];
            *reinterpret_cast<u32x4*>(vb + (lrow + kLoadRows * i) * kVPitch + piece * 16) = vst[i];
        }
    };
    // Direct copies (fast pass): wave w fills rows 4(w*kDmaPerWave + u) + lane/16,
    // u < kDmaPerWave, of both tiles; lane l lands in slot l%16 of its row.  Slot s of
    // K row r holds 16-byte piece s ^ (r % 16), of V row r piece s ^ 4(r % 4): the
    // MFMA operand reads below then touch every bank once per group of lanes.
    constexpr int kDmaPerWave = kKT / 4 / NW;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int drow = lane >> 4, dslot = lane & 15;
    // byte offsets from the tile's first row (< 127 * 2^25 + 256: fit 32 bits unsigned)
    uint32_t kdoff[kDmaPerWave], vdoff[kDmaPerWave];
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
        const int r = 4 * (wave_u * kDmaPerWave + u) + drow;
        kdoff[u] = 2u * (uint32_t)(r * krs32 + ((dslot ^ (r & 15)) * 8));
        vdoff[u] = 2u * (uint32_t)(r * vrs32 + ((dslot ^ (4 * (r & 3))) * 8));
    }
    // Full tile with a usable block id: asynchronous copies, waited for at the next
    // barrier -- the K half right after the barrier, the V half after the QK^T phase
    // (spreading the LDS writes over the tile: measured +2%).  Each half is one asm
    // block: the scalar-base form (tile base in SGPRs + the lane's 32-bit byte offset:
    // no address arithmetic per tile), M0 carries each copy's LDS address (1 KB
    // chunk), and the compiler, which
    // does not see these copies, adds no waits of its own for them before the LDS
    // reads of the other buffer.  The explicit vmcnt(0) and the barrier (a
    // workgroup fence) order them against every later read of the buffer they fill.
    static_assert(kDmaPerWave == 4, "one asm block moves a wave's 4 chunks of K or of V");
    auto issue_half = [&](int t, int stage, int32_t blk, bool vhalf) {
        bool ok;
        const int64_t r0 = row0_of(t, blk, ok);
        const uint16_t* p = (vhalf ? vbase : kbase) + r0 * (vhalf ? vrs : krs);   // uniform: a scalar base
        const uint32_t* off = vhalf ? vdoff : kdoff;
        const uint32_t l = (uint32_t)(uintptr_t)(vhalf ? v_lds3 : k_lds3) +
                           stage * (vhalf ? kVTileBytes : kKTileBytes) + 1024 * (wave_u * kDmaPerWave);
        uint32_t saved;
        asm volatile(
            "s_mov_b32 %[sv], m0\n\t"
            "s_mov_b32 m0, %[l0]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a0], %[base]\n\t"
            "s_mov_b32 m0, %[l1]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a1], %[base]\n\t"
            "s_mov_b32 m0, %[l2]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a2], %[base]\n\t"
            "s_mov_b32 m0, %[l3]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a3], %[base]\n\t"
            "s_mov_b32 m0, %[sv]"
            : [sv] "=&s"(saved)
            : [a0] "v"(off[0]), [a1] "v"(off[1]), [a2] "v"(off[2]), [a3] "v"(off[3]), [base] "s"(p),
              [l0] "s"(l), [l1] "s"(l + 1024), [l2] "s"(l + 2048), [l3] "s"(l + 3072));
    };
    // Partial or unusable tile: through registers, rows past the end clamped for K and
    // zeroed for V (their weights are 0; zeros keep NaN-carrying slots out of P V).
    auto fill_tile_sync = [&](int t, int stage, int32_t blk) {
        bool ok;
        const int64_t r0 = row0_of(t, blk, ok);
        const int last = Lk - 1 - t * kKT;
        const uint16_t* kp = kbase + r0 * krs;
        const uint16_t* vp = vbase + r0 * vrs;
#pragma unroll
        for (int u = 0; u < kDmaPerWave; ++u) {
            const int r = 4 * (wave_u * kDmaPerWave + u) + drow;
            const int row = ok ? min(r, last) : 0;
            const u32x4 kx = ldg128(kp + (row * krs32 + (dslot ^ (r & 15)) * 8));
            u32x4 vx = ldg128(vp + (row * vrs32 + (dslot ^ (4 * (r & 3))) * 8));
            if (!ok || r > last) vx = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(k_lds + stage * kKTileBytes + r * 256 + dslot * 16) = kx;
            *reinterpret_cast<u32x4*>(v_lds + stage * kVTileBytes + r * 256 + dslot * 16) = vx;
        }
    };
    auto tile_full = [&](int t, int32_t blk) {
        bool ok;
        (void)row0_of(t, blk, ok);
        return ok && Lk - 1 - t * kKT >= kKT - 1;
    };

    const int h32 = lane >> 5;  // which half of the k-slots this lane feeds

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_run = -INFINITY, l_part = 0.f;   // reference max (raw score units), partial row sum
    const float lazy_raw = kLazyLog2 / a.scale_log2;

    // One pass over the key tiles.  Double-buffered LDS tiles: one barrier per tile.
    // Exact pass: tile t is computed from buffer t&1 while tile t+1 (loaded into
    // registers one iteration earlier) is stored into the other buffer; tile t+2 is
    // loaded after the barrier.  Fast pass: right after the barrier, tile t+1 is
    // copied straight into the other buffer while tile t is computed.
    //   Fast pass (kExact false): the weights are exp2(score * scale * log2 e)
    //   against a fixed reference of 0 -- no row max, no rescale, one VALU op less
    //   per score.  Softmax does not depend on the reference and floating point is
    //   scale-invariant away from overflow and underflow, so this is the same
    //   computation while a row's sum stays inside [2^-64, 2^64] and its O finite
    //   (scores within about +-64 in base-2 units); checked afterwards.  Weights
    //   below 2^-126 then sit more than 2^-62 / keys under the row's largest and
    //   do not matter.
    //   Exact pass (kExact true): the online softmax with a lazy reference max that
    //   moves only when a row grows by more than 2^8, so the O rescale is skipped
    //   on most tiles.  Exact for any input: O and l always share the reference.
    {
        bool ok_cur = false;   // fast pass: whether tile t's block id is usable, found when its copies were issued
        int32_t blk_next = 0;  // fast pass: block id of tile t+1
        if (kDma) {
            const int32_t blk0 = blk_of(t_begin, load_blk(t_begin));
            blk_next = load_blk(min(t_begin + 1, n_tiles - 1));
            (void)row0_of(t_begin, blk0, ok_cur);
            if (tile_full(t_begin, blk0)) {
                issue_half(t_begin, t_begin & 1, blk0, false);
                issue_half(t_begin, t_begin & 1, blk0, true);
            } else {
                fill_tile_sync(t_begin, t_begin & 1, blk0);
            }
        } else {
            load_tile(0);
            store_tile(0, k_lds, v_lds);
            if (1 < n_tiles) load_tile(1);
            __syncthreads();
        }
        for (int t = t_begin; t < t_end; ++t) {
            unsigned char* kb = k_lds + (t & 1) * kKTileBytes;
            unsigned char* vb = v_lds + (t & 1) * kVTileBytes;
            if (kDma) {
                // this wave's copies of tile t have landed; after the barrier every
                // wave's have, and every wave is done with tile t-1, whose buffer the
                // copies of tile t+1 then fill while tile t is computed
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                __syncthreads();
            }
            bool ok_next = false;
            bool v_later = false;   // V copies of tile t+1 issued after the QK^T phase
            int32_t blk1 = 0;
            if (kDma && t + 1 < t_end) {
                const int32_t blk = blk_of(t + 1, blk_next);
                blk1 = blk;
                (void)row0_of(t + 1, blk, ok_next);
                if (tile_full(t + 1, blk)) { issue_half(t + 1, (t + 1) & 1, blk, false); v_later = true; }
                else fill_tile_sync(t + 1, (t + 1) & 1, blk);
                // issued after the copies: the wait for them at the next barrier covers it
                blk_next = load_blk(min(t + 2, n_tiles - 1));
            }
            const bool live_t = t < wave_tiles;   // this wave still has visible keys in tile t
            const int j0 = t * kKT;
            bool ok = ok_cur;
            if (!kDma) (void)tile_row0(t, ok);
            f32x16 s[kKH];
            // Fast pass: the QK^T phase (MFMA only) runs at raised wave priority and the
            // softmax + P V phase (VALU-heavy) at the normal one, so of the two waves on a
            // SIMD the one still issuing QK^T MFMAs goes first while the other works
            // through its exponentials (measured +1.5 to 2.5% on the 8B prefix batch).
            if (kDma) __builtin_amdgcn_s_setprio(3);
            if (live_t) {
                // ---- S^T = K Q^T for the tile's 32-key blocks
                // The key blocks are independent accumulation chains; interleaving them
                // keeps consecutive MFMAs independent so each issues without waiting for the
                // previous result.
#pragma unroll
                for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kh][r] = 0.f;
#pragma unroll
                for (int st = 0; st < 8; ++st)
#pragma unroll
                    for (int kh = 0; kh < kKH; ++kh) {
                        // piece 2st + h32 of row 32kh + lane%32; swizzled, it sits in slot
                        // piece ^ (row % 16) = piece ^ (lane % 16)
                        const unsigned char* kr =
                            kDma ? kb + (32 * kh + (lane & 31)) * 256 + (((2 * st + h32) ^ (lane & 15)) << 4)
                                 : kb + (32 * kh + (lane & 31)) * kKPitch + 16 * h32 + 32 * st;
                        const bf16x8 av = *reinterpret_cast<const bf16x8*>(kr);
                        s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[st], s[kh], 0, 0, 0);
                    }
                if (kDma) {
                    // three K operand reads in flight ahead of the MFMAs (measured: +2% over
                    // the compiler's own one-to-two; four is no better)
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
                    for (int i = 0; i < 8 * kKH - 3; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                }
            }
            if (kDma) __builtin_amdgcn_s_setprio(0);
            if (v_later) issue_half(t + 1, (t + 1) & 1, blk1, true);
            if (live_t) {
                // s[kh][r] = raw score (q . k, unscaled) of key j0 + 32kh + 8(r/4) + 4*h32 + r%4
                // for query qi.
                const bool need_mask = !ok || (j0 + kKT - 1 > off + wp0) || (j0 + kKT > Lk);
                if (need_mask) {
                    // key j0 + 4*h32 + c (c a compile-time offset) is visible iff c <= lim
                    const int lim = ok ? min(qpos, Lk - 1) - (j0 + 4 * h32) : -1;
#pragma unroll
                    for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int c = 32 * kh + 8 * (r >> 2) + (r & 3);
                            s[kh][r] = c > lim ? -INFINITY : s[kh][r];
                        }
                }
                float moff = 0.f;
                if (kExact) {
                    float tmax = -INFINITY;
#pragma unroll
                    for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
                        for (int r = 0; r < 16; r += 2)
                            tmax = __builtin_fmaxf(__builtin_fmaxf(tmax, s[kh][r]), s[kh][r + 1]);
                    {
                        // exchange with the lane 32 away without an LDS round trip (v_permlane32_swap)
                        const uint32_t tb = __float_as_uint(tmax);
                        const auto sw = __builtin_amdgcn_permlane32_swap(tb, tb, false, false);
                        tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                    }
                    const bool grow = tmax > m_run + lazy_raw;
                    if (__any(grow)) {
                        const float mn = grow ? tmax : m_run;
                        const float alpha =
                            m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - mn) * a.scale_log2);
                        m_run = mn;
                        l_part *= alpha;
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
                    }
                    moff = m_run == -INFINITY ? 0.f : -m_run * a.scale_log2;
                }
                // The weights enter P V rounded to bf16; the row sum adds up those same
                // rounded weights (bf16 dot2 with (1, 1), fp32 accumulate), so numerator
                // and denominator agree: a row dominated by one key returns that key's
                // value, not the value scaled by that weight's rounding error.
                float psum0 = 0.f, psum1 = 0.f;
                uint32_t pk[kKH][8];
#pragma unroll
                for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const float x0 = kExact ? fmaf(s[kh][r], a.scale_log2, moff) : s[kh][r] * a.scale_log2;
                        const float x1 = kExact ? fmaf(s[kh][r + 1], a.scale_log2, moff) : s[kh][r + 1] * a.scale_log2;
                        const float e0 = __builtin_amdgcn_exp2f(x0);
                        const float e1 = __builtin_amdgcn_exp2f(x1);
                        const uint32_t pw = pack_bf16x2(e0, e1);
                        pk[kh][r >> 1] = pw;
                        if (r & 2)
                            psum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw), kOnes2, psum1, false);
                        else
                            psum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw), kOnes2, psum0, false);
                    }
                l_part += psum0 + psum1;

                // ---- O^T += V^T P^T: per 16-key step (kh, v) the B operand is registers 8v..8v+7 of s[kh].
                // The A operand (V^T: row d = lane%32, 8 keys) comes from row-major V with two
                // transposing LDS reads: lane j of a 16-lane group addresses key j/4, dims 4*(j%4)
                // of a 4-key x 16-dim tile and receives its own dim across the 4 keys.
                const int grp16 = lane >> 4, j16 = lane & 15;
#pragma unroll
                for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        u32x4 bw = {pk[kh][4 * v], pk[kh][4 * v + 1], pk[kh][4 * v + 2], pk[kh][4 * v + 3]};
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
                        const int kcol = 32 * kh + 16 * v + 4 * h32;   // first key of this lane's k-slots
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) {
                            const int d0 = 32 * dt + 16 * (grp16 & 1) + 4 * (j16 & 3);
                            // swizzled: piece (2 d0)/16 of row kcol + j16/4 (row % 4 = j16/4) sits in
                            // slot piece ^ 4(j16/4), i.e. dims 32 dt move to 32 (dt ^ j16/4)
                            const int vo = kDma ? 64 * (dt ^ (j16 >> 2)) + 32 * (grp16 & 1) + 8 * (j16 & 3) : 2 * d0;
                            lds_ptr_t p0 = (lds_ptr_t)(vb + (kcol + (j16 >> 2)) * kVP + vo);
                            lds_ptr_t p1 = (lds_ptr_t)(vb + (kcol + 8 + (j16 >> 2)) * kVP + vo);
                            const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0);
                            const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1);
                            const bf16x8 av = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, oacc[dt], 0, 0, 0);
                        }
                    }
            }
            if (!kDma) {
                if (t + 1 < n_tiles)
                    store_tile(t + 1, k_lds + ((t + 1) & 1) * kKTileBytes, v_lds + ((t + 1) & 1) * kVTileBytes);
                __syncthreads();
                if (t + 2 < n_tiles) load_tile(t + 2);
            }
            ok_cur = ok_next;
        }
    }

    if (split) {
        // this chunk's share: O^T accumulators and row sums, summed by the merge kernel
        const int lane_e = __lane_id();
        float* pp = part + ((size_t)(work * nc + c) * NW + (threadIdx.x >> 6)) * kPartFloats;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) pp[(dt * 16 + r) * 64 + lane_e] = oacc[dt][r];
        pp[64 * 64 + lane_e] = l_part;
        return;
    }
    prefill_finish<!kExact>(a, call, cq0, Lq, wp0, head, wave_live, oacc, l_part);
}

// Work item of the kx-th workgroup of XCD xcd (XCDs take workgroups round-robin
// by id).  Work items are numbered unit * m_blocks + i, where a unit is one
// (sequence, kv head, head group) and i = 0 is its heaviest (last) query block.
// With fewer units than XCDs (chunk < m_blocks) the items go out in chunks of 2
// blocks, round-robin.  Otherwise XCD x runs units x, x+8, x+16, ..., so each
// unit's K/V stays in one L2, taken `win` units at a time: within such a window
// the 4 heaviest blocks of every unit come first, then the next 4, and so on.  A
// window of one unit runs each unit's blocks in turn; wider windows let the long
// sequences of a ragged batch start at once instead of after the units dealt
// before them (the XCD dispatches in order, so a late heavy block is a late end).
// Blocks of one unit dealt together: an XCD hands consecutive workgroups to its 4
// shader engines in turn, so a group of 4 spreads each unit over all of them.
constexpr int kDealGroup = 4;
__device__ __forceinline__ int deal_item(int xcd, int kx, int chunk, int win, int m_blocks, int n_work) {
    if (chunk < m_blocks || win <= 1) return (xcd + 8 * (kx / chunk)) * chunk + kx % chunk;
    const int nu = (n_work / m_blocks + 7) / 8;    // units per XCD in the grid
    const int span = win * m_blocks;
    const int w = kx / span, r = kx - w * span;
    const int ws = min(win, nu - w * win);          // units in this window (the last may be short)
    if (ws <= 0) return n_work;                     // past the grid's items: none
    // rounds of kDealGroup blocks per unit, so each unit's blocks still go to
    // consecutive workgroup slots (spread over the XCD's shader engines)
    const int full = m_blocks / kDealGroup, head = full * ws * kDealGroup;
    int j, i;
    if (r < head) {
        const int round = r / (ws * kDealGroup), rr = r - round * ws * kDealGroup;
        j = rr / kDealGroup;
        i = round * kDealGroup + rr % kDealGroup;
    } else {
        const int last = m_blocks - full * kDealGroup, rr = r - head;
        j = rr / last;
        i = full * kDealGroup + rr % last;
    }
    return (xcd + 8 * (w * win + j)) * m_blocks + i;
}

// The two passes are separate kernels so that the exact pass's code does not
// change how the compiler schedules the fast pass's loop.  The launcher runs the
// fast pass, then the exact pass as a persistent kernel of at most one
// workgroup per CU slot, which exits at once unless this call flagged something.
template <int GW, bool PAGED, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) prefill_kernel(PrefillArgs a, int32_t m_blocks, int32_t n_work,
                                                                  int32_t head_groups, int32_t chunk, int32_t win,
                                                                  uint64_t call, int32_t nc, float* part) {
    constexpr int kKT = kTileKeys<NW>;
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[2 * kKT * kHeadDim * 2];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[2 * kKT * kHeadDim * 2];

    // Work items by deal_item.  With a key split (nc > 1) the nc chunks of each item take consecutive slots of
    // its XCD, so they run side by side and share the item's K/V in one L2.
    const int xcd = blockIdx.x & 7;
    int kx = blockIdx.x >> 3, c = 0;
    if (nc > 1) {
        c = kx % nc;
        kx /= nc;
    }
    const int work = deal_item(xcd, kx, chunk, win, m_blocks, n_work);
    if (work >= n_work) return;
    prefill_block<GW, PAGED, NW, false>(a, m_blocks, head_groups, work, (lds_byte*)k_lds, (lds_byte*)v_lds, call, c,
                                        nc, part);
}


// Key split: one wave per (work item, 32-row block).  Sums the chunks' partial O^T
// and row sums in chunk order (deterministic), then finishes as the fast pass does
// (range check, marker or normalised store).
template <int GW, bool PAGED, int NW>
__global__ void __launch_bounds__(64) prefill_merge_kernel(PrefillArgs a, int32_t m_blocks, int32_t n_work,
                                                           int32_t head_groups, int32_t nc, const float* part,
                                                           uint64_t call) {
    constexpr int kKT = kTileKeys<NW>;
    constexpr int kBM = kRowsPerWave * (NW / GW);
    const int work = blockIdx.x / NW, wave = blockIdx.x % NW;
    if (work >= n_work) return;
    const int mb = m_blocks - 1 - (work % m_blocks);
    int rest = work / m_blocks;
    const int hg = rest % head_groups;
    rest /= head_groups;
    const int g = rest % a.hkv;
    const int b = rest / a.hkv;
    const int cq0 = a.cu_q[b], cq1 = a.cu_q[b + 1];
    const int ck0 = a.cu_k[b], ck1 = a.cu_k[b + 1];
    const int Lq = cq1 - cq0, Lk = ck1 - ck0;
    const int p0 = mb * kBM;
    if (p0 >= Lq || Lk < Lq || Lq <= 0) return;
    if (cq0 < 0 || cq1 > a.total_q || ck0 < 0) return;
    const int off = Lk - Lq;
    const int n_tiles = (off + min(p0 + kBM, Lq) + kKT - 1) / kKT;
    const int nc_item = item_chunks(n_tiles, nc);
    if (nc_item < 2) return;
    const int lane = threadIdx.x;
    const int head = g * (a.hq / a.hkv) + hg * GW + (wave % GW);
    const int wp0 = p0 + kRowsPerWave * (wave / GW);
    f32x16 oacc[4];
    float l_part = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    // each chunk's 65 loads issued together, then added in chunk order
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c >= nc_item) break;
        const float* pp = part + ((size_t)(work * nc + c) * NW + wave) * kPartFloats;
        f32x16 t[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) t[dt][r] = __builtin_nontemporal_load(pp + (dt * 16 + r) * 64 + lane);
        const float tl = __builtin_nontemporal_load(pp + 64 * 64 + lane);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] += t[dt];
        l_part += tl;
    }
    prefill_finish<true>(a, call, cq0, Lq, wp0, head, wp0 < Lq, oacc, l_part);
}

// call != 0: after the fast pass, recompute the work items it flagged (exits at
// once if this call flagged none).  call == 0: the whole batch with the exact
// pass, one workgroup per work item in the fast pass's XCD order (small batches,
// where a second launch would cost more than the fast pass saves).
template <int GW, bool PAGED, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) prefill_exact_kernel(PrefillArgs a, int32_t m_blocks,
                                                                        int32_t n_work, int32_t head_groups,
                                                                        int32_t chunk, int32_t win, int32_t n_iter,
                                                                        uint64_t call) {
    constexpr int kKT = kTileKeys<NW>;
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[2 * kKT * kKPitch];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[2 * kKT * kVPitch];
    if (call != 0 &&
        __hip_atomic_load(&g_prefill_flagged_call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < call)
        return;
    // Every workgroup walks the same item sequence, so the barriers inside match.
    for (int i = blockIdx.x; i < n_iter; i += gridDim.x) {
        const int xcd = i & 7, kx = i >> 3;
        const int work = call != 0 ? i : deal_item(xcd, kx, chunk, win, m_blocks, n_work);
        if (work >= n_work) continue;
        prefill_block<GW, PAGED, NW, true>(a, m_blocks, head_groups, work, (lds_byte*)k_lds, (lds_byte*)v_lds, call);
    }
}

namespace {
// Launch shape of a call, shared by the launcher and the workspace query.
struct PrefillPlan {
    bool ok = false;
    int gw = 0, head_groups = 0, nw = 0, m_blocks = 0, n_work = 0, grid = 0, grid_exact = 0, n_iter = 0;
    int64_t chunk = 0;
    int win = 1;               // units per dealing window (deal_item)
    bool wide = false, two_pass = false;
    int split_nc = 1;          // chunks per split item (1: no split)
    size_t split_bytes = 0;    // workspace the split needs
};

PrefillPlan plan_prefill(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                         int32_t hkv) {
    PrefillPlan p;
    if (num_seqs <= 0 || total_q <= 0 || max_seqlen_q <= 0 || hq <= 0 || hkv <= 0 || hq % hkv) return p;
    const int G = hq / hkv;
    p.gw = G >= 4 ? 4 : G;                 // query heads per workgroup
    if (G % p.gw) return p;
    p.head_groups = G / p.gw;
    // 8 waves (64 positions x 4 heads, or 128 x 2, 128-key tiles) for long
    // sequences; 4 waves (smaller workgroups, more of them) for short ones.  With
    // 4 heads a workgroup, queries of 1024+ positions on average that sit after
    // cached prefixes (the longest key range at least twice the longest query)
    // also take 8 waves: 5-7% faster on such prefix hits, equal on the rest; with
    // 2 heads the same rule was faster on some prefix batches and slower on others.
    p.wide = p.gw >= 2 && ((int64_t)total_q >= (int64_t)2048 * num_seqs ||
                           (p.gw == 4 && (int64_t)total_q >= (int64_t)1024 * num_seqs &&
                            (int64_t)max_seqlen_k >= (int64_t)2 * max_seqlen_q));
    p.nw = p.wide ? 8 : 4;
    const int bm = kRowsPerWave * (p.nw / p.gw);
    p.m_blocks = (int)(((int64_t)max_seqlen_q + bm - 1) / bm);
    const int64_t n_work64 = (int64_t)num_seqs * hkv * p.head_groups * p.m_blocks;
    if (n_work64 > (int64_t)0x7FFFFFF0) return p;
    p.n_work = (int)n_work64;
    // Whole units (all query blocks of a sequence and kv head) per XCD keep their
    // K/V in one L2; with fewer units than XCDs they are cut into 2-block chunks.
    const int64_t units = n_work64 / p.m_blocks;
    p.chunk = units >= 8 ? p.m_blocks : (p.m_blocks < 2 ? p.m_blocks : 2);
    const int64_t n_chunks = (n_work64 + p.chunk - 1) / p.chunk;
    const int64_t grid64 = ((n_chunks + 7) / 8) * 8 * p.chunk;
    if (grid64 > (int64_t)0x7FFFFFF0 / 4) return p;
    p.grid = (int)grid64;
    // Dealing window (deal_item): an XCD share of at most kWindowUnits units whose
    // K/V (at most max_seqlen_k keys each) fits in kWindowBytes is dealt as one
    // window, so the long sequences of a small ragged batch start at once (the
    // 0.6B varlen batch: 60 -> 56 us).  Larger shares keep one unit at a time:
    // windows there cost 2-7% (16 x 2048, 64 x 512, 8B prefix hits) and up to 13%
    // with long cached prefixes, as the units' K/V no longer share the L2.
    if (p.chunk == p.m_blocks) {
        const int64_t unit_bytes = std::max<int64_t>(max_seqlen_k, 1) * kHeadDim * 2 * 2;
        const int64_t nu = (units + 7) / 8;
        if (nu > 1 && nu <= kWindowUnits && nu * unit_bytes <= kWindowBytes) p.win = (int)nu;
    }
    // Batches under 2e10 FLOP (counted without the causal half, so roughly under
    // 20 us of work) run the exact pass alone in one launch: there the second
    // launch of the two-pass scheme (~4 us when nothing is flagged) costs more than
    // the fast pass saves (measured: two passes 10% slower at 16 x 128 tokens,
    // even at 4 x 512, 7-9% faster from 8 x 1024 and on 16 x 2048 queries over
    // 4096 keys).
    p.two_pass = (double)total_q * max_seqlen_k * hq * 4.0 * kHeadDim >= 2e10;
    // Exact pass after the fast one: one workgroup per CU slot (two 4-wave or one
    // 8-wave per CU), walking the work items.
    const int slots = p.nw == 8 ? 256 : 512;
    p.grid_exact = p.two_pass ? (int)std::min<int64_t>(n_work64, slots) : p.grid;
    p.n_iter = p.two_pass ? p.n_work : p.grid;
    // Key split: when the items that hold queries (at most one partial query block
    // per sequence beyond total_q / block) do not fill the CU slots and keys run
    // long, the fast pass cuts every item of at least 2 * kSplitMinChunkTiles tiles
    // into slots / items + 1 chunks (2 to 4), whose partial sums a merge kernel
    // adds.  Measured on 4 x 256 queries over 16384 cached keys at 32/8 heads (288
    // items): 322 -> 279 us per call with two chunks (dealing every unit's heaviest
    // block first on top of that: no change).  The 0.6B varlen batch (944
    // items for 512 slots) is left whole: split in two, it ran 56 -> 69 us (the
    // merge over all its items alone takes 9 us).
    const int kt = p.nw == 8 ? 128 : 64;
    const int64_t max_tiles = ((int64_t)max_seqlen_k + kt - 1) / kt;
    const int64_t n_real = (((int64_t)total_q + bm - 1) / bm + num_seqs) * hkv * p.head_groups;
    if (p.two_pass && n_real <= slots && max_tiles >= 2 * kSplitMinChunkTiles) {
        const int nc = (int)std::min<int64_t>(4, slots / std::max<int64_t>(n_real, 1) + 1);
        const size_t bytes = (size_t)p.n_work * nc * p.nw * kPartFloats * sizeof(float);
        if (nc >= 2 && bytes <= kSplitMaxBytes) {
            p.split_nc = nc;
            p.split_bytes = bytes;
        }
    }
    p.ok = true;
    return p;
}
}  // namespace

size_t prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t hq, int32_t hkv) {
    const PrefillPlan p = plan_prefill(num_seqs, total_q, max_seqlen_q, max_seqlen_k, hq, hkv);
    return p.ok && p.split_nc > 1 ? p.split_bytes : 0;
}

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.total_q == 0 || a.max_seqlen_q == 0) return hipSuccess;
    const PrefillPlan p = plan_prefill(a.num_seqs, a.total_q, a.max_seqlen_q, a.max_seqlen_k, a.hq, a.hkv);
    if (!p.ok) return hipErrorInvalidValue;
    const int gw = p.gw, head_groups = p.head_groups, m_blocks = p.m_blocks, n_work = p.n_work, grid = p.grid;
    const int grid_exact = p.grid_exact, n_iter = p.n_iter;
    const int64_t chunk = p.chunk;
    const int win = p.win;
    const bool wide = p.wide, two_pass = p.two_pass;
    // The key split runs only with a workspace of the planned size (else the call
    // runs unsplit, with the same results up to summation order).
    const int nc = p.split_nc > 1 && a.workspace && a.workspace_bytes >= p.split_bytes &&
                           (uintptr_t)a.workspace % 256 == 0
                       ? p.split_nc
                       : 1;
    float* part = nc > 1 ? (float*)a.workspace : nullptr;
    // Each two-pass call gets a number of its own, so the exact pass can tell
    // whether this call's fast pass flagged anything (the device keeps the
    // highest number seen).  0 means exact pass only.
    static std::atomic<uint64_t> s_calls{0};
    const uint64_t call = two_pass ? s_calls.fetch_add(1, std::memory_order_relaxed) + 1 : 0;
    const bool paged = a.block_table != nullptr;
#define PKV_PREFILL(GW_, PG_, NW_)                                                                               \
    do {                                                                                                         \
        if (two_pass)                                                                                            \
            hipLaunchKernelGGL((prefill_kernel<GW_, PG_, NW_>), dim3(grid * nc), dim3(64 * NW_), 0, stream, a,   \
                               m_blocks, n_work, head_groups, (int32_t)chunk, win, call, nc, part);              \
        if (nc > 1)                                                                                              \
            hipLaunchKernelGGL((prefill_merge_kernel<GW_, PG_, NW_>), dim3(n_work * NW_), dim3(64), 0, stream,   \
                               a, m_blocks, n_work, head_groups, nc, part, call);                                \
        hipLaunchKernelGGL((prefill_exact_kernel<GW_, PG_, NW_>), dim3(grid_exact), dim3(64 * NW_), 0, stream,   \
                           a, m_blocks, n_work, head_groups, (int32_t)chunk, win, n_iter, call);                 \
    } while (0)
    if (gw == 4) {
        if (wide) {
            if (paged) PKV_PREFILL(4, true, 8); else PKV_PREFILL(4, false, 8);
        } else {
            if (paged) PKV_PREFILL(4, true, 4); else PKV_PREFILL(4, false, 4);
        }
    } else if (gw == 2) {
        if (wide) {
            if (paged) PKV_PREFILL(2, true, 8); else PKV_PREFILL(2, false, 8);
        } else {
            if (paged) PKV_PREFILL(2, true, 4); else PKV_PREFILL(2, false, 4);
        }
    } else if (gw == 1) {
        if (paged) PKV_PREFILL(1, true, 4); else PKV_PREFILL(1, false, 4);
    } else {
        return hipErrorInvalidValue;
    }
#undef PKV_PREFILL
    return hipGetLastError();
}

}  // namespace pkv
