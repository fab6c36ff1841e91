/*
 * pkv.h -- C ABI of libpkv: the Qwen3 attention-sublayer core on MI355X (gfx950).
 *
 * The library runs four steps of one attention sublayer, each on the caller's
 * HIP stream, in the order the attention pages describe them:
 *
 *   pkv_qk_norm_rope         per-head RMSNorm of q and k, then RoPE
 *   pkv_store_kvcache        scatter of k and v rows into the paged KV cache
 *   pkv_attn_prefill_varlen  varlen causal GQA prefill (fresh K/V or paged)
 *   pkv_attn_prefill_workspace_bytes  its optional key-split workspace
 *   pkv_attn_decode_paged    single-token paged decode
 *
 * plus pkv_rope_cache_build, which fills the cos/sin table once at set-up,
 * pkv_qk_norm_rope_store, the first two steps in one pass (rotated k and v go
 * straight to their cache rows), the decode step (pkv_decode_step) with
 * its HIP-graph replay per batch bucket (pkv_decode_graph_*), and the
 * elementwise steps on either side of attention in a decoder layer:
 * pkv_add_rms_norm, pkv_silu_and_mul and the sampler pkv_sample_gumbel.
 *
 * Conventions for every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     stated otherwise.  The library keeps no pointer after a call returns.
 *   - bf16 tensors are passed as raw 16-bit patterns (void*).  Integer
 *     metadata is int32 except positions (int64).
 *   - Row strides are counted in ELEMENTS, not bytes.  Inside a row, heads
 *     are contiguous blocks of head_dim elements and head_dim elements are
 *     contiguous (the pages' stride(-1) == 1, stride(1) == head_dim).
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued asynchronously; no entry point synchronises, allocates or
 *     frees device memory.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid argument returns a negative status and nothing is launched.
 *     pkv_last_error() then returns a thread-local message.
 *   - Contents of device arrays (slot ids, block ids, lengths) cannot be
 *     checked on the host.  Kernels never access memory outside the buffers
 *     the sizes describe: a slot outside [0, num_slots) is not written, a
 *     block id outside [0, num_blocks) is not read and the key it would hold
 *     is dropped from the softmax.  Results for rows whose metadata is
 *     invalid are unspecified.
 *   - Only head_dim == 128 and block_size == 256 are built (Qwen3 shapes);
 *     other values return PKV_ERR_UNSUPPORTED.
 *
 * Citations name the page and section that defines each operation:
 *   "3.3 Model skeleton and core operators" (infra-guide)        = [Ops]
 *   "Nano-vLLM 源码解读 #17 注意力层" (yeyulingfeng)             = [Attn17]
 *   "同一个 Qwen3，两种写法" (violet-quartz)                      = [TwoWays]
 *   "nano-vllm code walkthrough" (roba269)                        = [Walk]
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef PKV_API
#define PKV_API __attribute__((visibility("default")))
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1,  /* null pointer, bad size or stride, Hq % Hkv != 0, ... */
    PKV_ERR_UNSUPPORTED = -2,  /* head_dim != 128, block_size != 256, causal == 0, ... */
    PKV_ERR_LAUNCH = -3,       /* the HIP runtime refused a launch */
    PKV_ERR_WORKSPACE = -4     /* decode workspace missing or too small */
} pkv_status;

/* Message describing the last failure on the calling thread ("" if none).
 * The string stays valid until the next pkv_* call on the same thread. */
PKV_API const char* pkv_last_error(void);

/* Library version, (major << 16) | minor. */
PKV_API int pkv_version(void);

/*
 * pkv_rope_cache_build -- cos/sin table for RoPE, [Ops] s3; [TwoWays] s3.5.
 *
 *   cos_sin_cache  device fp32 [max_position][rotary_dim], written entirely.
 *                  Row p = [cos(p f_0) .. cos(p f_{r/2-1}) | sin(p f_0) .. sin(p f_{r/2-1})]
 *                  with f_i = fp32(theta^(-2i/rotary_dim)); the angle is the fp32
 *                  product fp32(p) * f_i and cos/sin of it are rounded to fp32.
 *   max_position   number of rows (the pages use 40960), > 0.
 *   rotary_dim     must equal head_dim (the pages assert rotary_dim == head_size): 128.
 *   theta          rope_theta (1e6 for Qwen3), > 0.
 * One table serves every layer; build it once and keep it.
 */
PKV_API int pkv_rope_cache_build(float* cos_sin_cache, int32_t max_position, int32_t rotary_dim, double theta,
                         void* stream);

/*
 * pkv_qk_norm_rope -- QK-Norm then RoPE on q and k, [Ops] s2, s3, s8;
 * [Attn17] s4.  For every token t and head h of q (and of k):
 *     r   = 1 / sqrt(mean_i x_i^2 + eps)
 *     y_i = x_i * r * gamma_i                    (gamma = q_norm / k_norm weight)
 *     (c, s) = cos_sin_cache[positions[t]] halves
 *     out[i]      = y_i * c_i - y_{i+64} * s_i
 *     out[i + 64] = y_{i+64} * c_i + y_i * s_i    (i < 64)
 * computed in fp32 and rounded once to bf16 (round to nearest even).
 *
 *   q, q_row_stride     bf16 rows of num_q_heads*head_dim elements (e.g. the q
 *                       columns of the fused qkv rows: stride = qkv width).
 *   k, k_row_stride     bf16 rows of num_kv_heads*head_dim elements.
 *   q_out, k_out        bf16, contiguous [n_tokens][heads][head_dim].  They may
 *                       alias q / k exactly (in place) when the strides equal
 *                       the contiguous row length; partial overlap is invalid.
 *   positions           int64 [n_tokens]; each in [0, max_position) (positions
 *                       outside are clamped to the table range).
 *   q_norm_weight, k_norm_weight   bf16 [head_dim].
 *   cos_sin_cache       fp32 [max_position][head_dim] from pkv_rope_cache_build.
 * n_tokens == 0 is valid and launches nothing.  V is not touched ([Ops] s3).
 */
PKV_API int pkv_qk_norm_rope(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride, void* q_out,
                     void* k_out, const int64_t* positions, int32_t n_tokens, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, const void* q_norm_weight, const void* k_norm_weight,
                     float eps, const float* cos_sin_cache, int32_t max_position, void* stream);

/*
 * pkv_store_kvcache -- scatter of this step's K/V rows into the paged cache,
 * [Ops] s7.1; [Attn17] s5.1.  For each token t with s = slot_mapping[t]:
 *     s == -1           -> nothing is written (padding rows)
 *     0 <= s < num_slots -> k_cache row s = key row t, v_cache row s = value row t
 * A row is D = num_kv_heads * head_dim elements of elem_bytes bytes, copied
 * bit for bit.  The caches are [num_blocks][block_size][num_kv_heads][head_dim]
 * viewed as num_slots = num_blocks * block_size contiguous rows of D elements
 * (the pages' k_cache.stride(1) == D).  Duplicate slots within one call are
 * invalid input: which row lands is unspecified.
 *
 *   key, key_row_stride       rows of D elements, key_row_stride >= D.
 *   value, value_row_stride   rows of D elements (e.g. the v columns of qkv).
 *   slot_mapping              int32 [n_tokens].
 *   elem_bytes                2 for bf16 (any of 1, 2, 4 is accepted).
 */
PKV_API int pkv_store_kvcache(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                      void* k_cache, void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                      int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes, void* stream);

/*
 * pkv_qk_norm_rope_store -- pkv_qk_norm_rope and pkv_store_kvcache in one
 * pass, [Ops] s3, s7.1, s8; [Attn17] s4, s5.1.  Per token t the rotated key
 * heads are written straight into k_cache row slot_mapping[t] and the value
 * heads into v_cache row slot_mapping[t]; the rotated query heads go to q_out.
 * Every value written is bit-identical to calling pkv_qk_norm_rope and then
 * pkv_store_kvcache(k_out, ..., v, ...) with the same arguments.
 *
 *   q, k, q_out, positions, norm weights, cos_sin_cache, max_position:
 *                   as for pkv_qk_norm_rope (q_out may alias q exactly).
 *   v, v_row_stride value rows of num_kv_heads*head_dim bf16 (e.g. the v
 *                   columns of the qkv rows); read only.
 *   k_out           optional contiguous [n_tokens][num_kv_heads][head_dim] copy
 *                   of the rotated keys (NULL: not written).  It may alias k
 *                   exactly when k is contiguous.
 *   k_cache, v_cache, num_slots, slot_mapping:
 *                   as for pkv_store_kvcache with elem_bytes 2; a slot outside
 *                   [0, num_slots), -1 included, writes no cache row (q_out and
 *                   k_out are still written).  The caches must not overlap
 *                   q, k, v or the outputs.
 */
PKV_API int pkv_qk_norm_rope_store(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                                   const void* v, int64_t v_row_stride, void* q_out, void* k_out, void* k_cache,
                                   void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                                   const int64_t* positions, int32_t n_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, const void* q_norm_weight,
                                   const void* k_norm_weight, float eps, const float* cos_sin_cache,
                                   int32_t max_position, void* stream);

/*
 * pkv_attn_prefill_varlen -- causal GQA attention over a packed batch of
 * variable-length sequences, [Ops] s7.2; [TwoWays] s3.2, s3.4; [Walk]
 * "Prefill stage".  Sequence b owns query rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 (Lq_b of them) and Lk_b = cu_seqlens_k[b+1]-cu_seqlens_k[b]
 * >= Lq_b keys.  Query i of sequence b sits at absolute position Lk_b - Lq_b + i
 * and attends keys 0 .. Lk_b - Lq_b + i:
 *     o[t][h] = sum_j softmax_j(softmax_scale * q[t][h] . k_j) v_j
 * with q head h reading kv head h / (num_q_heads / num_kv_heads).
 *
 *   block_table == NULL ("case 1", fresh K/V): key j of sequence b is row
 *       cu_seqlens_k[b] + j of k / v (row strides k_row_stride / v_row_stride,
 *       each at most 2^24 elements).
 *   block_table != NULL ("case 2", prefix hit or later chunk): k and v are the
 *       caches [num_blocks][block_size][num_kv_heads][head_dim]; key j of
 *       sequence b is cache row block_table[b][j / block_size] * block_size
 *       + j % block_size.  The row strides must be num_kv_heads*head_dim.
 *       num_blocks bounds the ids read (ids outside are never dereferenced).
 *   q, q_row_stride   bf16 rows of num_q_heads*head_dim elements.
 *   o                 bf16 contiguous [Tq][num_q_heads][head_dim], Tq = cu_seqlens_q[num_seqs];
 *                     must not overlap q.
 *   cu_seqlens_q/k    int32 [num_seqs+1], non-decreasing, starting at 0.
 *   max_seqlen_q      >= every Lq_b (sizes the launch grid); max_seqlen_k >= every Lk_b.
 *   total_q           cu_seqlens_q[num_seqs] (host copy, bounds the q/o rows touched).
 *   causal            must be 1 (the pages only use causal attention).
 * Sequences with Lq_b == 0 contribute nothing.  Output rows are written in
 * full for every query row.
 *
 *   workspace, workspace_bytes
 *                     optional device scratch (NULL, 0: none), 256-byte aligned,
 *                     not overlapping any other argument.  When it holds at least
 *                     pkv_attn_prefill_workspace_bytes(...) (> 0) bytes, a batch
 *                     with few query blocks and long key ranges splits each long
 *                     block's keys over several workgroups and adds their partial
 *                     sums in a fixed order; otherwise the call runs unsplit.  The
 *                     two differ only in fp32 summation order.  Contents on entry
 *                     do not matter; the call owns the bytes until its work on
 *                     `stream` completes.
 *
 * Large batches run as two kernels on `stream`: a fast pass, then a pass that
 * recomputes any work item whose softmax sums left the fast pass's range (until
 * then such rows of o hold a marker value, so o is complete only when the call's
 * work on `stream` is); a split call adds a merge kernel between them.  The
 * library keeps one 8-byte device word per GPU for this; calls on several streams
 * may overlap (each with its own workspace), and a call may be captured into a
 * HIP graph and replayed.
 */
PKV_API int pkv_attn_prefill_varlen(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                            const void* v, int64_t v_row_stride, void* o, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            float softmax_scale, int32_t causal, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pkv_attn_prefill_workspace_bytes -- workspace pkv_attn_prefill_varlen splits
 * key ranges with for a call of these sizes (arguments as there); 0 when such a
 * call does not split (many query blocks, short keys, or invalid sizes).  At
 * most 512 MiB.
 */
PKV_API size_t pkv_attn_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                                int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim);

/*
 * pkv_attn_decode_workspace_bytes -- device workspace pkv_attn_decode_paged
 * needs for these sizes (0 on invalid sizes, and on sizes past the launch grid:
 * more than 65535 sequences, or tables so long that a sequence would need more
 * than 65535 splits; the decode calls refuse those with PKV_ERR_UNSUPPORTED).
 * Host-only, no HIP call.
 */
PKV_API size_t pkv_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size);

/*
 * pkv_attn_decode_paged -- one new query per sequence against its paged KV,
 * [Ops] s7.2; [Walk] "Decode Stage"; [Attn17] s5.3.  Sequence b attends its
 * first context_lens[b] cached keys (the token written this step included):
 *     o[b][h] = sum_{j < ctx_b} softmax_j(softmax_scale * q[b][h] . k_j) v_j
 * key j at cache row block_table[b][j / block_size] * block_size + j % block_size,
 * q head h reading kv head h / (num_q_heads / num_kv_heads).  context_lens[b] == 0
 * gives a zero output row (padded rows of a fixed-size batch).
 *
 *   q                 bf16 contiguous [num_seqs][num_q_heads][head_dim].
 *   k_cache, v_cache  bf16 [num_blocks][block_size][num_kv_heads][head_dim].
 *   o                 bf16 contiguous [num_seqs][num_q_heads][head_dim].
 *   context_lens      int32 [num_seqs], each <= max_blocks_per_seq * block_size.
 *   block_table       int32 [num_seqs][max_blocks_per_seq], -1 padded.
 *   workspace         device scratch of at least
 *                     pkv_attn_decode_workspace_bytes(...) bytes, 256-byte aligned,
 *                     sharing no byte with q, o or the caches (else PKV_ERR_WORKSPACE);
 *                     owned by the caller, contents need no initialisation.
 * The split of each context into chunks and their merge are deterministic:
 * the result does not depend on where the blocks sit in the pool.
 */
PKV_API int pkv_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o,
                          const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks_per_seq,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, float softmax_scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * pkv_attn_decode_paged_noalloc -- pkv_attn_decode_paged without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * same kernels run; the split-K partials live in a fixed device array inside
 * the library (one per GPU, 96 MiB, kept until the process ends).  Arguments,
 * layouts and results are those of pkv_attn_decode_paged, byte for byte.
 *
 *   Sizes: a call needing more than 96 MiB of workspace (see
 *   pkv_attn_decode_workspace_bytes; the Qwen3-8B batch of 256 sequences with
 *   128-block tables needs 65 MiB) returns PKV_ERR_WORKSPACE and launches
 *   nothing.  Nothing is allocated or freed; the first call on a device looks
 *   up the array's device address once.
 *   Concurrency: every call on one GPU uses the same array, so calls whose
 *   execution overlaps on one GPU (different streams, or different host
 *   threads) race and must be serialised by the caller; calls in order on one
 *   stream are safe.
 */
PKV_API int pkv_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                  const int32_t* context_lens, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  float softmax_scale, void* stream);

/*
 * pkv_add_rms_norm -- residual add folded into RMSNorm, [Ops] s2 (RMSNorm
 * and its residual entry point); [TwoWays] s3.6 (one pass: read x and the
 * residual, write y and the new residual).  Per row of `hidden` elements:
 *     s_i      = fp32(x_i) + fp32(residual_i)        (one IEEE fp32 add)
 *     res'_i   = bf16(s_i)                           (the new residual)
 *     r        = 1 / sqrt(mean_i s_i^2 + eps)        (fp32)
 *     y_i      = bf16(bf16(s_i * r) * gamma_i)       (rounded, then times gamma)
 * With residual == NULL (and residual_out == NULL) the input itself is
 * normalised: s_i = x_i (the pages' rms_forward, used before the first layer).
 *
 *   x, residual, y, residual_out   bf16 contiguous [n_tokens][hidden]; y may
 *                                  alias x and residual_out may alias residual
 *                                  (in place); y != residual_out.
 *   weight                         bf16 [hidden] (gamma).
 *   hidden                         multiple of 8, at most 16384.
 */
PKV_API int pkv_add_rms_norm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                             int32_t n_tokens, int32_t hidden, float eps, void* stream);

/*
 * pkv_silu_and_mul -- SwiGLU activation, [Ops] s4.  Row t of x holds gate
 * (columns 0..I-1) then up (columns I..2I-1):
 *     out[t][i] = bf16(silu(gate_i) * up_i),  silu(g) = g / (1 + exp(-g)),
 * in fp32 with one rounding.
 *   x, x_row_stride       bf16 rows of >= 2 * intermediate elements.
 *   out, out_row_stride   bf16 rows of >= intermediate elements; must not
 *                         overlap x.  Strides multiples of 8 elements.
 */
PKV_API int pkv_silu_and_mul(const void* x, int64_t x_row_stride, void* out, int64_t out_row_stride,
                             int32_t n_tokens, int32_t intermediate, void* stream);

#define PKV_DTYPE_BF16 0
#define PKV_DTYPE_F32 1

/*
 * pkv_sample_gumbel -- one token per row by the Gumbel-max form of sampling,
 * [Ops] s9: logits / temperature, softmax p, E ~ Exp(1) clamped below at
 * 1e-10, token = argmax_i p_i / E_i (lowest index on ties).  The kernel takes
 * the argmax of the equivalent score (l_i / T) log2(e) - log2(E_i) (the
 * softmax normaliser is the same for every token of a row), in fp32.
 *
 *   logits, logits_row_stride, logits_dtype   [num_rows][vocab] bf16 or fp32
 *                      (PKV_DTYPE_*), rows 16-byte aligned.
 *   temperatures       fp32 [num_rows], each > 0 (values below 1e-10 act as 1e-10).
 *   noise              NULL: E is drawn in the kernel from Philox4x32-10 with
 *                      key (seed low 32 bits, seed high 32 bits) and counter
 *                      (column / 4, row, offset low, offset high), word column % 4;
 *                      the top 24 bits k give u = (k + 1) / 2^24 and E = -ln(u).
 *                      Otherwise fp32 [num_rows][noise_row_stride] holding E.
 *   tokens             int64 [num_rows], 8-byte aligned, written.  During the
 *                      call it also serves as each row's reduction slot (the
 *                      row's workgroups combine their winners there with 64-bit
 *                      atomics), so it must not overlap the other arguments.
 * Rows whose scores are all NaN return token 0.  Three launches on `stream`:
 * clear the slots, sample, turn each slot's key into the token index.
 */
PKV_API int pkv_sample_gumbel(const void* logits, int64_t logits_row_stride, int32_t logits_dtype,
                              const float* temperatures, const float* noise, int64_t noise_row_stride, uint64_t seed,
                              uint64_t offset, int64_t* tokens, int32_t num_rows, int32_t vocab, void* stream);

/*
 * The decode step of the attention core, eager or from HIP graphs,
 * [Walk] "Misc implementation details" (graphs for the decode stage, one per
 * batch size 1, 2, 4, 8, ...; the smallest one that fits is replayed);
 * [Ops] s7.1 (padded rows carry slot -1 and are not written).
 *
 * One step over `batch` sequences is
 *     pkv_qk_norm_rope_store(q, k, v columns of qkv rows 0..batch-1 -> q_out,
 *                            k_cache / v_cache at slot_mapping)
 *     pkv_attn_decode_paged(q_out -> o, context_lens, block_table)
 * on the buffers the descriptor names, with the same checks and, bit for bit,
 * the same results, run as two kernels: the decode split kernel applies
 * QK-Norm + RoPE to the rows it attends with and stores each row's new k' / v,
 * then the merge.  The equality needs what the engine's metadata gives: each
 * row's slot is the cache row of its key context_lens[b] - 1 (or -1 for a
 * padded row).  Otherwise the slot is still written, but the row's attention
 * reads whatever that key's cache row holds.  Those buffers are owned by the caller,
 * sized for max_batch rows, and must stay allocated and at the same addresses
 * while a graph built from the descriptor exists (a graph bakes them in): a
 * caller writes each step's inputs into them, then launches.
 */
/* pkv_decode_step_desc.flags: the caller keeps rows [batch, bucket) of
 * slot_mapping and context_lens at -1 and 0 itself (as the pages' runner fills
 * its static buffers before a replay), so pkv_decode_graph_launch enqueues the
 * captured graph alone, without its one-kernel padding step. */
#define PKV_DECODE_CALLER_PADS 1

typedef struct {
    const void* qkv;             /* bf16 [max_batch][qkv_row_stride]: q | k | v column blocks (a1 views) */
    int64_t qkv_row_stride;      /* elements, >= (Hq + 2 Hkv) * head_dim, multiple of 8 */
    void* q_out;                 /* bf16 [max_batch][Hq][head_dim], q' of the step */
    void* o;                     /* bf16 [max_batch][Hq][head_dim], attention output */
    void* k_cache;               /* bf16 [num_blocks][block_size][Hkv][head_dim] */
    void* v_cache;
    int64_t num_blocks;
    const int64_t* positions;    /* int64 [max_batch] */
    int32_t* slot_mapping;       /* int32 [max_batch]; a graph launch writes -1 into padded rows
                                    (unless flags has PKV_DECODE_CALLER_PADS) */
    int32_t* context_lens;       /* int32 [max_batch]; a graph launch writes 0 into padded rows
                                    (unless flags has PKV_DECODE_CALLER_PADS) */
    const int32_t* block_table;  /* int32 [max_batch][max_blocks_per_seq] */
    int32_t max_blocks_per_seq;
    int32_t max_batch;
    const void* q_norm_weight;   /* bf16 [head_dim] */
    const void* k_norm_weight;
    const float* cos_sin_cache;  /* fp32 [max_position][head_dim] */
    int32_t max_position;
    float eps;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;            /* 128 */
    int32_t block_size;          /* 256 */
    float softmax_scale;
    int32_t flags;               /* 0 or PKV_DECODE_CALLER_PADS */
    void* workspace;             /* >= pkv_decode_step_workspace_bytes(max_batch, ...), 256-byte aligned */
    size_t workspace_bytes;
} pkv_decode_step_desc;

#define PKV_DECODE_GRAPH_MAX_BUCKETS 16

/* Decode workspace that serves every batch size 1..max_batch (0 on invalid sizes). */
PKV_API size_t pkv_decode_step_workspace_bytes(int32_t max_batch, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size);

/* One eager decode step over rows 0..batch-1 (0 <= batch <= max_batch) on `stream`. */
PKV_API int pkv_decode_step(const pkv_decode_step_desc* desc, int32_t batch, void* stream);

typedef struct pkv_decode_graph_s* pkv_decode_graph;

/*
 * Captures one graph per bucket (strictly increasing, each in [1, max_batch],
 * at most PKV_DECODE_GRAPH_MAX_BUCKETS) on a private stream of the current
 * device; graph n is the eager step at batch n.  The descriptor is copied.
 * Set-up only: capture and instantiation allocate host and driver objects.
 * On failure *out is NULL and nothing is kept.
 */
PKV_API int pkv_decode_graph_create(const pkv_decode_step_desc* desc, const int32_t* buckets, int32_t num_buckets,
                                    pkv_decode_graph* out);

/* The bucket a batch of this size runs in (the smallest that holds it), or -1. */
PKV_API int32_t pkv_decode_graph_bucket(pkv_decode_graph graph, int32_t batch);

/*
 * Runs a step for rows 0..batch-1: with n = pkv_decode_graph_bucket(batch),
 * rows batch..n-1 of slot_mapping / context_lens are set to -1 / 0 by one
 * small kernel, then graph n is launched on `stream` (same device as the
 * capture).  Outputs of padded rows are zero.  batch == 0 does nothing;
 * batch above the largest bucket is PKV_ERR_INVALID_ARG.  No allocation.
 */
PKV_API int pkv_decode_graph_launch(pkv_decode_graph graph, int32_t batch, void* stream);

/* Releases the graphs (NULL is ignored).  Work already launched is unaffected. */
PKV_API void pkv_decode_graph_destroy(pkv_decode_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
