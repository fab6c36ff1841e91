/*
 * pkv_oracle.c -- CPU reference for the Qwen3 attention-sublayer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source with the HIP library.
 *
 * Plain loops, fp64 arithmetic for every float operation (sums, products,
 * square roots, exponentials), OpenMP over independent outputs.  Inputs that
 * the pages hold in bf16 arrive as raw uint16 bit patterns; the one table the
 * pages keep in fp32 (RoPE cos/sin) is produced as fp32.
 *
 * Sources, cited by page title and section:
 *   [P1] "3.3 Model skeleton and core operators" (infra-guide):
 *        s2 RMSNorm, s3 RoPE, s7.1 store_kvcache, s7.2 the two attention paths.
 *   [P3] "Nano-vLLM 源码解读 #17 注意力层": s3 GQA grouping, s4 QK-Norm,
 *        s5.1 scatter examples, s5.2 FlashAttention / online softmax, s5.3.
 *   [P4] "同一个 Qwen3，两种写法": s1.2 attention definition with causal mask,
 *        s3.2 flat [T,H] layout and block-diagonal mask, s3.4 GQA repeat,
 *        s3.5 RoPE table.
 *   [P5] "nano-vllm code walkthrough": "Prefill stage" case 1 / case 2 and
 *        "Decode Stage" argument meanings.
 *
 * Readings where the pages are silent (each restated in the design notes):
 *   - q head h uses kv head h / (Hq/Hkv) (contiguous groups, [P3] s3, [P4] s3.4);
 *   - with fewer queries than keys, query i of a sequence sits at absolute
 *     position Lk - Lq + i and sees keys 0..Lk-Lq+i ([P5] case 2);
 *   - eps is added to the mean square inside the root ([P1] s2);
 *   - the RoPE table is fp32: inv_freq_i = fp32(theta^(-2i/d)), the angle is
 *     the fp32 product fp32(p) * inv_freq_i, cos/sin of that fp32 angle are
 *     rounded to fp32 ([P1] s3, [P4] s3.5);
 *   - fp -> bf16 conversions round to nearest, ties to even;
 *   - slot values outside [0, num_slots) other than -1 are invalid and are
 *     not written; a context of 0 tokens yields a zero output row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* bf16 <-> double                                                           */
/* ------------------------------------------------------------------------ */

static double bf16_val(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Direct double -> bf16 with round-to-nearest-even (no fp32 step, so no
 * double rounding).  bf16 = 1 sign, 8 exponent, 7 fraction bits. */
static uint16_t bf16_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                    /* a = m * 2^e, 0.5 <= m < 1 */
    int unb = e - 1;                 /* a = 1.f * 2^unb */
    if (unb < -126) {                /* subnormal range: quantum 2^-133 */
        double q = nearbyint(ldexp(a, 133));
        if (q >= 128.0) return sign | 0x0080;      /* rounds up to min normal */
        return sign | (uint16_t)q;
    }
    double r = nearbyint(ldexp(a, 7 - unb));       /* in [128, 256] */
    if (r >= 256.0) { r = 128.0; unb += 1; }
    if (unb > 127) return sign | 0x7F80;
    return sign | (uint16_t)(((unb + 127) << 7) | ((int)r - 128));
}

static float f32_rn(double x) { return (float)x; } /* IEEE conversion: RNE */

ORC_EXPORT void orc_round_bf16(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}

ORC_EXPORT void orc_bf16_to_double(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_val(in[i]);
}

/* ------------------------------------------------------------------------ */
/* RoPE cos/sin table  ([P1] s3, [P4] s3.5)                                  */
/*   row p = [cos(p*f_0) .. cos(p*f_{r/2-1}) | sin(p*f_0) .. sin(p*f_{r/2-1})]  */
/* ------------------------------------------------------------------------ */

ORC_EXPORT int orc_rope_table(float* out, int32_t max_pos, int32_t rot_dim, double theta) {
    if (!out || max_pos < 0 || rot_dim <= 0 || (rot_dim & 1) || !(theta > 0.0)) return -1;
    int half = rot_dim / 2;
    float* inv = (float*)malloc(sizeof(float) * (size_t)half);
    if (!inv) return -1;
    for (int i = 0; i < half; ++i)
        inv[i] = f32_rn(pow(theta, -(2.0 * i) / (double)rot_dim));
#pragma omp parallel for schedule(static)
    for (int32_t p = 0; p < max_pos; ++p) {
        float fp = (float)p;
        float* row = out + (int64_t)p * rot_dim;
        for (int i = 0; i < half; ++i) {
            float ang = fp * inv[i];            /* fp32 product, as the fp32 einsum */
            row[i] = f32_rn(cos((double)ang));
            row[half + i] = f32_rn(sin((double)ang));
        }
    }
    free(inv);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* QK-Norm then RoPE on one family of heads ([P1] s2, s3, s8; [P3] s4)       */
/*   x  : bf16 [n_tokens] rows, row_stride elements apart, heads of d at     */
/*        head stride d inside a row                                         */
/*   out: double [n_tokens][n_heads][d], unrounded                           */
/*   pages_rounding != 0: round to bf16 where the pages' code holds bf16     */
/*        tensors -- after normalising, after the product with gamma ([P1]   */
/*        s2: the row is cast back before the weight multiply) and after the */
/*        rotation ([P1] s3 / [P4] s3.5: the rotated row is cast to x's      */
/*        dtype); out then holds those bf16 values.                          */
/* ------------------------------------------------------------------------ */

ORC_EXPORT int orc_rmsnorm_rope(const uint16_t* x, int64_t row_stride, int32_t n_tokens, int32_t n_heads,
                                int32_t d, const uint16_t* gamma, double eps, const int64_t* positions,
                                const float* table, int32_t max_pos, int32_t pages_rounding, double* out) {
    if (d <= 0 || d > 512 || (d & 1) || n_tokens < 0 || n_heads <= 0) return -1;
    int half = d / 2;
    for (int32_t t = 0; t < n_tokens; ++t)
        if (positions[t] < 0 || positions[t] >= max_pos) return -2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t t = 0; t < n_tokens; ++t) {
        for (int32_t h = 0; h < n_heads; ++h) {
            const uint16_t* xr = x + (int64_t)t * row_stride + (int64_t)h * d;
            double y[512];
            double ss = 0.0;
            for (int i = 0; i < d; ++i) { double v = bf16_val(xr[i]); ss += v * v; }
            double r = 1.0 / sqrt(ss / (double)d + eps);
            if (pages_rounding) {
                /* the pages' precision steps: the normalised row is cast to bf16,
                   multiplied by gamma in bf16 (one rounding of the exact product) */
                for (int i = 0; i < d; ++i)
                    y[i] = bf16_val(bf16_rne(bf16_val(bf16_rne(bf16_val(xr[i]) * r)) * bf16_val(gamma[i])));
            } else {
                for (int i = 0; i < d; ++i) y[i] = bf16_val(xr[i]) * r * bf16_val(gamma[i]);
            }
            const float* cs = table + positions[t] * (int64_t)d;
            double* o = out + ((int64_t)t * n_heads + h) * d;
            for (int i = 0; i < half; ++i) {
                double c = (double)cs[i], s = (double)cs[half + i];
                double x1 = y[i], x2 = y[half + i];
                o[i] = x1 * c - x2 * s;
                o[half + i] = x2 * c + x1 * s;
                if (pages_rounding) {   /* the rotated row is cast back to bf16 */
                    o[i] = bf16_val(bf16_rne(o[i]));
                    o[half + i] = bf16_val(bf16_rne(o[half + i]));
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* store_kvcache scatter ([P1] s7.1, [P3] s5.1)                              */
/*   Row t of key (row_stride elements apart, D contiguous elements) is      */
/*   copied byte for byte to cache row slot_mapping[t]; -1 means skip.       */
/* ------------------------------------------------------------------------ */

ORC_EXPORT int orc_store_kvcache(const void* key, int64_t key_row_stride, const void* value,
                                 int64_t value_row_stride, void* k_cache, void* v_cache, int64_t num_slots,
                                 const int32_t* slot_mapping, int32_t n_tokens, int32_t row_elems,
                                 int32_t elem_bytes) {
    if (n_tokens < 0 || row_elems <= 0 || elem_bytes <= 0) return -1;
    size_t row_bytes = (size_t)row_elems * (size_t)elem_bytes;
    for (int32_t t = 0; t < n_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s == -1) continue;
        if (s < 0 || s >= num_slots) continue;
        memcpy((char*)k_cache + (size_t)s * row_bytes,
               (const char*)key + (size_t)t * (size_t)key_row_stride * elem_bytes, row_bytes);
        memcpy((char*)v_cache + (size_t)s * row_bytes,
               (const char*)value + (size_t)t * (size_t)value_row_stride * elem_bytes, row_bytes);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* One attention row ([P4] s1.2; [P3] s5.2)                                  */
/*   s_j = scale * q . k_j ; m = max s_j ; e_j = exp(s_j - m) ; l = sum e_j  */
/*   o = sum e_j v_j / l                                                      */
/* The n keys are fetched through key_row(j) -> pointer to d bf16.           */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t* k;     /* contiguous case: base of key rows  */
    const uint16_t* v;
    int64_t k_stride, v_stride;   /* elements between consecutive rows */
    int64_t row0;          /* first row of this sequence (contiguous case) */
    const int32_t* bt;     /* paged case: this sequence's block-table row (NULL: contiguous) */
    int32_t block_size;
    int32_t kv_head, d;
} key_src;

static const uint16_t* key_ptr(const key_src* s, int64_t j, int which_v) {
    int64_t row;
    if (s->bt) {
        int64_t blk = s->bt[j / s->block_size];
        row = blk * s->block_size + j % s->block_size;
    } else {
        row = s->row0 + j;
    }
    const uint16_t* base = which_v ? s->v : s->k;
    int64_t stride = which_v ? s->v_stride : s->k_stride;
    return base + row * stride + (int64_t)s->kv_head * s->d;
}

static void attn_row(const double* q, const key_src* src, int64_t n_keys, double scale, double* out,
                     double* scratch /* n_keys */) {
    int d = src->d;
    if (n_keys <= 0) { for (int i = 0; i < d; ++i) out[i] = 0.0; return; }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        const uint16_t* kr = key_ptr(src, j, 0);
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += q[i] * bf16_val(kr[i]);
        scratch[j] = scale * dot;
        if (scratch[j] > m) m = scratch[j];
    }
    double l = 0.0;
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        double e = exp(scratch[j] - m);
        l += e;
        const uint16_t* vr = key_ptr(src, j, 1);
        for (int i = 0; i < d; ++i) out[i] += e * bf16_val(vr[i]);
    }
    for (int i = 0; i < d; ++i) out[i] /= l;
}

/* ------------------------------------------------------------------------ */
/* Varlen causal prefill ([P1] s7.2; [P4] s3.2; [P5] "Prefill stage")        */
/*   q: bf16 rows [Tq], head h at offset h*d, q_row_stride elements apart.   */
/*   Without block_table (case 1): keys of sequence b are rows               */
/*     cu_k[b] .. cu_k[b+1]-1 of k/v.                                         */
/*   With block_table (case 2): k/v are the caches [num_slots] rows and key  */
/*     j of sequence b sits at slot bt[b][j/bs]*bs + j%bs.                   */
/*   Query i of sequence b sees keys 0 .. (Lk-Lq)+i.                          */
/*   out: double [Tq][Hq][d].  Optional row list (pairs t, h) restricts the  */
/*   work to those outputs (n_rows < 0: all rows).                            */
/* ------------------------------------------------------------------------ */

/* Every key a sequence attends must exist: in the paged case its block id is
 * in [0, num_slots / block_size) for each of the first ceil(n_keys / bs) table
 * entries (and the table is wide enough); in the contiguous case its rows lie
 * inside the num_slots rows given.  The pages never define what an unusable id
 * means (the kernels drop such keys); the oracle refuses the input instead, so a
 * test cannot read outside the host arrays by accident.  Returns 0 or -3. */
static int check_keys(const int32_t* bt_row, int32_t max_blocks, int32_t block_size, int64_t row0,
                      int64_t n_keys, int64_t num_slots) {
    if (n_keys <= 0) return 0;
    if (!bt_row) return (row0 >= 0 && row0 + n_keys <= num_slots) ? 0 : -3;
    if (block_size <= 0) return -3;
    int64_t nblk = (n_keys + block_size - 1) / block_size;
    if (nblk > max_blocks) return -3;
    int64_t pool = num_slots / block_size;
    for (int64_t i = 0; i < nblk; ++i)
        if (bt_row[i] < 0 || (int64_t)bt_row[i] >= pool) return -3;
    return 0;
}

static int find_seq(const int32_t* cu, int32_t nseq, int64_t t) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {            /* last b with cu[b] <= t */
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

ORC_EXPORT int orc_attn_prefill(const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,
                                const uint16_t* v, int64_t v_row_stride, const int32_t* cu_q, const int32_t* cu_k,
                                int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, double scale,
                                const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                                int64_t num_slots, const int64_t* rows, int64_t n_rows, double* out) {
    if (num_seqs <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || d > 512) return -1;
    int32_t group = hq / hkv;
    int64_t Tq = cu_q[num_seqs];
    int64_t maxk = 0;
    if (cu_q[0] != 0) return -2;
    for (int b = 0; b < num_seqs; ++b) {
        int64_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
        if (lq < 0 || lk < lq) return -2;
        if (lk > maxk) maxk = lk;
        if (check_keys(block_table ? block_table + (int64_t)b * max_blocks : NULL, max_blocks, block_size,
                       cu_k[b], lk, num_slots))
            return -3;
    }
    for (int64_t r = 0; n_rows >= 0 && r < n_rows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= Tq || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= hq) return -4;
    int64_t total = n_rows < 0 ? Tq * hq : n_rows;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (size_t)(maxk > 0 ? maxk : 1));
        double qd[512];
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < total; ++r) {
            int64_t t = n_rows < 0 ? r / hq : rows[2 * r];
            int32_t h = n_rows < 0 ? (int32_t)(r % hq) : (int32_t)rows[2 * r + 1];
            int b = find_seq(cu_q, num_seqs, t);
            int64_t i = t - cu_q[b];
            int64_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
            key_src src;
            src.k = k; src.v = v; src.k_stride = k_row_stride; src.v_stride = v_row_stride;
            src.row0 = cu_k[b];
            src.bt = block_table ? block_table + (int64_t)b * max_blocks : NULL;
            src.block_size = block_size;
            src.kv_head = h / group;
            src.d = d;
            const uint16_t* qr = q + t * q_row_stride + (int64_t)h * d;
            for (int x = 0; x < d; ++x) qd[x] = bf16_val(qr[x]);
            int64_t n_keys = (lk - lq) + i + 1;
            double* o = out + (n_rows < 0 ? (t * hq + h) * d : r * d);
            attn_row(qd, &src, n_keys, scale, o, scratch);
        }
        free(scratch);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Paged decode ([P1] s7.2; [P5] "Decode Stage")                             */
/*   q: bf16 [B][Hq][d] contiguous.  Sequence b sees its context_lens[b]     */
/*   cached keys (the token decoded this step included).                     */
/*   out: double [B][Hq][d]; seq list restricts the work (n_sel < 0: all).    */
/* ------------------------------------------------------------------------ */

ORC_EXPORT int orc_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
                               int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t block_size,
                               int64_t num_slots, double scale, const int32_t* seqs, int32_t n_sel, double* out) {
    if (num_seqs < 0 || hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || d > 512) return -1;
    int32_t group = hq / hkv;
    int32_t nsel = n_sel < 0 ? num_seqs : n_sel;
    int64_t maxk = 1;
    for (int32_t s = 0; s < nsel; ++s) {
        int32_t b = n_sel < 0 ? s : seqs[s];
        if (b < 0 || b >= num_seqs) return -4;
        if (context_lens[b] < 0) return -2;
        if (context_lens[b] > maxk) maxk = context_lens[b];
        if (check_keys(block_table + (int64_t)b * max_blocks, max_blocks, block_size, 0, context_lens[b], num_slots))
            return -3;
    }
    int64_t row_stride = (int64_t)hkv * d;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (size_t)maxk);
        double qd[512];
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int32_t s = 0; s < nsel; ++s) {
            for (int32_t h = 0; h < hq; ++h) {
                int32_t b = n_sel < 0 ? s : seqs[s];
                key_src src;
                src.k = k_cache; src.v = v_cache; src.k_stride = row_stride; src.v_stride = row_stride;
                src.row0 = 0;
                src.bt = block_table + (int64_t)b * max_blocks;
                src.block_size = block_size;
                src.kv_head = h / group;
                src.d = d;
                const uint16_t* qr = q + ((int64_t)b * hq + h) * d;
                for (int x = 0; x < d; ++x) qd[x] = bf16_val(qr[x]);
                double* o = out + ((int64_t)s * hq + h) * d;
                attn_row(qd, &src, context_lens[b], scale, o, scratch);
            }
        }
        free(scratch);
    }
    return 0;
}

ORC_EXPORT int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following oracle calls use (n > 0); returns the count now in force. */
ORC_EXPORT int orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return orc_num_threads();
}
