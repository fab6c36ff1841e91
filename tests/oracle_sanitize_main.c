/*
 * oracle_sanitize_main.c -- drives every entry point of oracle/pkv_oracle.c on
 * small inputs, edge cases included, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's own memory accesses.
 * Test infrastructure only: built and run by tests/test_oracle_robustness.py
 * with gcc on the host (no GPU code is involved).
 *
 * Every array is sized exactly for what the call may touch, so an access one
 * element past an end is reported.  Exit status 0 means every call returned
 * what it should; the sanitizers abort on any finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_round_bf16(const double* in, uint16_t* out, int64_t n);
void orc_bf16_to_double(const uint16_t* in, double* out, int64_t n);
int orc_rope_table(float* out, int32_t max_pos, int32_t rot_dim, double theta);
int orc_rmsnorm_rope(const uint16_t* x, int64_t row_stride, int32_t n_tokens, int32_t n_heads, int32_t d,
                     const uint16_t* gamma, double eps, const int64_t* positions, const float* table,
                     int32_t max_pos, int32_t pages_rounding, double* out);
int orc_store_kvcache(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                      void* k_cache, void* v_cache, int64_t num_slots, const int32_t* slot_mapping, int32_t n_tokens,
                      int32_t row_elems, int32_t elem_bytes);
int orc_attn_prefill(const uint16_t* q, int64_t q_row_stride, const uint16_t* k, int64_t k_row_stride,
                     const uint16_t* v, int64_t v_row_stride, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, double scale,
                     const int32_t* block_table, int32_t max_blocks, int32_t block_size, int64_t num_slots,
                     const int64_t* rows, int64_t n_rows, double* out);
int orc_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks, int32_t num_seqs,
                    int32_t hq, int32_t hkv, int32_t d, int32_t block_size, int64_t num_slots, double scale,
                    const int32_t* seqs, int32_t n_sel, double* out);
int orc_num_threads(void);
int orc_set_num_threads(int n);

static int failures = 0;
#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);    \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint32_t lcg = 12345u;
static uint16_t rnd_bf16(void) {
    lcg = lcg * 1664525u + 1013904223u;
    /* values in about [-2, 2): sign, exponent 126..128, random fraction */
    uint16_t sign = (lcg >> 31) << 15;
    uint16_t expo = (uint16_t)(126 + ((lcg >> 20) % 3)) << 7;
    return sign | expo | ((lcg >> 8) & 0x7F);
}
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static uint16_t* rnd_array(size_t n) {
    uint16_t* a = xmalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) a[i] = rnd_bf16();
    return a;
}

int main(void) {
    const int D = 128, HQ = 4, HKV = 2, BS = 256;
    const double scale = 1.0 / sqrt(128.0);

    /* bf16 conversions, special values included */
    {
        double in[8] = {1.0, -2.5, 0.0, -0.0, 1e39, -1e39, NAN, 1e-41};
        uint16_t b[8];
        double back[8];
        orc_round_bf16(in, b, 8);
        orc_bf16_to_double(b, back, 8);
        EXPECT(b[0] == 0x3F80 && back[1] == -2.5 && isinf(back[4]) && isnan(back[6]));
    }

    /* RoPE table: odd sizes and the refused arguments */
    const int max_pos = 300;
    float* table = xmalloc(sizeof(float) * (size_t)max_pos * D);
    EXPECT(orc_rope_table(table, max_pos, D, 1e6) == 0);
    EXPECT(table[0] == 1.0f && table[64] == 0.0f);
    EXPECT(orc_rope_table(table, 1, 3, 1e6) != 0);
    EXPECT(orc_rope_table(table, 1, D, 0.0) != 0);

    /* QK-Norm + RoPE in both rounding modes, a strided row layout, out-of-table positions refused */
    {
        const int n = 5, heads = 3, stride = heads * D + 64;
        uint16_t* x = rnd_array((size_t)(n - 1) * stride + heads * D);
        uint16_t* g = rnd_array(D);
        int64_t pos[5] = {0, 1, 17, 298, 299};
        double* out = xmalloc(sizeof(double) * n * heads * D);
        for (int mode = 0; mode < 2; ++mode)
            EXPECT(orc_rmsnorm_rope(x, stride, n, heads, D, g, 1e-6, pos, table, max_pos, mode, out) == 0);
        EXPECT(orc_rmsnorm_rope(x, stride, 0, heads, D, g, 1e-6, pos, table, max_pos, 0, out) == 0);
        int64_t bad[1] = {300};
        EXPECT(orc_rmsnorm_rope(x, stride, 1, heads, D, g, 1e-6, bad, table, max_pos, 0, out) == -2);
        free(x); free(g); free(out);
    }

    /* scatter: -1, out-of-pool and negative slots are skipped; fp32 rows too */
    {
        const int n = 6, row = HKV * D, slots = 4;
        uint16_t* key = rnd_array((size_t)n * row);
        uint16_t* val = rnd_array((size_t)n * row);
        uint16_t* kc = xmalloc(sizeof(uint16_t) * slots * row);
        uint16_t* vc = xmalloc(sizeof(uint16_t) * slots * row);
        memset(kc, 0, sizeof(uint16_t) * slots * row);
        memset(vc, 0, sizeof(uint16_t) * slots * row);
        int32_t sm[6] = {3, -1, 0, 4, -7, 1};
        EXPECT(orc_store_kvcache(key, row, val, row, kc, vc, slots, sm, n, row, 2) == 0);
        EXPECT(memcmp(kc + 3 * row, key, sizeof(uint16_t) * row) == 0);
        EXPECT(orc_store_kvcache(key, row, val, row, kc, vc, slots, sm, 0, row, 2) == 0);
        float fk[3 * 4], fcache[3 * 4];
        for (int i = 0; i < 12; ++i) { fk[i] = (float)i; fcache[i] = 0.f; }
        int32_t sm2[3] = {2, 0, -1};
        EXPECT(orc_store_kvcache(fk, 4, fk, 4, fcache, fcache, 3, sm2, 3, 4, 4) == 0);
        free(key); free(val); free(kc); free(vc);
    }

    /* prefill, contiguous K/V: ragged and zero-length sequences, every row and a row list */
    {
        int32_t lens[4] = {5, 0, 300, 1};
        int32_t cu[5] = {0};
        for (int b = 0; b < 4; ++b) cu[b + 1] = cu[b] + lens[b];
        const int T = cu[4];
        uint16_t* q = rnd_array((size_t)T * HQ * D);
        uint16_t* k = rnd_array((size_t)T * HKV * D);
        uint16_t* v = rnd_array((size_t)T * HKV * D);
        double* out = xmalloc(sizeof(double) * T * HQ * D);
        EXPECT(orc_attn_prefill(q, HQ * D, k, HKV * D, v, HKV * D, cu, cu, 4, HQ, HKV, D, scale, NULL, 0, BS, T,
                                NULL, -1, out) == 0);
        int64_t rows[4] = {0, 0, T - 1, HQ - 1};
        EXPECT(orc_attn_prefill(q, HQ * D, k, HKV * D, v, HKV * D, cu, cu, 4, HQ, HKV, D, scale, NULL, 0, BS, T,
                                rows, 2, out) == 0);
        int64_t bad_rows[2] = {T, 0};
        EXPECT(orc_attn_prefill(q, HQ * D, k, HKV * D, v, HKV * D, cu, cu, 4, HQ, HKV, D, scale, NULL, 0, BS, T,
                                bad_rows, 1, out) == -4);
        /* keys past the rows given are refused instead of read */
        EXPECT(orc_attn_prefill(q, HQ * D, k, HKV * D, v, HKV * D, cu, cu, 4, HQ, HKV, D, scale, NULL, 0, BS, T - 1,
                                NULL, -1, out) == -3);
        free(q); free(k); free(v); free(out);
    }

    /* prefill over the paged cache and decode; -1 padding past the context is fine, an
       unusable id inside it is refused before any key is read */
    {
        const int nb = 5, slots = nb * BS, mb = 3;
        uint16_t* kc = rnd_array((size_t)slots * HKV * D);
        uint16_t* vc = rnd_array((size_t)slots * HKV * D);
        int32_t bt[2 * 3] = {4, 1, -1, 0, 2, 3};
        int32_t cuq[3] = {0, 10, 11};
        int32_t cuk[3] = {0, 300, 600};     /* seq 0: 300 keys (blocks 4, 1); seq 1: 300 keys */
        uint16_t* q = rnd_array((size_t)11 * HQ * D);
        double* out = xmalloc(sizeof(double) * 11 * HQ * D);
        EXPECT(orc_attn_prefill(q, HQ * D, kc, HKV * D, vc, HKV * D, cuq, cuk, 2, HQ, HKV, D, scale, bt, mb, BS,
                                slots, NULL, -1, out) == 0);
        int32_t bt_bad[2 * 3] = {4, -1, 0, 0, 2, 3};
        EXPECT(orc_attn_prefill(q, HQ * D, kc, HKV * D, vc, HKV * D, cuq, cuk, 2, HQ, HKV, D, scale, bt_bad, mb, BS,
                                slots, NULL, -1, out) == -3);
        int32_t bt_far[2 * 3] = {4, 1, -1, 0, 5, 3};
        EXPECT(orc_attn_prefill(q, HQ * D, kc, HKV * D, vc, HKV * D, cuq, cuk, 2, HQ, HKV, D, scale, bt_far, mb, BS,
                                slots, NULL, -1, out) == -3);

        int32_t ctx[3] = {300, 0, 513};
        int32_t btd[3 * 3] = {4, 1, -1, -1, -1, -1, 0, 2, 3};
        uint16_t* qd = rnd_array((size_t)3 * HQ * D);
        double* od = xmalloc(sizeof(double) * 3 * HQ * D);
        EXPECT(orc_attn_decode(qd, kc, vc, ctx, btd, mb, 3, HQ, HKV, D, BS, slots, scale, NULL, -1, od) == 0);
        for (int i = 0; i < HQ * D; ++i) EXPECT(od[HQ * D + i] == 0.0);
        int32_t sel[2] = {2, 0};
        EXPECT(orc_attn_decode(qd, kc, vc, ctx, btd, mb, 3, HQ, HKV, D, BS, slots, scale, sel, 2, od) == 0);
        int32_t ctx_long[3] = {300, 0, 769};    /* needs a 4th table entry */
        EXPECT(orc_attn_decode(qd, kc, vc, ctx_long, btd, mb, 3, HQ, HKV, D, BS, slots, scale, NULL, -1, od) == -3);
        int32_t btd_bad[3 * 3] = {4, 7, -1, -1, -1, -1, 0, 2, 3};
        EXPECT(orc_attn_decode(qd, kc, vc, ctx, btd_bad, mb, 3, HQ, HKV, D, BS, slots, scale, NULL, -1, od) == -3);
        int32_t sel_bad[1] = {3};
        EXPECT(orc_attn_decode(qd, kc, vc, ctx, btd, mb, 3, HQ, HKV, D, BS, slots, scale, sel_bad, 1, od) == -4);
        free(kc); free(vc); free(q); free(out); free(qd); free(od);
    }

    EXPECT(orc_set_num_threads(1) >= 1 && orc_num_threads() >= 1);
    free(table);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
