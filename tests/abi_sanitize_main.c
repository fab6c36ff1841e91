/*
 * Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the library's host code (tests/test_abi_sanitize.py).
 * Every call here is refused by argument validation or is a size query, so no
 * device work is issued: the run needs no GPU.  Sizes at the extremes of their
 * types exercise the overflow guards of the size arithmetic.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int failures = 0, checks = 0;

static void expect(int got, int want, const char* what) {
    ++checks;
    const char* msg = pkv_last_error();
    if (got != want) {
        ++failures;
        printf("FAIL %s: got %d, want %d (%s)\n", what, got, want, msg ? msg : "");
    } else if (want != 0 && (msg == NULL || msg[0] == 0)) {
        ++failures;
        printf("FAIL %s: no error message\n", what);
    }
}

static void expect_size(size_t got, int positive, const char* what) {
    ++checks;
    if ((got > 0) != (positive != 0)) {
        ++failures;
        printf("FAIL %s: size %zu\n", what, got);
    }
}

#define FAKE ((void*)(uintptr_t)0x1000)
#define FAR(n) ((void*)(((uintptr_t)1 << 40) + ((uintptr_t)(n) << 32)))

int main(void) {
    const int32_t I32MAX = 2147483647;
    expect(pkv_version() > 0 ? 0 : 1, 0, "version");

    /* size queries: valid, invalid and extreme arguments */
    expect_size(pkv_attn_prefill_workspace_bytes(4, 1024, 256, 16384, 32, 8, 128), 1, "prefill split query");
    expect_size(pkv_attn_prefill_workspace_bytes(16, 32768, 2048, 4096, 32, 8, 128), 0, "prefill no split");
    expect_size(pkv_attn_prefill_workspace_bytes(I32MAX, I32MAX, I32MAX, I32MAX, 64, 8, 128), 0, "prefill extreme");
    expect_size(pkv_attn_prefill_workspace_bytes(1, I32MAX, I32MAX, I32MAX, 64, 1, 128), 0, "prefill extreme 2");
    expect_size(pkv_attn_prefill_workspace_bytes(-1, 4, 4, 4, 32, 8, 128), 0, "prefill negative");
    expect_size(pkv_attn_prefill_workspace_bytes(4, 1024, 256, 16384, 0, 8, 128), 0, "prefill no heads");
    expect_size(pkv_attn_decode_workspace_bytes(256, 32, 8, 128, 128, 256), 1, "decode query");
    expect_size(pkv_attn_decode_workspace_bytes(0, 32, 8, 128, 128, 256), 1, "decode empty batch");
    expect_size(pkv_attn_decode_workspace_bytes(I32MAX, 128, 8, 128, I32MAX, 256), 0, "decode extreme");
    expect_size(pkv_attn_decode_workspace_bytes(4, 32, 8, 64, 16, 256), 0, "decode head_dim");
    expect_size(pkv_attn_decode_workspace_bytes(4, 12, 8, 128, 16, 256), 0, "decode Hq % Hkv");
    expect_size(pkv_decode_step_workspace_bytes(512, 32, 8, 128, 128, 256), 1, "step query");
    expect_size(pkv_decode_step_workspace_bytes(I32MAX, 128, 8, 128, I32MAX, 256), 0, "step extreme");
    expect_size(pkv_decode_step_workspace_bytes(-3, 32, 8, 128, 16, 256), 0, "step negative");

    /* argument validation: each refused before any device call */
    expect(pkv_rope_cache_build(NULL, 40960, 128, 1e6, NULL), PKV_ERR_INVALID_ARG, "rope NULL");
    expect(pkv_rope_cache_build((float*)FAKE, 40960, 64, 1e6, NULL), PKV_ERR_UNSUPPORTED, "rope dim");
    expect(pkv_rope_cache_build((float*)FAKE, -1, 128, 1e6, NULL), PKV_ERR_INVALID_ARG, "rope positions");
    expect(pkv_qk_norm_rope(FAKE, 4096, FAKE, 1024, NULL, NULL, (const int64_t*)FAKE, 4, 32, 8, 128, FAKE, FAKE, 1e-6f,
                            (const float*)FAKE, 40960, NULL),
           PKV_ERR_INVALID_ARG, "norm_rope NULL output");
    expect(pkv_qk_norm_rope(FAKE, 4096, FAKE, 1024, FAR(1), FAR(2), (const int64_t*)FAKE, -1, 32, 8, 128, FAKE, FAKE,
                            1e-6f, (const float*)FAKE, 40960, NULL),
           PKV_ERR_INVALID_ARG, "norm_rope negative tokens");
    expect(pkv_store_kvcache(FAKE, 1024, FAKE, 1024, FAR(1), FAR(2), 4096, (const int32_t*)FAKE, 4, 8, 128, 3, NULL),
           PKV_ERR_INVALID_ARG, "store elem_bytes");
    expect(pkv_store_kvcache(FAKE, 512, FAKE, 1024, FAR(1), FAR(2), 4096, (const int32_t*)FAKE, 4, 8, 128, 2, NULL),
           PKV_ERR_INVALID_ARG, "store short stride");
    expect(pkv_qk_norm_rope_store(FAKE, 6144, FAKE, 6144, FAKE, 512, FAR(1), NULL, FAR(2), FAR(3), 4096,
                                  (const int32_t*)FAKE, (const int64_t*)FAKE, 4, 32, 8, 128, FAKE, FAKE, 1e-6f,
                                  (const float*)FAKE, 40960, NULL),
           PKV_ERR_INVALID_ARG, "norm_rope_store short v stride");
    expect(pkv_attn_prefill_varlen(FAKE, 4096, FAKE, 1024, FAKE, 1024, FAR(1), (const int32_t*)FAKE,
                                   (const int32_t*)FAKE, 2, 337, 300, 300, 32, 8, 128, 0.088f, 0, NULL, 0, 256, 0,
                                   NULL, 0, NULL),
           PKV_ERR_UNSUPPORTED, "prefill non-causal");
    expect(pkv_attn_prefill_varlen(FAKE, 4096, FAKE, 1024, FAKE, 1024, FAR(1), (const int32_t*)FAKE,
                                   (const int32_t*)FAKE, 2, 337, 400, 300, 32, 8, 128, 0.088f, 1, NULL, 0, 256, 0,
                                   NULL, 0, NULL),
           PKV_ERR_INVALID_ARG, "prefill max_seqlen_q > max_seqlen_k");
    expect(pkv_attn_prefill_varlen(FAKE, 4096, FAKE, 1024, FAKE, 1024, FAR(1), (const int32_t*)FAKE,
                                   (const int32_t*)FAKE, 2, I32MAX, I32MAX, I32MAX, 32, 8, 128, 0.088f, 1, NULL, 0,
                                   256, 0, NULL, 0, NULL),
           PKV_ERR_INVALID_ARG, "prefill o overlapping a huge q");
    expect(pkv_attn_prefill_varlen(FAKE, 4096, FAKE, 1024, FAKE, 1024, FAR(1), (const int32_t*)FAKE,
                                   (const int32_t*)FAKE, 2, 337, 300, 300, 32, 8, 128, 0.088f, 1, NULL, 0, 256, 0,
                                   (void*)(uintptr_t)(UINT64_MAX & ~(uint64_t)255), (size_t)1 << 20, NULL),
           PKV_ERR_WORKSPACE, "prefill workspace wrapping");
    expect(pkv_attn_decode_paged(FAR(0), FAR(1), FAR(2), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE, 16, 4,
                                 32, 8, 128, 256, 100, 0.088f, NULL, 0, NULL),
           PKV_ERR_WORKSPACE, "decode no workspace");
    expect(pkv_attn_decode_paged(FAR(0), FAR(1), FAR(2), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE, 16, 4,
                                 32, 8, 128, 256, 100, 0.088f, FAR(1), (size_t)1 << 30, NULL),
           PKV_ERR_WORKSPACE, "decode workspace on the k cache");
    expect(pkv_attn_decode_paged(FAR(0), FAR(1), FAR(1), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE, 16, 4,
                                 32, 8, 128, 256, 100, 0.088f, FAR(5), (size_t)1 << 30, NULL),
           PKV_ERR_INVALID_ARG, "decode k_cache == v_cache");
    expect(pkv_attn_decode_paged_noalloc(FAR(0), FAR(1), FAR(2), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE,
                                         4096, 4096, 32, 8, 128, 256, 100, 0.088f, NULL),
           PKV_ERR_WORKSPACE, "decode noalloc beyond its array");
    expect(pkv_attn_decode_paged_noalloc(FAR(0), FAR(1), FAR(2), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE,
                                         I32MAX, 4096, 32, 8, 128, 256, 100, 0.088f, NULL),
           PKV_ERR_UNSUPPORTED, "decode tables beyond the launch grid");
    expect(pkv_attn_decode_paged(FAR(0), FAR(1), FAR(2), FAR(3), (const int32_t*)FAKE, (const int32_t*)FAKE, 16,
                                 70000, 32, 8, 128, 256, 100, 0.088f, FAR(5), (size_t)1 << 30, NULL),
           PKV_ERR_UNSUPPORTED, "decode batch beyond the launch grid");
    expect(pkv_add_rms_norm(FAKE, FAKE, FAKE, FAR(1), FAR(2), 4, 4100, 1e-6f, NULL), PKV_ERR_INVALID_ARG,
           "add_rms_norm hidden");
    expect(pkv_silu_and_mul(FAKE, 100, FAR(1), 100, 4, 64, NULL), PKV_ERR_INVALID_ARG, "silu short row");
    expect(pkv_sample_gumbel(FAKE, 151936, 7, (const float*)FAKE, NULL, 0, 1, 0, (int64_t*)FAR(1), 4, 151936, NULL),
           PKV_ERR_UNSUPPORTED, "sampler dtype");

    pkv_decode_step_desc d;
    memset(&d, 0, sizeof d);
    d.qkv = FAR(0);
    d.qkv_row_stride = 6144;
    d.q_out = FAR(1);
    d.o = FAR(2);
    d.k_cache = FAR(3);
    d.v_cache = FAR(4);
    d.num_blocks = 64;
    d.positions = (const int64_t*)FAR(5);
    d.slot_mapping = (int32_t*)FAR(6);
    d.context_lens = (int32_t*)FAR(7);
    d.block_table = (const int32_t*)FAR(8);
    d.max_blocks_per_seq = 8;
    d.max_batch = 32;
    d.q_norm_weight = FAR(9);
    d.k_norm_weight = FAR(10);
    d.cos_sin_cache = (const float*)FAR(11);
    d.max_position = 40960;
    d.eps = 1e-6f;
    d.num_q_heads = 32;
    d.num_kv_heads = 8;
    d.head_dim = 128;
    d.block_size = 256;
    d.softmax_scale = 0.088f;
    d.workspace = FAR(3);   /* on the k cache */
    d.workspace_bytes = (size_t)1 << 30;
    expect(pkv_decode_step(&d, 4, NULL), PKV_ERR_WORKSPACE, "step workspace on the k cache");
    expect(pkv_decode_step(&d, 33, NULL), PKV_ERR_INVALID_ARG, "step batch above max_batch");
    expect(pkv_decode_step(NULL, 4, NULL), PKV_ERR_INVALID_ARG, "step NULL descriptor");
    {
        pkv_decode_graph g = (pkv_decode_graph)FAKE;
        const int32_t buckets[3] = {4, 2, 8};
        expect(pkv_decode_graph_create(&d, buckets, 3, &g), PKV_ERR_INVALID_ARG, "graph buckets not increasing");
        expect(g == NULL ? 0 : 1, 0, "graph handle cleared on failure");
        expect(pkv_decode_graph_create(&d, buckets, -1, &g), PKV_ERR_INVALID_ARG, "graph bucket count");
    }
    expect(pkv_decode_graph_bucket(NULL, 4) == -1 ? 0 : 1, 0, "bucket of no graph");
    pkv_decode_graph_destroy(NULL);

    printf("%d checks, %d failures\n", checks, failures);
    return failures != 0;
}
