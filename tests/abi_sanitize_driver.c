/* Calls every C-ABI entry point with arguments its checks must reject: NULL pointers,
 * out-of-range and extreme sizes (near INT32_MAX, products beyond 64 bits), bad patterns,
 * small or misaligned workspaces.  Built and run by tests/test_abi_sanitized.py against a
 * copy of the library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer,
 * so an out-of-bounds read, a signed overflow or a shift out of range in argument checking
 * aborts the run.  No call here may pass validation: the pointers are placeholders and no
 * kernel is ever launched.  Exit status 0 when every call returned the expected status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "indexcache.h"

static int failures = 0;

static void expect(int line, const char* what, ic_status got, ic_status want) {
    const char* msg = ic_last_error();
    if (got != want) {
        fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, (int)got, (int)want,
                msg ? msg : "(null)");
        ++failures;
    } else if (want != IC_OK && (!msg || strlen(msg) == 0)) {
        fprintf(stderr, "line %d: %s failed without a message\n", line, what);
        ++failures;
    }
}
#define EXPECT(call, want) expect(__LINE__, #call, (call), (want))

static void expect_size(int line, const char* what, size_t got, int zero) {
    if (zero ? got != 0 : got == 0) {
        fprintf(stderr, "line %d: %s returned %zu\n", line, what, got);
        ++failures;
    }
}
#define EXPECT_ZERO(call) expect_size(__LINE__, #call, (call), 1)
#define EXPECT_NONZERO(call) expect_size(__LINE__, #call, (call), 0)

#define FAKE ((void*)0x1000)
#define FAKE_WS ((void*)0x10000)
#define BIG (1u << 30)

static ic_shape shape(void) {
    ic_shape s = {1, 512, 512, 0, 4, 32, 64, 4, 64, IC_BF16, 0};
    return s;
}

static ic_layer layers[8];

static const ic_layer* make_layers(const char* pattern) {
    for (int i = 0; i < 8 && pattern[i]; ++i) {
        const int full = pattern[i] == 'F' || pattern[i] == '1';
        layers[i].q_I = full ? FAKE : NULL;
        layers[i].w = full ? (const float*)FAKE : NULL;
        layers[i].k_I = full ? FAKE : NULL;
        layers[i].q = FAKE;
        layers[i].kv = FAKE;
        layers[i].out = FAKE;
    }
    return layers;
}

static ic_status stack(const char* pattern, int32_t n, ic_shape s, size_t ws_bytes) {
    return ic_run_stack(pattern, n, make_layers("FSSSFSSS"), &s, (int32_t*)FAKE, FAKE_WS, ws_bytes, NULL, NULL);
}

int main(void) {
    if (ic_version() < 100) {
        fprintf(stderr, "version %d\n", ic_version());
        ++failures;
    }
    ic_stats st;
    EXPECT(ic_get_stats(NULL), IC_ERR_ARG);
    EXPECT(ic_get_stats(&st), IC_OK);

    /* workspace queries: every op on a valid shape, then invalid shapes and ops */
    ic_shape s = shape();
    for (int op = 0; op <= 7; ++op) (void)ic_workspace_size(&s, op);
    EXPECT_NONZERO(ic_workspace_size(&s, IC_OP_RUN_STACK));
    EXPECT_ZERO(ic_workspace_size(&s, 99));
    EXPECT_ZERO(ic_workspace_size(NULL, IC_OP_RUN_STACK));
    ic_shape h = shape();
    h.B = INT32_MAX; h.Lq = INT32_MAX; h.Lk = INT32_MAX; h.k = 4096; h.H = 4096; h.d = 128;
    for (int op = 0; op <= 7; ++op) (void)ic_workspace_size(&h, op);      /* extreme sizes: no overflow */
    h = shape(); h.chunk = 65536; h.Lq = 1 << 20; h.Lk = 1 << 20; h.B = 1 << 20;
    for (int op = 0; op <= 7; ++op) (void)ic_workspace_size(&h, op);
    /* the largest valid shapes: the size arithmetic runs on them without overflow */
    h = shape(); h.d = 64; h.Lk = (1 << 24) - 1; h.Lq = h.Lk; h.B = 127; h.chunk = 65536; h.k = 4096; h.H = 4096;
    h.H_I = 64; h.d_I = 128;
    for (int op = 0; op <= 7; ++op) (void)ic_workspace_size(&h, op);
    EXPECT_NONZERO(ic_workspace_size(&h, IC_OP_RUN_STACK));
    (void)ic_run_stack_dynamic_ws(&h, 1);
    h.Lq = 1; h.B = INT32_MAX;                                           /* decode: many long sequences */
    EXPECT_NONZERO(ic_workspace_size(&h, IC_OP_DECODE_STEP));
    (void)ic_workspace_size(&h, IC_OP_DECODE_ATTN);                    /* one split per query: none */
    EXPECT_ZERO(ic_run_stack_dynamic_ws(&s, 0));
    EXPECT_ZERO(ic_run_stack_dynamic_ws(NULL, 16));
    h = shape(); h.B = INT32_MAX; h.Lq = INT32_MAX; h.Lk = INT32_MAX;
    (void)ic_run_stack_dynamic_ws(&h, 1);
    (void)ic_run_stack_dynamic_ws(&s, INT32_MAX);
    (void)ic_run_stack_dynamic_ws(&s, INT32_MIN);

    /* the stack: patterns, shapes, workspace, pointers */
    EXPECT(stack("SFSS", 4, s, BIG), IC_ERR_NO_CACHED_INDICES);
    EXPECT(stack("0100", 4, s, BIG), IC_ERR_NO_CACHED_INDICES);
    EXPECT(stack("FXSS", 4, s, BIG), IC_ERR_PATTERN);
    EXPECT(stack("FSS", 4, s, BIG), IC_ERR_PATTERN);
    EXPECT(stack("FSSS", -1, s, BIG), IC_ERR_ARG);
    EXPECT(stack("", 0, s, BIG), IC_ERR_ARG);
    EXPECT(ic_run_stack(NULL, 4, make_layers("FSSS"), &s, (int32_t*)FAKE, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack("FSSS", 4, NULL, &s, (int32_t*)FAKE, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack("FSSS", 4, make_layers("FSSS"), NULL, (int32_t*)FAKE, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack("FSSS", 4, make_layers("FSSS"), &s, NULL, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    ic_shape b;
    b = shape(); b.d = 96;          EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.d_I = 48;        EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.H_I = 65;        EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.H_I = 0;         EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.k = 0;           EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.k = 4097;        EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.H = 0;           EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.B = 0;           EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.Lq = 600;        EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.pos0 = -1;       EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.pos0 = INT32_MAX; EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.Lq = INT32_MAX; b.pos0 = INT32_MAX; b.Lk = INT32_MAX; EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.idx_dtype = 7;   EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_DTYPE);
    b = shape(); b.chunk = 100;     EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.chunk = -16;     EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    b = shape(); b.Lk = 1 << 24;    EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);    /* 4 GiB of KV rows */
    b = shape(); b.B = INT32_MAX; b.Lq = 512; b.Lk = 512;                              /* 2^40 query rows */
    EXPECT(stack("FSSS", 4, b, BIG), IC_ERR_SHAPE);
    EXPECT(stack("FSSS", 4, s, 16), IC_ERR_WORKSPACE);
    EXPECT(ic_run_stack("FSSS", 4, make_layers("FSSS"), &s, (int32_t*)FAKE, NULL, BIG, NULL, NULL), IC_ERR_WORKSPACE);
    EXPECT(ic_run_stack("FSSS", 4, make_layers("FSSS"), &s, (int32_t*)FAKE, (void*)0x10010, BIG, NULL, NULL),
           IC_ERR_WORKSPACE);
    make_layers("FSSS");
    layers[0].k_I = NULL;
    EXPECT(ic_run_stack("FSSS", 4, layers, &s, (int32_t*)FAKE, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    make_layers("FSSS");
    layers[2].kv = NULL;
    EXPECT(ic_run_stack("FSSS", 4, layers, &s, (int32_t*)FAKE, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);

    /* one F layer, its scores, the attention */
    EXPECT(ic_indexer_topk(&s, NULL, (const float*)FAKE, FAKE, (int32_t*)FAKE, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_indexer_topk(&s, FAKE, (const float*)FAKE, FAKE, (int32_t*)FAKE, FAKE_WS, 16, NULL), IC_ERR_WORKSPACE);
    b = shape(); b.d_I = 0;
    EXPECT(ic_indexer_topk(&b, FAKE, (const float*)FAKE, FAKE, (int32_t*)FAKE, FAKE_WS, BIG, NULL), IC_ERR_SHAPE);
    EXPECT(ic_indexer_scores(&s, FAKE, (const float*)FAKE, FAKE, NULL, 512, NULL), IC_ERR_ARG);
    EXPECT(ic_indexer_scores(&s, FAKE, (const float*)FAKE, FAKE, (float*)FAKE, 100, NULL), IC_ERR_SHAPE);
    EXPECT(ic_indexer_scores(&s, FAKE, (const float*)FAKE, FAKE, (float*)FAKE, INT64_MIN, NULL), IC_ERR_SHAPE);
    EXPECT(ic_sparse_attn(&s, NULL, FAKE, (const int32_t*)FAKE, FAKE, NULL, 0, NULL), IC_ERR_ARG);
    EXPECT(ic_sparse_attn(NULL, FAKE, FAKE, (const int32_t*)FAKE, FAKE, NULL, 0, NULL), IC_ERR_ARG);
    b = shape(); b.d = 32;
    EXPECT(ic_sparse_attn(&b, FAKE, FAKE, (const int32_t*)FAKE, FAKE, NULL, 0, NULL), IC_ERR_SHAPE);

    /* top-k of score rows */
    EXPECT(ic_topk_rows(NULL, 100, 4, 10, 8, (int32_t*)FAKE, NULL), IC_ERR_ARG);
    EXPECT(ic_topk_rows((const float*)FAKE, 100, 0, 10, 8, (int32_t*)FAKE, NULL), IC_ERR_SHAPE);
    EXPECT(ic_topk_rows((const float*)FAKE, 100, 4, 0, 8, (int32_t*)FAKE, NULL), IC_ERR_SHAPE);
    EXPECT(ic_topk_rows((const float*)FAKE, 100, 4, 98, 8, (int32_t*)FAKE, NULL), IC_ERR_SHAPE);
    EXPECT(ic_topk_rows((const float*)FAKE, 100, 4, 10, 5000, (int32_t*)FAKE, NULL), IC_ERR_SHAPE);
    EXPECT(ic_topk_rows((const float*)FAKE, INT64_MAX, INT32_MAX, INT32_MAX, 8, (int32_t*)FAKE, NULL), IC_ERR_SHAPE);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 100, 4, NULL, 100, 8, (int32_t*)FAKE, NULL, 0, NULL), IC_ERR_ARG);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 100, 4, (const int32_t*)FAKE, 100, 0, (int32_t*)FAKE, NULL, 0, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 100, 4, (const int32_t*)FAKE, 101, 8, (int32_t*)FAKE, NULL, 0, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 100, 4, (const int32_t*)FAKE, 0, 8, (int32_t*)FAKE, NULL, 0, NULL),
           IC_ERR_SHAPE);
    const size_t need = ic_topk_rows_seq_ws(32, 65600, 2048);
    EXPECT_NONZERO(need);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 65600, 32, (const int32_t*)FAKE, 65600, 2048, (int32_t*)FAKE, FAKE_WS,
                            need - 1, NULL), IC_ERR_WORKSPACE);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 65600, 32, (const int32_t*)FAKE, 65600, 2048, (int32_t*)FAKE,
                            (void*)0x10010, need, NULL), IC_ERR_WORKSPACE);
    (void)ic_topk_rows_seq_ws(8, INT32_MAX, 2048);                        /* extreme sizes: no overflow */
    (void)ic_topk_rows_seq_ws(INT32_MAX, INT32_MAX, 4096);
    (void)ic_topk_rows_seq_ws(-5, -5, -5);
    EXPECT_ZERO(ic_topk_rows_seq_ws(8, 65536, 0));

    /* ragged batches */
    ic_shape v = shape(); v.B = 2; v.Lq = 30; v.Lk = 100;
    int32_t ql[2] = {10, 20}, p0[2] = {0, 50}, sum_bad[2] = {10, 21}, far[2] = {0, 90}, neg[2] = {-1, 31};
    int32_t huge[2] = {INT32_MAX, INT32_MAX}, pneg[2] = {0, -1};
    int32_t* I = (int32_t*)FAKE;
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, NULL, p0, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack_varlen("SF", 2, make_layers("SF"), &v, ql, p0, I, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_NO_CACHED_INDICES);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, sum_bad, p0, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, ql, far, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, neg, p0, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, huge, p0, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, ql, pneg, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    ic_shape v2 = v; v2.pos0 = 5;
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v2, ql, p0, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_SHAPE);
    EXPECT(ic_run_stack_varlen("FS", 2, make_layers("FS"), &v, ql, p0, I, FAKE_WS, 16, NULL, NULL), IC_ERR_WORKSPACE);

    /* dynamic refresh */
    EXPECT(ic_run_stack_dynamic("SFSS", 4, make_layers("SFSS"), &s, 16, 0.5, I, NULL, NULL, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_NO_CACHED_INDICES);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, 0, 0.5, I, NULL, NULL, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_ARG);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, -3, 0.5, I, NULL, NULL, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_ARG);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, 16, -0.1, I, NULL, NULL, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_ARG);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, 16, NAN, I, NULL, NULL, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_ARG);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, 16, 0.5, I, NULL, NULL, FAKE_WS, 16, NULL, NULL),
           IC_ERR_WORKSPACE);

    /* decode */
    ic_shape d = shape(); d.B = 32; d.Lq = 1; d.Lk = 65600; d.k = 2048; d.H = 16; d.d = 128; d.H_I = 64; d.d_I = 128;
    d.idx_dtype = IC_FP8_E4M3;
    ic_shape d2 = d; d2.Lq = 2;
    EXPECT(ic_decode_step("FSSS", 4, make_layers("FSSS"), &d2, (const int32_t*)FAKE, I, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_decode_step("FSSS", 4, make_layers("FSSS"), &d, NULL, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_step("FSSS", 4, make_layers("FSSS"), &d, (const int32_t*)FAKE, I, FAKE_WS, 16, NULL, NULL),
           IC_ERR_WORKSPACE);
    EXPECT(ic_decode_step("SSSS", 4, make_layers("SSSS"), &d, (const int32_t*)FAKE, I, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_NO_CACHED_INDICES);
    ic_shape dbig = d; dbig.B = 64; dbig.Lk = 1 << 20;                  /* needs more than the static scratch */
    EXPECT(ic_decode_step_static("FSSS", 4, make_layers("FSSS"), &dbig, (const int32_t*)FAKE, I, NULL, NULL),
           IC_ERR_WORKSPACE);
    EXPECT(ic_decode_step_static("FSSS", 4, make_layers("FSSS"), &d, NULL, I, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_step_static("FSSS", 4, make_layers("FSSS"), &d2, (const int32_t*)FAKE, I, NULL, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_decode_indexer_scores(&d, FAKE, (const float*)FAKE, FAKE, NULL, (float*)FAKE, 65600, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_indexer_scores(&d, FAKE, (const float*)FAKE, FAKE, (const int32_t*)FAKE, (float*)FAKE, 100, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_decode_attn(&d, NULL, FAKE, (const int32_t*)FAKE, FAKE, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_attn(&d2, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE_WS, BIG, NULL), IC_ERR_SHAPE);
    EXPECT(ic_decode_attn(&d, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE_WS, 16, NULL), IC_ERR_WORKSPACE);

    /* cross-layer overlap */
    EXPECT(ic_index_overlap(NULL, (const int32_t*)FAKE, 4, 8, NULL, NULL, NULL, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_index_overlap((const int32_t*)FAKE, (const int32_t*)FAKE, 4, 0, NULL, NULL, NULL, NULL, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_index_overlap((const int32_t*)FAKE, (const int32_t*)FAKE, 4, 5000, NULL, NULL, NULL, NULL, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_index_overlap((const int32_t*)FAKE, (const int32_t*)FAKE, -1, 8, NULL, NULL, NULL, NULL, NULL),
           IC_ERR_SHAPE);
    EXPECT(ic_index_overlap((const int32_t*)FAKE, (const int32_t*)FAKE, 4, 8, NULL, NULL, NULL, (float*)FAKE, NULL),
           IC_ERR_ARG);

    /* distillation loss */
    const void* ptrs[2] = {FAKE, FAKE};
    const void* holes[2] = {FAKE, NULL};
    const float* W = (const float*)FAKE;
    float* KL = (float*)FAKE;
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 0, ptrs, ptrs, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 17, ptrs, ptrs, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, NULL, ptrs, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, ptrs, holes, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, ptrs, ptrs, NULL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    b = shape(); b.d = 96;
    EXPECT(ic_distill_kl(&b, FAKE, W, FAKE, I, 2, ptrs, ptrs, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_SHAPE);
    b = shape(); b.idx_dtype = 7;
    EXPECT(ic_distill_kl(&b, FAKE, W, FAKE, I, 2, ptrs, ptrs, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_DTYPE);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, ptrs, ptrs, KL, NULL, FAKE_WS, 16, NULL), IC_ERR_WORKSPACE);

    /* misaligned tensor pointers (views starting at an odd element): 16 bytes for q_I, k_I,
     * q, kv and out, 4 for the fp32 / int32 arrays */
    const uintptr_t odd2 = 0x1002, odd8 = 0x1008;
    make_layers("FSSS");
    layers[1].kv = (const void*)odd2;
    EXPECT(ic_run_stack("FSSS", 4, layers, &s, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    make_layers("FSSS");
    layers[0].q_I = (const void*)odd8;
    EXPECT(ic_run_stack("FSSS", 4, layers, &s, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    make_layers("FSSS");
    layers[0].w = (const float*)odd2;
    EXPECT(ic_run_stack("FSSS", 4, layers, &s, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    make_layers("FSSS");
    layers[3].out = (void*)odd8;
    EXPECT(ic_decode_step("FSSS", 4, layers, &d, (const int32_t*)FAKE, I, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack("FSSS", 4, make_layers("FSSS"), &s, (int32_t*)odd2, FAKE_WS, BIG, NULL, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_step("FSSS", 4, make_layers("FSSS"), &d, (const int32_t*)odd2, I, FAKE_WS, BIG, NULL, NULL),
           IC_ERR_ARG);
    EXPECT(ic_indexer_topk(&s, FAKE, (const float*)FAKE, (const void*)odd8, I, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_indexer_scores(&s, FAKE, (const float*)FAKE, FAKE, (float*)odd2, 512, NULL), IC_ERR_ARG);
    EXPECT(ic_sparse_attn(&s, FAKE, FAKE, (const int32_t*)FAKE, (void*)odd2, NULL, 0, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_attn(&d, (const void*)odd8, FAKE, (const int32_t*)FAKE, FAKE, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_decode_indexer_scores(&d, FAKE, (const float*)FAKE, (const void*)odd2, (const int32_t*)FAKE,
                                    (float*)FAKE, 65600, NULL), IC_ERR_ARG);
    EXPECT(ic_topk_rows((const float*)(uintptr_t)0x1001, 100, 4, 10, 8, I, NULL), IC_ERR_ARG);
    EXPECT(ic_topk_rows_seq((const float*)FAKE, 100, 4, (const int32_t*)odd2, 100, 8, I, NULL, 0, NULL), IC_ERR_ARG);
    EXPECT(ic_index_overlap((const int32_t*)odd2, (const int32_t*)FAKE, 4, 8, NULL, NULL, NULL, NULL, NULL),
           IC_ERR_ARG);
    const void* odd_kv[2] = {FAKE, (const void*)odd8};
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, ptrs, odd_kv, KL, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_distill_kl(&s, FAKE, W, FAKE, I, 2, ptrs, ptrs, (float*)odd2, NULL, FAKE_WS, BIG, NULL), IC_ERR_ARG);
    EXPECT(ic_run_stack_dynamic("FSSS", 4, make_layers("FSSS"), &s, 16, 0.5, I, (int32_t*)odd2, NULL, FAKE_WS, BIG,
                                NULL, NULL), IC_ERR_ARG);

    if (failures) fprintf(stderr, "%d unexpected results\n", failures);
    else printf("all argument checks behaved\n");
    return failures ? 1 : 0;
}
