/*
 * Host-side checks of the corrector C-ABI, built and run under AddressSanitizer
 * and UndefinedBehaviorSanitizer (host code only).  Every call made here either
 * fails host validation or is a no-op, so nothing is launched and no GPU is
 * needed; the weight and buffer pointers are aligned host addresses that the
 * library only validates and never dereferences.
 *
 * Covered: create with a valid descriptor and with each class of invalid
 * descriptor, the workspace and table sizes, each entry point's argument
 * checks, n_req = 0 no-ops, and the life cycle of a handle: calls and a
 * second destroy on a destroyed handle are rejected with CORR_E_HANDLE
 * without reading freed memory.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/corrector.h"

static int failures = 0;

#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static _Alignas(256) unsigned char arena[1 << 16];

static corrector_desc base_desc(void)
{
    corrector_desc d;
    memset(&d, 0, sizeof d);
    d.vocab = 1000;
    d.slots = 3;
    d.k = 4;
    d.d_hidden = 64;
    d.d_embed = 64;
    d.r = 16;
    d.mlp_hidden = 32;
    d.d_vec = 16;
    d.variant = CORR_VARIANT_MLP;
    d.logits_dtype = CORR_DTYPE_F32;
    d.max_requests = 4;
    d.ln_eps = 1e-5f;
    d.sigma = 1.0f;
    d.path_rule = CORR_PATH_GREEDY;
    d.path_lambda = 0.75f;
    d.beam_width = 2;
    return d;
}

static corrector_weights base_weights(void)
{
    corrector_weights w;
    w.embed = arena;
    w.w_cand = arena + 256;
    w.w_ctx = arena + 512;
    w.w_fuse = arena + 768;
    w.w_pair = arena + 1024;
    w.ln_gamma = (const float *)(arena + 1280);
    w.ln_beta = (const float *)(arena + 1536);
    w.w1 = arena + 1792;
    w.b1 = (const float *)(arena + 2048);
    w.w2 = (const float *)(arena + 2304);
    w.b2 = (const float *)(arena + 2560);
    w.w_out = arena + 2816;
    w.w_in = arena + 3072;
    return w;
}

static int create_with(corrector_desc d, corrector_weights w, corrector **h)
{
    *h = (corrector *)0x1;  /* must be reset to NULL on error */
    int rc = corrector_create(&d, &w, h);
    if (rc != CORR_OK) EXPECT(*h == NULL);
    return rc;
}

static void invalid_descriptors(void)
{
    corrector_weights w = base_weights();
    corrector *h;
    corrector_desc d;
#define BAD(field, value, code)                                  \
    do {                                                         \
        d = base_desc();                                         \
        d.field = value;                                         \
        EXPECT(create_with(d, w, &h) == (code));                 \
    } while (0)
    BAD(variant, 7, CORR_E_UNSUPPORTED);
    BAD(logits_dtype, 9, CORR_E_UNSUPPORTED);
    BAD(path_rule, 11, CORR_E_UNSUPPORTED);
    BAD(vocab, 0, CORR_E_SHAPE);
    BAD(vocab, 3, CORR_E_SHAPE);              /* K > V */
    BAD(slots, 0, CORR_E_SHAPE);
    BAD(slots, 65, CORR_E_SHAPE);
    BAD(k, 0, CORR_E_SHAPE);
    BAD(k, 65, CORR_E_SHAPE);
    BAD(d_hidden, 48, CORR_E_SHAPE);
    BAD(d_embed, 0, CORR_E_SHAPE);
    BAD(r, 48, CORR_E_UNSUPPORTED);
    BAD(mlp_hidden, 24, CORR_E_UNSUPPORTED);
    BAD(max_requests, 0, CORR_E_SHAPE);
    BAD(ln_eps, 0.0f, CORR_E_SHAPE);
    BAD(succ_top_m, 5, CORR_E_SHAPE);
    BAD(succ_top_m, -1, CORR_E_SHAPE);
    d = base_desc();
    d.path_rule = CORR_PATH_GEOMETRIC;
    d.path_lambda = 0.0f;
    EXPECT(create_with(d, w, &h) == CORR_E_SHAPE);
    d.path_lambda = 1.5f;
    EXPECT(create_with(d, w, &h) == CORR_E_SHAPE);
    d = base_desc();
    d.path_rule = CORR_PATH_BEAM;
    d.beam_width = 5;
    EXPECT(create_with(d, w, &h) == CORR_E_SHAPE);
    d = base_desc();
    d.variant = CORR_VARIANT_COSINE;
    d.d_vec = 24;
    EXPECT(create_with(d, w, &h) == CORR_E_UNSUPPORTED);
#undef BAD
    /* null and misaligned weights */
    d = base_desc();
    EXPECT(corrector_create(&d, &w, NULL) == CORR_E_NULL);
    EXPECT(create_with(d, w, &h) == CORR_OK);
    corrector_destroy(h);
    corrector_weights w2 = w;
    w2.w1 = NULL;
    EXPECT(create_with(d, w2, &h) == CORR_E_NULL);
    w2 = w;
    w2.w_cand = arena + 2;
    EXPECT(create_with(d, w2, &h) == CORR_E_ALIGN);
    /* the cosine variant needs w_out / w_in, not the MLP weights */
    d.variant = CORR_VARIANT_COSINE;
    w2 = w;
    w2.w_in = NULL;
    EXPECT(create_with(d, w2, &h) == CORR_E_NULL);
    w2 = w;
    w2.w1 = NULL;
    w2.w_pair = NULL;
    EXPECT(create_with(d, w2, &h) == CORR_OK);
    corrector_destroy(h);
}

static void argument_checks(corrector *h)
{
    const corrector_desc d = base_desc();
    /* ws: the size for one request, which every n_req = 1 call below uses */
    const size_t ws = corrector_workspace_bytes(h, 1);
    EXPECT(ws > 0);
    EXPECT(corrector_workspace_bytes(h, d.max_requests) >= ws);
    EXPECT(corrector_workspace_bytes(h, d.max_requests + 1) == 0);
    EXPECT(corrector_workspace_bytes(h, -1) == 0);
    EXPECT(corrector_table_bytes(h) == sizeof(float) * (size_t)d.vocab * d.r);
    void *p = arena + 4096;
    int32_t *ip = (int32_t *)(arena + 8192);
    float *fp = (float *)(arena + 12288);
    const int64_t V = d.vocab, B1 = d.slots + 1;
    /* n_req = 0 is a no-op on every call, whatever the buffers */
    EXPECT(corrector_topk(h, 0, NULL, 0, 0, NULL, NULL, NULL, 0, NULL) == CORR_OK);
    EXPECT(corrector_score(h, 0, NULL, NULL, NULL, 0, 0, NULL, NULL, 0, NULL) == CORR_OK);
    EXPECT(corrector_walk(h, 0, NULL, NULL, NULL, NULL, NULL) == CORR_OK);
    EXPECT(corrector_run(h, 0, NULL, 0, 0, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == CORR_OK);
    /* too many requests */
    EXPECT(corrector_topk(h, d.max_requests + 1, p, B1 * V, V, ip, fp, p, ws, NULL) == CORR_E_SHAPE);
    EXPECT(corrector_run(h, -1, p, B1 * V, V, p, B1 * 64, 64, ip, NULL, NULL, NULL, NULL, p, ws, NULL) ==
           CORR_E_SHAPE);
    /* null, misaligned, negative strides, short workspace */
    EXPECT(corrector_topk(h, 1, NULL, B1 * V, V, ip, fp, p, ws, NULL) == CORR_E_NULL);
    EXPECT(corrector_topk(h, 1, p, B1 * V, V, NULL, fp, p, ws, NULL) == CORR_E_NULL);
    EXPECT(corrector_topk(h, 1, (char *)p + 4, B1 * V, V, ip, fp, p, ws, NULL) == CORR_E_ALIGN);
    EXPECT(corrector_topk(h, 1, p, B1 * V + 1, V, ip, fp, p, ws, NULL) == CORR_E_ALIGN);
    EXPECT(corrector_topk(h, 1, p, -1, V, ip, fp, p, ws, NULL) == CORR_E_SHAPE);
    EXPECT(corrector_topk(h, 1, p, B1 * V, V, ip, fp, NULL, ws, NULL) == CORR_E_NULL);
    EXPECT(corrector_topk(h, 1, p, B1 * V, V, ip, fp, (char *)p + 8, ws, NULL) == CORR_E_ALIGN);
    EXPECT(corrector_topk(h, 1, p, B1 * V, V, ip, fp, p, 16, NULL) == CORR_E_WORKSPACE);
    EXPECT(corrector_topk_softmax(h, 1, p, B1 * V, V, ip, fp, NULL, NULL, p, ws, NULL) == CORR_E_NULL);
    EXPECT(corrector_score(h, 1, ip, fp, (char *)p + 2, 64, 64, fp, p, ws, NULL) == CORR_E_ALIGN);
    EXPECT(corrector_score(h, 1, ip, fp, p, B1 * 64, 64, NULL, p, ws, NULL) == CORR_E_NULL);
    EXPECT(corrector_score(h, 1, ip, fp, p, B1 * 64, 64, fp, p, 0, NULL) == CORR_E_WORKSPACE);
    EXPECT(corrector_walk(h, 1, NULL, ip, ip, NULL, NULL) == CORR_E_NULL);
    EXPECT(corrector_walk(h, 1, fp, ip, NULL, NULL, NULL) == CORR_E_NULL);
    EXPECT(corrector_run(h, 1, p, B1 * V, V, p, B1 * 64, 64, NULL, NULL, NULL, NULL, NULL, p, ws, NULL) ==
           CORR_E_NULL);
    EXPECT(corrector_run(h, 1, p, B1 * V, V, p, B1 * 64, 64, ip, NULL, NULL, NULL, NULL, p, ws - 1, NULL) ==
           CORR_E_WORKSPACE);
    EXPECT(corrector_run_static(h, 1, p, B1 * V, V, p, B1 * 64, 64, NULL, NULL, NULL, NULL, NULL, NULL) ==
           CORR_E_NULL);
    EXPECT(corrector_run_static(h, 1, (char *)p + 4, B1 * V, V, p, B1 * 64, 64, ip, NULL, NULL, NULL, NULL, NULL) ==
           CORR_E_ALIGN);
    EXPECT(corrector_run_static(h, d.max_requests + 1, p, B1 * V, V, p, B1 * 64, 64, ip, NULL, NULL, NULL, NULL,
                                NULL) == CORR_E_SHAPE);
    EXPECT(corrector_intermediates(h, 1, p, 8, NULL, NULL, NULL, NULL) == CORR_E_WORKSPACE);
    EXPECT(corrector_fold_table(h, NULL, NULL) == CORR_E_NULL);
    EXPECT(corrector_fold_table(h, (float *)((char *)p + 4), NULL) == CORR_E_ALIGN);
    EXPECT(corrector_use_table(h, (const float *)((char *)p + 4)) == CORR_E_ALIGN);
    EXPECT(corrector_use_table(h, NULL) == CORR_OK);
    /* timing off: no events exist, no kernel times */
    EXPECT(corrector_set_timing(h, 0) == CORR_OK);
    EXPECT(corrector_kernel_times(h, NULL, NULL, 0) == 0);
}

static void handle_lifecycle(void)
{
    corrector_desc d = base_desc();
    corrector_weights w = base_weights();
    corrector *a, *b;
    EXPECT(create_with(d, w, &a) == CORR_OK);
    EXPECT(create_with(d, w, &b) == CORR_OK);
    EXPECT(a != b);
    argument_checks(a);
    corrector_destroy(a);
    /* a is gone: every call rejects it without reading through it */
    EXPECT(corrector_workspace_bytes(a, 1) == 0);
    EXPECT(corrector_table_bytes(a) == 0);
    EXPECT(corrector_run(a, 1, arena, 0, 0, arena, 0, 0, (int32_t *)arena, NULL, NULL, NULL, NULL, arena, 1 << 20,
                         NULL) == CORR_E_HANDLE);
    EXPECT(corrector_walk(a, 1, (const float *)arena, (const int32_t *)arena, (int32_t *)arena, NULL, NULL) ==
           CORR_E_HANDLE);
    EXPECT(corrector_use_table(a, NULL) == CORR_E_HANDLE);
    EXPECT(corrector_set_timing(a, 0) == CORR_E_HANDLE);
    EXPECT(corrector_kernel_times(a, NULL, NULL, 0) == -CORR_E_HANDLE);
    EXPECT(corrector_fold_table(a, (float *)arena, NULL) == CORR_E_HANDLE);
    corrector_destroy(a);  /* second destroy: ignored */
    corrector_destroy(NULL);
    /* b is unaffected */
    EXPECT(corrector_workspace_bytes(b, 1) > 0);
    corrector_destroy(b);
    EXPECT(corrector_workspace_bytes(b, 1) == 0);
    EXPECT(corrector_run_static(b, 1, arena, 0, 0, arena, 0, 0, (int32_t *)arena, NULL, NULL, NULL, NULL, NULL) ==
           CORR_E_HANDLE);
    /* a batch whose workspace exceeds the static array is refused on the host */
    corrector_desc big = base_desc();
    big.vocab = 151936;
    big.slots = 15;
    big.k = 64;
    big.d_hidden = 4096;
    big.d_embed = 4096;
    big.r = 128;
    big.mlp_hidden = 256;
    big.max_requests = 4096;
    corrector *c;
    EXPECT(create_with(big, w, &c) == CORR_OK);
    EXPECT(corrector_workspace_bytes(c, 4096) > ((size_t)64 << 20));
    EXPECT(corrector_run_static(c, 4096, arena, 0, 0, arena, 0, 0, (int32_t *)arena, NULL, NULL, NULL, NULL, NULL) ==
           CORR_E_WORKSPACE);
    corrector_destroy(c);
    /* a pointer that never was a handle */
    EXPECT(corrector_workspace_bytes((const corrector *)arena, 1) == 0);
    corrector_destroy((corrector *)arena);
    /* many handles created and destroyed in interleaved order */
    corrector *hs[64];
    for (int i = 0; i < 64; ++i) EXPECT(create_with(d, w, &hs[i]) == CORR_OK);
    for (int i = 0; i < 64; i += 2) corrector_destroy(hs[i]);
    for (int i = 1; i < 64; i += 2) EXPECT(corrector_workspace_bytes(hs[i], 2) > 0);
    for (int i = 1; i < 64; i += 2) corrector_destroy(hs[i]);
}

int main(void)
{
    for (int s = -1; s <= 8; ++s) EXPECT(corrector_status_string(s) != NULL);
    invalid_descriptors();
    handle_lifecycle();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi host checks passed\n");
    return 0;
}
