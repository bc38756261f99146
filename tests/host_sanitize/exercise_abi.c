/* Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built against a host-instrumented copy of the library (device code is not
 * built) and run without a GPU: every call below either fails validation, only
 * sizes a workspace, or validates and plans a step and then fails at its first
 * HIP call.  That drives the host code -- argument checks, overlap tests, the
 * shape-group plan, the workspace layout, the launch tables, the schedule
 * cache and its eviction -- under the sanitizers.  Device pointers are fake,
 * distinct addresses; nothing dereferences them on the host.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "muonstep.h"

static int failures = 0;
#define EXPECT(cond)                                                                                   \
    do {                                                                                               \
        if (!(cond)) {                                                                                 \
            fprintf(stderr, "FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond,            \
                    muon_last_error());                                                                \
            ++failures;                                                                                \
        }                                                                                              \
    } while (0)

static const uintptr_t kBase = (uintptr_t)1 << 44;

/* Tensor k's buffers: five fake, disjoint 1 GiB ranges. */
static muon_tensor_t tensor(int k, int rows, int cols) {
    const uintptr_t b = kBase + ((uintptr_t)k << 33);
    muon_tensor_t t;
    t.param = (float*)(b);
    t.grad = (const float*)(b + ((uintptr_t)1 << 30));
    t.momentum = (float*)(b + ((uintptr_t)2 << 30));
    t.update_out = NULL;
    t.ema = (float*)(b + ((uintptr_t)3 << 30));
    t.rows = rows;
    t.cols = cols;
    return t;
}

static float coeffs[MUON_MAX_NS_STEPS * 3];

static int step(const muon_tensor_t* t, int n, float lr, int steps, int precision, void* ws, size_t ws_bytes) {
    return muon_step(t, n, lr, 0.95f, 1, 0.1f, 1, steps, coeffs, precision, 0.99f, ws, ws_bytes, NULL);
}

static void check_workspace_and_validation(void) {
    muon_tensor_t t[4] = {tensor(0, 512, 512), tensor(1, 256, 512), tensor(2, 2048, 512), tensor(3, 512, 2048)};
    const size_t ws = muon_workspace_size(t, 4, MUON_NS_BF16);
    EXPECT(ws > 0);
    EXPECT(muon_workspace_size(t, 4, MUON_NS_FP32) > 0);
    EXPECT(muon_workspace_size(t, 4, MUON_NS_BF16X3) > 0);
    EXPECT(muon_workspace_size(t, 1, MUON_NS_BF16) < ws);
    void* wsp = (void*)(kBase - ((uintptr_t)1 << 40));
    EXPECT(step(t, 4, NAN, 5, MUON_NS_BF16, wsp, ws) == MUON_ERR_INVALID_ARG);
    EXPECT(step(t, 0, 0.02f, 5, MUON_NS_BF16, wsp, ws) == MUON_ERR_INVALID_ARG);
    EXPECT(step(t, 4, 0.02f, MUON_MAX_NS_STEPS + 1, MUON_NS_BF16, wsp, ws) == MUON_ERR_INVALID_ARG);
    EXPECT(step(t, 4, 0.02f, 5, 7, wsp, ws) == MUON_ERR_INVALID_ARG);
    EXPECT(step(t, 4, 0.02f, 5, MUON_NS_BF16, wsp, ws - 1) == MUON_ERR_WORKSPACE);
    EXPECT(step(t, 4, 0.02f, 5, MUON_NS_BF16, NULL, ws) != MUON_OK);
    coeffs[4] = NAN;
    EXPECT(step(t, 4, 0.02f, 5, MUON_NS_BF16, wsp, ws) == MUON_ERR_INVALID_ARG);
    coeffs[4] = -4.775f;
    muon_tensor_t bad[2] = {tensor(0, 512, 512), tensor(1, 512, 512)};
    bad[1].grad = bad[0].param + 64;                    /* aliases another tensor's weights */
    EXPECT(step(bad, 2, 0.02f, 5, MUON_NS_BF16, wsp, muon_workspace_size(bad, 2, MUON_NS_BF16)) ==
           MUON_ERR_UNSUPPORTED);
    bad[1] = tensor(1, 512, 512);
    bad[1].param = NULL;
    EXPECT(step(bad, 2, 0.02f, 5, MUON_NS_BF16, wsp, ws) == MUON_ERR_INVALID_ARG);
    bad[1] = tensor(1, 0, 512);
    EXPECT(step(bad, 2, 0.02f, 5, MUON_NS_BF16, wsp, ws) != MUON_OK);
    bad[1] = tensor(1, MUON_MAX_SHORT_SIDE + 1, MUON_MAX_SHORT_SIDE + 1);
    EXPECT(step(bad, 2, 0.02f, 5, MUON_NS_BF16, wsp, ws) == MUON_ERR_UNSUPPORTED);
    /* the workspace overlapping a tensor */
    EXPECT(step(t, 4, 0.02f, 5, MUON_NS_BF16, (void*)t[2].param, ws) == MUON_ERR_UNSUPPORTED);
    EXPECT(muon_step_static(t, 0, 0.02f, 0.95f, 1, 0.1f, 1, 5, coeffs, MUON_NS_BF16, 0.99f, NULL) ==
           MUON_ERR_INVALID_ARG);
}

/* Valid calls: validation and planning run, then the first HIP call fails. */
static void check_planning_and_cache(void) {
    enum { kMany = 90 };
    muon_tensor_t* t = (muon_tensor_t*)calloc(kMany, sizeof(muon_tensor_t));
    for (int i = 0; i < kMany; ++i) {
        /* 80+ distinct oriented shapes, ragged on both sides, some tall, one with an update output */
        const int r = 33 + 37 * (i % 41), c = 65 + 29 * (i % 23);
        t[i] = tensor(10 + i, (i % 3 == 0) ? c : r, (i % 3 == 0) ? r : c);
        if (i == 5) t[i].update_out = (float*)((uintptr_t)t[i].param + ((uintptr_t)4 << 30));
    }
    const int precisions[3] = {MUON_NS_BF16, MUON_NS_FP32, MUON_NS_BF16X3};
    for (int schedule = MUON_NS_SCHEDULE_PHASES; schedule <= MUON_NS_SCHEDULE_CHAIN; ++schedule) {
        EXPECT(muon_set_ns_schedule(schedule) >= 0);
        for (int p = 0; p < 3; ++p) {
            const size_t ws = muon_workspace_size(t, kMany, precisions[p]);
            EXPECT(ws > 0);
            void* wsp = (void*)(kBase - ((uintptr_t)1 << 42));
            int64_t built0 = 0, hits0 = 0, built1 = 0, hits1 = 0;
            muon_plan_cache_stats(&built0, &hits0);
            int rc = step(t, kMany, 0.02f, 5, precisions[p], wsp, ws);
            EXPECT(rc == MUON_ERR_HIP || rc == MUON_OK);
            rc = step(t, kMany, 0.03f, 3, precisions[p], wsp, ws);
            EXPECT(rc == MUON_ERR_HIP || rc == MUON_OK);
            muon_plan_cache_stats(&built1, &hits1);
            EXPECT(built1 == built0 + 1 && hits1 == hits0 + 1);
        }
    }
    EXPECT(muon_set_ns_schedule(7) < 0);
    EXPECT(muon_set_ns_schedule(MUON_NS_SCHEDULE_PHASES) == MUON_NS_SCHEDULE_CHAIN);
    /* more signatures than the cache holds: eviction */
    for (int k = 0; k < 12; ++k) {
        muon_tensor_t one[2] = {tensor(200 + k, 512, 512 + 128 * k), tensor(300 + k, 256, 512)};
        const size_t ws = muon_workspace_size(one, 2, MUON_NS_BF16);
        int rc = step(one, 2, 0.02f, 5, MUON_NS_BF16, (void*)(kBase - ((uintptr_t)1 << 42)), ws);
        EXPECT(rc == MUON_ERR_HIP || rc == MUON_OK);
    }
    /* the static entry point refuses what its workspace cannot hold, before any HIP call */
    muon_tensor_t big[30];
    for (int i = 0; i < 30; ++i) big[i] = tensor(400 + i, 2048, 512);
    EXPECT(muon_step_static(big, 30, 0.02f, 0.95f, 1, 0.1f, 1, 5, coeffs, MUON_NS_BF16, 0.99f, NULL) ==
           MUON_ERR_WORKSPACE);
    free(t);
}

static void check_streaming_entry_points(void) {
    float* e[3];
    const float* p[3];
    float* pw[3];
    int64_t ne[3] = {100, 4097, 1 << 20};
    for (int i = 0; i < 3; ++i) {
        e[i] = (float*)(kBase + ((uintptr_t)(500 + i) << 33));
        p[i] = (const float*)(kBase + ((uintptr_t)(600 + i) << 33));
        pw[i] = (float*)p[i];
    }
    EXPECT(ema_update(e, p, ne, 3, NAN, NULL) == MUON_ERR_INVALID_ARG);
    EXPECT(ema_update(e, p, ne, -1, 0.5f, NULL) == MUON_ERR_INVALID_ARG);
    EXPECT(ema_update(NULL, p, ne, 3, 0.5f, NULL) == MUON_ERR_INVALID_ARG);
    int64_t neg[3] = {100, -1, 5};
    EXPECT(ema_update(e, p, neg, 3, 0.5f, NULL) == MUON_ERR_INVALID_ARG);
    int64_t huge[3] = {100, (int64_t)1 << 41, 5};
    EXPECT(ema_update(e, p, huge, 3, 0.5f, NULL) == MUON_ERR_UNSUPPORTED);
    const float* alias[3] = {(const float*)(e[0] + 10), p[1], p[2]};
    EXPECT(ema_update(e, alias, ne, 3, 0.5f, NULL) == MUON_ERR_UNSUPPORTED);
    EXPECT(ema_swap(e, pw, neg, 3, NULL) == MUON_ERR_INVALID_ARG);
    adamw_tensor_t a[2];
    for (int i = 0; i < 2; ++i) {
        const uintptr_t b = kBase + ((uintptr_t)(700 + i) << 33);
        a[i].param = (float*)b;
        a[i].grad = (const float*)(b + ((uintptr_t)1 << 30));
        a[i].exp_avg = (float*)(b + ((uintptr_t)2 << 30));
        a[i].exp_avg_sq = (float*)(b + ((uintptr_t)3 << 30));
        a[i].ema = NULL;
        a[i].numel = 1000 + i;
    }
    EXPECT(adamw_step(a, 2, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 0, 0.0f, NULL) == MUON_ERR_INVALID_ARG);
    EXPECT(adamw_step(a, 2, 1e-3f, 1.5f, 0.999f, 1e-8f, 0.01f, 10, 0.0f, NULL) == MUON_ERR_INVALID_ARG);
    a[1].grad = a[0].param;
    EXPECT(adamw_step(a, 2, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 10, 0.0f, NULL) == MUON_ERR_UNSUPPORTED);
    /* the step with the other tensors' EMA: a valid call plans and fails at its first HIP call; an extra
     * buffer inside a matrix's is refused before anything */
    muon_tensor_t m2[2] = {tensor(800, 512, 512), tensor(801, 256, 512)};
    const size_t ws2 = muon_workspace_size(m2, 2, MUON_NS_BF16);
    void* wsp2 = (void*)(kBase - ((uintptr_t)1 << 42));
    int rc = muon_step_ema(m2, 2, 0.02f, 0.95f, 1, 0.1f, 1, 5, coeffs, MUON_NS_BF16, 0.99f, e, p, ne, 3, wsp2, ws2,
                           NULL);
    EXPECT(rc == MUON_ERR_HIP || rc == MUON_OK);
    float* e_bad[3] = {e[0], (float*)m2[1].grad + 8, e[2]};
    EXPECT(muon_step_ema(m2, 2, 0.02f, 0.95f, 1, 0.1f, 1, 5, coeffs, MUON_NS_BF16, 0.99f, e_bad, p, ne, 3, wsp2,
                         ws2, NULL) == MUON_ERR_UNSUPPORTED);
    EXPECT(muon_step_ema(m2, 2, 0.02f, 0.95f, 1, 0.1f, 1, 5, coeffs, MUON_NS_BF16, 0.99f, e, p, ne, -2, wsp2, ws2,
                         NULL) == MUON_ERR_INVALID_ARG);
    EXPECT(muon_profile_enable(0) == 0);
    EXPECT(muon_profile_read(NULL, NULL, NULL, 0, 1) == 0);
}

int main(void) {
    for (int k = 0; k < MUON_MAX_NS_STEPS; ++k) {
        coeffs[3 * k] = 3.4445f;
        coeffs[3 * k + 1] = -4.775f;
        coeffs[3 * k + 2] = 2.0315f;
    }
    EXPECT(muon_version() > 0);
    EXPECT(muon_last_error() != NULL);
    check_workspace_and_validation();
    check_planning_and_cache();
    check_streaming_entry_points();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
