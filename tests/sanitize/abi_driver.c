/*
 * Calls the C ABI of librr through its host-side argument checks (no GPU
 * work is enqueued: every call fails validation or only sizes a buffer), for
 * a build of the host code under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Prints "ok" and exits 0 when every call
 * returns the documented status.
 */
#include <stdio.h>
#include <stdint.h>
#include <stddef.h>
#include "rr.h"
int main(void) {
    void *F = (void *)0x1000;
    int bad = 0;
    bad += rr_estimate(NULL, F, 1024, 8, 2, 128, 128, 8, F, F, 1ull << 40, NULL) != RR_E_NULL;
    bad += rr_estimate(F, F, 1004, 8, 2, 128, 128, 8, F, F, 1ull << 40, NULL) != RR_E_SHAPE;
    bad += rr_estimate(F, F, 1024, 8, 2, 96, 128, 8, F, F, 1ull << 40, NULL) != RR_E_UNSUPPORTED;
    bad += rr_estimate(F, F, 1024, 8, 2, 128, 128, 8, F, F, 16, NULL) != RR_E_WORKSPACE;
    bad += rr_select(F, 8, 1024, 128, 1.5f, F, F, NULL) != RR_E_TAU;
    bad += rr_sparse_attn(F, F, F, 1024, 8, 2, 128, 128, F, F, F, 7, F, 1ull << 40, NULL) != RR_E_UNSUPPORTED;
    bad += rr_prefill(F, F, F, 128 * 4097, 8, 2, 128, 128, 8, 0.9f, F, 0, F, F, F, 1ull << 40, NULL) != RR_E_UNSUPPORTED;
    bad += rr_estimate_materialized(F, F, 1024, 8, 2, 128, 128, 64, F, F, F, 1ull << 40, NULL) != RR_E_UNSUPPORTED;
    bad += rr_estimate_workspace_bytes(1024, 8, 2, 128, 128, 8) == 0;
    bad += rr_stride_scores_count(1216, 8, 2, 128, 128, 8) != 8LL * 16 * 16 * 10 * 11 / 2;
    for (int c = 0; c < 7; ++c) bad += rr_status_str(c) == NULL;
    printf(bad ? "bad %d\n" : "ok\n", bad);
    return bad != 0;
}
