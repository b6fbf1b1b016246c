/* The C ABI of include/moe_expert.h used from plain C99 (no C++ and no Python):
 * host-side entry points and the validation that rejects bad arguments before any
 * launch, so it runs without a GPU.  Prints one "name value" line per result and
 * exits non-zero on the first failed check. */
#include <stdio.h>
#include <stdlib.h>

#include "moe_expert.h"

static int fails = 0;

static void check(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "FAIL %s\n", what);
        fails++;
    }
}

int main(void) {
    /* a DeepSeek-V2-Lite-shaped layer: 64 experts, top-6, d 2048, d_ff 1408, bf16 */
    moe_layer_desc d = {64, 6, 2048, 1408, MOE_BF16, 0u, 0};
    const int32_t ids[2 * 6] = {0, 1, 2, 3, 4, 5, 0, 1, 2, 3, 4, 63};
    const int64_t w = 3ll * 2048 * 1408 * 2;

    int64_t slot = bytes_requested(MOE_KIND_SLOT, &d, ids, 2);
    int64_t dedup = bytes_requested(MOE_KIND_DEDUP, &d, ids, 2);
    printf("bytes_slot %lld\nbytes_dedup %lld\n", (long long)slot, (long long)dedup);
    check(slot == 12 * w, "per-slot bytes = n m w");
    check(dedup == 7 * w, "dedup bytes = X(n) w (7 distinct experts)");

    size_t ws = moe_workspace_bytes(&d, 8, MOE_KIND_SLOT);
    printf("workspace_slot_n8 %zu\n", ws);
    check(ws > 0, "workspace size for n = 8");

    /* rejected before any launch */
    moe_layer_desc bad = d;
    bad.m = 0;
    moe_layer_weights W = {0, 0, 0, 0, 0, 0};
    check(moe_expert_perslot(&bad, &W, 0, 0, 0, 1, 0, 0, 0, 0, 0) == MOE_E_INVAL, "m = 0 rejected");
    check(moe_expert_dedup(&d, &W, 0, 0, 0, 1, 0, 0, 0, 0, 0) == MOE_E_INVAL, "null pointers rejected");
    check(moe_pack_tiled(&d, (void*)0x1000, (void*)0x900000, 7, 0) == MOE_E_INVAL, "bad matrix code rejected");
    bad = d;
    bad.flags = MOE_FLAG_TILED | MOE_FLAG_WDOWN_PACKED;
    check(moe_workspace_bytes(&bad, 4, MOE_KIND_SLOT) == 0, "tiled and packed together rejected");

    /* Table 2 factors at eps = 0.1: delta = eps / (1 - eps) */
    double eb[5];
    check(moe_error_bounds(0.1, eb) == MOE_OK, "error bounds");
    printf("delta %.6f\n", eb[2]);
    check(eb[2] > 0.1111 && eb[2] < 0.1112, "delta = 1/9");

    /* Eq. (E.1) fit of exact data t = 10 us + 1e-15 s/B * U b + 0.5 us * n (b = 1 GB) */
    int32_t n[5] = {1, 2, 2, 3, 4}, U[5] = {1, 2, 3, 4, 6};
    double t[5], coef[3];
    for (int i = 0; i < 5; ++i) t[i] = 10e-6 + 1e-6 * U[i] + 0.5e-6 * n[i];
    check(moe_fit_times(MOE_KIND_DEDUP, 5, n, U, 2, t, 1e9, coef) == MOE_OK, "fit");
    printf("fit %.6e %.6e %.6e\n", coef[0], coef[1], coef[2]);
    check(coef[0] > 9.999e-6 && coef[0] < 10.001e-6, "t_op");
    check(coef[1] > 0.9999e-15 && coef[1] < 1.0001e-15, "c_g");
    check(coef[2] > 0.4999e-6 && coef[2] < 0.5001e-6, "c_t");
    int32_t nn[3] = {1, 2, 3}, UU[3] = {1, 2, 3};  /* U = n: the three constants are not determined */
    check(moe_fit_times(MOE_KIND_DEDUP, 3, nn, UU, 1, t, 1e9, coef) == MOE_E_INVAL, "undetermined fit rejected");

    printf("failures %d\n", fails);
    return fails ? 1 : 0;
}
