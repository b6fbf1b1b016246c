/* Drives the host entry points of host_model.cpp (byte accounting, step-time model,
 * fits, error bounds, subtree selection) over seeded random and edge-case inputs,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer: any invalid
 * memory access, leak or undefined operation aborts the run.  Prints "ok" and the
 * number of calls at the end. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_expert.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}
static int ri(int lo, int hi) { return lo + (int)(rnd() % (uint64_t)(hi - lo + 1)); }
static double rd(double lo, double hi) { return lo + (hi - lo) * (double)(rnd() >> 11) * 0x1.0p-53; }

int main(void) {
    long calls = 0;
    /* bytes_requested: valid, out-of-range and repeated ids, bad descriptors */
    for (int it = 0; it < 2000; ++it) {
        moe_layer_desc d = {ri(1, 1024), 1, 8 * ri(1, 64), 8 * ri(1, 64), ri(0, 1) ? MOE_BF16 : MOE_F32, 0u, 0};
        d.m = ri(1, d.N < 16 ? d.N : 16);
        int n = ri(1, 16);
        int32_t ids[256];
        for (int s = 0; s < n * d.m; ++s) ids[s] = ri(-2, d.N + 1);
        (void)bytes_requested(ri(-1, 2), &d, ids, n);
        (void)bytes_requested(MOE_KIND_DEDUP, &d, ids, ri(-1, 0));
        calls += 2;
    }
    (void)bytes_requested(MOE_KIND_SLOT, NULL, NULL, 1);
    /* step_time_model: random sizes and values, then invalid inputs */
    for (int it = 0; it < 400; ++it) {
        moe_step_in in;
        moe_step_out out;
        memset(&in, 0, sizeof in);
        in.n_max = ri(1, MOE_STEP_NMAX + 1);
        in.n_a = ri(0, MOE_STEP_AMAX + 1);
        for (int i = 0; i < MOE_STEP_AMAX; ++i) in.a[i] = rd(0.0, 1.0);
        in.m_W = ri(0, 9) ? rd(1e6, 1e10) : 0.0;
        in.t0 = rd(0, 1e-5);
        in.D = rd(0, 1e9);
        in.beta_D = rd(1e11, 8e12);
        for (int k = 0; k < MOE_STEP_NMAX; ++k) {
            in.kv[k] = rd(0, 1e8) * k;
            in.h[k] = rd(0, 1e-5);
            for (int p = 0; p < 2; ++p) {
                in.E[p][k] = rd(1e6, 1e10);
                in.beta[p][k] = ri(0, 30) ? rd(1e11, 8e12) : 0.0;
                in.phi[p][k] = rd(0, 1e-5);
            }
        }
        (void)step_time_model(&in, &out);
        calls++;
    }
    (void)step_time_model(NULL, NULL);
    /* moe_fit_times */
    for (int it = 0; it < 400; ++it) {
        int count = ri(-1, 40), m = ri(1, 8);
        int32_t n[40], U[40];
        double t[40], coef[3];
        for (int i = 0; i < 40; ++i) {
            n[i] = ri(1, 9);
            U[i] = ri(0, n[i] * m + 1);
            t[i] = rd(1e-6, 1e-3);
        }
        (void)moe_fit_times(ri(-1, 2), count, n, U, m, t, rd(-1.0, 1e9), coef);
        calls++;
    }
    /* moe_error_bounds */
    double eb[5];
    for (int it = 0; it < 200; ++it) {
        (void)moe_error_bounds(rd(-0.2, 0.7), eb);
        calls++;
    }
    (void)moe_error_bounds(0.1, NULL);
    /* moe_tree_select: random trees (parents before children), layers, bitmaps */
    for (int it = 0; it < 150; ++it) {
        int V = ri(0, 24), L = ri(1, 4), words = ri(1, 4), K = ri(0, 8);
        int32_t parent[64], level[64];
        double p[64], b[MOE_TREE_MAXK + 1];
        static uint64_t bm[64 * 4 * 4];
        parent[0] = -1;
        level[0] = 0;
        p[0] = 1.0;
        for (int v = 1; v <= V; ++v) {
            parent[v] = ri(0, v - 1);
            level[v] = level[parent[v]] + 1;
            p[v] = p[parent[v]] * rd(0.0, 1.0);
        }
        for (int i = 0; i < (V + 1) * L * words; ++i) bm[i] = rnd() & rnd();
        for (int k = 0; k <= MOE_TREE_MAXK; ++k) b[k] = rd(1e-6, 1e-4);
        moe_tree_in in = {V, L, words, K, parent, p, bm, b, rd(1e-7, 1e-5), ri(-1, 3), level};
        moe_tree_out out;
        (void)moe_tree_select(&in, &out);
        calls++;
    }
    (void)moe_tree_select(NULL, NULL);
    printf("ok %ld\n", calls);
    return 0;
}
