/* Drives the CPU oracle (moe_oracle.c: grouping, union count, bytes, one expert, the
 * expert operation) over seeded random and edge-case inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "ok" and the number of
 * calls at the end. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_route_group(const int32_t* ids, int32_t n, int32_t m, int32_t N, int32_t* count, int32_t* offset,
                       int32_t* slot_by_expert, int32_t* distinct, int32_t* U);
int32_t oracle_union_count(const int32_t* ids, int32_t n, int32_t m, int32_t N);
int64_t oracle_bytes(int32_t kind, int32_t N, int32_t m, int32_t d, int32_t d_ff, int32_t elem_bytes,
                     const int32_t* ids, int32_t n);
int oracle_expert_apply(int32_t d, int32_t d_ff, int32_t wdtype, const void* wg, const void* wu, const void* wd,
                        int32_t xdtype, const void* x, double* o);
int oracle_moe_ffn(int32_t N, int32_t m, int32_t d, int32_t d_ff, int32_t wdtype, const void* Wg, const void* Wu,
                   const void* Wd, int32_t xdtype, const void* x, const int32_t* ids, const float* w, int32_t n,
                   double* acc);

static uint64_t st = 0x2545F4914F6CDD1Dull;
static uint64_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}
static int ri(int lo, int hi) { return lo + (int)(rnd() % (uint64_t)(hi - lo + 1)); }

int main(void) {
    long calls = 0;
    int32_t ids[256], count[1025], offset[1026], sbe[256], distinct[1025], U;
    for (int it = 0; it < 3000; ++it) {
        int N = ri(1, 1024), m = ri(1, 8), n = ri(1, 256 / m);
        for (int s = 0; s < n * m; ++s) ids[s] = ri(-1, N);
        (void)oracle_route_group(ids, n, m, N, count, offset, sbe, distinct, &U);
        (void)oracle_union_count(ids, n, m, N);
        (void)oracle_bytes(ri(0, 1), N, m, 8 * ri(1, 8), 8 * ri(1, 8), ri(0, 1) ? 2 : 4, ids, n);
        calls += 3;
    }
    (void)oracle_route_group(NULL, 1, 1, 1, count, offset, sbe, distinct, &U);
    /* the expert operation on small layers, both dtypes, valid and invalid ids */
    for (int it = 0; it < 60; ++it) {
        int N = ri(1, 6), m = ri(1, N), d = ri(1, 24), d_ff = ri(1, 24), n = ri(1, 5);
        int wdt = ri(0, 1), xdt = ri(0, 1);
        size_t es = wdt ? 2 : 4, xs = xdt ? 2 : 4;
        size_t per = (size_t)N * d * d_ff;
        unsigned char* W = malloc(3 * per * es);
        unsigned char* x = malloc((size_t)n * d * xs);
        float* w = malloc(sizeof(float) * n * m);
        double* acc = calloc((size_t)n * d, sizeof(double));
        for (size_t i = 0; i < 3 * per * es; ++i) W[i] = (unsigned char)(rnd() & 0x3f);
        for (size_t i = 0; i < (size_t)n * d * xs; ++i) x[i] = (unsigned char)(rnd() & 0x3f);
        for (int s = 0; s < n * m; ++s) {
            ids[s] = ri(-1, N);
            w[s] = (float)(rnd() % 100) / 100.f;
        }
        (void)oracle_moe_ffn(N, m, d, d_ff, wdt, W, W + per * es, W + 2 * per * es, xdt, x, ids, w, n, acc);
        double* o = malloc(sizeof(double) * d);
        (void)oracle_expert_apply(d, d_ff, wdt, W, W + per * es, W + 2 * per * es, xdt, x, o);
        free(o);
        free(W);
        free(x);
        free(w);
        free(acc);
        calls += 2;
    }
    printf("ok %ld\n", calls);
    return 0;
}
