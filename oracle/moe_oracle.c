/*
 * CPU oracle of the MoE expert operation of a speculative-decoding verification
 * pass.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the smoke check
 * and by the benchmark's CPU-baseline leg, never by the product path.  It shares
 * no code, header or constant with the GPU library.
 *
 * Source: Y. Lan, "Speculative Decoding for Mixture-of-Experts Models: Expert
 * Bytes, Kernel Bandwidth and the Best Draft Length" (arXiv:2610.34440):
 *   - Section 1 (Introduction): the expert operation is the gate, up and down
 *     projections of each token of a pass with the weights of its m selected
 *     experts; a slot is one of a token's m selections; a deduplicating kernel
 *     groups the pass's tokens by expert and reads each distinct expert once.
 *   - Section 1, "Routing, union and reuse": X(n) = |S_t u ... u S_{t+n-1}|.
 *   - Section 1, "Bytes": a per-slot kernel requests n m w bytes for a pass of
 *     n tokens, a deduplicating one w X(n).
 * The FFN of one expert is the SwiGLU form y = W_down (silu(W_gate x) * W_up x),
 * silu(z) = z / (1 + e^-z), and a token's output is the sum over its slots of
 * the routing weight times that expert's output.
 *
 * Arithmetic: every dot product and the silu are evaluated in double; the
 * caller rounds the double result to fp32 once.  Inputs are fp32 or bf16 bit
 * patterns (decoded exactly).  Loops are the plain definition: no blocking,
 * no reordering beyond what the definition states.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_OK = 0, OR_E_INVAL = -1, OR_E_DTYPE = -2, OR_E_IDS = -5 };
enum { OR_F32 = 0, OR_BF16 = 1 };

static double elem(const void* base, int32_t dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Validity of slot s = t*m + j: id in [0, N) and not equal to an earlier id of
 * the same token (the m selections of a token are distinct experts). */
static int slot_valid(const int32_t* ids, int32_t m, int32_t N, int32_t s) {
    int32_t e = ids[s];
    if (e < 0 || e >= N) return 0;
    return 1;
}

static int slot_duplicate(const int32_t* ids, int32_t m, int32_t s) {
    int32_t t = s / m, j = s % m;
    for (int32_t jj = 0; jj < j; ++jj)
        if (ids[t * m + jj] == ids[s]) return 1;
    return 0;
}

/*
 * Grouping of a pass's slots by expert ("groups the pass's tokens by expert",
 * Section 1):
 *   count[e]  = number of in-range slots with id e
 *   offset    = exclusive prefix sum of count, offset[N] = in-range slots
 *   slot_by_expert[offset[e] .. offset[e+1]) = those slots s = t*m + j in
 *               increasing s; entries from offset[N] to n*m-1 are -1
 *   distinct  = the ids with count > 0 in increasing order, then -1 up to N
 *   *U        = number of distinct ids, X(n) of the pass
 * Slots whose id is outside [0, N) take no part.  Returns OR_E_IDS when any id
 * is out of range or repeats within its token, OR_OK otherwise; the arrays are
 * filled in both cases.
 */
int oracle_route_group(const int32_t* ids, int32_t n, int32_t m, int32_t N, int32_t* count,
                       int32_t* offset, int32_t* slot_by_expert, int32_t* distinct, int32_t* U) {
    if (!ids || n < 1 || m < 1 || N < 1) return OR_E_INVAL;
    int status = OR_OK;
    int32_t nm = n * m;
    for (int32_t e = 0; e < N; ++e) count[e] = 0;
    for (int32_t s = 0; s < nm; ++s) {
        if (!slot_valid(ids, m, N, s)) {
            status = OR_E_IDS;
            continue;
        }
        if (slot_duplicate(ids, m, s)) status = OR_E_IDS;
        count[ids[s]] += 1;
    }
    offset[0] = 0;
    for (int32_t e = 0; e < N; ++e) offset[e + 1] = offset[e] + count[e];
    for (int32_t i = 0; i < nm; ++i) slot_by_expert[i] = -1;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    for (int32_t e = 0; e < N; ++e) cursor[e] = offset[e];
    for (int32_t s = 0; s < nm; ++s) {
        if (!slot_valid(ids, m, N, s)) continue;
        slot_by_expert[cursor[ids[s]]++] = s;
    }
    free(cursor);
    int32_t u = 0;
    for (int32_t e = 0; e < N; ++e)
        if (count[e] > 0) distinct[u++] = e;
    for (int32_t e = u; e < N; ++e) distinct[e] = -1;
    *U = u;
    return status;
}

/* X(n): number of distinct in-range ids among the n*m slots of a pass. */
int32_t oracle_union_count(const int32_t* ids, int32_t n, int32_t m, int32_t N) {
    char* seen = (char*)calloc((size_t)N, 1);
    int32_t u = 0;
    for (int32_t s = 0; s < n * m; ++s) {
        int32_t e = ids[s];
        if (e < 0 || e >= N) continue;
        if (!seen[e]) {
            seen[e] = 1;
            ++u;
        }
    }
    free(seen);
    return u;
}

void oracle_union_count_batch(const int32_t* ids, int64_t B, int32_t n, int32_t m, int32_t N,
                              int32_t* out) {
    for (int64_t b = 0; b < B; ++b) out[b] = oracle_union_count(ids + b * (int64_t)n * m, n, m, N);
}

/*
 * Requested expert bytes of one pass (Section 1, "Bytes"): w = 3 d d_ff sizeof(W)
 * per expert; per-slot kernel (kind 0): n m w; deduplicating kernel (kind 1):
 * X(n) w.  Returns a negative status for invalid ids.
 */
int64_t oracle_bytes(int32_t kind, int32_t N, int32_t m, int32_t d, int32_t d_ff, int32_t elem_bytes,
                     const int32_t* ids, int32_t n) {
    for (int32_t s = 0; s < n * m; ++s)
        if (!slot_valid(ids, m, N, s) || slot_duplicate(ids, m, s)) return OR_E_IDS;
    int64_t w = 3LL * d * d_ff * elem_bytes;
    if (kind == 0) return (int64_t)n * m * w;
    if (kind == 1) return (int64_t)oracle_union_count(ids, n, m, N) * w;
    return OR_E_INVAL;
}

/*
 * One expert applied to one token, in double:
 *   a_f = sum_i Wg[f][i] x[i],  b_f = sum_i Wu[f][i] x[i]      (f < d_ff)
 *   h_f = silu(a_f) b_f,        silu(z) = z / (1 + exp(-z))
 *   o_i = sum_f Wd[i][f] h_f                                  (i < d)
 * wg, wu point at the expert's [d_ff][d] blocks, wd at its [d][d_ff] block.
 */
int oracle_expert_apply(int32_t d, int32_t d_ff, int32_t wdtype, const void* wg, const void* wu,
                        const void* wd, int32_t xdtype, const void* x, double* o) {
    if (d < 1 || d_ff < 1) return OR_E_INVAL;
    if ((wdtype != OR_F32 && wdtype != OR_BF16) || (xdtype != OR_F32 && xdtype != OR_BF16))
        return OR_E_DTYPE;
    double* h = (double*)malloc(sizeof(double) * (size_t)d_ff);
    for (int32_t f = 0; f < d_ff; ++f) {
        double a = 0.0, b = 0.0;
        for (int32_t i = 0; i < d; ++i) {
            double xi = elem(x, xdtype, i);
            a += elem(wg, wdtype, (int64_t)f * d + i) * xi;
            b += elem(wu, wdtype, (int64_t)f * d + i) * xi;
        }
        h[f] = a / (1.0 + exp(-a)) * b;
    }
    for (int32_t i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int32_t f = 0; f < d_ff; ++f) acc += elem(wd, wdtype, (int64_t)i * d_ff + f) * h[f];
        o[i] = acc;
    }
    free(h);
    return OR_OK;
}

/*
 * The expert operation of a pass, accumulated in double into acc [n][d]
 * (acc += ...; the caller zeroes it and rounds to fp32 once):
 *   acc[t] += sum_{j=0..m-1} w[t][j] * FFN_{ids[t][j]}(x_t)
 * Weights Wg, Wu: [N][d_ff][d]; Wd: [N][d][d_ff]; x: [n][d]; ids, w: [n][m].
 * Every slot is computed on its own (the definition); no grouping.
 */
int oracle_moe_ffn(int32_t N, int32_t m, int32_t d, int32_t d_ff, int32_t wdtype, const void* Wg,
                   const void* Wu, const void* Wd, int32_t xdtype, const void* x, const int32_t* ids,
                   const float* w, int32_t n, double* acc) {
    if (n < 1 || m < 1 || m > N) return OR_E_INVAL;
    for (int32_t s = 0; s < n * m; ++s)
        if (!slot_valid(ids, m, N, s) || slot_duplicate(ids, m, s)) return OR_E_IDS;
    int64_t eb_w = (wdtype == OR_F32) ? 4 : 2, eb_x = (xdtype == OR_F32) ? 4 : 2;
    int64_t mat = (int64_t)d * d_ff * eb_w;
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (int32_t t = 0; t < n; ++t) {
        const char* xt = (const char*)x + (int64_t)t * d * eb_x;
        for (int32_t j = 0; j < m; ++j) {
            int32_t e = ids[t * m + j];
            int rc = oracle_expert_apply(d, d_ff, wdtype, (const char*)Wg + e * mat,
                                         (const char*)Wu + e * mat, (const char*)Wd + e * mat, xdtype,
                                         xt, o);
            if (rc != OR_OK) {
                free(o);
                return rc;
            }
            double wt = (double)w[t * m + j];
            for (int32_t i = 0; i < d; ++i) acc[(int64_t)t * d + i] += wt * o[i];
        }
    }
    free(o);
    return OR_OK;
}
