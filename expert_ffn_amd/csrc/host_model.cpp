// Host-side byte accounting, step-time model, fits and error bounds (double precision).
//
// Lan, arXiv:2610.34440:
//   Section 1 "Bytes":  per-slot requests n m w, deduplicating requests X(n) w.
//   Section 1 "Speculative decoding", Section 3.1 Eq. (5)-(6), Section 3.2
//   Eqs. (8)-(9), Section 3.3 and Appendix B.3 (staircase, step points (B.31),
//   convex case (B.36)), Section 3.4 Eqs. (14) and (16).
//   Section 2 Eq. (4) and Appendix E Eq. (E.1): least-squares fits of the kernels'
//   times over passes with chosen ids.  Section 3.5, Table 2 and Appendix C: the
//   error bounds for a relative bandwidth error eps.
// SpecFit, arXiv:2610.15417, Sections 3.1-3.3 and Algorithm 1: the exact search for
// the verification subtree with the largest reward over predicted cycle time.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "moe_expert.h"

namespace {

double geo(double a, int k) {  // G_a(k) = 1 + a + ... + a^k, summed from the top for accuracy
    double g = 0.0;
    for (int i = k; i >= 0; --i) g = g * a + 1.0;
    return g;
}

// T_a(k) > T_a(i)  <=>  G_a(k) V(i) > G_a(i) V(k)   (V > 0)
bool beats(double a, int k, int i, const double* V) { return geo(a, k) * V[i] > geo(a, i) * V[k]; }

// alpha_{k,i} = inf{a in [0,1) : T_a(k) > T_a(i)}, 1 if empty.  The set is upward
// closed (Appendix B.3, (B.26)-(B.27)), so bisection applies.
double alpha(int k, int i, const double* V) {
    if (beats(0.0, k, i, V)) return 0.0;
    const double near1 = nextafter(1.0, 0.0);
    if (!beats(near1, k, i, V)) return 1.0;
    double lo = 0.0, hi = near1;
    for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (beats(mid, k, i, V)) hi = mid;
        else lo = mid;
    }
    return hi;
}

int kstar(double a, const double* V, int K) {
    int best = 0;
    for (int k = 1; k <= K; ++k)
        if (geo(a, k) * V[best] > geo(a, best) * V[k]) best = k;
    return best;
}

}  // namespace

extern "C" {

int64_t bytes_requested(int32_t kind, const moe_layer_desc* d, const int32_t* ids, int32_t n) {
    if (!d || !ids) return -(int64_t)(-MOE_E_INVAL);
    if (kind != MOE_KIND_SLOT && kind != MOE_KIND_DEDUP) return -(int64_t)(-MOE_E_INVAL);
    if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return -(int64_t)(-MOE_E_DTYPE);
    if (d->N < 1 || d->N > MOE_MAX_EXPERTS || d->m < 1 || d->m > d->N || n < 1 || d->d_model < 1 || d->d_ff < 1)
        return -(int64_t)(-MOE_E_INVAL);
    const int64_t esize = d->dtype == MOE_BF16 ? 2 : 4;
    const int64_t w = 3 * (int64_t)d->d_model * d->d_ff * esize;
    const int m = d->m;
    std::vector<char> seen((size_t)d->N, 0);
    int64_t U = 0;
    for (int64_t s = 0; s < (int64_t)n * m; ++s) {
        const int32_t e = ids[s];
        if (e < 0 || e >= d->N) return -(int64_t)(-MOE_E_IDS);
        const int64_t t = s / m, j = s % m;
        for (int64_t jj = 0; jj < j; ++jj)
            if (ids[t * m + jj] == e) return -(int64_t)(-MOE_E_IDS);
        if (!seen[e]) {
            seen[e] = 1;
            ++U;
        }
    }
    return kind == MOE_KIND_SLOT ? (int64_t)n * m * w : U * w;
}

int step_time_model(const moe_step_in* in, moe_step_out* out) {
    if (!in || !out) return MOE_E_INVAL;
    const int NM = in->n_max;
    if (NM < 2 || NM > MOE_STEP_NMAX || in->n_a < 1 || in->n_a > MOE_STEP_AMAX) return MOE_E_INVAL;
    if (!(in->m_W > 0.0) || !(in->beta_D > 0.0)) return MOE_E_INVAL;
    for (int p = 0; p < 2; ++p)
        for (int i = 0; i < NM; ++i)
            if (!(in->beta[p][i] > 0.0)) return MOE_E_INVAL;
    for (int i = 0; i < in->n_a; ++i)
        if (!(in->a[i] >= 0.0 && in->a[i] <= 1.0)) return MOE_E_INVAL;
    memset(out, 0, sizeof(*out));
    const int K = NM - 1;  // k_max

    for (int p = 0; p < 2; ++p)
        for (int n = 1; n <= NM; ++n)
            out->tau[p][n - 1] = in->t0 + (in->D + in->kv[n - 1]) / in->beta_D +
                                 in->E[p][n - 1] / in->beta[p][n - 1] + in->phi[p][n - 1];
    for (int n = 1; n <= NM; ++n) out->S[n - 1] = out->tau[0][n - 1] - out->tau[1][n - 1];
    out->crossover = 0;
    for (int n = NM; n >= 2; --n) {
        if (out->S[n - 1] > 0.0) out->crossover = n;
        else break;
    }

    for (int p = 0; p < 2; ++p) {
        double* V = out->V[p];
        V[0] = out->tau[0][0] + in->h[0];  // a one-token pass runs the same kernel either way
        for (int k = 1; k <= K; ++k) V[k] = out->tau[p][k] + in->h[k];
        bool pos = true;
        for (int k = 0; k <= K; ++k) pos = pos && V[k] > 0.0;
        if (!pos) return MOE_E_INVAL;
        out->a0[p] = V[1] / V[0] - 1.0;
        for (int ia = 0; ia < in->n_a; ++ia) {
            const double a = in->a[ia];
            const int ks = kstar(a, V, K);
            out->kstar[p][ia] = ks;
            out->speedup[p][ia] = geo(a, ks) * V[0] / V[ks];
        }
        for (int j = 1; j <= K; ++j) {
            double mx = 0.0;
            for (int i = 0; i < j; ++i) {
                double mn = 1.0;
                for (int k = j; k <= K; ++k) {
                    const double al = alpha(k, i, V);
                    if (al < mn) mn = al;
                }
                if (mn > mx) mx = mn;
            }
            out->step_point[p][j] = mx;
        }
        bool convex = true;
        double cprev = -1.0;
        for (int k = 1; k <= K; ++k) {
            const double c = V[k] - V[k - 1];
            if (c < 0.0 || (k > 1 && c < cprev)) convex = false;
            cprev = c;
        }
        out->convex[p] = convex ? 1 : 0;
        const double a1 = (V[1] - V[0]) / V[0];
        out->a1_convex[p] = a1 < 1.0 ? a1 : 1.0;
    }

    const double mW = in->m_W;
    const double tau1 = out->tau[0][0];
    const double beta1 = in->beta[0][0];
    for (int ia = 0; ia < in->n_a; ++ia) {
        const double a = in->a[ia];
        for (int k = 1; k <= K; ++k) {
            const double Gm1 = geo(a, k) - 1.0;
            const double Bk = in->beta[1][k];
            const double dD = in->kv[k] - in->kv[0];
            const double dphi = in->phi[1][k] - in->phi[0][0];
            const double bracket = Gm1 * tau1 - dD / in->beta_D - dphi;
            out->rho_star[ia][k] = 1.0 - Bk / (mW * k) * bracket - (Bk / beta1 - 1.0) / k;
            const double V0b = in->D + mW + in->kv[0];
            out->rho_star_bytes[ia][k] = 1.0 - (Gm1 * V0b - dD) / (mW * k);
        }
    }
    return MOE_OK;
}

// Least squares min |A c - t| for A with three columns (count rows, row-major),
// by Householder reflections on the column-scaled matrix.  Returns false when a
// column is (numerically) dependent on the others.
static bool lsq3(std::vector<double>& A, std::vector<double>& t, int count, double* c) {
    double scale[3];
    for (int j = 0; j < 3; ++j) {
        double mx = 0.0;
        for (int r = 0; r < count; ++r) mx = fmax(mx, fabs(A[r * 3 + j]));
        if (!(mx > 0.0)) return false;
        scale[j] = mx;
        for (int r = 0; r < count; ++r) A[r * 3 + j] /= mx;
    }
    double R[3][3] = {};
    for (int j = 0; j < 3; ++j) {
        double nrm = 0.0;
        for (int r = j; r < count; ++r) nrm += A[r * 3 + j] * A[r * 3 + j];
        nrm = sqrt(nrm);
        if (!(nrm > 1e-12)) return false;
        const double alpha = A[j * 3 + j] > 0.0 ? -nrm : nrm;
        // v = x - alpha e_1, stored in place; H = I - 2 v v^T / (v^T v)
        A[j * 3 + j] -= alpha;
        double vv = 0.0;
        for (int r = j; r < count; ++r) vv += A[r * 3 + j] * A[r * 3 + j];
        for (int jj = j + 1; jj < 3; ++jj) {
            double dot = 0.0;
            for (int r = j; r < count; ++r) dot += A[r * 3 + j] * A[r * 3 + jj];
            const double f = 2.0 * dot / vv;
            for (int r = j; r < count; ++r) A[r * 3 + jj] -= f * A[r * 3 + j];
        }
        double dot = 0.0;
        for (int r = j; r < count; ++r) dot += A[r * 3 + j] * t[r];
        const double f = 2.0 * dot / vv;
        for (int r = j; r < count; ++r) t[r] -= f * A[r * 3 + j];
        R[j][j] = alpha;
        for (int jj = j + 1; jj < 3; ++jj) R[j][jj] = A[j * 3 + jj];
    }
    for (int j = 2; j >= 0; --j) {
        double v = t[j];
        for (int jj = j + 1; jj < 3; ++jj) v -= R[j][jj] * c[jj];
        c[j] = v / R[j][j];
    }
    for (int j = 0; j < 3; ++j) c[j] /= scale[j];
    return true;
}

int moe_fit_times(int32_t kind, int32_t count, const int32_t* n, const int32_t* U, int32_t m, const double* t,
                  double b, double* coef) {
    if (kind != MOE_KIND_SLOT && kind != MOE_KIND_DEDUP) return MOE_E_INVAL;
    if (!n || !U || !t || !coef || count < 3 || count > (1 << 24) || m < 1 || !(b > 0.0) || !isfinite(b))
        return MOE_E_INVAL;
    std::vector<double> A((size_t)count * 3), y((size_t)count);
    for (int r = 0; r < count; ++r) {
        if (n[r] < 1 || U[r] < 1 || (int64_t)U[r] > (int64_t)n[r] * m || !isfinite(t[r])) return MOE_E_INVAL;
        A[r * 3 + 0] = 1.0;
        A[r * 3 + 1] = (double)U[r] * b;
        A[r * 3 + 2] = kind == MOE_KIND_SLOT ? ((double)n[r] * m - U[r]) * b : (double)n[r];
        y[r] = t[r];
    }
    double c[3];
    if (!lsq3(A, y, count, c)) return MOE_E_INVAL;
    for (int j = 0; j < 3; ++j) coef[j] = c[j];
    return MOE_OK;
}

int moe_error_bounds(double eps, double* out) {
    if (!out || !(eps >= 0.0) || !(eps < 0.5)) return MOE_E_INVAL;
    const double f = eps / (1.0 - eps);
    const double delta = f;
    out[0] = f;                                    // (17), (18)
    out[1] = log((1.0 + eps) / (1.0 - eps));       // (19)
    out[2] = delta;                                // from eps to delta
    out[3] = (1.0 - delta) / (1.0 + delta);        // (20)
    out[4] = (1.0 + delta) / (1.0 - delta);        // (21)
    return MOE_OK;
}

}  // extern "C"

namespace {

struct TreeSearch {
    const moe_tree_in* in;
    int V, L, W;
    std::vector<uint64_t> stack;  // per depth: L * W words of the carried unions
    int ids[MOE_TREE_MAXK];       // current subset, increasing ids
    // incumbent
    double bR, bT;
    int bF, bn;
    int bids[MOE_TREE_MAXK];
    int64_t visited;

    bool usable(int v) const { return in->max_level <= 0 || in->level[v] <= in->max_level; }

    // candidate (R, T, F, n, ids) against the incumbent: ratio, then R, then -F, then
    // -n; otherwise the earlier subset in enumeration order (the lexicographically
    // smaller id list) stays
    void offer(double R, double T, int F, int n) {
        ++visited;
        const double lhs = R * bT, rhs = bR * T;  // R/T vs bR/bT, T > 0
        bool better = lhs > rhs;
        if (lhs == rhs) {
            if (R != bR) better = R > bR;
            else if (F != bF) better = F < bF;
            else better = n < bn;
        }
        if (better) {
            bR = R;
            bT = T;
            bF = F;
            bn = n;
            for (int i = 0; i < n; ++i) bids[i] = ids[i];
        }
    }

    int popcount_state(const uint64_t* st) const {
        int f = 0;
        for (int i = 0; i < L * W; ++i) f += __builtin_popcountll(st[i]);
        return f;
    }

    // S = ids[0..n) with unions in stack[n]; extend by every later eligible node
    void dfs(int n, int last, double R, const std::vector<char>& in_s) {
        if (n == in->K) return;
        std::vector<char> mark(in_s);
        for (int v = last + 1; v <= V; ++v) {
            if (!usable(v)) continue;
            const int pa = in->parent[v];
            if (pa != 0 && !mark[pa]) continue;
            const uint64_t* cur = &stack[(size_t)n * L * W];
            uint64_t* nxt = &stack[(size_t)(n + 1) * L * W];
            const uint64_t* bv = in->bitmap + (size_t)v * L * W;
            for (int i = 0; i < L * W; ++i) nxt[i] = cur[i] | bv[i];
            ids[n] = v;
            const double Rv = R + in->p[v];
            const int F = popcount_state(nxt);
            offer(Rv, in->b[n + 1] + in->beta * F, F, n + 1);
            mark[v] = 1;
            dfs(n + 1, v, Rv, mark);
            mark[v] = 0;
        }
    }
};

}  // namespace

extern "C" {

int moe_tree_select(const moe_tree_in* in, moe_tree_out* out) {
    if (!in || !out || !in->parent || !in->p || !in->bitmap || !in->b) return MOE_E_INVAL;
    if (in->V < 0 || in->V > MOE_TREE_MAXV || in->L < 1 || in->words < 1 || in->words > MOE_TREE_MAXW ||
        in->K < 0 || in->K > MOE_TREE_MAXK)
        return MOE_E_INVAL;
    if (!(in->beta > 0.0) || !isfinite(in->beta)) return MOE_E_INVAL;
    if (in->max_level > 0 && !in->level) return MOE_E_INVAL;
    for (int k = 0; k <= in->K; ++k)
        if (!(in->b[k] > 0.0) || !isfinite(in->b[k])) return MOE_E_INVAL;
    for (int v = 1; v <= in->V; ++v) {
        if (in->parent[v] < 0 || in->parent[v] >= v) return MOE_E_INVAL;
        if (!(in->p[v] >= 0.0) || !isfinite(in->p[v])) return MOE_E_INVAL;
    }
    TreeSearch ts;
    ts.in = in;
    ts.V = in->V;
    ts.L = in->L;
    ts.W = in->words;
    ts.stack.assign((size_t)(in->K + 1) * in->L * in->words, 0ull);
    for (int i = 0; i < in->L * in->words; ++i) ts.stack[i] = in->bitmap[i];  // the root's experts
    ts.visited = 0;
    const int F0 = ts.popcount_state(ts.stack.data());
    ts.bR = 1.0;
    ts.bT = in->b[0] + in->beta * F0;
    ts.bF = F0;
    ts.bn = 0;
    ts.visited = 1;
    std::vector<char> mark((size_t)in->V + 1, 0);
    ts.dfs(0, 0, 1.0, mark);
    out->selected = 0;
    for (int i = 0; i < ts.bn; ++i) out->selected |= 1ull << (ts.bids[i] - 1);
    out->count = ts.bn;
    out->F = ts.bF;
    out->R = ts.bR;
    out->T = ts.bT;
    out->visited = ts.visited;
    return MOE_OK;
}

}  // extern "C"
