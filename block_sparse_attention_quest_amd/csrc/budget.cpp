// budget.cpp - the critical-path-aware speculation budget (host code, no GPU work).
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text), §4.4 (critical-path-aware speculation budget), A.6 (profiling
//           grid and polynomial regression), Eq. 1 (|P| <= delta |A|).
//
// The budget ratio delta bounds the predicted set, |P| <= delta |A|.  A larger delta covers more of A but
// lengthens the speculative pass; the pages keep that pass inside the selection window.  They profile,
// once per configuration, the selection latency and the speculative-attention latency over a grid of
// context lengths and budget ratios, keep the results in a table indexed by context length, estimate
// lengths outside the grid by polynomial regression, and at run time pick the biggest ratio for which
// speculation ends no later than selection.
//
// Readings where the pages leave a step open:
//   * the regression is an ordinary least-squares polynomial in x = T / T_max (T_max the longest
//     profiled length; the scaling keeps the Vandermonde columns of comparable size), one polynomial for the
//     selection latency and one per profiled delta for the speculative latency, of a degree the caller
//     picks (the pages name none);
//   * a length in the grid reads the table itself; any other length reads the polynomials;
//   * a ratio qualifies when est_spec(delta) <= est_select; when no profiled delta does, the choice
//     is -1 and the caller decides (a grid that holds delta = 0 always has a fitting entry).
//
// The fit solves the least-squares problem by Householder QR of the Vandermonde matrix (no normal
// equations), in float64.

#include <algorithm>
#include <cmath>

#include "prr.h"

namespace {

constexpr int kMaxPoints = PRR_BUDGET_MAX_POINTS;
constexpr int kMaxCoef = PRR_BUDGET_MAX_DEGREE + 1;

bool is_fin(double x) { return std::isfinite(x); }

prr_status check_table(const double *ctx, int32_t n_ctx, const double *t_select, const double *deltas,
                       int32_t n_delta, const double *t_spec, int32_t degree) {
    if (!ctx || !t_select || !deltas || !t_spec) return PRR_EINVAL;
    if (n_ctx < 1 || n_ctx > kMaxPoints || n_delta < 1 || n_delta > kMaxPoints) return PRR_EINVAL;
    if (degree < 0 || degree > PRR_BUDGET_MAX_DEGREE || degree > n_ctx - 1) return PRR_EINVAL;
    for (int i = 0; i < n_ctx; ++i) {
        if (!is_fin(ctx[i]) || ctx[i] <= 0.0 || (i > 0 && !(ctx[i] > ctx[i - 1]))) return PRR_EINVAL;
        if (!is_fin(t_select[i])) return PRR_EINVAL;
    }
    for (int j = 0; j < n_delta; ++j) {
        if (!is_fin(deltas[j]) || deltas[j] < 0.0 || (j > 0 && !(deltas[j] > deltas[j - 1]))) return PRR_EINVAL;
        for (int i = 0; i < n_ctx; ++i)
            if (!is_fin(t_spec[(size_t)j * n_ctx + i])) return PRR_EINVAL;
    }
    return PRR_OK;
}

// Least-squares coefficients c[0..nc) of sum_k c_k x^k through the points (x[i], y[i]), i < m, m >= nc:
// Householder QR of the m x nc Vandermonde matrix, Q^T applied to y, then back substitution.
void lsq_poly(const double *x, const double *y, int m, int nc, double *c) {
    double a[kMaxPoints][kMaxCoef];
    double b[kMaxPoints];
    for (int i = 0; i < m; ++i) {
        double p = 1.0;
        for (int k = 0; k < nc; ++k) {
            a[i][k] = p;
            p *= x[i];
        }
        b[i] = y[i];
    }
    double diag[kMaxCoef];
    for (int k = 0; k < nc; ++k) {
        double norm = 0.0;
        for (int i = k; i < m; ++i) norm += a[i][k] * a[i][k];
        norm = std::sqrt(norm);
        // reflect column k onto -sign(a_kk) |a_k| e_k (the sign that avoids cancellation)
        const double alpha = a[k][k] > 0.0 ? -norm : norm;
        diag[k] = alpha;
        if (norm == 0.0) continue;
        a[k][k] -= alpha;  // v = a_k - alpha e_k, stored in place
        double vv = 0.0;
        for (int i = k; i < m; ++i) vv += a[i][k] * a[i][k];
        if (vv == 0.0) continue;
        for (int j = k + 1; j < nc; ++j) {
            double s = 0.0;
            for (int i = k; i < m; ++i) s += a[i][k] * a[i][j];
            const double f = 2.0 * s / vv;
            for (int i = k; i < m; ++i) a[i][j] -= f * a[i][k];
        }
        double s = 0.0;
        for (int i = k; i < m; ++i) s += a[i][k] * b[i];
        const double f = 2.0 * s / vv;
        for (int i = k; i < m; ++i) b[i] -= f * a[i][k];
    }
    for (int k = nc - 1; k >= 0; --k) {
        double s = b[k];
        for (int j = k + 1; j < nc; ++j) s -= a[k][j] * c[j];
        c[k] = diag[k] != 0.0 ? s / diag[k] : 0.0;
    }
}

double horner(const double *c, int nc, double x) {
    double r = 0.0;
    for (int k = nc - 1; k >= 0; --k) r = r * x + c[k];
    return r;
}

}  // namespace

extern "C" {

prr_status prr_budget_fit(const double *ctx, int32_t n_ctx, const double *t_select, const double *deltas,
                          int32_t n_delta, const double *t_spec, int32_t degree, double *coef) {
    const prr_status st = check_table(ctx, n_ctx, t_select, deltas, n_delta, t_spec, degree);
    if (st != PRR_OK) return st;
    if (!coef) return PRR_EINVAL;
    const int nc = degree + 1;
    double x[kMaxPoints];
    for (int i = 0; i < n_ctx; ++i) x[i] = ctx[i] / ctx[n_ctx - 1];
    lsq_poly(x, t_select, n_ctx, nc, coef);
    for (int j = 0; j < n_delta; ++j) lsq_poly(x, t_spec + (size_t)j * n_ctx, n_ctx, nc, coef + (size_t)(1 + j) * nc);
    return PRR_OK;
}

prr_status prr_budget_choose(const double *ctx, int32_t n_ctx, const double *t_select, const double *deltas,
                             int32_t n_delta, const double *t_spec, int32_t degree, const double *coef,
                             double context, int32_t *choice, double *est, int32_t topk, int32_t *budget_blocks) {
    const prr_status st = check_table(ctx, n_ctx, t_select, deltas, n_delta, t_spec, degree);
    if (st != PRR_OK) return st;
    if (!coef || !choice || !is_fin(context) || context <= 0.0) return PRR_EINVAL;
    if (budget_blocks && topk < 0) return PRR_EINVAL;
    const int nc = degree + 1;
    int row = -1;
    for (int i = 0; i < n_ctx; ++i)
        if (ctx[i] == context) row = i;
    const double x = context / ctx[n_ctx - 1];
    const double sel = row >= 0 ? t_select[row] : horner(coef, nc, x);
    if (est) est[0] = sel;
    int best = -1;
    for (int j = 0; j < n_delta; ++j) {
        const double sp = row >= 0 ? t_spec[(size_t)j * n_ctx + row] : horner(coef + (size_t)(1 + j) * nc, nc, x);
        if (est) est[1 + j] = sp;
        if (sp <= sel) best = j;
    }
    // |P| <= delta |A| (Eq. 1): the largest admissible set, floor(delta K), with a relative slack of 1e-9 for
    // products that round just below an integer; no fitting delta: the smallest profiled one
    if (budget_blocks) {
        const double x = deltas[best >= 0 ? best : 0] * (double)topk;
        const double n = std::floor(x + 1e-9 * std::max(1.0, x));
        if (!(n <= (double)INT32_MAX)) return PRR_EINVAL;
        *budget_blocks = (int32_t)n;
    }
    *choice = best;
    return PRR_OK;
}

}  // extern "C"
