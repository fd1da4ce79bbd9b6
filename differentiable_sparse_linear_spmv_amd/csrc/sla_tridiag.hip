// sla_tridiag.hip -- host code: wanted eigenpairs of the small symmetric tridiagonal
// matrix T that the Lanczos eigensolver builds (sla_eigsh).
//
// Eigenvalues by bisection on the Sturm count (the number of negative pivots of the
// LDL^T factorization of T - x I equals the number of eigenvalues below x), each to
// the full precision of the count.  Eigenvectors by inverse iteration: three solves
// with T - theta I, factored by Gaussian elimination with partial pivoting (a
// tridiagonal matrix keeps one extra superdiagonal), each followed by normalization;
// the wanted vectors are then orthogonalized in order (modified Gram-Schmidt), which
// separates vectors of close eigenvalues.  Cost O(k m) per eigenpair, for the few k
// wanted out of m.
#include <algorithm>
#include <cfloat>
#include <cmath>
#include <vector>

#include "sla_internal.h"

namespace sla {
namespace {

struct Tri {
    const double* a;   // diagonal, m entries
    const double* b;   // off-diagonal, m - 1 entries
    int m;
    double pivmin;     // smallest pivot magnitude allowed in the Sturm count
};

// Number of eigenvalues of T strictly below x.
int count_below(const Tri& T, double x)
{
    int c = 0;
    double q = T.a[0] - x;
    if (std::fabs(q) < T.pivmin) q = -T.pivmin;
    if (q < 0.0) ++c;
    for (int l = 1; l < T.m; ++l) {
        q = (T.a[l] - x) - T.b[l - 1] * T.b[l - 1] / q;
        if (std::fabs(q) < T.pivmin) q = -T.pivmin;
        if (q < 0.0) ++c;
    }
    return c;
}

// Eigenvalue number i (0-based, ascending) inside the Gershgorin interval [lo, hi].
double bisect(const Tri& T, int i, double lo, double hi)
{
    for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;   // interval at the resolution of doubles
        if (hi - lo <= 2.0 * DBL_EPSILON * std::max(std::fabs(lo), std::fabs(hi)) + T.pivmin) break;
        if (count_below(T, mid) > i) hi = mid;
        else lo = mid;
    }
    return 0.5 * (lo + hi);
}

// Unit vector y with (T - theta I) y ~ 0 by inverse iteration.
void inverse_iteration(const Tri& T, double theta, double tnorm, double* y)
{
    const int m = T.m;
    if (m == 1) {
        y[0] = 1.0;
        return;
    }
    std::vector<double> dl(m - 1), d(m), du(m - 1), du2(m > 2 ? m - 2 : 1, 0.0);
    std::vector<char> swap(m - 1, 0);
    for (int l = 0; l < m; ++l) d[l] = T.a[l] - theta;
    for (int l = 0; l < m - 1; ++l) dl[l] = du[l] = T.b[l];
    const double tiny = DBL_EPSILON * tnorm + DBL_MIN;
    for (int l = 0; l < m - 1; ++l) {
        if (std::fabs(d[l]) >= std::fabs(dl[l])) {
            if (d[l] == 0.0) d[l] = tiny;
            const double f = dl[l] / d[l];
            dl[l] = f;
            d[l + 1] = d[l + 1] - f * du[l];
            if (l < m - 2) du2[l] = 0.0;
        } else {   // rows l and l + 1 exchanged
            swap[l] = 1;
            const double f = d[l] / dl[l];
            d[l] = dl[l];
            dl[l] = f;
            const double t = du[l];
            du[l] = d[l + 1];
            d[l + 1] = t - f * d[l + 1];
            if (l < m - 2) {
                du2[l] = du[l + 1];
                du[l + 1] = -f * du[l + 1];
            }
        }
    }
    if (d[m - 1] == 0.0) d[m - 1] = tiny;
    for (int l = 0; l < m; ++l) y[l] = 1.0;
    for (int it = 0; it < 3; ++it) {
        for (int l = 0; l < m - 1; ++l) {   // L^{-1} with the row exchanges
            if (swap[l]) {
                const double t = y[l];
                y[l] = y[l + 1];
                y[l + 1] = t - dl[l] * y[l];
            } else {
                y[l + 1] = y[l + 1] - dl[l] * y[l];
            }
        }
        y[m - 1] = y[m - 1] / d[m - 1];   // U^{-1}: diagonal d, superdiagonals du, du2
        y[m - 2] = (y[m - 2] - du[m - 2] * y[m - 1]) / d[m - 2];
        for (int l = m - 3; l >= 0; --l) y[l] = (y[l] - du[l] * y[l + 1] - du2[l] * y[l + 2]) / d[l];
        double big = 0.0;
        for (int l = 0; l < m; ++l) big = std::max(big, std::fabs(y[l]));
        if (!(big > 0.0) || !std::isfinite(big)) big = 1.0;
        double s = 0.0;
        for (int l = 0; l < m; ++l) {
            y[l] /= big;
            s += y[l] * y[l];
        }
        s = std::sqrt(s);
        for (int l = 0; l < m; ++l) y[l] /= s;
    }
}

}  // namespace

void tridiag_eigpairs(const double* a, const double* b, int m, int k, bool largest, double* theta, double* S)
{
    double lo = a[0], hi = a[0], tnorm = 0.0, bmax = 0.0;
    for (int l = 0; l < m; ++l) {
        const double r = (l > 0 ? std::fabs(b[l - 1]) : 0.0) + (l < m - 1 ? std::fabs(b[l]) : 0.0);
        lo = std::min(lo, a[l] - r);
        hi = std::max(hi, a[l] + r);
        tnorm = std::max(tnorm, std::fabs(a[l]) + r);
        if (l < m - 1) bmax = std::max(bmax, b[l] * b[l]);
    }
    const double pad = 2.0 * DBL_EPSILON * tnorm + DBL_MIN;
    lo -= pad;
    hi += pad;
    const Tri T{a, b, m, DBL_MIN * std::max(1.0, bmax)};
    for (int r = 0; r < k; ++r) {
        const int i = largest ? m - 1 - r : r;
        theta[r] = bisect(T, i, lo, hi);
        double* y = S + static_cast<size_t>(r) * m;
        inverse_iteration(T, theta[r], tnorm, y);
        for (int q = 0; q < r; ++q) {   // against the vectors already found
            const double* z = S + static_cast<size_t>(q) * m;
            double d = 0.0;
            for (int l = 0; l < m; ++l) d += z[l] * y[l];
            for (int l = 0; l < m; ++l) y[l] -= d * z[l];
        }
        double s = 0.0;
        for (int l = 0; l < m; ++l) s += y[l] * y[l];
        s = std::sqrt(s);
        for (int l = 0; l < m; ++l) y[l] /= s;
    }
}

}  // namespace sla
