// sla_tridiag.hip -- host code: wanted eigenpairs of the small symmetric tridiagonal
// matrix T that the Lanczos eigensolver builds (sla_eigsh), and of the dense projected
// matrix of a thick-restarted basis.
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
#include <cstddef>
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

// Dense symmetric H (m x m, row-major): Householder reduction H = Q T Q^T (for c = 0 ..
// m - 3 the reflector I - 2 v v^T zeroes column c below its subdiagonal, applied from
// both sides as H -= v q^T + q v^T with p = 2 H v, q = p - (v^T p) v, and accumulated
// into Q; columns already zero there are skipped, so the tridiagonal part of a
// restarted basis costs nothing), the wanted eigenpairs of T, and back to H's
// eigenvectors Q y.  O(c m^2) for c columns to reduce.
void sym_eigpairs(const double* Hm, int m, int k, bool largest, double* theta, double* S)
{
    std::vector<double> H(Hm, Hm + static_cast<size_t>(m) * m), Q(static_cast<size_t>(m) * m, 0.0);
    for (int i = 0; i < m; ++i) Q[static_cast<size_t>(i) * m + i] = 1.0;
    std::vector<double> v(m), p(m), q(m);
    auto at = [&](std::vector<double>& X, int r, int c) -> double& { return X[static_cast<size_t>(r) * m + c]; };
    for (int c = 0; c + 2 < m; ++c) {
        double tail = 0.0;   // column c below its subdiagonal: already tridiagonal if zero
        for (int r = c + 2; r < m; ++r) tail += at(H, r, c) * at(H, r, c);
        if (tail == 0.0) continue;
        const double nx = std::sqrt(at(H, c + 1, c) * at(H, c + 1, c) + tail);
        const double x0 = at(H, c + 1, c);
        const double alpha = x0 >= 0.0 ? -nx : nx;
        double nv = 0.0;
        for (int r = c + 1; r < m; ++r) {
            v[r] = at(H, r, c) - (r == c + 1 ? alpha : 0.0);
            nv += v[r] * v[r];
        }
        nv = std::sqrt(nv);
        if (nv == 0.0) continue;
        for (int r = c + 1; r < m; ++r) v[r] /= nv;
        double K = 0.0;
        for (int r = c + 1; r < m; ++r) {
            double t = 0.0;
            for (int s2 = c + 1; s2 < m; ++s2) t += at(H, r, s2) * v[s2];
            p[r] = 2.0 * t;
            K += v[r] * p[r];
        }
        for (int r = c + 1; r < m; ++r) q[r] = p[r] - K * v[r];
        for (int r = c + 1; r < m; ++r)
            for (int s2 = c + 1; s2 < m; ++s2) at(H, r, s2) -= v[r] * q[s2] + q[r] * v[s2];
        at(H, c + 1, c) = at(H, c, c + 1) = alpha;
        for (int r = c + 2; r < m; ++r) at(H, r, c) = at(H, c, r) = 0.0;
        for (int r = 0; r < m; ++r) {   // Q (I - 2 v v^T)
            double t = 0.0;
            for (int s2 = c + 1; s2 < m; ++s2) t += at(Q, r, s2) * v[s2];
            t *= 2.0;
            for (int s2 = c + 1; s2 < m; ++s2) at(Q, r, s2) -= t * v[s2];
        }
    }
    std::vector<double> d(m), e(m > 1 ? m - 1 : 1), Y(static_cast<size_t>(k) * m);
    for (int i = 0; i < m; ++i) d[i] = at(H, i, i);
    for (int i = 0; i + 1 < m; ++i) e[i] = at(H, i + 1, i);
    tridiag_eigpairs(d.data(), e.data(), m, k, largest, theta, Y.data());
    for (int r = 0; r < k; ++r)
        for (int i = 0; i < m; ++i) {
            double t = 0.0;
            for (int c = 0; c < m; ++c) t += at(Q, i, c) * Y[static_cast<size_t>(r) * m + c];
            S[static_cast<size_t>(r) * m + i] = t;
        }
}

}  // namespace sla
