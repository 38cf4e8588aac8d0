// Host-side offline factorisation for DyRA (float64, OpenMP).
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Algorithm 1 Offline Preparation (lines 2-5): the structured weight
// W_hat is the rank-r truncated SVD of W (Appendix B), W_res = W - W_hat
// (§2.1 Eq. 1), R0 is fixed to the top-k right singular vectors of W_res
// (Appendix D), which for an SVD-truncated W_hat are V_{r+1..r+k}^T
// (Proposition 1's assumption), and P_L = W_res R0^T (R0 R0^T + lambda I)^-1
// (Eq. 7).
//
// No LAPACK is linked.  The SVD comes from the symmetric eigenproblem of the
// float64 Gram matrix on the smaller side, solved with textbook methods
// (Golub & Van Loan, "Matrix Computations", ch. 8):
//   1. Householder reduction to tridiagonal form (each reflector's rank-2
//      update is fused with the next reflector's matrix-vector product, so the
//      trailing matrix is swept once per step);
//   2. the wanted eigenvalues by bisection on Sturm counts;
//   3. their eigenvectors by inverse iteration on the tridiagonal matrix, with
//      classical Gram-Schmidt (twice) against the earlier vectors of the same
//      cluster;
//   4. back-transformation by the stored reflectors.
// Only the r + k leading eigenpairs are formed.
#include "dyra_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

namespace dyra {
namespace {

using Vec = std::vector<double>;

// G = S S^T for S row-major [p][q]; G row-major [p][p] (both triangles filled).
void gram_rows(const double *S, int64_t p, int64_t q, double *G) {
    const int64_t BT = 64;   // output tile
    const int64_t BQ = 512;  // contraction chunk
    const int64_t nt = (p + BT - 1) / BT;
    std::vector<std::pair<int64_t, int64_t>> tiles;
    for (int64_t a = 0; a < nt; ++a)
        for (int64_t b = 0; b <= a; ++b) tiles.emplace_back(a, b);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < (int64_t)tiles.size(); ++t) {
        const int64_t i0 = tiles[t].first * BT, j0 = tiles[t].second * BT;
        const int64_t i1 = std::min(p, i0 + BT), j1 = std::min(p, j0 + BT);
        double acc[64][64];
        for (int64_t i = 0; i < i1 - i0; ++i)
            for (int64_t j = 0; j < j1 - j0; ++j) acc[i][j] = 0.0;
        for (int64_t q0 = 0; q0 < q; q0 += BQ) {
            const int64_t q1 = std::min(q, q0 + BQ);
            for (int64_t i = i0; i < i1; ++i) {
                const double *si = S + i * q;
                for (int64_t j = j0; j < j1; ++j) {
                    const double *sj = S + j * q;
                    double s = 0.0;
#pragma omp simd reduction(+ : s)
                    for (int64_t c = q0; c < q1; ++c) s += si[c] * sj[c];
                    acc[i - i0][j - j0] += s;
                }
            }
        }
        for (int64_t i = i0; i < i1; ++i)
            for (int64_t j = j0; j < j1; ++j) {
                G[i * p + j] = acc[i - i0][j - j0];
                G[j * p + i] = acc[i - i0][j - j0];
            }
    }
}

// Householder vector of x (length m): v with v[0] = x[0] - alpha, beta = 2 / v^T v,
// so that (I - beta v v^T) x = alpha e_1.  Returns alpha; beta = 0 if x = 0.
double householder(const double *x, int64_t m, double *v, double *beta) {
    double ss = 0.0;
    for (int64_t i = 0; i < m; ++i) ss += x[i] * x[i];
    const double nx = std::sqrt(ss);
    if (nx == 0.0) {
        for (int64_t i = 0; i < m; ++i) v[i] = 0.0;
        *beta = 0.0;
        return 0.0;
    }
    const double alpha = x[0] >= 0.0 ? -nx : nx;
    for (int64_t i = 0; i < m; ++i) v[i] = x[i];
    v[0] -= alpha;
    const double vv = ss - x[0] * x[0] + v[0] * v[0];
    *beta = vv > 0.0 ? 2.0 / vv : 0.0;
    return alpha;
}

// Reduces symmetric A (row-major p x p, full storage, overwritten) to tridiagonal
// T = Q^T A Q with diagonal d[p] and off-diagonal e[p-1].  Reflector k acts on
// indices k+1..p-1; its vector is stored in A's row k from column k+1 on, its
// beta in beta[k].
void tridiagonalize(double *A, int64_t p, double *d, double *e, double *beta) {
    if (p == 1) {
        d[0] = A[0];
        return;
    }
    Vec v(p), y(p), w(p);
    // first reflector and its product y = A_trail v
    auto start_reflector = [&](int64_t k) {
        const int64_t m = p - k - 1;
        double b;
        const double alpha = householder(A + k * p + k + 1, m, v.data(), &b);
        beta[k] = b;
        e[k] = alpha;
        d[k] = A[k * p + k];
        return m;
    };
    int64_t m = start_reflector(0);
    {
        const int64_t off = 1;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < m; ++i) {
            const double *row = A + (off + i) * p + off;
            double s = 0.0;
#pragma omp simd reduction(+ : s)
            for (int64_t j = 0; j < m; ++j) s += row[j] * v[j];
            y[i] = s;
        }
    }
    for (int64_t k = 0; k <= p - 3; ++k) {
        // trailing block S = A[k+1.., k+1..] of size m; y = S v (unscaled)
        const int64_t off = k + 1;
        const double b = beta[k];
        // p = b y; w = p - (b/2)(p^T v) v
        double pv = 0.0;
        for (int64_t i = 0; i < m; ++i) pv += y[i] * v[i];
        const double K = 0.5 * b * b * pv;
        for (int64_t i = 0; i < m; ++i) w[i] = b * y[i] - K * v[i];
        // store this reflector's vector in row k (it is no longer needed as data)
        for (int64_t i = 0; i < m; ++i) A[k * p + off + i] = v[i];
        // update row 0 of S first: it defines the next reflector
        {
            double *row = A + off * p + off;
            const double v0 = v[0], w0 = w[0];
            for (int64_t j = 0; j < m; ++j) row[j] -= v0 * w[j] + w0 * v[j];
        }
        if (k == p - 3) {
            // S is 2x2: update the remaining row and read off the last entries
            double *row = A + (off + 1) * p + off;
            const double v1 = v[1], w1 = w[1];
            for (int64_t j = 0; j < m; ++j) row[j] -= v1 * w[j] + w1 * v[j];
            d[p - 2] = A[(p - 2) * p + (p - 2)];
            d[p - 1] = A[(p - 1) * p + (p - 1)];
            e[p - 2] = A[(p - 1) * p + (p - 2)];
            beta[p - 2] = 0.0;
            break;
        }
        // next reflector from row 0 of S (entries 1..m-1)
        const int64_t k2 = k + 1;
        const int64_t m2 = m - 1;
        Vec vn(m2);
        double b2;
        const double alpha2 = householder(A + k2 * p + k2 + 1, m2, vn.data(), &b2);
        beta[k2] = b2;
        e[k2] = alpha2;
        d[k2] = A[k2 * p + k2];
        // fused pass: update rows 1..m-1 of S and form y2 = S'[1..,1..] vn
        Vec y2(m2);
#pragma omp parallel for schedule(static)
        for (int64_t i = 1; i < m; ++i) {
            double *row = A + (off + i) * p + off;
            const double vi = v[i], wi = w[i];
            double s = 0.0;
            row[0] -= vi * w[0] + wi * v[0];
#pragma omp simd reduction(+ : s)
            for (int64_t j = 1; j < m; ++j) {
                const double a = row[j] - (vi * w[j] + wi * v[j]);
                row[j] = a;
                s += a * vn[j - 1];
            }
            y2[i - 1] = s;
        }
        std::copy(vn.begin(), vn.end(), v.begin());
        std::copy(y2.begin(), y2.end(), y.begin());
        m = m2;
    }
    if (p == 2) {
        d[0] = A[0];
        d[1] = A[3];
        e[0] = A[2];
        beta[0] = 0.0;
    }
}

// Number of eigenvalues of the tridiagonal (d, e) that are < x (Sturm count via
// the LDL^T pivots of T - x I).
int64_t sturm_count(const double *d, const double *e2, int64_t p, double x, double pivmin) {
    int64_t cnt = 0;
    double q = d[0] - x;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++cnt;
    for (int64_t i = 1; i < p; ++i) {
        q = d[i] - x - e2[i - 1] / q;
        if (std::fabs(q) < pivmin) q = -pivmin;
        if (q < 0) ++cnt;
    }
    return cnt;
}

// The `want` largest eigenvalues of the tridiagonal (d, e), descending, by bisection.
void top_eigenvalues(const double *d, const double *e, int64_t p, int64_t want, double *lam) {
    Vec e2(std::max<int64_t>(p - 1, 1));
    double lo = d[0], hi = d[0], emax2 = 0.0;
    for (int64_t i = 0; i < p; ++i) {
        const double r = (i > 0 ? std::fabs(e[i - 1]) : 0.0) + (i < p - 1 ? std::fabs(e[i]) : 0.0);
        lo = std::min(lo, d[i] - r);
        hi = std::max(hi, d[i] + r);
    }
    for (int64_t i = 0; i + 1 < p; ++i) {
        e2[i] = e[i] * e[i];
        emax2 = std::max(emax2, e2[i]);
    }
    const double eps = std::numeric_limits<double>::epsilon();
    const double tnorm = std::max(std::fabs(lo), std::fabs(hi));
    const double pivmin = std::max(std::numeric_limits<double>::min() * std::max(1.0, emax2),
                                   std::numeric_limits<double>::min());
    lo -= 2 * eps * tnorm + pivmin;
    hi += 2 * eps * tnorm + pivmin;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t j = 0; j < want; ++j) {
        const int64_t idx = p - 1 - j;  // ascending index of the j-th largest
        double a = lo, b = hi;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (a + b);
            if (b - a <= 2 * eps * std::max(std::fabs(a), std::fabs(b)) + pivmin) break;
            if (mid <= a || mid >= b) break;
            if (sturm_count(d, e2.data(), p, mid, pivmin) <= idx) a = mid;
            else b = mid;
        }
        lam[j] = 0.5 * (a + b);
    }
}

// LU factorisation with partial pivoting of the tridiagonal T - lambda I, and
// solves with it (the factor U has two super-diagonals).
struct TriLU {
    int64_t p;
    Vec u0, u1, u2, l;
    std::vector<unsigned char> swap;
    void factor(const double *d, const double *e, double lambda, double tiny) {
        u0.assign(p, 0.0);
        u1.assign(p, 0.0);
        u2.assign(p, 0.0);
        l.assign(p, 0.0);
        swap.assign(p, 0);
        // row i holds (diag, super1, super2) in (u0, u1, u2) after elimination
        double cd = d[0] - lambda, cu = p > 1 ? e[0] : 0.0, cu2 = 0.0;
        for (int64_t i = 0; i + 1 < p; ++i) {
            const double sub = e[i];
            const double nd = d[i + 1] - lambda;
            const double nu = i + 2 < p ? e[i + 1] : 0.0;
            if (std::fabs(cd) >= std::fabs(sub)) {
                if (cd == 0.0) cd = tiny;
                const double f = sub / cd;
                l[i] = f;
                u0[i] = cd;
                u1[i] = cu;
                u2[i] = cu2;
                cd = nd - f * cu;
                cu = nu - f * cu2;
                cu2 = 0.0;
            } else {
                const double f = cd / sub;
                l[i] = f;
                swap[i] = 1;
                u0[i] = sub;
                u1[i] = nd;
                u2[i] = nu;
                const double ncd = cu - f * nd;
                const double ncu = cu2 - f * nu;
                cd = ncd;
                cu = ncu;
                cu2 = 0.0;
            }
        }
        if (cd == 0.0) cd = tiny;
        u0[p - 1] = cd;
        if (p > 1) u1[p - 1] = 0.0;
    }
    // solves (T - lambda I) x = b in place
    void solve(double *b, double tiny) const {
        for (int64_t i = 0; i + 1 < p; ++i) {
            if (swap[i]) {
                const double t = b[i];
                b[i] = b[i + 1];
                b[i + 1] = t - l[i] * b[i + 1];
            } else {
                b[i + 1] -= l[i] * b[i];
            }
        }
        for (int64_t i = p - 1; i >= 0; --i) {
            double s = b[i];
            if (i + 1 < p) s -= u1[i] * b[i + 1];
            if (i + 2 < p) s -= u2[i] * b[i + 2];
            double piv = u0[i];
            if (std::fabs(piv) < tiny) piv = piv < 0 ? -tiny : tiny;
            b[i] = s / piv;
        }
    }
};

// Eigenvectors of the tridiagonal for eigenvalues lam[0..want) (descending):
// Z row-major [want][p], rows orthonormal.
void tridiag_eigenvectors(const double *d, const double *e, int64_t p, const double *lam,
                          int64_t want, double *Z) {
    const double eps = std::numeric_limits<double>::epsilon();
    double tnorm = 0.0;
    for (int64_t i = 0; i < p; ++i) {
        const double r = std::fabs(d[i]) + (i > 0 ? std::fabs(e[i - 1]) : 0.0) +
                         (i < p - 1 ? std::fabs(e[i]) : 0.0);
        tnorm = std::max(tnorm, r);
    }
    if (tnorm == 0.0) tnorm = 1.0;
    const double ortol = 1e-3 * tnorm;
    const double tiny = eps * tnorm;
    TriLU lu;
    lu.p = p;
    Vec x(p), dots(want);
    int64_t cluster_start = 0;
    uint64_t state = 0x9E3779B97F4A7C15ull;
    auto next_uniform = [&]() {
        // splitmix64, a fixed deterministic start vector
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        return (double)(z >> 11) * (1.0 / 9007199254740992.0) - 0.5;
    };
    double prev_shift = 0.0;
    for (int64_t j = 0; j < want; ++j) {
        if (j > 0 && lam[j - 1] - lam[j] > ortol) cluster_start = j;
        // separate numerically equal eigenvalues so each iteration differs
        double shift = lam[j];
        if (j > cluster_start && shift >= prev_shift - 10 * eps * std::fabs(prev_shift))
            shift = prev_shift - 10 * eps * std::max(std::fabs(prev_shift), tnorm);
        prev_shift = shift;
        lu.factor(d, e, shift, tiny);
        for (int64_t i = 0; i < p; ++i) x[i] = next_uniform();
        const int64_t nclus = j - cluster_start;
        for (int it = 0; it < 4; ++it) {
            lu.solve(x.data(), tiny);
            // classical Gram-Schmidt twice against the earlier members of the cluster
            for (int pass = 0; pass < 2 && nclus > 0; ++pass) {
#pragma omp parallel for schedule(static) if (nclus * p > 200000)
                for (int64_t c = 0; c < nclus; ++c) {
                    const double *z = Z + (cluster_start + c) * p;
                    double s = 0.0;
                    for (int64_t i = 0; i < p; ++i) s += z[i] * x[i];
                    dots[c] = s;
                }
                const int64_t IB = 512;
#pragma omp parallel for schedule(static) if (nclus * p > 200000)
                for (int64_t i0 = 0; i0 < p; i0 += IB) {
                    const int64_t i1 = std::min(p, i0 + IB);
                    for (int64_t c = 0; c < nclus; ++c) {
                        const double *z = Z + (cluster_start + c) * p;
                        const double dc = dots[c];
#pragma omp simd
                        for (int64_t i = i0; i < i1; ++i) x[i] -= dc * z[i];
                    }
                }
            }
            double nrm = 0.0;
            for (int64_t i = 0; i < p; ++i) nrm += x[i] * x[i];
            nrm = std::sqrt(nrm);
            if (nrm == 0.0) {
                for (int64_t i = 0; i < p; ++i) x[i] = next_uniform();
                continue;
            }
            for (int64_t i = 0; i < p; ++i) x[i] /= nrm;
        }
        std::memcpy(Z + j * p, x.data(), sizeof(double) * p);
    }
}

// Z[j] <- Q Z[j] for every row j of Z ([want][p]), Q = H_0 H_1 ... H_{p-3} with
// H_k = I - beta_k v_k v_k^T, v_k stored in A's row k from column k+1.
void back_transform(const double *A, const double *beta, int64_t p, double *Z, int64_t want) {
    const int64_t VB = 16;
    const int64_t nblk = (want + VB - 1) / VB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int64_t j0 = blk * VB, j1 = std::min(want, j0 + VB);
        for (int64_t k = p - 3; k >= 0; --k) {
            const double b = beta[k];
            if (b == 0.0) continue;
            const double *v = A + k * p + k + 1;
            const int64_t m = p - k - 1;
            for (int64_t j = j0; j < j1; ++j) {
                double *z = Z + j * p + k + 1;
                double s = 0.0;
#pragma omp simd reduction(+ : s)
                for (int64_t i = 0; i < m; ++i) s += v[i] * z[i];
                s *= b;
#pragma omp simd
                for (int64_t i = 0; i < m; ++i) z[i] -= s * v[i];
            }
        }
    }
}

// Solves the k x k SPD system (lower Cholesky) for each column of B [k][cols] in place.
bool spd_solve(const double *Gin, int64_t k, double *B, int64_t cols) {
    Vec L(Gin, Gin + k * k);
    for (int64_t j = 0; j < k; ++j) {
        double s = L[j * k + j];
        for (int64_t t = 0; t < j; ++t) s -= L[j * k + t] * L[j * k + t];
        if (!(s > 0.0)) return false;
        const double ljj = std::sqrt(s);
        L[j * k + j] = ljj;
        for (int64_t i = j + 1; i < k; ++i) {
            double u = L[i * k + j];
            for (int64_t t = 0; t < j; ++t) u -= L[i * k + t] * L[j * k + t];
            L[i * k + j] = u / ljj;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        Vec y(k);
        for (int64_t i = 0; i < k; ++i) {
            double s = B[i * cols + c];
            for (int64_t t = 0; t < i; ++t) s -= L[i * k + t] * y[t];
            y[i] = s / L[i * k + i];
        }
        for (int64_t i = k - 1; i >= 0; --i) {
            double s = y[i];
            for (int64_t t = i + 1; t < k; ++t) s -= L[t * k + i] * y[t];
            y[i] = s / L[i * k + i];
        }
        for (int64_t i = 0; i < k; ++i) B[i * cols + c] = y[i];
    }
    return true;
}

}  // namespace

namespace {

// Float64 copy of a float32 array; false if any value is not finite.
bool widen(const float *src, int64_t count, Vec &dst) {
    dst.resize((size_t)count);
    bool finite = true;
#pragma omp parallel for schedule(static) reduction(&& : finite)
    for (int64_t i = 0; i < count; ++i) {
        const double w = src[i];
        finite = finite && std::isfinite(w);
        dst[(size_t)i] = w;
    }
    return finite;
}

// Lines 2-5 of the Offline Preparation on a float64 W (arguments checked by
// the callers): the rank-r truncated SVD as W_hat, W_res, R0 and P_L.
dyra_status factorize_core(Vec &&W, int64_t c1, int64_t c2, int32_t r, int32_t k, double lambda, Factors *out,
                           const float *R0_in) {
    // singular vectors needed: the static r, plus k for the default R0
    const int64_t want = (int64_t)r + (R0_in ? 0 : k);
    out->c1 = c1;
    out->c2 = c2;
    out->r = r;
    out->k = k;
    out->lambda = lambda;

    out->A_s.assign((size_t)(c1 * r), 0.0);
    out->V_s.assign((size_t)(c2 * r), 0.0);
    out->R0.assign((size_t)(k * c2), 0.0);
    out->P_L.assign((size_t)(c1 * k), 0.0);
    out->sigma.assign((size_t)want, 0.0);
    out->W_res = W;
    if (R0_in) {
        for (int64_t i = 0; i < (int64_t)k * c2; ++i) out->R0[i] = R0_in[i];
    }
    if (want == 0 && !(R0_in && k > 0)) return DYRA_OK;
    if (want > 0) {

        // Gram matrix on the smaller side: rows of S are the vectors whose inner
        // products are taken (the columns of W if c2 <= c1, else its rows).
        const bool right_side = c2 <= c1;
        const int64_t p = right_side ? c2 : c1;
        const int64_t q = right_side ? c1 : c2;
        Vec G((size_t)(p * p));
        {
            Vec St;
            const double *S = W.data();
            if (right_side) {
                St.resize((size_t)(c2 * c1));
#pragma omp parallel for schedule(static)
                for (int64_t j = 0; j < c2; ++j)
                    for (int64_t i = 0; i < c1; ++i) St[j * c1 + i] = W[i * c2 + j];
                S = St.data();
            }
            gram_rows(S, p, q, G.data());
        }
        Vec d(p), e(std::max<int64_t>(p, 1)), beta(std::max<int64_t>(p, 1), 0.0);
        tridiagonalize(G.data(), p, d.data(), e.data(), beta.data());
        Vec lam((size_t)want);
        top_eigenvalues(d.data(), e.data(), p, want, lam.data());
        Vec Z((size_t)(want * p));
        tridiag_eigenvectors(d.data(), e.data(), p, lam.data(), want, Z.data());
        back_transform(G.data(), beta.data(), p, Z.data(), want);

        // Right singular vectors V [c2][want] (column j = v_j).
        Vec V((size_t)(c2 * want));
        if (right_side) {
            for (int64_t j = 0; j < want; ++j)
                for (int64_t i = 0; i < c2; ++i) V[i * want + j] = Z[j * p + i];
        } else {
            // v_j = W^T u_j / ||W^T u_j||
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < want; ++j) {
                const double *u = Z.data() + j * p;
                Vec t((size_t)c2, 0.0);
                for (int64_t a = 0; a < c1; ++a) {
                    const double ua = u[a];
                    const double *wr = W.data() + a * c2;
                    for (int64_t b = 0; b < c2; ++b) t[b] += ua * wr[b];
                }
                double nrm = 0.0;
                for (int64_t b = 0; b < c2; ++b) nrm += t[b] * t[b];
                nrm = std::sqrt(nrm);
                const double inv = nrm > 0.0 ? 1.0 / nrm : 0.0;
                for (int64_t b = 0; b < c2; ++b) V[b * want + j] = t[b] * inv;
            }
            // W^T u / ||W^T u|| loses orthogonality as sigma_j / sigma_0 approaches
            // the Gram's rounding level; re-orthonormalise those columns (twice)
            // against all earlier ones so V_s stays an orthonormal row-space basis.
            const double cut = 1e-4 * std::sqrt(std::max(lam[0], 0.0));
            for (int64_t j = 0; j < want; ++j) {
                if (std::sqrt(std::max(lam[j], 0.0)) >= cut) continue;
                for (int attempt = 0; attempt < 3; ++attempt) {
                    double nrm = 0.0;
                    for (int pass = 0; pass < 2; ++pass) {
                        for (int64_t i = 0; i < j; ++i) {
                            double d = 0.0;
                            for (int64_t b = 0; b < c2; ++b) d += V[b * want + i] * V[b * want + j];
                            for (int64_t b = 0; b < c2; ++b) V[b * want + j] -= d * V[b * want + i];
                        }
                        nrm = 0.0;
                        for (int64_t b = 0; b < c2; ++b) nrm += V[b * want + j] * V[b * want + j];
                        nrm = std::sqrt(nrm);
                        if (nrm > 1e-8) {
                            for (int64_t b = 0; b < c2; ++b) V[b * want + j] /= nrm;
                        }
                    }
                    if (nrm > 1e-8) break;
                    // a null direction of W: complete the basis from a fixed start vector
                    for (int64_t b = 0; b < c2; ++b)
                        V[b * want + j] = std::sin(0.7 * (double)(b + 1) * (double)(j + 2 + attempt));
                }
            }
        }
        // A = W V (= U Sigma); sigma_j = ||W v_j||
        Vec A((size_t)(c1 * want), 0.0);
#pragma omp parallel for schedule(static)
        for (int64_t a = 0; a < c1; ++a) {
            const double *wr = W.data() + a * c2;
            double *ar = A.data() + a * want;
            for (int64_t b = 0; b < c2; ++b) {
                const double wab = wr[b];
                const double *vb = V.data() + b * want;
                for (int64_t j = 0; j < want; ++j) ar[j] += wab * vb[j];
            }
        }
        for (int64_t j = 0; j < want; ++j) {
            double s = 0.0;
            for (int64_t a = 0; a < c1; ++a) s += A[a * want + j] * A[a * want + j];
            out->sigma[j] = std::sqrt(s);
        }
        for (int64_t a = 0; a < c1; ++a)
            for (int64_t j = 0; j < r; ++j) out->A_s[a * r + j] = A[a * want + j];
        for (int64_t b = 0; b < c2; ++b)
            for (int64_t j = 0; j < r; ++j) out->V_s[b * r + j] = V[b * want + j];
        if (!R0_in) {
            for (int64_t j = 0; j < k; ++j)
                for (int64_t b = 0; b < c2; ++b) out->R0[j * c2 + b] = V[b * want + r + j];
        }
    }

    // W_res = W - A_s V_s^T  (§2.1 Eq. 1)
    if (r > 0) {
#pragma omp parallel for schedule(static)
        for (int64_t a = 0; a < c1; ++a) {
            const double *ar = out->A_s.data() + a * r;
            double *wr = out->W_res.data() + a * c2;
            for (int64_t b = 0; b < c2; ++b) {
                const double *vb = out->V_s.data() + b * r;
                double s = 0.0;
                for (int64_t j = 0; j < r; ++j) s += ar[j] * vb[j];
                wr[b] -= s;
            }
        }
    }
    // P_L = W_res R0^T (R0 R0^T + lambda I)^-1  (Eq. 7).  Solve with the SPD
    // matrix on the right: P_L^T = (R0 R0^T + lambda I)^-1 (R0 W_res^T).
    if (k > 0) {
        Vec Gk((size_t)(k * k), 0.0);
        for (int64_t i = 0; i < k; ++i)
            for (int64_t j = 0; j < k; ++j) {
                double s = 0.0;
                for (int64_t b = 0; b < c2; ++b) s += out->R0[i * c2 + b] * out->R0[j * c2 + b];
                Gk[i * k + j] = s + (i == j ? lambda : 0.0);
            }
        Vec PLt((size_t)(k * c1), 0.0);  // [k][c1] = R0 W_res^T
#pragma omp parallel for schedule(static)
        for (int64_t a = 0; a < c1; ++a) {
            const double *wr = out->W_res.data() + a * c2;
            for (int64_t i = 0; i < k; ++i) {
                const double *r0 = out->R0.data() + i * c2;
                double s = 0.0;
                for (int64_t b = 0; b < c2; ++b) s += r0[b] * wr[b];
                PLt[i * c1 + a] = s;
            }
        }
        if (!spd_solve(Gk.data(), k, PLt.data(), c1)) return DYRA_ERR_NUMERIC;
        for (int64_t a = 0; a < c1; ++a)
            for (int64_t i = 0; i < k; ++i) out->P_L[a * k + i] = PLt[i * c1 + a];
    }
    for (double s : out->sigma)
        if (!std::isfinite(s)) return DYRA_ERR_NUMERIC;
    return DYRA_OK;
}

}  // namespace

dyra_status factorize(const float *W32, int64_t c1, int64_t c2, int32_t r, int32_t k,
                      double lambda, Factors *out, const float *R0_in) {
    if (!W32 || !out) return DYRA_ERR_ARG;
    if (c1 <= 0 || c2 <= 0 || r < 0 || k < 0) return DYRA_ERR_ARG;
    if ((int64_t)r + k > std::min(c1, c2)) return DYRA_ERR_ARG;
    if (!(lambda >= 0.0) || !std::isfinite(lambda)) return DYRA_ERR_ARG;
    if (R0_in) {
        for (int64_t i = 0; i < (int64_t)k * c2; ++i)
            if (!std::isfinite(R0_in[i])) return DYRA_ERR_NUMERIC;
    }
    Vec W;
    if (!widen(W32, c1 * c2, W)) return DYRA_ERR_NUMERIC;
    return factorize_core(std::move(W), c1, c2, r, k, lambda, out, R0_in);
}

// BLAST (Appendix B): W_hat's block (i, j) is U_i diag(s_ij) V_j^T.  W_res =
// W - W_hat is formed here, and the rest of the preparation is the r = 0 case
// of the truncated-SVD one on W_res: R0 = its top-k right singular vectors,
// P_L from Eq. 7.
dyra_status factorize_blast(const float *W32, int64_t c1, int64_t c2, int32_t nb, int32_t rb, const float *U32,
                            const float *S32, const float *V32, int32_t k, double lambda, Factors *out) {
    if (!W32 || !U32 || !S32 || !V32 || !out) return DYRA_ERR_ARG;
    if (c1 <= 0 || c2 <= 0 || nb < 1 || rb < 1 || k < 0) return DYRA_ERR_ARG;
    if (c1 % nb != 0 || c2 % nb != 0 || k > std::min(c1, c2)) return DYRA_ERR_ARG;
    if (!(lambda >= 0.0) || !std::isfinite(lambda)) return DYRA_ERR_ARG;
    Vec W, U, S, V;
    if (!widen(W32, c1 * c2, W) || !widen(U32, c1 * rb, U) || !widen(S32, (int64_t)nb * nb * rb, S) ||
        !widen(V32, c2 * rb, V))
        return DYRA_ERR_NUMERIC;
    const int64_t p = c1 / nb, q = c2 / nb;
#pragma omp parallel for schedule(static)
    for (int64_t a = 0; a < c1; ++a) {
        const int64_t i = a / p;
        Vec us((size_t)rb);
        for (int64_t j = 0; j < nb; ++j) {
            const double *s = S.data() + (i * nb + j) * rb;
            for (int32_t c = 0; c < rb; ++c) us[(size_t)c] = U[(size_t)(a * rb + c)] * s[c];
            for (int64_t b = j * q; b < (j + 1) * q; ++b) {
                const double *v = V.data() + b * rb;
                double acc = 0.0;
                for (int32_t c = 0; c < rb; ++c) acc += us[(size_t)c] * v[c];
                W[(size_t)(a * c2 + b)] -= acc;
            }
        }
    }
    return factorize_core(std::move(W), c1, c2, 0, k, lambda, out, nullptr);
}

}  // namespace dyra

extern "C" dyra_status dyra_factorize_host(const float *W, int64_t c1, int64_t c2, int32_t r,
                                           int32_t k, double lambda, double *A_s, double *V_s,
                                           double *R0, double *P_L, double *sigma) {
    dyra::Factors f;
    const dyra_status st = dyra::factorize(W, c1, c2, r, k, lambda, &f);
    if (st != DYRA_OK) return st;
    if (A_s) std::copy(f.A_s.begin(), f.A_s.end(), A_s);
    if (V_s) std::copy(f.V_s.begin(), f.V_s.end(), V_s);
    if (R0) std::copy(f.R0.begin(), f.R0.end(), R0);
    if (P_L) std::copy(f.P_L.begin(), f.P_L.end(), P_L);
    if (sigma) std::copy(f.sigma.begin(), f.sigma.end(), sigma);
    return DYRA_OK;
}

extern "C" dyra_status dyra_factorize_blast_host(const float *W, int64_t c1, int64_t c2, int32_t nb, int32_t rb,
                                                 const float *U, const float *S, const float *V, int32_t k,
                                                 double lambda, double *W_res, double *R0, double *P_L) {
    dyra::Factors f;
    const dyra_status st = dyra::factorize_blast(W, c1, c2, nb, rb, U, S, V, k, lambda, &f);
    if (st != DYRA_OK) return st;
    if (W_res) std::copy(f.W_res.begin(), f.W_res.end(), W_res);
    if (R0) std::copy(f.R0.begin(), f.R0.end(), R0);
    if (P_L) std::copy(f.P_L.begin(), f.P_L.end(), P_L);
    return DYRA_OK;
}
