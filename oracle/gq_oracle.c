/*
 * gq_oracle.c -- plain, slow, fp64 CPU reference for the calibration-Hessian
 * GPTQ int4 path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * Every stage computes the plain definition, in the order the pages give it:
 *
 *   Gram           H = X^T X, summed over tokens (dataset card hipfire-calib-data,
 *                  "Hessian storage": full Hessians, not diagonals) and additive
 *                  over chunks (AtomicChat GGUF page, "The importance matrix":
 *                  the statistic is a sum over chunks, merging is addition).
 *   tril storage   Bf16TrilDiagF32: exact f32 diagonal, then the strict lower
 *                  triangle as bf16 by truncation (f32 bits >> 16) at index
 *                  i*(i-1)/2 + j for i > j, mirrored on read (hipfire-calib-data,
 *                  "Hessian storage: Bf16TrilDiagF32").
 *   PSD projection eigendecompose, clip negative eigenvalues to zero, rebuild,
 *                  symmetrise (hipfire-calib-data, "The fix").  The eigensolvers
 *                  are written here from the textbook algorithms (cyclic Jacobi;
 *                  Householder tridiagonalisation followed by implicit
 *                  Wilkinson-shift QR), with no LAPACK.
 *   GPTQ           damping in units of mean(diag H) (hipfire-calib-data, damping
 *                  table in "The fix"), a Cholesky-based inverse and the
 *                  error-feedback column sweep emitting symmetric int4 codes in
 *                  [-8, 7] with a per-(row, group) scale absmax/7 so that
 *                  w = code * scale (ork-driver wiki "Exp 2026-08-18 GPTQ Int4",
 *                  opening description; GPTQ is Frantar et al. 2022).
 *   qerr           sqrt(sum imp[k] (w - q)^2 / sum imp[k] w^2), imp = 1 when
 *                  absent (same wiki page, qerr definition).
 *   variants       static groups (every scale from the original weights, fixed
 *                  before the sweep) and the NF4 codebook (the wiki's qerr
 *                  section scores an NF4 pack beside the uniform one): scale
 *                  absmax, code = the nearest of 16 levels in [-1, 1], passed
 *                  in by the caller.
 *
 * Readings where the pages are silent are stated at each function.  Decisions
 * that turn floating point into an integer (the scale and the rounded code) are
 * taken in fp32, the precision the device path uses; everything else is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ORC_MUTANT selects a deliberately wrong variant for the CPU mutation tests,
 * which check that the pins catch plausible mistakes.  The default build has
 * ORC_MUTANT == 0 and none of them. */
#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif

#define ORC_OK 0
#define ORC_ERR_INVALID_ARG 1
#define ORC_ERR_NOT_PD 2
#define ORC_ERR_NONFINITE 3
#define ORC_ERR_NO_CALIBRATION 4
#define ORC_ERR_NO_CONVERGENCE 6

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float f32_from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------ Gram */

/* H (K x K fp64, both triangles) += X^T X, X is T x K row-major fp32.
 * Entry (i, j) is the plain sum over tokens t of X[t][i] * X[t][j]. */
void orc_gram_accumulate(double *H, const float *X, int64_t T, int64_t K)
{
    double *Xc = (double *)malloc((size_t)(T * K) * sizeof(double));
    for (int64_t t = 0; t < T; t++)
        for (int64_t i = 0; i < K; i++)
            Xc[i * T + t] = (double)X[t * K + i];          /* column i of X */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t i = 0; i < K; i++) {
        const double *xi = Xc + i * T;
        for (int64_t j = 0; j <= i; j++) {
            const double *xj = Xc + j * T;
            double s = 0.0;
            int64_t tend = T;
#if ORC_MUTANT == 7
            tend = T - 1;   /* mutant: drops the last token */
#endif
            for (int64_t t = 0; t < tend; t++) s += xi[t] * xj[t];
            H[i * K + j] += s;
            if (j != i) H[j * K + i] += s;
        }
    }
    free(Xc);
}

/* out[s] = sum_t X[t][I[s]] * X[t][J[s]]: single Gram entries, one by one. */
void orc_gram_entries(double *out, const float *X, int64_t T, int64_t K,
                      const int64_t *I, const int64_t *J, int64_t S)
{
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < S; s++) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; t++)
            acc += (double)X[t * K + I[s]] * (double)X[t * K + J[s]];
        out[s] = acc;
    }
}

/* ------------------------------------------------------------------ tril */

int64_t orc_tril_bytes(int64_t K) { return 4 * K + K * (K - 1); }

/* Blob = K little-endian f32 diagonal words, then K(K-1)/2 little-endian u16
 * words, word i*(i-1)/2 + j holding bits(H[i][j]) >> 16 for i > j.  Only the
 * strict lower triangle of H is read. */
void orc_pack_tril(uint8_t *blob, const float *H, int64_t K)
{
    for (int64_t i = 0; i < K; i++) {
        uint32_t u = f32_bits(H[i * K + i]);
        blob[4 * i + 0] = (uint8_t)(u);
        blob[4 * i + 1] = (uint8_t)(u >> 8);
        blob[4 * i + 2] = (uint8_t)(u >> 16);
        blob[4 * i + 3] = (uint8_t)(u >> 24);
    }
    uint8_t *tril = blob + 4 * K;
    for (int64_t i = 1; i < K; i++)
        for (int64_t j = 0; j < i; j++) {
            int64_t idx = i * (i - 1) / 2 + j;
            uint32_t hi = f32_bits(H[i * K + j]) >> 16;
#if ORC_MUTANT == 1
            {   /* mutant: round to nearest even instead of truncating */
                uint32_t u = f32_bits(H[i * K + j]);
                hi = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
            }
#endif
#if ORC_MUTANT == 8
            idx = i * (i - 1) / 2 + (i - 1 - j);   /* mutant: row stored in reverse */
#endif
            tril[2 * idx + 0] = (uint8_t)(hi);
            tril[2 * idx + 1] = (uint8_t)(hi >> 8);
        }
}

/* Full symmetric K x K fp32 from a blob: diagonal exact, H[i][j] = H[j][i] =
 * f32(u16 << 16). */
void orc_unpack_tril(float *H, const uint8_t *blob, int64_t K)
{
    for (int64_t i = 0; i < K; i++) {
        uint32_t u = (uint32_t)blob[4 * i] | ((uint32_t)blob[4 * i + 1] << 8) |
                     ((uint32_t)blob[4 * i + 2] << 16) | ((uint32_t)blob[4 * i + 3] << 24);
        H[i * K + i] = f32_from(u);
    }
    const uint8_t *tril = blob + 4 * K;
    for (int64_t i = 1; i < K; i++)
        for (int64_t j = 0; j < i; j++) {
            int64_t idx = i * (i - 1) / 2 + j;
            uint32_t w = (uint32_t)tril[2 * idx] | ((uint32_t)tril[2 * idx + 1] << 8);
            float v = f32_from(w << 16);
            H[i * K + j] = v;
            H[j * K + i] = v;
        }
}

/* ------------------------------------------------------------ eigensolvers */

/* fp64 copy of a symmetric matrix given by the lower triangle of fp32 H. */
static double *sym_lower_f64(const float *H, int64_t K)
{
    double *A = (double *)malloc((size_t)(K * K) * sizeof(double));
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j <= i; j++) {
            A[i * K + j] = (double)H[i * K + j];
            A[j * K + i] = (double)H[i * K + j];
        }
    return A;
}

/* Cyclic two-sided Jacobi (Golub & Van Loan, "Matrix Computations", the
 * symmetric Schur decomposition and cyclic-by-row Jacobi).  A (K x K, full,
 * symmetric) is destroyed; w gets the eigenvalues, Vt (K x K) the eigenvectors
 * as rows (Vt[k][:] belongs to w[k]).  Unsorted. */
int orc_eigh_jacobi(double *A, double *w, double *Vt, int64_t K, int max_sweeps)
{
    for (int64_t i = 0; i < K * K; i++) Vt[i] = 0.0;
    for (int64_t i = 0; i < K; i++) Vt[i * K + i] = 1.0;
    double fro = 0.0;
    for (int64_t i = 0; i < K * K; i++) fro += A[i] * A[i];
    int converged = 0;
    for (int sweep = 0; sweep < max_sweeps && !converged; sweep++) {
        double off = 0.0;
        for (int64_t p = 0; p < K; p++)
            for (int64_t q = p + 1; q < K; q++) off += 2.0 * A[p * K + q] * A[p * K + q];
        if (off <= 1e-30 * fro) { converged = 1; break; }
        for (int64_t p = 0; p < K - 1; p++)
            for (int64_t q = p + 1; q < K; q++) {
                double apq = A[p * K + q];
                if (apq == 0.0) continue;
                double tau = (A[q * K + q] - A[p * K + p]) / (2.0 * apq);
                double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                double c = 1.0 / sqrt(1.0 + t * t), s = t * c;
                /* A <- A J on columns p, q */
                for (int64_t k = 0; k < K; k++) {
                    double akp = A[k * K + p], akq = A[k * K + q];
                    A[k * K + p] = c * akp - s * akq;
                    A[k * K + q] = s * akp + c * akq;
                }
                /* A <- J^T A on rows p, q */
                for (int64_t k = 0; k < K; k++) {
                    double apk = A[p * K + k], aqk = A[q * K + k];
                    A[p * K + k] = c * apk - s * aqk;
                    A[q * K + k] = s * apk + c * aqk;
                }
                A[p * K + q] = 0.0;
                A[q * K + p] = 0.0;
                /* V <- V J: columns p, q of V are rows p, q of Vt */
                for (int64_t k = 0; k < K; k++) {
                    double vp = Vt[p * K + k], vq = Vt[q * K + k];
                    Vt[p * K + k] = c * vp - s * vq;
                    Vt[q * K + k] = s * vp + c * vq;
                }
            }
    }
    if (!converged) {
        double off = 0.0;
        for (int64_t p = 0; p < K; p++)
            for (int64_t q = p + 1; q < K; q++) off += 2.0 * A[p * K + q] * A[p * K + q];
        if (off > 1e-30 * fro) return ORC_ERR_NO_CONVERGENCE;
    }
    for (int64_t i = 0; i < K; i++) w[i] = A[i * K + i];
    return ORC_OK;
}

/* Householder reduction of symmetric A (full, destroyed) to tridiagonal form
 * T = Q^T A Q (Golub & Van Loan, Householder tridiagonalisation).  d gets the
 * diagonal, e the sub-diagonal (e[k] = T[k+1][k]).  If Qt is non-NULL it gets
 * Q^T (row i of Qt = column i of Q). */
static void householder_tridiag(double *A, int64_t K, double *d, double *e, double *Qt)
{
    double *v = (double *)malloc((size_t)K * sizeof(double));
    double *p = (double *)malloc((size_t)K * sizeof(double));
    double *vs = Qt ? (double *)malloc((size_t)(K * K) * sizeof(double)) : NULL;
    double *betas = (double *)calloc((size_t)K, sizeof(double));
    for (int64_t k = 0; k + 2 < K; k++) {
        int64_t m = K - k - 1;                 /* length of x = A[k+1:, k] */
        double alpha = 0.0;
        for (int64_t i = 0; i < m; i++) {
            v[i] = A[(k + 1 + i) * K + k];
            alpha += v[i] * v[i];
        }
        alpha = sqrt(alpha);
        double beta = 0.0;
        if (alpha > 0.0) {
            double sg = v[0] >= 0.0 ? 1.0 : -1.0;
            v[0] += sg * alpha;
            double vv = 0.0;
            for (int64_t i = 0; i < m; i++) vv += v[i] * v[i];
            beta = 2.0 / vv;
            e[k] = -sg * alpha;
            /* p = beta * A22 v */
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                const double *row = A + (k + 1 + i) * K + (k + 1);
                double s = 0.0;
                for (int64_t j = 0; j < m; j++) s += row[j] * v[j];
                p[i] = beta * s;
            }
            double pv = 0.0;
            for (int64_t i = 0; i < m; i++) pv += p[i] * v[i];
            double half = 0.5 * beta * pv;
            for (int64_t i = 0; i < m; i++) p[i] -= half * v[i];   /* p is now q */
            /* A22 -= v q^T + q v^T */
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                double *row = A + (k + 1 + i) * K + (k + 1);
                for (int64_t j = 0; j < m; j++) row[j] -= v[i] * p[j] + p[i] * v[j];
            }
        } else {
            e[k] = 0.0;
        }
        betas[k] = beta;
        if (vs) memcpy(vs + k * K, v, (size_t)m * sizeof(double));
    }
    for (int64_t k = 0; k < K; k++) d[k] = A[k * K + k];
    if (K >= 2) e[K - 2] = A[(K - 1) * K + (K - 2)];
    if (Qt) {
        /* Q^T = P_{K-3} ... P_1 P_0: apply P_0 first to the identity. */
        for (int64_t i = 0; i < K * K; i++) Qt[i] = 0.0;
        for (int64_t i = 0; i < K; i++) Qt[i * K + i] = 1.0;
        double *wrow = (double *)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k + 2 < K; k++) {
            double beta = betas[k];
            if (beta == 0.0) continue;
            int64_t m = K - k - 1;
            const double *vk = vs + k * K;
            /* wrow = sum_i v_i Qt[k+1+i][:], each column summed in order of i */
#pragma omp parallel for schedule(static)
            for (int64_t cb = 0; cb < K; cb += 64) {
                int64_t ce = cb + 64 < K ? cb + 64 : K;
                double acc[64];
                for (int64_t c = cb; c < ce; c++) acc[c - cb] = 0.0;
                for (int64_t i = 0; i < m; i++) {
                    const double *row = Qt + (k + 1 + i) * K;
                    double f = vk[i];
                    for (int64_t c = cb; c < ce; c++) acc[c - cb] += f * row[c];
                }
                for (int64_t c = cb; c < ce; c++) wrow[c] = acc[c - cb];
            }
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                double *row = Qt + (k + 1 + i) * K;
                double f = beta * vk[i];
                for (int64_t c = 0; c < K; c++) row[c] -= f * wrow[c];
            }
        }
        free(wrow);
    }
    free(v);
    free(p);
    free(vs);
    free(betas);
}

/* Implicit symmetric QR with Wilkinson shift on the tridiagonal (d, e)
 * (Golub & Van Loan, implicit symmetric QR step).  If Zt is non-NULL its rows
 * are rotated along: on entry Zt = Q^T from the reduction, on exit row k is
 * the eigenvector of d[k]. */
static int tridiag_qr(double *d, double *e, int64_t K, double *Zt)
{
    const double eps = DBL_EPSILON;
    int64_t m = K - 1;
    int iter = 0;
    while (m > 0) {
        if (fabs(e[m - 1]) <= eps * (fabs(d[m - 1]) + fabs(d[m])) || fabs(e[m - 1]) < DBL_MIN) {
            e[m - 1] = 0.0;
            m--;
            iter = 0;
            continue;
        }
        int64_t l = m - 1;
        while (l > 0) {
            if (fabs(e[l - 1]) <= eps * (fabs(d[l - 1]) + fabs(d[l])) || fabs(e[l - 1]) < DBL_MIN) {
                e[l - 1] = 0.0;
                break;
            }
            l--;
        }
        if (++iter > 100) return ORC_ERR_NO_CONVERGENCE;
        double delta = 0.5 * (d[m - 1] - d[m]);
        double bb = e[m - 1];
        double sg = delta >= 0.0 ? 1.0 : -1.0;
        double mu = d[m] - bb * bb / (delta + sg * hypot(delta, bb));
        double x = d[l] - mu, z = e[l];
        for (int64_t k = l; k < m; k++) {
            double r = hypot(x, z);
            double c = 1.0, s = 0.0;
            if (r != 0.0) { c = x / r; s = z / r; }
            if (k > l) e[k - 1] = r;
            double pp = d[k], qq = d[k + 1], rr = e[k];
            d[k] = c * c * pp + 2.0 * c * s * rr + s * s * qq;
            d[k + 1] = s * s * pp - 2.0 * c * s * rr + c * c * qq;
            e[k] = c * s * (qq - pp) + (c * c - s * s) * rr;
            if (k + 1 < m) {
                z = s * e[k + 1];
                e[k + 1] = c * e[k + 1];
                x = e[k];
            }
            if (Zt) {
                double *zk = Zt + k * K, *zk1 = Zt + (k + 1) * K;
                for (int64_t j = 0; j < K; j++) {
                    double a = zk[j], b = zk1[j];
                    zk[j] = c * a + s * b;
                    zk1[j] = -s * a + c * b;
                }
            }
        }
    }
    return ORC_OK;
}

/* Eigen-decomposition through tridiagonalisation + implicit QR.  A destroyed. */
int orc_eigh_tridiag(double *A, double *w, double *Vt, int64_t K)
{
    if (K == 1) { w[0] = A[0]; if (Vt) Vt[0] = 1.0; return ORC_OK; }
    double *e = (double *)calloc((size_t)K, sizeof(double));
    householder_tridiag(A, K, w, e, Vt);
    int st = tridiag_qr(w, e, K, Vt);
    free(e);
    return st;
}

/* Eigenvalues only, of the symmetric matrix given by the lower triangle of H. */
int orc_eigvalsh(double *w, const float *H, int64_t K)
{
    double *A = sym_lower_f64(H, K);
    int st = orc_eigh_tridiag(A, w, NULL, K);
    free(A);
    return st;
}

/* Same, from an fp64 full symmetric matrix (copied, not destroyed). */
int orc_eigvalsh_f64(double *w, const double *S, int64_t K)
{
    double *A = (double *)malloc((size_t)(K * K) * sizeof(double));
    memcpy(A, S, (size_t)(K * K) * sizeof(double));
    int st = orc_eigh_tridiag(A, w, NULL, K);
    free(A);
    return st;
}

/* Eigenpairs of the matrix given by the lower triangle of H (method 0: Jacobi,
 * 1: tridiagonal QR).  w: K eigenvalues, Vt: K x K eigenvectors as rows. */
int orc_eigh(double *w, double *Vt, const float *H, int64_t K, int method)
{
    double *A = sym_lower_f64(H, K);
    int st = method == 0 ? orc_eigh_jacobi(A, w, Vt, K, 100) : orc_eigh_tridiag(A, w, Vt, K);
    free(A);
    return st;
}

/* ------------------------------------------------------------ PSD projection */

/* P = sym(V max(Lambda, 0) V^T) of the symmetric matrix given by the lower
 * triangle of H, in fp64, rounded to fp32 at the end (hipfire-calib-data,
 * "The fix": eigh, clip at zero, rebuild, (P + P^T)/2).  P64 (nullable)
 * receives the fp64 result before rounding. */
int orc_psd_project(float *P, double *P64, const float *H, int64_t K, int method)
{
    double *w = (double *)malloc((size_t)K * sizeof(double));
    double *Vt = (double *)malloc((size_t)(K * K) * sizeof(double));
    int st = orc_eigh(w, Vt, H, K, method);
    if (st != ORC_OK) { free(w); free(Vt); return st; }
    double *R = (double *)malloc((size_t)(K * K) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < K; i++) {
        double *row = R + i * K;
        for (int64_t j = 0; j < K; j++) row[j] = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double lam = w[k] > 0.0 ? w[k] : 0.0;
#if ORC_MUTANT == 5
            lam = fabs(w[k]);   /* mutant: flips negative eigenvalues instead of clipping */
#endif
            if (lam == 0.0) continue;
            double f = lam * Vt[k * K + i];
            const double *vk = Vt + k * K;
            for (int64_t j = 0; j < K; j++) row[j] += f * vk[j];
        }
    }
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j < K; j++) {
            double s = 0.5 * (R[i * K + j] + R[j * K + i]);
            if (P64) P64[i * K + j] = s;
            P[i * K + j] = (float)s;
        }
    free(R);
    free(w);
    free(Vt);
    return ORC_OK;
}

/* ------------------------------------------------------------ factorisation */

/* In-place lower Cholesky of the full symmetric fp64 matrix A (lower triangle
 * read): A = L L^T.  A pivot that is not > 0 (which includes NaN) means the
 * matrix is not positive definite.  The strict upper triangle is zeroed. */
int orc_cholesky_lower(double *A, int64_t K)
{
    for (int64_t j = 0; j < K; j++) {
        const double *rj = A + j * K;
        double dsum = A[j * K + j];
        for (int64_t k = 0; k < j; k++) dsum -= rj[k] * rj[k];
        if (!(dsum > 0.0)) return ORC_ERR_NOT_PD;
        double ljj = sqrt(dsum);
        A[j * K + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < K; i++) {
            const double *ri = A + i * K;
            double s = A[i * K + j];
            for (int64_t k = 0; k < j; k++) s -= ri[k] * rj[k];
            A[i * K + j] = s / ljj;
        }
    }
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = i + 1; j < K; j++) A[i * K + j] = 0.0;
    return ORC_OK;
}

static int all_finite_f32(const float *x, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* mean of the diagonal of the lower-triangle symmetric H (fp64 sum). */
double orc_diag_mean(const float *H, int64_t K)
{
    double s = 0.0;
    for (int64_t i = 0; i < K; i++) s += (double)H[i * K + i];
    return s / (double)K;
}

/* U (K x K fp64, upper triangular, lower part zero) with H_d^{-1} = U^T U, where
 * H_d = H + damp * mean(diag H) * I.  Literal route: L = chol(H_d),
 * H_d^{-1} = L^{-T} L^{-1}, U = the upper Cholesky factor of H_d^{-1}.
 * Returns NONFINITE for NaN/Inf in H's lower triangle, NO_CALIBRATION when
 * mean(diag H) <= 0, NOT_PD when a Cholesky pivot is not positive. */
int orc_gptq_U(double *U, const float *H, int64_t K, double damp, double *mu_out)
{
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j <= i; j++)
            if (!isfinite(H[i * K + j])) return ORC_ERR_NONFINITE;
    double mu = orc_diag_mean(H, K);
    if (mu_out) *mu_out = mu;
    if (!(mu > 0.0)) return ORC_ERR_NO_CALIBRATION;
    double *A = sym_lower_f64(H, K);
    for (int64_t i = 0; i < K; i++) A[i * K + i] += damp * mu;
    int st = orc_cholesky_lower(A, K);
    if (st != ORC_OK) { free(A); return st; }
    /* LinvT[j][:] = column j of L^{-1}: solve L x = e_j by forward substitution */
    double *LinvT = (double *)calloc((size_t)(K * K), sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < K; j++) {
        double *x = LinvT + j * K;
        for (int64_t i = j; i < K; i++) {
            const double *li = A + i * K;
            double s = (i == j) ? 1.0 : 0.0;
            for (int64_t k = j; k < i; k++) s -= li[k] * x[k];
            x[i] = s / li[i];
        }
    }
    /* Hinv[a][b] = sum_i Linv[i][a] Linv[i][b], i >= max(a, b) */
    double *Hinv = A;   /* reuse storage */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t a = 0; a < K; a++) {
        const double *xa = LinvT + a * K;
        for (int64_t b = 0; b <= a; b++) {
            const double *xb = LinvT + b * K;
            double s = 0.0;
            for (int64_t i = a; i < K; i++) s += xa[i] * xb[i];
            Hinv[a * K + b] = s;
            Hinv[b * K + a] = s;
        }
    }
    free(LinvT);
    st = orc_cholesky_lower(Hinv, K);
    if (st != ORC_OK) { free(A); return st; }
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j < K; j++) U[i * K + j] = (j >= i) ? Hinv[j * K + i] : 0.0;
#if ORC_MUTANT == 4
    /* mutant: rows of the Cholesky factor of H_d^{-1} taken in reversed order */
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j < K; j++)
            U[i * K + j] = (j >= i) ? Hinv[(K - 1 - i) * K + (K - 1 - j)] : 0.0;
#endif
    free(A);
    return ORC_OK;
}

/* ------------------------------------------------------------ quantisation */

/* fp32 scale of a group from its absolute maximum: fl32(amax) / 7 in fp32. */
static float group_scale(double amax) { return (float)amax / 7.0f; }

/* Sweep and pack switches.  ORC_STATIC_GROUPS: every group's scale is fixed
 * before the sweep from the original weights (AutoGPTQ's static_groups), instead
 * of at the group's first column from its error-updated values.  ORC_NF4: the
 * codes index a 16-level codebook (NF4, the comparison pack of the ork-driver
 * wiki's qerr section) instead of the uniform int4 grid. */
#define ORC_STATIC_GROUPS 1
#define ORC_NF4 2
/* ORC_ACT_ORDER (with ORC_STATIC_GROUPS only): columns are quantised in order of
 * decreasing diag(H) (AutoGPTQ's desc_act), each with its original group's
 * static scale; codes come back in the original column order. */
#define ORC_ACT_ORDER 4

/* Scale on the chosen grid: absmax/7 for the uniform grid; absmax itself for a
 * codebook, whose levels span [-1, 1]. */
static float grid_scale(double amax, const float *book)
{
#if ORC_MUTANT == 9
    if (book) return (float)amax / 7.0f;   /* mutant: the uniform grid's step as the codebook scale */
#endif
    return book ? (float)amax : group_scale(amax);
}

/* Index of the codebook level nearest to x = fl32(w) / s, decided in fp32: the
 * number of midpoints fl32(L[j] + L[j+1]) / 2 that x exceeds, so a value exactly
 * on a midpoint takes the lower level.  s == 0 gives the level 0.0 (an all-zero
 * group reconstructs exactly). */
static int book_code(double w, float s, const float *L)
{
    float x = 0.0f;
    if (s != 0.0f) x = (float)w / s;
    int c = 0;
    for (int j = 0; j < 15; j++) {
        float mid = (L[j] + L[j + 1]) * 0.5f;
#if ORC_MUTANT == 10
        mid = L[j + 1];                     /* mutant: the level below instead of the nearest */
#endif
        if (x > mid) c++;
    }
    return c;
}

/* Code of value w under scale s, decided in fp32: clamp(rint(fl32(w) / s), -8, 7),
 * ties to even; an all-zero group (s == 0) gives code 0. */
static int quant_code(double w, float s)
{
    if (s == 0.0f) return 0;
    float v = (float)w / s;
    float r = nearbyintf(v);
    if (r > 7.0f) r = 7.0f;
    if (r < -8.0f) r = -8.0f;
    return (int)r;
}

/* Code of w under scale s on the chosen grid, and the value it stands for. */
static int grid_code(double w, float s, const float *book)
{
    return book ? book_code(w, s, book) : quant_code(w, s);
}
static double grid_value(int c, float s, const float *book)
{
    return (book ? (double)book[c] : (double)c) * (double)s;
}

/* absmax of w[i .. i+G-1] in fp64. */
static double group_amax_f32(const float *w, int64_t i, int64_t G)
{
    double amax = 0.0;
    for (int64_t k = i; k < i + G; k++) amax = fmax(amax, fabs((double)w[k]));
    return amax;
}

/* GPTQ error-feedback sweep of the listed rows, natural column order, fp64
 * working copy (ork-driver wiki, GPTQ Int4: error-compensated
 * column-sequential rounding).  For column i of row n:
 *   at a group start (i % G == 0) the scale is absmax/7 of the group's current,
 *   error-updated values (with ORC_STATIC_GROUPS: of the original weights);
 *   c = clamp(rint(w_i / s), -8, 7)  (ORC_NF4: the nearest level of `book`,
 *   scale absmax);  e = (w_i - value(c)) / U[i][i];
 *   w_j -= e * U[i][j] for every later column j.
 * codes: nrows x K (one code per byte: signed int4, or the NF4 level index),
 * scales: nrows x K/G. */
/* Static scales of one row: stab[g] = the grid's scale of the absolute maximum
 * of the original values w0[k] over the columns k of group g (gidx[k] == g, or
 * k / G when gidx is NULL). */
static void static_scales(float *stab, const float *w0, int64_t K, int64_t G, const int64_t *gidx,
                          const float *book)
{
    double *amax = (double *)calloc((size_t)(K / G), sizeof(double));
    for (int64_t k = 0; k < K; k++) {
        int64_t g = gidx ? gidx[k] : k / G;
        amax[g] = fmax(amax[g], fabs((double)w0[k]));
    }
    for (int64_t g = 0; g < K / G; g++) stab[g] = grid_scale(amax[g], book);
    free(amax);
}

/* The sweep, with an optional group map for static groups: column i takes the
 * static scale of group gidx[i] (the act-order permutation's original groups);
 * gidx NULL means contiguous groups, i / G. */
void orc_gptq_sweep_gx(int8_t *codes, float *scales, const float *W, const double *U,
                       int64_t K, int64_t G, const int64_t *rows, int64_t nrows, int flags,
                       const float *book, const int64_t *gidx)
{
    int stat = (flags & ORC_STATIC_GROUPS) != 0;
#if ORC_MUTANT == 13
    stat = 0;                               /* mutant: the static switch ignored */
#endif
    if (!(flags & ORC_NF4)) book = NULL;
    if (!stat) gidx = NULL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
        const float *w0 = W + rows[r] * K;
        double *wk = (double *)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) wk[k] = (double)w0[k];
        float *srow = scales + r * (K / G);
        if (stat) static_scales(srow, w0, K, G, gidx, book);
        float s = 0.0f;
        for (int64_t i = 0; i < K; i++) {
            if (stat) {
                s = srow[gidx ? gidx[i] : i / G];
            } else if (i % G == 0) {
                double amax = 0.0;
                for (int64_t k = i; k < i + G; k++) amax = fmax(amax, fabs(wk[k]));
#if ORC_MUTANT == 3
                amax = group_amax_f32(w0, i, G);   /* mutant: static scales in the default sweep */
#endif
                s = grid_scale(amax, book);
                srow[i / G] = s;
            }
            int c = grid_code(wk[i], s, book);
            codes[r * K + i] = (int8_t)c;
            double e = (wk[i] - grid_value(c, s, book)) / U[i * K + i];
#if ORC_MUTANT == 2
            e = -e;   /* mutant: wrong sign of the error feedback */
#endif
            const double *ui = U + i * K;
            for (int64_t j = i + 1; j < K; j++) wk[j] -= e * ui[j];
        }
        free(wk);
    }
}

void orc_gptq_sweep_ex(int8_t *codes, float *scales, const float *W, const double *U,
                       int64_t K, int64_t G, const int64_t *rows, int64_t nrows, int flags,
                       const float *book)
{
    orc_gptq_sweep_gx(codes, scales, W, U, K, G, rows, nrows, flags, book, NULL);
}

void orc_gptq_sweep(int8_t *codes, float *scales, const float *W, const double *U,
                    int64_t K, int64_t G, const int64_t *rows, int64_t nrows)
{
    orc_gptq_sweep_ex(codes, scales, W, U, K, G, rows, nrows, 0, NULL);
}

/* Round-to-nearest on the same grid (flags: ORC_NF4 with `book`): scales from
 * the original weights. */
void orc_rtn_ex(int8_t *codes, float *scales, const float *W, int64_t N, int64_t K, int64_t G, int flags,
                const float *book)
{
    if (!(flags & ORC_NF4)) book = NULL;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const float *w = W + n * K;
        for (int64_t g = 0; g < K / G; g++) {
            float s = grid_scale(group_amax_f32(w, g * G, G), book);
            scales[n * (K / G) + g] = s;
            for (int64_t k = g * G; k < (g + 1) * G; k++) codes[n * K + k] = (int8_t)grid_code(w[k], s, book);
        }
    }
}

void orc_rtn(int8_t *codes, float *scales, const float *W, int64_t N, int64_t K, int64_t G)
{
    orc_rtn_ex(codes, scales, W, N, K, G, 0, NULL);
}

/* qerr = sqrt(sum_n sum_k imp[k] (w - c s)^2 / sum_n sum_k imp[k] w^2), w the
 * original weights, imp = 1 when NULL; 0 when the denominator is 0.  Also
 * returns the two sums (num_den[0], num_den[1]) when num_den is non-NULL. */
double orc_qerr_ex(const int8_t *codes, const float *scales, const float *W, const float *imp,
                   int64_t N, int64_t K, int64_t G, const float *book, double *num_den)
{
    double num = 0.0, den = 0.0;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double wi = imp ? (double)imp[k] : 1.0;
            double w = (double)W[n * K + k];
            double q = grid_value(codes[n * K + k], scales[n * (K / G) + k / G], book);
#if ORC_MUTANT == 6
            num += (w - q) * (w - q);   /* mutant: numerator ignores the importance */
#else
            num += wi * (w - q) * (w - q);
#endif
            den += wi * w * w;
        }
    if (num_den) { num_den[0] = num; num_den[1] = den; }
    return den > 0.0 ? sqrt(num / den) : 0.0;
}

double orc_qerr(const int8_t *codes, const float *scales, const float *W, const float *imp,
                int64_t N, int64_t K, int64_t G, double *num_den)
{
    return orc_qerr_ex(codes, scales, W, imp, N, K, G, NULL, num_den);
}

/* Two signed codes per byte: column 2m in the low nibble of byte m, column
 * 2m+1 in the high nibble, two's complement. */
void orc_pack_codes(uint8_t *out, const int8_t *codes, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < K / 2; m++) {
            uint8_t lo = (uint8_t)codes[n * K + 2 * m] & 0xF;
            uint8_t hi = (uint8_t)codes[n * K + 2 * m + 1] & 0xF;
            out[n * (K / 2) + m] = (uint8_t)(lo | (hi << 4));
        }
}

void orc_unpack_codes(int8_t *codes, const uint8_t *packed, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < K / 2; m++) {
            uint8_t b = packed[n * (K / 2) + m];
            int lo = b & 0xF, hi = b >> 4;
            codes[n * K + 2 * m] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            codes[n * K + 2 * m + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
}

/* Act-order permutation: perm[a] = the column with the a-th largest diagonal
 * entry of H (fp32 values of the stored diagonal), equal entries in increasing
 * column order (a stable sort), so the result is unique. */
static const float *g_perm_diag;
static int cmp_desc_diag(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    float da = g_perm_diag[a], db = g_perm_diag[b];
#if ORC_MUTANT == 11
    { float t = da; da = db; db = t; }     /* mutant: increasing diagonal */
#endif
    if (da > db) return -1;
    if (da < db) return 1;
    return (a > b) - (a < b);
}

void orc_act_order_perm(int64_t *perm, const float *H, int64_t K)
{
    float *d = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t i = 0; i < K; i++) { d[i] = H[i * K + i]; perm[i] = i; }
    g_perm_diag = d;
    qsort(perm, (size_t)K, sizeof(int64_t), cmp_desc_diag);
    free(d);
}

/* Full GPTQ of W (N x K) under H: codes (N x K, one per byte), scales, qerr.
 * imp NULL => 1, qerr_out NULL => not computed; flags and book as for
 * orc_gptq_sweep_ex.  With ORC_ACT_ORDER (and ORC_STATIC_GROUPS) the columns of W
 * and the rows and columns of H are permuted by orc_act_order_perm, U is formed
 * from the permuted H, the sweep runs in that order with each column's original
 * group's static scale, and the codes are put back in the original order. */
int orc_gptq_ex(int8_t *codes, float *scales, double *qerr_out, const float *W, const float *H,
                const float *imp, int64_t N, int64_t K, int64_t G, double damp, int flags,
                const float *book)
{
    if (!(flags & ORC_NF4)) book = NULL;
    if ((flags & ORC_NF4) && !book) return ORC_ERR_INVALID_ARG;
    if ((flags & ORC_ACT_ORDER) && !(flags & ORC_STATIC_GROUPS)) return ORC_ERR_INVALID_ARG;
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j <= i; j++)
            if (!isfinite(H[i * K + j])) return ORC_ERR_NONFINITE;
    if (N < 1 || K < 2 || (K & 1) || G < 1 || K % G != 0) return ORC_ERR_INVALID_ARG;
    if (!all_finite_f32(W, N * K)) return ORC_ERR_NONFINITE;
    if (imp && !all_finite_f32(imp, K)) return ORC_ERR_NONFINITE;
    double *U = (double *)malloc((size_t)(K * K) * sizeof(double));
    int64_t *rows = (int64_t *)malloc((size_t)N * sizeof(int64_t));
    for (int64_t n = 0; n < N; n++) rows[n] = n;
    int st;
    if (flags & ORC_ACT_ORDER) {
        int64_t *perm = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        int64_t *gidx = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        float *Hp = (float *)malloc((size_t)(K * K) * sizeof(float));
        float *Wp = (float *)malloc((size_t)(N * K) * sizeof(float));
        int8_t *cp = (int8_t *)malloc((size_t)(N * K));
        orc_act_order_perm(perm, H, K);     /* H is finite here (checked above) */
        /* Hp[a][b] = H[perm[a]][perm[b]], read from H's lower triangle */
        for (int64_t a = 0; a < K; a++)
            for (int64_t b = 0; b < K; b++) {
                int64_t i = perm[a], j = perm[b];
                Hp[a * K + b] = i >= j ? H[i * K + j] : H[j * K + i];
            }
        for (int64_t n = 0; n < N; n++)
            for (int64_t a = 0; a < K; a++) Wp[n * K + a] = W[n * K + perm[a]];
        for (int64_t a = 0; a < K; a++) gidx[a] = perm[a] / G;
#if ORC_MUTANT == 12
        for (int64_t a = 0; a < K; a++) gidx[a] = a / G;   /* mutant: groups of the permuted order */
#endif
        st = orc_gptq_U(U, Hp, K, damp, NULL);
        if (st == ORC_OK) {
            orc_gptq_sweep_gx(cp, scales, Wp, U, K, G, rows, N, flags, book, gidx);
            for (int64_t n = 0; n < N; n++)
                for (int64_t a = 0; a < K; a++) codes[n * K + perm[a]] = cp[n * K + a];
        }
        free(perm); free(gidx); free(Hp); free(Wp); free(cp);
    } else {
        st = orc_gptq_U(U, H, K, damp, NULL);
        if (st == ORC_OK) orc_gptq_sweep_ex(codes, scales, W, U, K, G, rows, N, flags, book);
    }
    free(rows);
    free(U);
    if (st != ORC_OK) return st;
    if (qerr_out) *qerr_out = orc_qerr_ex(codes, scales, W, imp, N, K, G, book, NULL);
    return ORC_OK;
}

int orc_gptq(int8_t *codes, float *scales, double *qerr_out, const float *W, const float *H,
             const float *imp, int64_t N, int64_t K, int64_t G, double damp)
{
    return orc_gptq_ex(codes, scales, qerr_out, W, H, imp, N, K, G, damp, 0, NULL);
}

/* ------------------------------------------------------------ replay checker */

/* Replays the sweep on the listed rows, feeding it the candidate codes and
 * scales, and classifies each candidate code against the decision the
 * reference arithmetic takes at the same point:
 *   stats[0] codes equal to the reference's                      (exact)
 *   stats[1] the other neighbour, with v within delta of a tie   (tie flips)
 *   stats[2] anything else                                       (inadmissible)
 *   stats[3] groups whose scale differs by more than scale_tol (relative)
 * v = fl32(w)/s with the reference's own scale (on the uniform grid v is in
 * steps and a tie is a half-integer; on a codebook a tie is the midpoint of two
 * neighbouring levels and delta is a fraction of their spacing); the trajectory
 * follows the candidate (w_j -= e U[i][j] with e from the candidate's code and
 * scale), so a tie flip's downstream effect is not counted again.  max_rel[0]
 * gets the largest relative scale difference.  flags and book as for
 * orc_gptq_sweep_ex.  flip_hist (nullable, 6 counters) sorts the accepted tie
 * flips by how far v was from the exact tie, in units of one step (of the
 * level spacing on a codebook): [0, 1e-7), [1e-7, 1e-6), [1e-6, 1e-5),
 * [1e-5, 1e-4), [1e-4, 1e-3), [1e-3, delta]. */
void orc_gptq_replay_hx(int64_t *stats, double *max_rel, const int8_t *cand_codes,
                        const float *cand_scales, const float *W, const double *U,
                        int64_t K, int64_t G, const int64_t *rows, int64_t nrows,
                        double delta, double scale_tol, int flags, const float *book,
                        const int64_t *gidx, int64_t *flip_hist)
{
    const int stat = (flags & ORC_STATIC_GROUPS) != 0;
    if (!(flags & ORC_NF4)) book = NULL;
    if (!stat) gidx = NULL;
    int64_t exact = 0, flips = 0, bad = 0, smis = 0;
    double mrel = 0.0;
    /* first[i]: column i is the first of its group in this order */
    char *first = (char *)calloc((size_t)K, 1);
    char *seen = (char *)calloc((size_t)(K / G), 1);
    for (int64_t i = 0; i < K; i++) {
        const int64_t gi = gidx ? gidx[i] : i / G;
        if (!seen[gi]) { seen[gi] = 1; first[i] = 1; }
    }
    free(seen);
    int64_t h0 = 0, h1 = 0, h2 = 0, h3 = 0, h4 = 0, h5 = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : exact, flips, bad, smis, h0, h1, h2, h3, h4, h5) reduction(max : mrel)
    for (int64_t r = 0; r < nrows; r++) {
        const float *w0 = W + rows[r] * K;
        double *wk = (double *)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) wk[k] = (double)w0[k];
        float s_ref = 0.0f, s_c = 0.0f;
        float *stab = (float *)malloc((size_t)(K / G) * sizeof(float));
        if (stat) static_scales(stab, w0, K, G, gidx, book);
        for (int64_t i = 0; i < K; i++) {
            const int64_t gi = gidx ? gidx[i] : i / G;
            if (stat) {
                s_ref = stab[gi];
                s_c = cand_scales[r * (K / G) + gi];
                if (first[i]) {         /* each group's scale is compared once */
                    double den = fabs((double)s_ref) > 0.0 ? fabs((double)s_ref) : 1e-30;
                    double rel = fabs((double)s_c - (double)s_ref) / den;
                    if (s_ref == 0.0f && s_c == 0.0f) rel = 0.0;
                    if (rel > mrel) mrel = rel;
                    if (rel > scale_tol) smis++;
                }
            } else if (i % G == 0) {
                double amax = 0.0;
                for (int64_t k = i; k < i + G; k++) amax = fmax(amax, fabs(wk[k]));
                s_ref = grid_scale(amax, book);
                s_c = cand_scales[r * (K / G) + i / G];
                double den = fabs((double)s_ref) > 0.0 ? fabs((double)s_ref) : 1e-30;
                double rel = fabs((double)s_c - (double)s_ref) / den;
                if (s_ref == 0.0f && s_c == 0.0f) rel = 0.0;
                if (rel > mrel) mrel = rel;
                if (rel > scale_tol) smis++;
            }
            int cg = cand_codes[r * K + i];
            int cr = grid_code(wk[i], s_ref, book);
            if (cg == cr) {
                exact++;
            } else if (s_ref != 0.0f && !book) {
                double v = (double)((float)wk[i] / s_ref);
                double rv = nearbyint(v);
                double dist = fabs(v - rv);
                double other = rv + (v > rv ? 1.0 : -1.0);
                if (other > 7.0) other = 7.0;
                if (other < -8.0) other = -8.0;
                if (dist >= 0.5 - delta && (double)cg == other) {
                    flips++;
                    const double gap = 0.5 - dist;
                    if (gap < 1e-7) h0++; else if (gap < 1e-6) h1++; else if (gap < 1e-5) h2++;
                    else if (gap < 1e-4) h3++; else if (gap < 1e-3) h4++; else h5++;
                } else {
                    bad++;
                }
            } else if (s_ref != 0.0f && (cg == cr + 1 || cg == cr - 1) && cg >= 0 && cg < 16) {
                int lo = cg < cr ? cg : cr;
                double v = (double)((float)wk[i] / s_ref);
                double mid = 0.5 * ((double)book[lo] + (double)book[lo + 1]);
                const double gap = fabs(v - mid) / ((double)book[lo + 1] - (double)book[lo]);
                if (gap <= delta) {
                    flips++;
                    if (gap < 1e-7) h0++; else if (gap < 1e-6) h1++; else if (gap < 1e-5) h2++;
                    else if (gap < 1e-4) h3++; else if (gap < 1e-3) h4++; else h5++;
                } else {
                    bad++;
                }
            } else {
                bad++;
            }
            double cv = (cg >= -8 && cg < 16 && (book ? cg >= 0 : cg < 8)) ? grid_value(cg, s_c, book) : 0.0;
            double e = (wk[i] - cv) / U[i * K + i];
            const double *ui = U + i * K;
            for (int64_t j = i + 1; j < K; j++) wk[j] -= e * ui[j];
        }
        free(stab);
        free(wk);
    }
    free(first);
    stats[0] = exact;
    stats[1] = flips;
    stats[2] = bad;
    stats[3] = smis;
    *max_rel = mrel;
    if (flip_hist) {
        flip_hist[0] = h0; flip_hist[1] = h1; flip_hist[2] = h2;
        flip_hist[3] = h3; flip_hist[4] = h4; flip_hist[5] = h5;
    }
}

void orc_gptq_replay_gx(int64_t *stats, double *max_rel, const int8_t *cand_codes,
                        const float *cand_scales, const float *W, const double *U,
                        int64_t K, int64_t G, const int64_t *rows, int64_t nrows,
                        double delta, double scale_tol, int flags, const float *book,
                        const int64_t *gidx)
{
    orc_gptq_replay_hx(stats, max_rel, cand_codes, cand_scales, W, U, K, G, rows, nrows, delta, scale_tol,
                       flags, book, gidx, NULL);
}

void orc_gptq_replay_ex(int64_t *stats, double *max_rel, const int8_t *cand_codes,
                        const float *cand_scales, const float *W, const double *U,
                        int64_t K, int64_t G, const int64_t *rows, int64_t nrows,
                        double delta, double scale_tol, int flags, const float *book)
{
    orc_gptq_replay_gx(stats, max_rel, cand_codes, cand_scales, W, U, K, G, rows, nrows, delta, scale_tol,
                       flags, book, NULL);
}

void orc_gptq_replay(int64_t *stats, double *max_rel, const int8_t *cand_codes,
                     const float *cand_scales, const float *W, const double *U,
                     int64_t K, int64_t G, const int64_t *rows, int64_t nrows,
                     double delta, double scale_tol)
{
    orc_gptq_replay_ex(stats, max_rel, cand_codes, cand_scales, W, U, K, G, rows, nrows, delta, scale_tol, 0,
                       NULL);
}
