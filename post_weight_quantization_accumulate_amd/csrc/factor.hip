// factor.hip -- element-wise and small kernels around the blocked fp64
// factorisation: damping in units of mean(diag H) (hipfire-calib-data, "The
// fix"), the order reversal that turns a lower-first Cholesky into the
// H_d = R R^T (R upper) factor whose inverse is the GPTQ factor U, the in-LDS
// factorisation and inversion of one diagonal block, and the fp64 reductions
// (deterministic single-workgroup trees, no atomics on floating point).
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int NT = 256;

__global__ void fill_f64_kernel(double *p, int64_t n, double v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void fill_u32_kernel(unsigned *p, int64_t n, unsigned v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void set_identity_f64_kernel(double *X, int64_t K)
{
    const int64_t n = K * K;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        X[e] = (e / K == e % K) ? 1.0 : 0.0;
}

// D[i][j] = D[j][i] = H[max][min] as fp64, from the lower triangle only.
__global__ __launch_bounds__(NT) void sym_lower_kernel(double *__restrict__ D, const float *__restrict__ H,
                                                      int64_t K, unsigned *status)
{
    const int64_t i = blockIdx.x;
    bool bad = false;
    for (int64_t j = threadIdx.x; j < K; j += NT) {
        const float h = (j <= i) ? H[i * K + j] : H[j * K + i];
        if (j <= i && !isfinite(h)) bad = true;
        D[i * K + j] = (double)h;
    }
    if (bad) atomicOr(status, ST_NONFINITE);
}

// Deterministic block reduction of 256 doubles in shared memory.
__device__ double block_sum(double v, double *sh)
{
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (t < s) sh[t] += sh[t + s];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

// Two-stage deterministic sum of squares: each of the first-stage workgroups
// owns a fixed contiguous chunk, the second stage adds the partials in order.
__global__ __launch_bounds__(NT) void sumsq_partial_kernel(double *partials, const double *a, int64_t n,
                                                          int64_t chunk)
{
    __shared__ double sh[NT];
    const int64_t b = blockIdx.x * chunk;
    const int64_t e = (b + chunk < n) ? b + chunk : n;
    double s = 0.0;
    for (int64_t i = b + threadIdx.x; i < e; i += NT) s += a[i] * a[i];
    const double tot = block_sum(s, sh);
    if (threadIdx.x == 0) partials[blockIdx.x] = tot;
}

__global__ __launch_bounds__(NT) void sqrt_sum_kernel(double *out, const double *partials, int64_t np)
{
    __shared__ double sh[NT];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < np; i += NT) s += partials[i];
    const double tot = block_sum(s, sh);
    if (threadIdx.x == 0) out[0] = sqrt(tot);
}

__global__ void scalar_combine_kernel(double *out, const double *x, double px, const double *y, double py)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const double u = x[0];
        const double v = y ? y[0] : 1.0;
        const bool ok = u > 0.0 && isfinite(u) && v > 0.0 && isfinite(v);
        out[0] = ok ? pow(u, px) * (y ? pow(v, py) : 1.0) : 0.0;
    }
}

__global__ __launch_bounds__(NT) void diag_mean_check_kernel(double *mu, const float *__restrict__ H,
                                                            int64_t K, unsigned *status)
{
    __shared__ double sh[NT];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += NT) s += (double)H[i * K + i];
    const double tot = block_sum(s, sh);
    if (threadIdx.x == 0) {
        const double m = tot / (double)K;
        mu[0] = m;
        if (!(m > 0.0) || !isfinite(m)) atomicOr(status, ST_NO_CALIB);
    }
}

// Non-finite scan of the lower triangle of H, one workgroup per row.
__global__ __launch_bounds__(NT) void lower_finite_kernel(const float *__restrict__ H, int64_t K,
                                                         unsigned *status)
{
    const int64_t i = blockIdx.x;
    bool bad = false;
    for (int64_t j = threadIdx.x; j <= i; j += NT)
        if (!isfinite(H[i * K + j])) bad = true;
    if (bad) atomicOr(status, ST_NONFINITE);
}

// M[i][j] = H[K-1-i][K-1-j] for i <= j (a lower-triangle element of H), plus the
// damping on the diagonal.  Row i of M reads row K-1-i of H backwards.
__global__ __launch_bounds__(NT) void damp_reverse_kernel(double *__restrict__ M, const float *__restrict__ H,
                                                         int64_t K, double damp, const double *mu)
{
    const int64_t i = blockIdx.x;
    const int64_t a = K - 1 - i;
    const double dm = damp * mu[0];
    for (int64_t j = i + threadIdx.x; j < K; j += NT) {
        const int64_t b = K - 1 - j;          // b <= a
        double v = (double)H[a * K + b];
        if (j == i) v += dm;
        M[i * K + j] = v;
    }
}

// Upper Cholesky (A = R^T R) of one nb x nb diagonal block in LDS, then its
// triangular inverse.  Writes R (upper) and R^T (lower) back into M, and the
// inverse / transposed inverse into Dinv / DinvT (nb x nb, row-major, ld = nb).
constexpr int NBMAX = 64;

__global__ __launch_bounds__(NT) void potrf_diag_kernel(double *__restrict__ M, int64_t K, int64_t p0,
                                                       int nb, double *__restrict__ Dinv,
                                                       double *__restrict__ DinvT, unsigned *status)
{
    __shared__ double a[NBMAX][NBMAX + 1];
    __shared__ double x[NBMAX][NBMAX + 1];
    __shared__ int bad;
    const int t = threadIdx.x;
    if (t == 0) bad = 0;
    for (int e = t; e < nb * nb; e += NT) {
        const int r = e / nb, c = e % nb;
        a[r][c] = (c >= r) ? M[(p0 + r) * K + p0 + c] : 0.0;
        x[r][c] = 0.0;
    }
    __syncthreads();
    for (int j = 0; j < nb; ++j) {
        if (t == 0) {
            double d = a[j][j];
            if (!(d > 0.0)) { bad = 1; d = 1.0; }
            a[j][j] = sqrt(d);
        }
        __syncthreads();
        const double rjj = a[j][j];
        for (int c = j + 1 + t; c < nb; c += NT) a[j][c] /= rjj;
        __syncthreads();
        // trailing update of the upper triangle: a[r][c] -= a[j][r] * a[j][c], j < r <= c
        const int m = nb - j - 1;
        for (int e = t; e < m * m; e += NT) {
            const int r = j + 1 + e / m, c = j + 1 + e % m;
            if (c >= r) a[r][c] -= a[j][r] * a[j][c];
        }
        __syncthreads();
    }
    // inverse of the upper triangular R by back substitution, one column per thread
    if (t < nb) {
        const int c = t;
        x[c][c] = 1.0 / a[c][c];
        for (int r = c - 1; r >= 0; --r) {
            double s = 0.0;
            for (int m2 = r + 1; m2 <= c; ++m2) s += a[r][m2] * x[m2][c];
            x[r][c] = -s / a[r][r];
        }
    }
    __syncthreads();
    for (int e = t; e < nb * nb; e += NT) {
        const int r = e / nb, c = e % nb;
        const double rv = (c >= r) ? a[r][c] : a[c][r];     // R above, R^T below
        M[(p0 + r) * K + p0 + c] = rv;
        Dinv[r * nb + c] = x[r][c];
        DinvT[c * nb + r] = x[r][c];
    }
    if (t == 0 && bad) atomicOr(status, ST_NOT_PD);
}

// U[i][j] = X[K-1-j][K-1-i] for i <= j, 0 below; transposed through LDS tiles.
constexpr int TF = 32;
__global__ __launch_bounds__(NT) void flip_transpose_kernel(float *__restrict__ U, const double *__restrict__ X,
                                                           int64_t K)
{
    __shared__ double tile[TF][TF + 1];
    const int64_t bi = blockIdx.y, bj = blockIdx.x;   // output tile (rows bi, cols bj)
    const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    // source rows a = K-1-j for j in the output column tile, cols b = K-1-i
    for (int r = r0; r < TF; r += NT / TF) {
        const int64_t j = bj * TF + r, i = bi * TF + c;
        double v = 0.0;
        if (i < K && j < K && i <= j) v = X[(K - 1 - j) * K + (K - 1 - i)];
        tile[r][c] = v;          // tile[j - j0][i - i0]
    }
    __syncthreads();
    for (int r = r0; r < TF; r += NT / TF) {
        const int64_t i = bi * TF + r, j = bj * TF + c;
        if (i < K && j < K) U[i * K + j] = (float)tile[c][r];
    }
}

}  // namespace

static unsigned grid_for(int64_t n)
{
    int64_t g = (n + NT - 1) / NT;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (unsigned)g;
}

hipError_t launch_fill_f64(double *p, int64_t n, double v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_f64_kernel, dim3(grid_for(n)), dim3(NT), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned *p, int64_t n, unsigned v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(NT), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_set_identity_f64(double *X, int64_t K, hipStream_t s)
{
    hipLaunchKernelGGL(set_identity_f64_kernel, dim3(grid_for(K * K)), dim3(NT), 0, s, X, K);
    return hipGetLastError();
}

hipError_t launch_sym_lower_to_f64(double *D, const float *H, int64_t K, unsigned *status,
                                   hipStream_t s)
{
    hipLaunchKernelGGL(sym_lower_kernel, dim3((unsigned)K), dim3(NT), 0, s, D, H, K, status);
    return hipGetLastError();
}

hipError_t launch_frobenius(double *out, const double *a, int64_t n, double *partials, hipStream_t s)
{
    const int64_t np = kFrobParts;
    const int64_t chunk = (n + np - 1) / np;
    hipLaunchKernelGGL(sumsq_partial_kernel, dim3((unsigned)np), dim3(NT), 0, s, partials, a, n, chunk);
    hipLaunchKernelGGL(sqrt_sum_kernel, dim3(1), dim3(NT), 0, s, out, partials, np);
    return hipGetLastError();
}

hipError_t launch_scalar_combine(double *out, const double *x, double px, const double *y, double py,
                                 hipStream_t s)
{
    hipLaunchKernelGGL(scalar_combine_kernel, dim3(1), dim3(64), 0, s, out, x, px, y, py);
    return hipGetLastError();
}

hipError_t launch_diag_mean_check(double *mu, const float *H, int64_t K, unsigned *status,
                                  hipStream_t s)
{
    hipLaunchKernelGGL(lower_finite_kernel, dim3((unsigned)K), dim3(NT), 0, s, H, K, status);
    hipLaunchKernelGGL(diag_mean_check_kernel, dim3(1), dim3(NT), 0, s, mu, H, K, status);
    return hipGetLastError();
}

hipError_t launch_damp_reverse(double *M, const float *H, int64_t K, double damp, const double *mu,
                               hipStream_t s)
{
    hipLaunchKernelGGL(damp_reverse_kernel, dim3((unsigned)K), dim3(NT), 0, s, M, H, K, damp, mu);
    return hipGetLastError();
}

hipError_t launch_potrf_diag(double *M, int64_t K, int64_t p0, int nb, double *Dinv, double *DinvT,
                             unsigned *status, hipStream_t s)
{
    if (nb < 1 || nb > NBMAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(NT), 0, s, M, K, p0, nb, Dinv, DinvT, status);
    return hipGetLastError();
}

hipError_t launch_flip_transpose(float *U, const double *X, int64_t K, hipStream_t s)
{
    const unsigned nt = (unsigned)((K + TF - 1) / TF);
    hipLaunchKernelGGL(flip_transpose_kernel, dim3(nt, nt), dim3(NT), 0, s, U, X, K);
    return hipGetLastError();
}

}  // namespace gq
