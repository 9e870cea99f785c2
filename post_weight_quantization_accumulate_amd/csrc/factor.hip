// factor.hip -- element-wise and small kernels around the blocked fp64
// factorisation: damping in units of mean(diag H) (hipfire-calib-data, "The
// fix"), the order reversal that turns a lower-first Cholesky into the
// H_d = R R^T (R upper) factor whose inverse is the GPTQ factor U, the
// factorisation of one diagonal block and the panel solves, and the fp64 reductions
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

// D[i][j] = D[j][i] = H[max][min] as fp64, from the lower triangle only.  One
// 64 x 64 lower tile of H per workgroup, read by rows into LDS and written to
// D both as it is and transposed (the mirror), so that every read and write
// runs along rows.  On a diagonal tile the entries above the diagonal come
// from their mirror inside the tile.  With rowmax set (zeroed beforehand) it
// also leaves there the largest magnitude of each row of D, as the bits of a
// non-negative fp64 (whose order is that of unsigned integers, so the rows'
// maxima over the tiles are taken with atomicMax, in any order).
constexpr int SYT = 64;
__global__ __launch_bounds__(NT) void sym_lower_kernel(double *__restrict__ D, const float *__restrict__ H,
                                                      int64_t K, unsigned *status,
                                                      unsigned long long *__restrict__ rowmax)
{
    __shared__ float t[SYT][SYT + 1];
    const int64_t id = blockIdx.x;
    int64_t ti = (int64_t)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
    while (ti * (ti + 1) / 2 > id) --ti;
    while ((ti + 1) * (ti + 2) / 2 <= id) ++ti;
    const int64_t tj = id - ti * (ti + 1) / 2;
    const int64_t i0 = ti * SYT, j0 = tj * SYT;
    const int tx = threadIdx.x & (SYT - 1), ty = threadIdx.x / SYT;
    bool bad = false;
    for (int r = ty; r < SYT; r += NT / SYT) {
        const int64_t gi = i0 + r, gj = j0 + tx;
        float h = 0.0f;
        if (gi < K && gj <= gi) {
            h = H[gi * K + gj];
            if (!isfinite(h)) bad = true;
        }
        t[r][tx] = h;
    }
    __syncthreads();
    for (int r = ty; r < SYT; r += NT / SYT) {
        const int64_t gi = i0 + r, gj = j0 + tx;
        if (gi < K && gj < K) D[gi * K + gj] = (double)(gj <= gi ? t[r][tx] : t[tx][r]);
        if (ti != tj) {
            const int64_t mi = j0 + r, mj = i0 + tx;        // mirror: D[mi][mj] = H[mj][mi]
            if (mj < K) D[mi * K + mj] = (double)t[tx][r];
        }
    }
    // rows i0 + r (this tile's rows) and j0 + r (its columns, the mirror's rows)
    if (rowmax && threadIdx.x < 2 * SYT) {
        const int r = threadIdx.x & (SYT - 1);
        const bool mirror = threadIdx.x >= SYT;
        float m = 0.0f;
        for (int c = 0; c < SYT; ++c) m = fmaxf(m, fabsf(mirror ? t[c][r] : t[r][c]));
        const int64_t row = (mirror ? j0 : i0) + r;
        if (row < K && m > 0.0f)
            atomicMax(rowmax + row, (unsigned long long)__double_as_longlong((double)m));
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

// Upper Cholesky (A = R^T R) of one nb x nb diagonal block (nb <= 128) in one
// workgroup, four columns per step, with the block in registers: thread t owns
// one 4 x 4 tile (tr, tc), tr <= tc, of the upper triangle (528 tiles, in row
// order).  Step jb takes the block row J = 4 jb .. 4 jb + 3 as
// it stands after steps 0 .. jb-1, published through LDS by its owners (two
// buffers, one barrier per step).  Every thread eliminates the 4 x 4 diagonal
// block D = A[J][J] in its registers, pivot by pivot: pivot e gives the
// multipliers l[e2][e] = D_e,e2 / D_ee (D as updated by the pivots before e),
// and the block row's rows become w_e = a_e - sum_{e' < e} l[e][e'] w_e'.  A
// tile below the block row then takes A[r][c] -= sum_e w_e[r] w_e[c] / D_ee,
// which is the four column steps of the unblocked algorithm, and the tile
// owners of the block row turn w_e into R's rows, R_e,c = w_e[c] / sqrt(D_ee).
// Writes R (upper) and R^T (lower) back into M, and 1 / R_kk for k < 128 to
// rinv (1 on padded rows), for the block substitutions that use the panel.
// Rows and columns beyond nb are padded with the identity, which decouples
// them.
constexpr int NBMAX = kPanel;
constexpr int SB = 32;
constexpr int PTE = 4;                                   // tile edge
constexpr int PTN = NBMAX / PTE;                         // tiles per block row
constexpr int PTILES = PTN * (PTN + 1) / 2;              // 528
constexpr int PNT = (PTILES + 63) / 64 * 64;             // 576 threads, 9 waves
static_assert(NBMAX % PTE == 0, "whole tiles");
constexpr size_t kPotrfReserveLds = 128 * 1024;

// 1 / sqrt(p) and 1 / p for p > 0: the hardware estimates and two Newton steps
// each (y <- y + y (1/2 - (p/2) y^2), y <- y + y (1 - p y)), each step doubling
// the correct bits, to full double precision
__device__ inline double rsqrt_f64(double p)
{
    double y = __builtin_amdgcn_rsq(p);
    const double hp = 0.5 * p;
    y = fma(y, fma(-hp * y, y, 0.5), y);
    y = fma(y, fma(-hp * y, y, 0.5), y);
    return y;
}
__device__ inline double rcp_f64(double p)
{
    double y = __builtin_amdgcn_rcp(p);
    y = fma(y, fma(-p, y, 1.0), y);
    y = fma(y, fma(-p, y, 1.0), y);
    return y;
}

__global__ __launch_bounds__(PNT) void potrf_diag_kernel(double *__restrict__ M, int64_t K, int64_t p0,
                                                        int nb, double *__restrict__ rinv_out, unsigned *status)
{
    __shared__ double rowb[2][PTE][NBMAX];   // the block row by step parity
    __shared__ double rinv[NBMAX];
    __shared__ int bad;
    const int t = threadIdx.x;
    const bool active = t < PTILES;
    // tiles in row order, so that a wave's tiles lie in a few neighbouring tile
    // rows and the wave has no work left once the steps have passed them
    int tr = 0, rs = 0;                                 // rs: index of tile (tr, tr)
    while (tr < PTN - 1 && rs + (PTN - tr) <= t) rs += PTN - tr++;
    const int tc = active ? tr + (t - rs) : PTN;
    if (!active) tr = PTN;                              // inactive: no rows
    const int r0 = PTE * tr, c0 = PTE * tc;
    double a[PTE][PTE];
    {
        // all 16 loads issued before any is used (clamped addresses, selects after)
        double v[PTE][PTE];
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) {
                const int r = r0 + i, c = c0 + k;
                const bool in = active && r < nb && c < nb && c >= r;
                v[i][k] = M[in ? (p0 + r) * K + p0 + c : p0 * K + p0];
            }
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) {
                const int r = r0 + i, c = c0 + k;
                const bool in = active && r < nb && c < nb && c >= r;
                a[i][k] = in ? v[i][k] : ((r == c) ? 1.0 : 0.0);
            }
    }
    if (t == 0) bad = 0;
    if (tr == 0) {
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) rowb[0][i][c0 + k] = a[i][k];
    }
    __syncthreads();
    bool badp = false;
#pragma unroll 1
    for (int jb = 0; jb < PTN; ++jb) {
        const int buf = jb & 1, j0 = PTE * jb;
        if (active && tr >= jb) {
            // D eliminated pivot by pivot (a pivot of a real row that is not
            // positive is replaced by 1 and flagged by the block row's owner)
            double d[PTE][PTE], q[PTE], pv[PTE], l[PTE][PTE];
#pragma unroll
            for (int e = 0; e < PTE; ++e)
#pragma unroll
                for (int c = 0; c < PTE; ++c) d[e][c] = rowb[buf][e][j0 + c];
#pragma unroll
            for (int e = 0; e < PTE; ++e) {
                if (tr == jb) badp |= !(d[e][e] > 0.0) & (j0 + e < nb);
                pv[e] = d[e][e] > 0.0 ? d[e][e] : 1.0;
                q[e] = rcp_f64(pv[e]);
#pragma unroll
                for (int e2 = e + 1; e2 < PTE; ++e2) {
                    l[e2][e] = d[e][e2] * q[e];
#pragma unroll
                    for (int c = e2; c < PTE; ++c) d[e2][c] = fma(-l[e2][e], d[e][c], d[e2][c]);
                }
            }
            if (tr > jb) {
                // the block row at this tile's rows (wr) and columns (wc), as w_e
                double wr[PTE][PTE], wc[PTE][PTE];
#pragma unroll
                for (int e = 0; e < PTE; ++e)
#pragma unroll
                    for (int i = 0; i < PTE; ++i) {
                        wr[e][i] = rowb[buf][e][r0 + i];
                        wc[e][i] = rowb[buf][e][c0 + i];
                    }
#pragma unroll
                for (int e = 1; e < PTE; ++e)
#pragma unroll
                    for (int e1 = 0; e1 < e; ++e1)
#pragma unroll
                        for (int i = 0; i < PTE; ++i) {
                            wr[e][i] = fma(-l[e][e1], wr[e1][i], wr[e][i]);
                            wc[e][i] = fma(-l[e][e1], wc[e1][i], wc[e][i]);
                        }
#pragma unroll
                for (int e = 0; e < PTE; ++e)
#pragma unroll
                    for (int i = 0; i < PTE; ++i) {
                        const double f = wr[e][i] * q[e];
#pragma unroll
                        for (int k = 0; k < PTE; ++k) a[i][k] = fma(-f, wc[e][k], a[i][k]);
                    }
            } else {
                // this tile's rows are the block row: w_e from its own (published)
                // values, then R's rows; on the diagonal tile the entries left of
                // the diagonal are never read
#pragma unroll
                for (int e = 1; e < PTE; ++e)
#pragma unroll
                    for (int e1 = 0; e1 < e; ++e1)
#pragma unroll
                        for (int k = 0; k < PTE; ++k) a[e][k] = fma(-l[e][e1], a[e1][k], a[e][k]);
#pragma unroll
                for (int e = 0; e < PTE; ++e) {
                    const double y = rsqrt_f64(pv[e]);
#pragma unroll
                    for (int k = 0; k < PTE; ++k) a[e][k] = (c0 + k == j0 + e) ? pv[e] * y : a[e][k] * y;
                    if (tc == jb) rinv[j0 + e] = y;
                }
            }
        }
        // publish the next block row
        if (active && tr == jb + 1) {
#pragma unroll
            for (int i = 0; i < PTE; ++i)
#pragma unroll
                for (int k = 0; k < PTE; ++k) rowb[buf ^ 1][i][c0 + k] = a[i][k];
        }
        __syncthreads();
    }
    if (active) {
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) {
                const int r = r0 + i, c = c0 + k;
                if (r < nb && c < nb && c >= r) {
                    M[(p0 + r) * K + p0 + c] = a[i][k];
                    M[(p0 + c) * K + p0 + r] = a[i][k];
                }
            }
    }
    if (t < NBMAX) rinv_out[t] = rinv[t];
    if (badp) atomicOr(&bad, 1);
    __syncthreads();
    if (t == 0 && bad) atomicOr(status, ST_NOT_PD);
}

// Y = R^-T B for the nb x nb upper block R at (p0, p0) of M (nb <= 128): block
// forward substitution by four rows, Y_J = R_JJ^-T (B_J - sum_{J' < J} R_J'J^T
// Y_J'), with 1 / R_kk from rinv (which the diagonal kernel wrote).  One
// workgroup per 64 columns of B (nb x ncols, ld ldb); thread t owns the 4 x 4
// tile (t / 16, t % 16) of the workgroup's 128 x 64 block of B in registers.
// R's upper triangle is staged in LDS, packed by rows.  Step jb: the tile row
// jb, which has every earlier step's update, solves its 4 x 4 diagonal system
// and publishes Y_J through LDS (two buffers, one barrier per step); every
// tile row below subtracts R_J,rows^T Y_J.  Y goes to out (ld ldo; out may be
// B: each workgroup reads its columns before it writes them) and, with out_t
// set, transposed to out_t (out_t[c ldt + a] = Y[a][c]).  Rows and columns
// beyond nb are padded with the identity.
constexpr int TSC = 64;
constexpr int TST = 512;
constexpr int TTC = TSC / PTE;                           // tile columns: 16
static_assert(TST == PTN * TTC, "one 4 x 4 tile per thread");
__device__ constexpr int rpack(int r) { return r * NBMAX - r * (r - 1) / 2; }   // entry (r, r)
__global__ __launch_bounds__(TST) void trsm_rt_kernel(const double *__restrict__ M, int64_t K, int64_t p0, int nb,
                                                      const double *__restrict__ rinv_in, const double *B,
                                                      int64_t ldb,
                                                      double *out, int64_t ldo, double *out_t, int64_t ldt,
                                                      int64_t ncols)
{
    __shared__ double Rp[NBMAX * (NBMAX + 1) / 2];
    __shared__ double Yp[2][PTE][TSC];
    __shared__ double rinv[NBMAX];
    const int t = threadIdx.x, tr = t / TTC, tcl = t % TTC;
    const int r0 = PTE * tr, c0 = PTE * tcl;
    const int64_t cb = (int64_t)blockIdx.x * TSC;
    double b[PTE][PTE];
    {
        // every load (R's block, this tile of B) issued before any is used
        // (clamped addresses, selects after)
        constexpr int PER = NBMAX * NBMAX / TST;
        double v[PER], w[PTE][PTE];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + TST * m, r = e / NBMAX, c = e % NBMAX;
            const bool in = r < nb && c < nb && c >= r;
            v[m] = M[in ? (p0 + r) * K + p0 + c : p0 * K + p0];
        }
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) {
                const bool in = r0 + i < nb && cb + c0 + k < ncols;
                w[i][k] = B[in ? (r0 + i) * ldb + cb + c0 + k : 0];
            }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + TST * m, r = e / NBMAX, c = e % NBMAX;
            if (c >= r) Rp[rpack(r) + c - r] = (r < nb && c < nb) ? v[m] : (r == c ? 1.0 : 0.0);
        }
#pragma unroll
        for (int i = 0; i < PTE; ++i)
#pragma unroll
            for (int k = 0; k < PTE; ++k) b[i][k] = (r0 + i < nb && cb + c0 + k < ncols) ? w[i][k] : 0.0;
    }
    if (t < NBMAX) rinv[t] = rinv_in[t];
    __syncthreads();
#pragma unroll 1
    for (int jb = 0; jb < PTN; ++jb) {
        const int buf = jb & 1, j0 = PTE * jb;
        if (tr == jb) {
            // y_e = (b_e - sum_{e1 < e} R[j0 + e1][j0 + e] y_e1) / R_ee, in place
#pragma unroll
            for (int e = 0; e < PTE; ++e) {
#pragma unroll
                for (int e1 = 0; e1 < e; ++e1) {
                    const double rr = Rp[rpack(j0 + e1) + e - e1];
#pragma unroll
                    for (int k = 0; k < PTE; ++k) b[e][k] = fma(-rr, b[e1][k], b[e][k]);
                }
                const double ri = rinv[j0 + e];
#pragma unroll
                for (int k = 0; k < PTE; ++k) b[e][k] *= ri;
            }
#pragma unroll
            for (int e = 0; e < PTE; ++e)
#pragma unroll
                for (int k = 0; k < PTE; ++k) Yp[buf][e][c0 + k] = b[e][k];
        }
        __syncthreads();
        if (tr > jb) {
            double y[PTE][PTE], rr[PTE][PTE];
#pragma unroll
            for (int e = 0; e < PTE; ++e)
#pragma unroll
                for (int k = 0; k < PTE; ++k) {
                    y[e][k] = Yp[buf][e][c0 + k];
                    rr[e][k] = Rp[rpack(j0 + e) + r0 + k - (j0 + e)];
                }
#pragma unroll
            for (int i = 0; i < PTE; ++i)
#pragma unroll
                for (int e = 0; e < PTE; ++e)
#pragma unroll
                    for (int k = 0; k < PTE; ++k) b[i][k] = fma(-rr[e][i], y[e][k], b[i][k]);
        }
    }
#pragma unroll
    for (int i = 0; i < PTE; ++i)
#pragma unroll
        for (int k = 0; k < PTE; ++k) {
            const int r = r0 + i;
            const int64_t c = cb + c0 + k;
            if (r < nb && c < ncols) {
                out[r * ldo + c] = b[i][k];
                if (out_t) out_t[c * ldt + r] = b[i][k];
            }
        }
}

// U[i][j] = X[K-1-i][K-1-j] (as fp32) for i <= j, 0 below: the lower triangular
// X turned by 180 degrees.
__global__ __launch_bounds__(NT) void flip_kernel(float *__restrict__ U, const double *__restrict__ X, int64_t K)
{
    const int64_t n = K * K;
    for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < n; e += (int64_t)gridDim.x * NT) {
        const int64_t i = e / K, j = e - i * K;
        U[e] = (i <= j) ? (float)X[(K - 1 - i) * K + (K - 1 - j)] : 0.0f;
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
                                   hipStream_t s, unsigned long long *rowmax)
{
    const int64_t ct = (K + SYT - 1) / SYT;
    hipLaunchKernelGGL(sym_lower_kernel, dim3((unsigned)(ct * (ct + 1) / 2)), dim3(NT), 0, s, D, H, K, status, rowmax);
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

hipError_t launch_potrf_diag(double *M, int64_t K, int64_t p0, int nb, double *rinv, unsigned *status,
                             hipStream_t s)
{
    if (nb < 1 || nb > NBMAX) return hipErrorInvalidValue;
    // The workgroup reserves most of a CU's LDS, which it does not use, so that
    // no workgroup of the concurrent trailing update shares its CU: the chain of
    // 128 barrier-separated steps runs at the speed of an idle CU.
    static const bool lds_ok = hipFuncSetAttribute((const void *)potrf_diag_kernel,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)kPotrfReserveLds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(PNT), kPotrfReserveLds, s, M, K, p0, nb, rinv, status);
    return hipGetLastError();
}

hipError_t launch_trsm_rt(const double *M, int64_t K, int64_t p0, int nb, const double *rinv, const double *B,
                          int64_t ldb, double *out, int64_t ldo, double *out_t, int64_t ldt, int64_t ncols,
                          hipStream_t s)
{
    if (nb < 1 || nb > NBMAX) return hipErrorInvalidValue;
    if (ncols < 1) return hipSuccess;
    hipLaunchKernelGGL(trsm_rt_kernel, dim3((unsigned)((ncols + TSC - 1) / TSC)), dim3(TST), 0, s, M, K, p0, nb, rinv,
                       B, ldb, out, ldo, out_t, ldt, ncols);
    return hipGetLastError();
}

hipError_t launch_flip(float *U, const double *X, int64_t K, hipStream_t s)
{
    hipLaunchKernelGGL(flip_kernel, dim3(grid_for(K * K)), dim3(NT), 0, s, U, X, K);
    return hipGetLastError();
}

}  // namespace gq
