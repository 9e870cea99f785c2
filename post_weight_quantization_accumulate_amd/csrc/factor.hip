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

// Upper Cholesky (A = R^T R) of one nb x nb diagonal block (nb <= 128), blocked
// by 32 so that the sequential part runs in one wave without workgroup barriers:
//   - one wave factors each 32 x 32 diagonal sub-block D in its
//     registers (each lane a 4 x 4 tile), publishing the pivot row (column) of
//     each step through LDS;
//   - then the strip solve R[D, rest] = R_DD^-T A[D, rest] by substitution, one
//     column per thread, and the trailing update A[rest, rest] -= R[D, rest]^T
//     R[D, rest] by all 8 waves.
// The block lives in LDS (R in the upper triangle).  Writes R (upper) and R^T
// (lower) back into M, and 1 / R_kk for k < 128 to rinv (1 on padded rows), for
// the block substitutions that use the panel.  Rows and columns beyond nb are
// padded with the identity, which decouples them.
constexpr int NBMAX = kPanel;
constexpr int SB = 32;
constexpr int PNT = 512;

// fp64 lane exchanges: the value of lane `lane` (compile-time), and of lane
// addr / 4 for each lane (ds_bpermute)
__device__ inline double readlane_f64(double v, int lane)
{
    const int2 w = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(w.x, lane), __builtin_amdgcn_readlane(w.y, lane)));
}
__device__ inline double bpermute_f64(int addr, double v)
{
    const int2 w = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_ds_bpermute(addr, w.x), __builtin_amdgcn_ds_bpermute(addr, w.y)));
}

// One wave: Cholesky of the 32 x 32 block at (o, o) of A.  Lane l owns rows
// 4 (l / 8) + i and columns 4 (l % 8) + k in registers.  Step j takes the pivot
// from the lane holding (j, j) (readlane) and the pivot row from the 8 lanes
// holding row j (one permute per value, issued while the pivot's inverse square
// root is computed).  Writes R (upper) into A and 1 / R_jj into rinv[o + j].
// Returns true if a pivot of a real (not padded) row was not positive.
__device__ __attribute__((noinline)) bool wave_factor32(double (*A)[NBMAX + 1], double *rinv, int o, int nb,
                                                        int lane)
{
    const int br = lane >> 3, bc = lane & 7;
    double a[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 4 * br + i, c = 4 * bc + k;
            a[i][k] = (c >= r) ? A[o + r][o + c] : 0.0;
        }
    bool badp = false;
    static_for<SB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int g = j >> 2, e = j & 3;             // row j: lanes 8 g + bc, register row e
        const double piv0 = readlane_f64(a[e][e], 9 * g);   // (j, j): lane 8 g + g
        // row j of the current matrix: columns 4 br + i (for the row factors) and
        // 4 bc + k (for the column factors)
        double vr[4], vc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = bpermute_f64(4 * (8 * g + br), a[e][i]);
#pragma unroll
        for (int k = 0; k < 4; ++k) vc[k] = bpermute_f64(4 * (8 * g + bc), a[e][k]);
        badp |= !(piv0 > 0.0) & (o + j < nb);
        const double piv = piv0 > 0.0 ? piv0 : 1.0;
        // 1/sqrt(piv) from the hardware estimate and two Newton steps
        // y <- y + y (1/2 - (piv/2) y^2) (quadratic convergence to full double
        // precision), then sqrt(piv) = piv y: a short dependent chain in place of
        // a square root and a division
        double inv = __builtin_amdgcn_rsq(piv);
        const double hp = 0.5 * piv;
        inv = fma(inv, fma(-hp * inv, inv, 0.5), inv);
        inv = fma(inv, fma(-hp * inv, inv, 0.5), inv);
        const double rjj = piv * inv;
        if (lane == 0) rinv[o + j] = inv;
        // A[r][c] -= R_jr R_jc = (A_jr / piv) A_jc for r > j, c >= r: the row
        // factor is 0 for r <= j, so every lane updates its whole tile with plain
        // fmas (entries below the diagonal are never read back)
        const double inv2 = inv * inv;
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = (4 * br + i > j) ? vr[i] * inv2 : 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) a[i][k] = fma(-vr[i], vc[k], a[i][k]);
        // row j of R: R_jj = sqrt(piv), R_jc = A_jc / sqrt(piv) for c > j
        if (br == g) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int c = 4 * bc + k;
                const double v = a[e][k];
                a[e][k] = (c == j) ? rjj : ((c > j) ? v * inv : v);
            }
        }
    });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 4 * br + i, c = 4 * bc + k;
            if (c >= r) A[o + r][o + c] = a[i][k];
        }
    return badp;
}

// In one thread: b <- R^-T b for the 32 x 32 upper block R at (o, o) of A (its
// 1 / R_kk in rinv[o + k]), b in registers; forward substitution, R read by
// broadcast.
__device__ inline void solve32(const double (*R)[NBMAX + 1], const double *rinv, int o, double (&b)[SB])
{
    static_for<SB>([&](auto KK) {
        constexpr int k = decltype(KK)::value;
        b[k] *= rinv[o + k];
        static_for<SB - 1 - k>([&](auto JJ) {
            constexpr int j = k + 1 + decltype(JJ)::value;
            b[j] = fma(-R[o + k][o + j], b[k], b[j]);
        });
    });
}

__global__ __launch_bounds__(PNT) void potrf_diag_kernel(double *__restrict__ M, int64_t K, int64_t p0,
                                                        int nb, double *__restrict__ rinv_out, unsigned *status)
{
    __shared__ double A[NBMAX][NBMAX + 1];
    __shared__ double rinv[NBMAX];
    __shared__ int bad;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    {
        // every thread's loads are issued before any LDS store (clamped
        // addresses, selects after), so they overlap instead of round-tripping
        constexpr int PER = NBMAX * NBMAX / PNT;
        double v[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + PNT * m, r = e >> 7, c = e & 127;
            const bool in = r < nb && c < nb && c >= r;
            v[m] = M[in ? (p0 + r) * K + p0 + c : p0 * K + p0];
        }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + PNT * m, r = e >> 7, c = e & 127;
            const bool in = r < nb && c < nb && c >= r;
            A[r][c] = in ? v[m] : ((r == c) ? 1.0 : 0.0);
        }
    }
    if (t == 0) bad = 0;
    __syncthreads();

    const int ty = t >> 5, tx = t & 31;              // trailing mapping: 16 x 32 grid
#pragma unroll 1
    for (int s = 0; s < NBMAX / SB; ++s) {
        const int o = s * SB;
        if (wave == 0) {
            const bool b = wave_factor32(A, rinv, o, nb, lane);
            if (b && lane == 0) bad = 1;
        }
        __syncthreads();
        if (o + SB >= NBMAX) break;
        // strip: R[o.., c] = R_DD^-T A[o.., c], one column per thread
        if (t < NBMAX - o - SB) {
            const int c = o + SB + t;
            double b[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) b[k] = A[o + k][c];
            solve32(A, rinv, o, b);
#pragma unroll
            for (int k = 0; k < SB; ++k) A[o + k][c] = b[k];
        }
        __syncthreads();
        // trailing: A[r][c] -= sum_k R[o+k][r] R[o+k][c], r <= c in [o+32, 128)
        const int base = o + SB;
        double acc[6][3];
#pragma unroll
        for (int i = 0; i < 6; ++i)
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) acc[i][kk] = 0.0;
#pragma unroll 2
        for (int k = 0; k < SB; ++k) {
            double vr[6], vc[3];
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int r = base + ty + 16 * i;
                vr[i] = A[o + k][r < NBMAX ? r : NBMAX - 1];
            }
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                const int c2 = base + tx + 32 * kk;
                vc[kk] = A[o + k][c2 < NBMAX ? c2 : NBMAX - 1];
            }
#pragma unroll
            for (int i = 0; i < 6; ++i)
#pragma unroll
                for (int kk = 0; kk < 3; ++kk) acc[i][kk] += vr[i] * vc[kk];
        }
#pragma unroll
        for (int i = 0; i < 6; ++i)
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                const int r = base + ty + 16 * i, c2 = base + tx + 32 * kk;
                if (r < NBMAX && c2 < NBMAX && r <= c2) A[r][c2] -= acc[i][kk];
            }
        __syncthreads();
    }

    // R is final: write it (upper) and R^T (lower) back, and 1 / R_kk
    if (t < NBMAX) rinv_out[t] = rinv[t];
    for (int e = t; e < NBMAX * NBMAX; e += PNT) {
        const int r = e >> 7, c = e & 127;
        if (r < nb && c < nb) M[(p0 + r) * K + p0 + c] = (c >= r) ? A[r][c] : A[c][r];
    }
    if (t == 0 && bad) atomicOr(status, ST_NOT_PD);
}

// Y = R^-T B for the nb x nb upper block R at (p0, p0) of M (nb <= 128), by block
// forward substitution over its 32 x 32 diagonal sub-blocks:
//     Y_s = R_ss^-T (B_s - sum_{t < s} R_ts^T Y_t),
// the update as small products (thread (a, g): row a of the block, columns
// 8 g .. 8 g + 7), the diagonal solve by substitution in one thread per
// column with 1 / R_kk from rinv (which the diagonal kernel wrote).  One
// workgroup per 64 columns of B (nb x ncols, ld ldb), held in LDS.  Y goes to
// out (ld ldo; out may be B: each workgroup reads its columns before it writes
// them) and, with out_t set, transposed to out_t (out_t[c ldt + a] = Y[a][c]).
// Memory is read in batches, every load of a batch issued before any of its
// values is stored (clamped addresses, selects after): B's block once, and for
// each s the column strip R[0 .. 32 s + 31][32 s .. 32 s + 31] it needs, so a
// workgroup waits on memory five times rather than once per element it reads.
constexpr int TSC = 64;
constexpr int TST = 256;
__global__ __launch_bounds__(TST) void trsm_rt_kernel(const double *__restrict__ M, int64_t K, int64_t p0, int nb,
                                                      const double *__restrict__ rinv_in, const double *B,
                                                      int64_t ldb,
                                                      double *out, int64_t ldo, double *out_t, int64_t ldt,
                                                      int64_t ncols)
{
    __shared__ double Ys[NBMAX][TSC + 1];
    __shared__ double Rs[NBMAX][SB + 1];          // R[0 .. 32 s + 31][32 s .. 32 s + 31]
    __shared__ double rinv[NBMAX];
    const int t = threadIdx.x, a = t & 31, cg = t >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * TSC;
    const int nsb = (nb + SB - 1) / SB;
    {
        constexpr int PER = NBMAX * TSC / TST;
        double v[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + TST * m, r = e / TSC, c = e % TSC;
            const bool in = r < nb && c0 + c < ncols;
            v[m] = B[in ? r * ldb + c0 + c : 0];
        }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + TST * m, r = e / TSC, c = e % TSC;
            const bool in = r < nb && c0 + c < ncols;
            Ys[r][c] = in ? v[m] : 0.0;
        }
    }
    if (t < NBMAX) rinv[t] = rinv_in[t];
#pragma unroll 1
    for (int s = 0; s < nsb; ++s) {
        // the strip of R this block row needs: rows 0 .. 32 s + 31 of its 32
        // columns (the identity past nb); element (rr, aa) is m-th of thread t
        // for rr * SB + aa = t + TST m
        {
            constexpr int PER = NBMAX * SB / TST;
            const int rows = SB * (s + 1);
            double v[PER];
#pragma unroll
            for (int m = 0; m < PER; ++m) {
                const int e = t + TST * m, rr = e / SB, cc = SB * s + e % SB;
                const bool in = rr < rows && rr < nb && cc < nb;
                v[m] = M[in ? (p0 + rr) * K + p0 + cc : p0 * K + p0];
            }
#pragma unroll
            for (int m = 0; m < PER; ++m) {
                const int e = t + TST * m, rr = e / SB, cc = SB * s + e % SB;
                if (rr < rows) Rs[rr][e % SB] = (rr < nb && cc < nb) ? v[m] : (rr == cc ? 1.0 : 0.0);
            }
        }
        __syncthreads();
        double acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = Ys[SB * s + a][8 * cg + j];
#pragma unroll 4
        for (int k = 0; k < SB * s; ++k) {
            const double r = Rs[k][a];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = fma(-r, Ys[k][8 * cg + j], acc[j]);
        }
        // (the update reads rows of Ys before block s only)
#pragma unroll
        for (int j = 0; j < 8; ++j) Ys[SB * s + a][8 * cg + j] = acc[j];
        __syncthreads();
        if (t < TSC) {
            // b <- R_ss^-T b, R_ss = Rs[32 s + k][j]
            double b[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) b[k] = Ys[SB * s + k][t];
            static_for<SB>([&](auto KK) {
                constexpr int k = decltype(KK)::value;
                b[k] *= rinv[SB * s + k];
                static_for<SB - 1 - k>([&](auto JJ) {
                    constexpr int j = k + 1 + decltype(JJ)::value;
                    b[j] = fma(-Rs[SB * s + k][j], b[k], b[j]);
                });
            });
#pragma unroll
            for (int k = 0; k < SB; ++k) Ys[SB * s + k][t] = b[k];
        }
        __syncthreads();
    }
    for (int e = t; e < NBMAX * TSC; e += TST) {
        const int r = e / TSC, c = e % TSC;
        if (r < nb && c0 + c < ncols) out[r * ldo + c0 + c] = Ys[r][c];
    }
    if (out_t) {
        for (int e = t; e < NBMAX * TSC; e += TST) {
            const int c = e / NBMAX, r = e % NBMAX;
            if (r < nb && c0 + c < ncols) out_t[(c0 + c) * ldt + r] = Ys[r][c];
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
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(PNT), 0, s, M, K, p0, nb, rinv, status);
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
