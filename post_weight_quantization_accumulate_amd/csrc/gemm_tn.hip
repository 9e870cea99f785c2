// gemm_tn.hip -- matrix-core GEMM C = alpha * A^T B + beta * Cin for the dense
// contractions of the path, with both operands "k-major" (row k of A holds a run
// of output rows, row k of B a run of output columns).
//
// Every contraction of the path has that shape without any transposition:
//   * the Gram matrix X^T X (rows of X are tokens),
//   * products of symmetric matrices X Y = X^T Y (the sign iteration),
//   * the upper Cholesky trailing update R^T R over a panel's rows,
//   * the triangular-inverse updates, and
//   * the GPTQ lazy-block update E U[blk, :] with E stored transposed.
// So operands stream from HBM with contiguous 16-byte loads straight into an LDS
// layout [k][m] from which each MFMA lane reads its element at a fixed k row:
// a whole wave reads contiguous LDS words, free of bank conflicts.
//
// Tiles are 128 x 128 per 256-thread workgroup (2 x 2 waves of 64 x 64), k in
// stages of 16 rows, LDS double-buffered so the global loads of stage k+1 are in
// flight while the matrix cores work on stage k.
//   fp32: v_mfma_f32_32x32x2f32, 2 x 2 blocks of 32 x 32 per wave.
//   fp64: v_mfma_f64_16x16x4f64, 4 x 4 blocks of 16 x 16 per wave.
#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16, NT = 256;

template <typename T> struct Mfma;

template <> struct Mfma<float> {
    static constexpr int BLK = 32;          // output block edge of one instruction
    static constexpr int NB = 64 / BLK;     // blocks per wave edge
    static constexpr int KSTEP = 2;         // k consumed per instruction
    static constexpr int LPK = 32;          // lanes per k row: lane -> (k = l / 32, m = l % 32)
    static constexpr int NACC = 16;
    typedef f32x16 acc_t;
    __device__ static acc_t mma(float a, float b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // accumulator element r of lane -> (row, col) inside the 32 x 32 block
    __device__ static int row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
    __device__ static int col(int lane, int) { return lane & 31; }
};

template <> struct Mfma<double> {
    static constexpr int BLK = 16;
    static constexpr int NB = 64 / BLK;
    static constexpr int KSTEP = 4;
    static constexpr int LPK = 16;          // lane -> (k = l / 16, m = l % 16)
    static constexpr int NACC = 4;
    typedef f64x4 acc_t;
    __device__ static acc_t mma(double a, double b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // the fp64 instruction interleaves rows across lane groups: element r of
    // lane l is row l/16 + 4 r (unlike the 4 (l/16) + r of the fp32 16x16 shapes)
    __device__ static int row(int lane, int r) { return (lane >> 4) + 4 * r; }
    __device__ static int col(int lane, int) { return lane & 15; }
};

__device__ inline double ipow(double x, int p)
{
    double r = 1.0;
    for (int i = 0; i < p; ++i) r *= x;
    return r;
}

// Linear index of a lower-triangular tile list -> (ti >= tj).
__device__ inline void tri_index(int64_t id, int64_t &ti, int64_t &tj)
{
    int64_t t = (int64_t)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
    while (t * (t + 1) / 2 > id) --t;
    while ((t + 1) * (t + 2) / 2 <= id) ++t;
    ti = t;
    tj = id - t * (t + 1) / 2;
}

template <typename T, typename OutT>
__global__ __launch_bounds__(NT) void gemm_tn_kernel(GemmDesc d, int64_t tiles_n, int vecA, int vecB)
{
    using MF = Mfma<T>;
    constexpr int V = 16 / (int)sizeof(T);          // elements per 16-byte vector
    constexpr int LDP = BM + V;                      // padded LDS row (elements)
    constexpr int VPR = BM / V;                      // vectors per tile row
    constexpr int NV = BK * VPR / NT;                // vectors per thread per operand
    typedef T vec_t __attribute__((ext_vector_type(V)));

    __shared__ __attribute__((aligned(16))) T As[2][BK][LDP];
    __shared__ __attribute__((aligned(16))) T Bs[2][BK][LDP];

    int64_t ti, tj;
    const int64_t bid = blockIdx.x;
    if (d.mode == TILE_RECT) {
        ti = bid / tiles_n;
        tj = bid % tiles_n;
    } else {
        tri_index(bid, ti, tj);
        if (d.mode == TILE_UPPER) { int64_t t = ti; ti = tj; tj = t; }
    }
    const int64_t i0 = ti * BM, j0 = tj * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const T *A = (const T *)d.A;
    const T *B = (const T *)d.B;

    vec_t ra[NV], rb[NV];
    auto gload = [&](int64_t kb) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int lin = tid + NT * v;
            const int kr = lin / VPR;
            const int cc = (lin % VPR) * V;
            const int64_t k = kb + kr;
            const int64_t gi = i0 + cc, gj = j0 + cc;
            if (k < d.Kd && vecA && gi + V <= d.M) {
                ra[v] = *(const vec_t *)(A + k * d.lda + gi);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    ra[v][e] = (k < d.Kd && gi + e < d.M) ? A[k * d.lda + gi + e] : (T)0;
            }
            if (k < d.Kd && vecB && gj + V <= d.N) {
                rb[v] = *(const vec_t *)(B + k * d.ldb + gj);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    rb[v][e] = (k < d.Kd && gj + e < d.N) ? B[k * d.ldb + gj + e] : (T)0;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int lin = tid + NT * v;
            const int kr = lin / VPR;
            const int cc = (lin % VPR) * V;
            *(vec_t *)&As[buf][kr][cc] = ra[v];
            *(vec_t *)&Bs[buf][kr][cc] = rb[v];
        }
    };

    typename MF::acc_t acc[MF::NB][MF::NB];
#pragma unroll
    for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
            for (int r = 0; r < MF::NACC; ++r) acc[bi][bj][r] = (T)0;

    const int64_t nk = (d.Kd + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int buf = (int)(kt & 1);
            if (kt + 1 < nk) gload((kt + 1) * BK);
            const int m = lane % MF::LPK;
#pragma unroll
            for (int kk = 0; kk < BK; kk += MF::KSTEP) {
                const int kr = kk + lane / MF::LPK;
                T a[MF::NB], b[MF::NB];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi) a[bi] = As[buf][kr][wr * 64 + bi * MF::BLK + m];
#pragma unroll
                for (int bj = 0; bj < MF::NB; ++bj) b[bj] = Bs[buf][kr][wc * 64 + bj * MF::BLK + m];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < MF::NB; ++bj) acc[bi][bj] = MF::mma(a[bi], b[bj], acc[bi][bj]);
            }
            if (kt + 1 < nk) sstore(buf ^ 1);
            __syncthreads();
        }
    }

    double alpha = d.alpha, beta = d.beta;
    if (d.alpha_dev) alpha *= ipow(*d.alpha_dev, d.alpha_pow);
    if (d.beta_dev) beta *= ipow(*d.beta_dev, d.beta_pow);
    OutT *out = (OutT *)d.out;
    OutT *out_t = (OutT *)d.out_t;
    const T *cin = (const T *)d.cin;
#pragma unroll
    for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
            for (int r = 0; r < MF::NACC; ++r) {
                const int64_t gi = i0 + wr * 64 + bi * MF::BLK + MF::row(lane, r);
                const int64_t gj = j0 + wc * 64 + bj * MF::BLK + MF::col(lane, r);
                if (gi >= d.M || gj >= d.N) continue;
                if (d.tri == 1 && gi < gj) continue;
                if (d.tri == 2 && gi > gj) continue;
                double v = alpha * (double)acc[bi][bj][r];
                if (beta != 0.0) v += beta * (double)cin[gi * d.ldc + gj];
                out[gi * d.ldo + gj] = (OutT)v;
                if (out_t) out_t[gj * d.ldo + gi] = (OutT)v;
            }
}

template <typename T, typename OutT>
hipError_t launch(const GemmDesc &d, hipStream_t s)
{
    if (d.M <= 0 || d.N <= 0) return hipSuccess;
    constexpr int V = 16 / (int)sizeof(T);
    const int64_t tm = (d.M + BM - 1) / BM, tn = (d.N + BN - 1) / BN;
    int64_t ntiles;
    if (d.mode == TILE_RECT) {
        ntiles = tm * tn;
    } else {
        if (d.M != d.N) return hipErrorInvalidValue;
        ntiles = tm * (tm + 1) / 2;
    }
    const int vecA = (d.lda % V == 0) && (((uintptr_t)d.A & 15) == 0);
    const int vecB = (d.ldb % V == 0) && (((uintptr_t)d.B & 15) == 0);
    hipLaunchKernelGGL((gemm_tn_kernel<T, OutT>), dim3((unsigned)ntiles), dim3(NT), 0, s, d, tn,
                       vecA, vecB);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_tn_f32(const GemmDesc &d, hipStream_t s) { return launch<float, float>(d, s); }
hipError_t gemm_tn_f64(const GemmDesc &d, hipStream_t s) { return launch<double, double>(d, s); }
hipError_t gemm_tn_f64_out_f32(const GemmDesc &d, hipStream_t s) { return launch<double, float>(d, s); }

}  // namespace gq
