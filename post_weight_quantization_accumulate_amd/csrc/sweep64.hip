// sweep64.hip -- the GPTQ error-feedback sweep with its state in fp64 (ork-driver
// wiki, "Exp 2026-08-18 GPTQ Int4": the column-sequential error-feedback sweep
// over the upper Cholesky factor U of H^-1).
//
// The fp32 sweep (gptq.hip) keeps U and the working weights in fp32.  Over long
// rows its trajectory drifts from an fp64 one by enough to decide a few rounding
// ties the other way (at K = 17408 about one per 37 rows), and each such flip
// changes the later codes of its row.  This path keeps U, the working weights
// and the errors in fp64, and the block updates run on the fp64 matrix cores;
// the rounding decisions stay in fp32 (the code of a value is taken from its
// fp32 rounding, divided by the fp32 scale), as in the fp32 sweep.  It serves
// the plain int4 grid with dynamic groups.
//
// One lazy block of 128 columns per launch.  Four lanes per row, each holding
// 32 consecutive columns of the block in registers (lane q of a row's quad
// holds columns 32 q .. 32 q + 31); 16 rows per wave, 32 per workgroup.  U's
// diagonal block sits in LDS, each row as four quarters of 32 values 34 apart
// (the quarters a quad reads fall on different banks; the 16 quads of a wave
// read the same addresses), with the reciprocals of its diagonal.  Column c:
// its value goes from its owner lane to the quad by a lane shuffle; at a
// group's first column the quad combines the group's absolute maximum; every
// lane takes the same decision, and each lane applies the error to its own
// later columns.  The owner keeps the error in place of the value, and the
// block's errors are written k-major (E^T) for the block and group updates
// that follow.  One unrolled body of 32 columns serves the four quarters, so
// the kernel's code stays within the instruction cache.
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int S64_NT = 128;               // 2 waves
constexpr int S64_ROWS = 32;              // rows per workgroup
constexpr int S64_BW = kSweepBlock;       // 128
constexpr int S64_QP = 34;                // doubles from one quarter of a U row to the next
constexpr int S64_UP = 4 * S64_QP;        // doubles per U row in LDS
constexpr size_t kSweep64Lds = ((size_t)S64_BW * S64_UP + S64_BW) * sizeof(double);

__global__ __launch_bounds__(256) void w64_kernel(double *__restrict__ dst, const float *__restrict__ src, int64_t n,
                                                  unsigned *status)
{
    bool bad = false;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = src[i];
        if (!isfinite(v)) bad = true;
        dst[i] = (double)v;
    }
    if (bad) atomicOr(status, ST_NONFINITE);
}

// U[i][j] = X[K-1-i][K-1-j] for i <= j, 0 below the diagonal (fp64)
__global__ __launch_bounds__(256) void flip64_kernel(double *__restrict__ U, const double *__restrict__ X, int64_t K)
{
    const int64_t n = K * K;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / K, j = e - i * K;
        U[e] = (i <= j) ? X[(K - 1 - i) * K + (K - 1 - j)] : 0.0;
    }
}

template <int LG>
__global__ __launch_bounds__(S64_NT, 1) void sweep64_kernel(double *__restrict__ Wk, double *__restrict__ ET,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                            const double *__restrict__ U, int64_t N, int64_t K,
                                                            int64_t b0)
{
    constexpr int G = 1 << LG;
    extern __shared__ __attribute__((aligned(16))) double Us[];
    double *rd = Us + S64_BW * S64_UP;                    // 1 / U_cc of the block's columns
    const int tid = threadIdx.x, lane = tid & 63;
    const int q = lane & 3;                               // quarter of the block this lane holds
    const int64_t row = (int64_t)blockIdx.x * S64_ROWS + (tid >> 2);
    const bool rv = row < N;
    const int bw = (int)((K - b0) < S64_BW ? (K - b0) : S64_BW);
    const int64_t ngroups = K / G;

    // U's diagonal block into LDS (zeros past bw), in pairs of values: each
    // thread loads a batch of 16 pairs before it stores any, so the loads are in
    // flight together (K is even and b0 a multiple of 128: 16-byte aligned)
    constexpr int kPairs = S64_BW * S64_BW / 2, kBatch = 16;
    static_assert(kPairs % (S64_NT * kBatch) == 0, "whole batches");
#pragma unroll 1
    for (int e0 = tid; e0 < kPairs; e0 += S64_NT * kBatch) {
        double2 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int e = e0 + b * S64_NT, r = e / (S64_BW / 2), c = 2 * (e % (S64_BW / 2));
            v[b] = (r < bw && c < bw) ? *(const double2 *)(U + (b0 + r) * K + b0 + c) : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int e = e0 + b * S64_NT, r = e / (S64_BW / 2), c = 2 * (e % (S64_BW / 2));
            *(double2 *)(Us + r * S64_UP + (c >> 5) * S64_QP + (c & 31)) = v[b];
        }
    }
    // this lane's 32 columns (zeros past bw and for rows past N)
    double w[32];
    {
        const double *src = Wk + (rv ? row : 0) * K + b0 + 32 * q;
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = (rv && 32 * q + j < bw) ? src[j] : 0.0;
    }
    __syncthreads();
    if (tid < bw) rd[tid] = 1.0 / Us[tid * S64_UP + (tid >> 5) * S64_QP + (tid & 31)];
    __syncthreads();

    unsigned cw[4] = {0u, 0u, 0u, 0u};                 // this lane's 32 codes, two per byte
    float s = 1.0f, y = 0.0f, f = 1.0f;                 // the group's scale, 1 / (s f) and guard factor
    const int qbase = lane & ~3;
    // One body of 32 columns serves the four quarters: quarter Q's column
    // c = 32 Q + t comes from lane Q of the quad.  Lanes of a later quarter
    // apply the error to all 32 of their columns, the owner to those past t, the
    // lanes of earlier quarters (whose columns hold errors by now) to none: the
    // error is zeroed per lane, so the body has no branch per column.
#pragma unroll 1
    for (int Q = 0; Q < 4 && 32 * Q < bw; ++Q) {
        const bool later = q > Q, from = q >= Q, own = q == Q;
        static_for<32>([&](auto I) {
            constexpr int t = decltype(I)::value;
            const int c = 32 * Q + t;
            if (c >= bw) return;
            const double wi = __shfl(w[t], qbase + Q, 64);
            bool start = false;
            if constexpr (G <= 32) start = (t % G) == 0;
            else start = t == 0 && (c & (G - 1)) == 0;
            if (start) {
                // the group's scale from its current values: s = fl32(fl32(absmax) / 7)
                double m = 0.0;
                if constexpr (G <= 32) {
                    // the group lies in the owner's columns t .. t + G - 1
#pragma unroll
                    for (int j = t; j < t + G && j < 32; ++j) m = fmax(m, fabs(w[j]));
                    m = __shfl(m, qbase + Q, 64);
                } else {
                    // quarters Q .. Q + G / 32 - 1, whole
                    const bool in = q >= Q && q < Q + G / 32;
#pragma unroll
                    for (int j = 0; j < 32; ++j) m = fmax(m, fabs(w[j]));
                    m = in ? m : 0.0;
                    m = fmax(m, __shfl_xor(m, 1, 4));
                    m = fmax(m, __shfl_xor(m, 2, 4));
                }
                const float sc = (float)m / 7.0f;
                if (q == 0 && rv) scales[row * ngroups + (b0 + c) / G] = sc;
                // A zero group takes the zero code (y = 0); a scale below 2^-60 is
                // scaled by f = 2^64 for the quotient, exactly, with the value, so
                // the correction step cannot underflow and 1/s cannot overflow.
                s = sc != 0.0f ? sc : 1.0f;
                f = sc < 0x1p-60f ? 0x1p64f : 1.0f;
                y = sc != 0.0f ? 1.0f / (s * f) : 0.0f;
            }
            // the code of fl32(wi) / s, the quotient correctly rounded by
            // Markstein's correction step from y = RN(1/s) (Markstein 1990)
            const float wq = (float)wi * f;
            const float q0 = wq * y;
            const float rr = fmaf(-(s * f), q0, wq);
            const float x = fmaf(rr, y, q0);
            const float code = fminf(fmaxf(rintf(x), -8.0f), 7.0f);
            const unsigned nib = (unsigned)(int)code & 0xFu;
            const double e = fma(-(double)code, (double)s, wi) * rd[c];
            const double e_to = from ? e : 0.0;          // columns past t
            const double e_at = later ? e : 0.0;         // columns up to t
            const double *ur = Us + c * S64_UP + q * S64_QP;
#pragma unroll
            for (int j = 0; j < 32; j += 2) {
                const double2 u = *(const double2 *)(ur + j);
                w[j] = fma(-(j > t ? e_to : e_at), u.x, w[j]);
                w[j + 1] = fma(-(j + 1 > t ? e_to : e_at), u.y, w[j + 1]);
            }
            w[t] = own ? e : w[t];
            cw[t / 8] |= own ? nib << (4 * (t % 8)) : 0u;
        });
    }

    if (!rv) return;
    // codes: two per byte, column 2m in the low nibble; this lane's 16 bytes
    uint8_t *crow = codes + row * (K / 2) + (b0 + 32 * q) / 2;
    if (32 * q + 32 <= bw && (((uintptr_t)crow & 3) == 0)) {
#pragma unroll
        for (int d = 0; d < 4; ++d) ((unsigned *)crow)[d] = cw[d];
    } else {
        for (int m = 0; m < 16; ++m)
            if (32 * q + 2 * m < bw) crow[m] = (uint8_t)(cw[m / 4] >> (8 * (m % 4)));
    }
    // errors, k-major: ET[k][row] for the block's columns k < bw
#pragma unroll
    for (int j = 0; j < 32; ++j)
        if (32 * q + j < bw) ET[(int64_t)(32 * q + j) * N + row] = w[j];
}

}  // namespace

hipError_t launch_w64(double *dst, const float *src, int64_t n, unsigned *status, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(w64_kernel, dim3((unsigned)g), dim3(256), 0, s, dst, src, n, status);
    return hipGetLastError();
}

hipError_t launch_flip64(double *U, const double *X, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    int64_t g = (K * K + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(flip64_kernel, dim3((unsigned)g), dim3(256), 0, s, U, X, K);
    return hipGetLastError();
}

template <int LG>
hipError_t launch_sweep64_lg(double *Wk, double *ET, uint8_t *codes, float *scales, const double *U, int64_t N,
                             int64_t K, int64_t b0, hipStream_t s)
{
    static const bool lds_ok = hipFuncSetAttribute((const void *)sweep64_kernel<LG>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)kSweep64Lds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int64_t grid = (N + S64_ROWS - 1) / S64_ROWS;
    hipLaunchKernelGGL(sweep64_kernel<LG>, dim3((unsigned)grid), dim3(S64_NT), kSweep64Lds, s, Wk, ET, codes, scales,
                       U, N, K, b0);
    return hipGetLastError();
}

hipError_t launch_sweep64_block(double *Wk, double *ET, uint8_t *codes, float *scales, const double *U, int64_t N,
                                int64_t K, int64_t G, int64_t b0, hipStream_t s)
{
    if (N <= 0 || b0 < 0 || b0 >= K || b0 % S64_BW != 0 || G < 1 || G > S64_BW || (G & (G - 1)) != 0 ||
        K % G != 0 || (K & 1))
        return hipErrorInvalidValue;
    switch (G) {
    case 1: return launch_sweep64_lg<0>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 2: return launch_sweep64_lg<1>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 4: return launch_sweep64_lg<2>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 8: return launch_sweep64_lg<3>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 16: return launch_sweep64_lg<4>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 32: return launch_sweep64_lg<5>(Wk, ET, codes, scales, U, N, K, b0, s);
    case 64: return launch_sweep64_lg<6>(Wk, ET, codes, scales, U, N, K, b0, s);
    default: return launch_sweep64_lg<7>(Wk, ET, codes, scales, U, N, K, b0, s);
    }
}

}  // namespace gq
