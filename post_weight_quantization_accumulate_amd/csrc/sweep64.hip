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
// read the same addresses).  Column c: its value is broadcast from its owner
// lane to the quad by DPP; at a group's first column the quad combines the
// group's absolute maximum; every lane takes the same decision, and each lane
// applies the error to its own later columns.  The owner keeps the error in
// place of the value, and the block's errors are written k-major (E^T) for the
// block and group updates that follow.
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int S64_NT = 128;               // 2 waves
constexpr int S64_ROWS = 32;              // rows per workgroup
constexpr int S64_BW = kSweepBlock;       // 128
constexpr int S64_QP = 34;                // doubles from one quarter of a U row to the next
constexpr int S64_UP = 4 * S64_QP;        // doubles per U row in LDS
constexpr size_t kSweep64Lds = (size_t)S64_BW * S64_UP * sizeof(double);

// lane qc of each quad's value, to the whole quad (DPP quad_perm)
template <int qc> __device__ inline double quad_bcast64(double x)
{
    constexpr int ctrl = qc | (qc << 2) | (qc << 4) | (qc << 6);
    const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)b, ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

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

__global__ __launch_bounds__(S64_NT, 1) void sweep64_kernel(double *__restrict__ Wk, double *__restrict__ ET,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                            const double *__restrict__ U, int64_t N, int64_t K,
                                                            int64_t G, int64_t b0)
{
    extern __shared__ __attribute__((aligned(16))) double Us[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int q = lane & 3;                               // quarter of the block this lane holds
    const int64_t row = (int64_t)blockIdx.x * S64_ROWS + (tid >> 2);
    const bool rv = row < N;
    const int64_t bw = (K - b0) < S64_BW ? (K - b0) : S64_BW;
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

    unsigned cw[4] = {0u, 0u, 0u, 0u};                 // this lane's 32 codes, two per byte
    float s = 1.0f, y = 0.0f, f = 1.0f;                 // the group's scale, 1 / (s f) and guard factor
    const double *urow_base = Us + q * S64_QP;
    auto column = [&](auto I) {
        constexpr int c = decltype(I)::value;
        constexpr int qc = c / 32, t = c % 32;
        if (c >= bw) return;
        const double wi = quad_bcast64<qc>(w[t]);
        if ((c & (G - 1)) == 0) {
            // the group's scale from its current values: s = fl32(fl32(absmax) / 7)
            double m = 0.0;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int col = 32 * q + j;
                m = (col >= c && col < c + G) ? fmax(m, fabs(w[j])) : m;
            }
            m = fmax(m, __shfl_xor(m, 1, 4));
            m = fmax(m, __shfl_xor(m, 2, 4));
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
        const double e = fma(-(double)code, (double)s, wi) / Us[c * S64_UP + qc * S64_QP + t];
        // later columns of this lane: all of them for a later quarter, those
        // past t for the column's own quarter, none for an earlier one
        const bool later = q > qc, from = q >= qc;
        const double *ur = urow_base + c * S64_UP;
#pragma unroll
        for (int j = 0; j < 32; j += 2) {
            const double2 u = *(const double2 *)(ur + j);
            const bool p0 = j > t ? from : later, p1 = j + 1 > t ? from : later;
            w[j] = p0 ? fma(-e, u.x, w[j]) : w[j];
            w[j + 1] = p1 ? fma(-e, u.y, w[j + 1]) : w[j + 1];
        }
        const bool own = q == qc;
        w[t] = own ? e : w[t];
        cw[t / 8] |= own ? nib << (4 * (t % 8)) : 0u;
    };
    static_for<S64_BW>(column);

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

hipError_t launch_sweep64_block(double *Wk, double *ET, uint8_t *codes, float *scales, const double *U, int64_t N,
                                int64_t K, int64_t G, int64_t b0, hipStream_t s)
{
    if (N <= 0 || b0 < 0 || b0 >= K || G < 1 || G > S64_BW || (G & (G - 1)) != 0 || K % G != 0 || (K & 1))
        return hipErrorInvalidValue;
    static const bool lds_ok = hipFuncSetAttribute((const void *)sweep64_kernel,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)kSweep64Lds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int64_t grid = (N + S64_ROWS - 1) / S64_ROWS;
    hipLaunchKernelGGL(sweep64_kernel, dim3((unsigned)grid), dim3(S64_NT), kSweep64Lds, s, Wk, ET, codes, scales, U,
                       N, K, G, b0);
    return hipGetLastError();
}

}  // namespace gq
