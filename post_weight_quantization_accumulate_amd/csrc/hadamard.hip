// hadamard.hip -- block Walsh-Hadamard rotation of weights and Hessians.
//
// The rotation composed with GPTQ (ork-driver wiki, "Exp 2026-08-18 GPTQ Int4":
// GPTQ composes with a Hadamard rotation, rotate then quantise, as in QuaRot):
// R = blockdiag(H_b, ..., H_b) D / sqrt(b) over the K input channels, H_b the
// Sylvester Hadamard matrix of order b (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]),
// D = diag(signs).  R is orthogonal, so rotating the weights (W' = W R^T) and the
// activations (X' = X R^T) leaves every output W X^T unchanged, and the Hessian
// of the rotated activations is H' = R H R^T.
//
// fwht_rows_kernel: the matrix, row r at A + r ld, is a sequence of segments of b
// consecutive columns (b divides K, so no segment straddles rows).  A workgroup
// takes E = max(b, 1024) elements -- E / b consecutive segments -- into LDS with
// the signs applied, runs the log2(b) butterfly stages (pair (i, i + h) of each
// segment becomes (x_i + x_j, x_i - x_j)), and writes them back scaled by
// 1/sqrt(b).  HBM-bound: one read and one write of the matrix.
#include "gq.h"
#include "gq_internal.h"

#include <cmath>

namespace gq {
namespace {

constexpr int HT = 256;              // threads per workgroup
constexpr int kMaxBlock = 4096;      // largest block order (16 elements per thread)

__global__ __launch_bounds__(HT) void fwht_rows_kernel(float *__restrict__ A, int64_t rows, int64_t K, int64_t ld,
                                                       int b, int E, const float *__restrict__ signs, float scale)
{
    __shared__ float x[kMaxBlock];
    const int64_t seg_per_row = K / b;
    const int64_t nseg = rows * seg_per_row;
    const int64_t seg0 = (int64_t)blockIdx.x * (E / b);
    // element e of the workgroup: segment seg0 + e / b, offset e % b
    auto addr = [&](int e, int64_t &col) -> float * {
        const int64_t g = seg0 + e / b;
        const int64_t r = g / seg_per_row;
        col = (g - r * seg_per_row) * b + e % b;
        return A + r * ld + col;
    };
    for (int e = threadIdx.x; e < E; e += HT) {
        float v = 0.0f;
        if (seg0 + e / b < nseg) {
            int64_t col;
            const float *p = addr(e, col);
            v = *p;
            if (signs) v *= signs[col];
        }
        x[e] = v;
    }
    __syncthreads();
    const int lb = __builtin_ctz(b);                 // b and h are powers of two
    for (int h = 1, lh = 0; h < b; h <<= 1, ++lh) {
        for (int q = threadIdx.x; q < E / 2; q += HT) {
            const int qq = q & ((b >> 1) - 1);
            const int i = ((q >> (lb - 1)) << lb) + ((qq >> lh) << (lh + 1)) + (qq & (h - 1)), j = i + h;
            const float u = x[i], v = x[j];
            x[i] = u + v;
            x[j] = u - v;
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < E; e += HT) {
        if (seg0 + e / b < nseg) {
            int64_t col;
            *addr(e, col) = x[e] * scale;
        }
    }
}

// The same transform for b >= 16 with K, ld and both matrices 16-byte aligned:
// thread t owns the P = E / 256 consecutive elements t P .. t P + P - 1 of the
// workgroup's E, all in one segment, loaded and stored as 16-byte vectors with
// one address computation per thread; the stages h < P (pairs inside a thread)
// run in registers, the rest through LDS.  It reads src and writes A (the same
// matrix for the in-place rotation; a thread stores only what it loaded).
template <int P>
__global__ __launch_bounds__(HT) void fwht_rows_vec_kernel(float *A, const float *src, int64_t rows, int64_t K,
                                                           int64_t ld, int b, const float *__restrict__ signs,
                                                           float scale)
{
    __shared__ float x[HT * P];
    constexpr int E = HT * P;
    const int64_t seg_per_row = K / b;
    const int64_t nseg = rows * seg_per_row;
    const int e0 = threadIdx.x * P;
    const int64_t g = (int64_t)blockIdx.x * (E / b) + e0 / b;    // this thread's segment
    const bool valid = g < nseg;
    const int64_t r = valid ? g / seg_per_row : 0;
    const int64_t col = valid ? (g - r * seg_per_row) * b + e0 % b : 0;
    float v[P];
    if (valid) {
#pragma unroll
        for (int u = 0; u < P; u += 4) {
            const float4 q = *(const float4 *)(src + r * ld + col + u);
            v[u] = q.x; v[u + 1] = q.y; v[u + 2] = q.z; v[u + 3] = q.w;
        }
        if (signs) {
#pragma unroll
            for (int u = 0; u < P; u += 4) {
                const float4 q = *(const float4 *)(signs + col + u);
                v[u] *= q.x; v[u + 1] *= q.y; v[u + 2] *= q.z; v[u + 3] *= q.w;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < P; ++u) v[u] = 0.0f;
    }
#pragma unroll
    for (int h = 1; h < P; h <<= 1)
#pragma unroll
        for (int u = 0; u < P; ++u)
            if ((u & h) == 0) {
                const float a = v[u], c = v[u + h];
                v[u] = a + c;
                v[u + h] = a - c;
            }
    if (b > P) {
#pragma unroll
        for (int u = 0; u < P; ++u) x[e0 + u] = v[u];
        __syncthreads();
        const int lb = __builtin_ctz(b);             // b and h are powers of two
        for (int h = P, lh = __builtin_ctz(P); h < b; h <<= 1, ++lh) {
#pragma unroll
            for (int k = 0; k < E / 2 / HT; ++k) {
                const int q = threadIdx.x + k * HT;
                const int qq = q & ((b >> 1) - 1);
                const int i = ((q >> (lb - 1)) << lb) + ((qq >> lh) << (lh + 1)) + (qq & (h - 1)), j = i + h;
                const float a = x[i], c = x[j];
                x[i] = a + c;
                x[j] = a - c;
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < P; ++u) v[u] = x[e0 + u];
    }
    if (valid) {
#pragma unroll
        for (int u = 0; u < P; u += 4)
            *(float4 *)(A + r * ld + col + u) = make_float4(v[u] * scale, v[u + 1] * scale, v[u + 2] * scale,
                                                            v[u + 3] * scale);
    }
}

// out[c][r] = in[r][c] for a K x K matrix (row stride K), 64 x 64 tiles.
__global__ __launch_bounds__(HT) void transpose_kernel(float *__restrict__ out, const float *__restrict__ in, int64_t K)
{
    __shared__ float t[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += HT / 64)
        if (r0 + r < K && c0 + tx < K) t[r][tx] = in[(r0 + r) * K + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += HT / 64)
        if (c0 + c < K && r0 + tx < K) out[(c0 + c) * K + r0 + tx] = t[tx][c];
}

}  // namespace

bool hadamard_block_ok(int64_t K, int64_t b)
{
    return b >= 1 && b <= kMaxBlock && (b & (b - 1)) == 0 && K % b == 0;
}

hipError_t launch_fwht_rows(float *A, int64_t rows, int64_t K, int64_t ld, int64_t b, const float *signs,
                            hipStream_t s, const float *src)
{
    if (rows <= 0 || K <= 0) return hipSuccess;
    if (!hadamard_block_ok(K, b) || ld < K) return hipErrorInvalidValue;
    const float scale = (float)(1.0 / std::sqrt((double)b));
    const bool vec = b >= 16 && K % 4 == 0 && ld % 4 == 0 && ((uintptr_t)A & 15) == 0 &&
                     ((uintptr_t)signs & 15) == 0 && ((uintptr_t)src & 15) == 0;
    // the vector kernel takes 16 elements per thread (4096 per workgroup): the
    // first four butterfly stages stay in registers; the generic one 1024
    const int E = vec ? 4096 : (b > 1024 ? (int)b : 1024);
    const int64_t nseg = rows * (K / b), per = E / b;
    const int64_t nwg = (nseg + per - 1) / per;
    if (src && !vec) return hipErrorInvalidValue;     // out of place: the vector kernel only
    if (!src) src = A;
    if (vec)
        hipLaunchKernelGGL(fwht_rows_vec_kernel<16>, dim3((unsigned)nwg), dim3(HT), 0, s, A, src, rows, K, ld, (int)b,
                           signs, scale);
    else
        hipLaunchKernelGGL(fwht_rows_kernel, dim3((unsigned)nwg), dim3(HT), 0, s, A, rows, K, ld, (int)b, E, signs,
                           scale);
    return hipGetLastError();
}

hipError_t launch_transpose(float *out, const float *in, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    const unsigned nt = (unsigned)((K + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, dim3(nt, nt), dim3(HT), 0, s, out, in, K);
    return hipGetLastError();
}

}  // namespace gq
