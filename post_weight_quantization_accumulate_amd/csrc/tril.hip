// tril.hip -- the Bf16TrilDiagF32 Hessian storage layout (hipfire-calib-data,
// "Hessian storage: Bf16TrilDiagF32 (quant_type 130)"):
//   K little-endian f32 words: the exact diagonal;
//   K*(K-1)/2 little-endian u16 words: word i*(i-1)/2 + j (i > j) holds the top
//   half of the f32 bit pattern of H[i][j] (truncation, bits >> 16), mirrored on
//   read.
// Pure bit movement, bound by HBM.  Pack takes one row per workgroup, writes its
// diagonal word and its packed words, in 16-byte stores where they fill an
// aligned 16-byte chunk.  Unpack works on 64 x 64 tiles of the lower triangle and writes
// each tile twice, 16 bytes per store: as is (rows of H) and transposed through
// LDS (the mirrored upper triangle).
#include <algorithm>

#include "gq_internal.h"

namespace gq {
namespace {

__global__ __launch_bounds__(256) void tril_pack_kernel(uint8_t *__restrict__ blob,
                                                       const float *__restrict__ H, int64_t K)
{
    const int64_t i = blockIdx.x;
    const float *row = H + i * K;
    uint32_t *diag = (uint32_t *)blob;
    uint16_t *tril = (uint16_t *)(blob + 4 * K);
    const int64_t base = i * (i - 1) / 2;
    for (int64_t j = threadIdx.x; j <= i; j += blockDim.x) {
        const uint32_t u = __float_as_uint(row[j]);
        if (j == i) diag[i] = u;
        else tril[base + j] = (uint16_t)(u >> 16);
    }
}

// One workgroup per row i >= 1: the row's packed words [b, b + i), b = i (i - 1) / 2,
// are cut at 16-byte boundaries of the blob; a thread takes one 8-word chunk,
// reads its floats (consecutive lanes, consecutive floats) and writes the chunk
// with one 16-byte store, or word by word where the chunk is shared with the
// neighbouring rows (at most the first and the last).  The triangle starts 4K
// bytes into a 16-byte aligned blob, so chunks are 16-byte aligned when
// K % 4 == 0 (the caller checks).
__global__ __launch_bounds__(256) void tril_pack8_kernel(uint8_t *__restrict__ blob, const float *__restrict__ H,
                                                        int64_t K)
{
    const int64_t i = blockIdx.x + 1;
    uint16_t *tril = (uint16_t *)(blob + 4 * K);
    const float *row = H + i * K;
    // the exact diagonal (row 1's workgroup also writes row 0's)
    if (threadIdx.x == 0) ((uint32_t *)blob)[i] = __float_as_uint(row[i]);
    if (i == 1 && threadIdx.x == 1) ((uint32_t *)blob)[0] = __float_as_uint(H[0]);
    const int64_t b = i * (i - 1) / 2, e = b + i;
    const int64_t k0 = b / 8, k1 = (e + 7) / 8;
    for (int64_t k = k0 + threadIdx.x; k < k1; k += blockDim.x) {
        const int64_t w0 = 8 * k;
        if (w0 >= b && w0 + 8 <= e) {
            const float *src = row + (w0 - b);
            unsigned v[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = __float_as_uint(src[x]) >> 16;
            uint4 q;
            q.x = v[0] | (v[1] << 16);
            q.y = v[2] | (v[3] << 16);
            q.z = v[4] | (v[5] << 16);
            q.w = v[6] | (v[7] << 16);
            *(uint4 *)(tril + w0) = q;
        } else {
            for (int64_t w = (w0 > b ? w0 : b); w < w0 + 8 && w < e; ++w)
                tril[w] = (uint16_t)(__float_as_uint(row[w - b]) >> 16);
        }
    }
}

__global__ __launch_bounds__(256) void tril_diag_kernel(uint8_t *__restrict__ blob, const float *__restrict__ H,
                                                       int64_t K)
{
    uint32_t *diag = (uint32_t *)blob;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < K; i += (int64_t)gridDim.x * blockDim.x)
        diag[i] = __float_as_uint(H[i * K + i]);
}

constexpr int TU = 64;

__device__ inline void tri_index(int64_t id, int64_t &ti, int64_t &tj)
{
    int64_t t = (int64_t)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
    while (t * (t + 1) / 2 > id) --t;
    while ((t + 1) * (t + 2) / 2 <= id) ++t;
    ti = t;
    tj = id - t * (t + 1) / 2;
}

__global__ __launch_bounds__(256) void tril_unpack_kernel(float *__restrict__ H,
                                                         const uint8_t *__restrict__ blob, int64_t K)
{
    __shared__ float tile[TU][TU + 1];
    int64_t ti, tj;
    tri_index(blockIdx.x, ti, tj);
    const int64_t i0 = ti * TU, j0 = tj * TU;
    const uint32_t *diag = (const uint32_t *)blob;
    const uint16_t *tril = (const uint16_t *)(blob + 4 * K);
    const int c = threadIdx.x & 63;      // column within the tile
    const int r0 = threadIdx.x >> 6;     // 0..3
    // lower part (and diagonal) of the tile, row by row
    for (int r = r0; r < TU; r += 4) {
        const int64_t i = i0 + r, j = j0 + c;
        float v = 0.0f;
        if (i < K && j < K && j <= i) {
            v = (j == i) ? __uint_as_float(diag[i]) : __uint_as_float((uint32_t)tril[i * (i - 1) / 2 + j] << 16);
            H[i * K + j] = v;
        }
        tile[r][c] = v;
    }
    __syncthreads();
    // mirrored upper part: H[j][i] = tile[i - i0][j - j0] for j < i
    for (int r = r0; r < TU; r += 4) {
        const int64_t j = j0 + r, i = i0 + c;
        if (i < K && j < K && j < i) H[j * K + i] = tile[c][r];
    }
}

// As tril_unpack_kernel with float4 stores (K % 4 == 0, 16-byte aligned H):
// thread t of a tile takes columns 4 (t % 16) .. + 3 of rows t / 16 + 16 k.
__global__ __launch_bounds__(256) void tril_unpack4_kernel(float *__restrict__ H, const uint8_t *__restrict__ blob,
                                                          int64_t K)
{
    __shared__ float tile[TU][TU + 1];
    int64_t ti, tj;
    tri_index(blockIdx.x, ti, tj);
    const int64_t i0 = ti * TU, j0 = tj * TU;
    const uint32_t *diag = (const uint32_t *)blob;
    const uint16_t *tril = (const uint16_t *)(blob + 4 * K);
    const int c4 = 4 * (threadIdx.x & 15);
    const int rq = threadIdx.x >> 4;      // 0..15
    // lower part (and diagonal) of the tile, row by row.  Every value the
    // thread needs is loaded first, from clamped addresses, so it waits on
    // memory once rather than once per element.
    uint16_t tv[TU / 16][4];
    uint32_t dv[TU / 16];
#pragma unroll
    for (int k = 0; k < TU / 16; ++k) {
        const int64_t i = i0 + rq + 16 * k;
        dv[k] = diag[i < K ? i : 0];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int64_t j = j0 + c4 + x;
            tv[k][x] = tril[(i < K && j < i) ? i * (i - 1) / 2 + j : 0];
        }
    }
#pragma unroll
    for (int k = 0; k < TU / 16; ++k) {
        const int r = rq + 16 * k;
        const int64_t i = i0 + r;
        float v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int64_t j = j0 + c4 + x;
            float f = 0.0f;
            if (i < K && j < i) f = __uint_as_float((uint32_t)tv[k][x] << 16);
            else if (i < K && j == i) f = __uint_as_float(dv[k]);
            v[x] = f;
            tile[r][c4 + x] = f;
        }
        const int64_t j = j0 + c4;
        if (i < K && j < K) {
            if (j + 3 <= i) {
                *(float4 *)(H + i * K + j) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                for (int x = 0; x < 4 && j + x <= i; ++x) H[i * K + j + x] = v[x];
            }
        }
    }
    __syncthreads();
    // mirrored upper part: H[j][i] = tile[i - i0][j - j0] for j < i
#pragma unroll
    for (int k = 0; k < TU / 16; ++k) {
        const int r = rq + 16 * k;
        const int64_t j = j0 + r, i = i0 + c4;
        if (j < K && i < K) {
            if (i > j) {
                *(float4 *)(H + j * K + i) = make_float4(tile[c4][r], tile[c4 + 1][r], tile[c4 + 2][r], tile[c4 + 3][r]);
            } else {
                for (int x = 0; x < 4; ++x)
                    if (i + x > j) H[j * K + i + x] = tile[c4 + x][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_tril_pack(uint8_t *blob, const float *H, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    if (K % 4 == 0 && ((uintptr_t)blob & 15) == 0) {
        if (K > 1)
            hipLaunchKernelGGL(tril_pack8_kernel, dim3((unsigned)(K - 1)), dim3(256), 0, s, blob, H, K);
        else
            hipLaunchKernelGGL(tril_diag_kernel, dim3(1), dim3(256), 0, s, blob, H, K);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(tril_pack_kernel, dim3((unsigned)K), dim3(256), 0, s, blob, H, K);
    return hipGetLastError();
}

hipError_t launch_tril_unpack(float *H, const uint8_t *blob, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    const int64_t nt = (K + TU - 1) / TU;
    if (K % 4 == 0 && ((uintptr_t)H & 15) == 0)
        hipLaunchKernelGGL(tril_unpack4_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, s, H, blob, K);
    else
        hipLaunchKernelGGL(tril_unpack_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, s, H, blob, K);
    return hipGetLastError();
}

}  // namespace gq
