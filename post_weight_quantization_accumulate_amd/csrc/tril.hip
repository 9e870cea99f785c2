// tril.hip -- the Bf16TrilDiagF32 Hessian storage layout (hipfire-calib-data,
// "Hessian storage: Bf16TrilDiagF32 (quant_type 130)"):
//   K little-endian f32 words: the exact diagonal;
//   K*(K-1)/2 little-endian u16 words: word i*(i-1)/2 + j (i > j) holds the top
//   half of the f32 bit pattern of H[i][j] (truncation, bits >> 16), mirrored on
//   read.
// Pure bit movement, bound by HBM.  Pack reads only the lower triangle, one
// workgroup per row, so every read and write is a contiguous run.  Unpack works
// on 64 x 64 tiles of the lower triangle and writes each tile twice: as is
// (rows of H) and transposed through LDS (the mirrored upper triangle), so both
// stores stay row-contiguous.
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

}  // namespace

hipError_t launch_tril_pack(uint8_t *blob, const float *H, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    hipLaunchKernelGGL(tril_pack_kernel, dim3((unsigned)K), dim3(256), 0, s, blob, H, K);
    return hipGetLastError();
}

hipError_t launch_tril_unpack(float *H, const uint8_t *blob, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    const int64_t nt = (K + TU - 1) / TU;
    hipLaunchKernelGGL(tril_unpack_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, s, H,
                       blob, K);
    return hipGetLastError();
}

}  // namespace gq
