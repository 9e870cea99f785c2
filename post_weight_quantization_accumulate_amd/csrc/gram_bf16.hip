// gram_bf16.hip -- H_lower += X^T X for bf16 activations on the bf16 matrix cores.
//
// The calibration Hessian is the Gram matrix of the activations, summed over
// tokens, and chunk sums add (hipfire-calib-data, "Hessian storage"; AtomicChat
// GGUF page, "The importance matrix").  Products of two bf16 values are exact
// in fp32; each launch accumulates its chunk in fp32 registers from zero and adds
// the result to H once, so streaming many chunks rounds once per chunk.
//
// Layout problem: v_mfma_f32_32x32x16_bf16 wants, per lane, 8 consecutive k
// values (tokens) of one output row (channel), but X is token-major.  Each
// thread therefore loads a 4-token x 8-channel patch with four 16-byte row
// loads, regroups it in registers into eight 4-token words and stores those to
// an LDS panel laid out [channel][token]; the MFMA operands are then single
// 16-byte LDS reads.  The token order inside a lane is irrelevant to the sum
// as long as A and B use the same one, which they do (same panel layout).
//
// Only lower tiles (ti >= tj) are launched; a diagonal tile reads one panel for
// both operands.  128 x 128 tiles, 256 threads (2 x 2 waves of 64 x 64), 32
// tokens per LDS stage, double-buffered.
#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BKT = 32, NT = 256;
constexpr int PITCH = BKT + 8;      // bf16 elements per LDS row (80 bytes)

__device__ inline void tri_index(int64_t id, int64_t &ti, int64_t &tj)
{
    int64_t t = (int64_t)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
    while (t * (t + 1) / 2 > id) --t;
    while ((t + 1) * (t + 2) / 2 <= id) ++t;
    ti = t;
    tj = id - t * (t + 1) / 2;
}

__global__ __launch_bounds__(NT) void gram_bf16_kernel(float *__restrict__ H,
                                                       const uint16_t *__restrict__ X,
                                                       int64_t T, int64_t K, int vec)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ps[2][2][BM][PITCH];  // [buf][panel][ch][tok]

    int64_t ti, tj;
    tri_index(blockIdx.x, ti, tj);
    const bool diag = (ti == tj);
    const int64_t i0 = ti * BM, j0 = tj * BM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // loader role: threads 0..127 -> panel A (channels i0..), 128..255 -> panel B
    const int panel = tid >> 7;
    const int u = tid & 127;
    const int q = u >> 4;          // token quad 0..7
    const int o = u & 15;          // channel octet 0..15
    const int64_t cbase = (panel ? j0 : i0) + 8 * o;
    const bool loader = !(diag && panel == 1);

    // Interior tiles and full token stages take unconditional 16-byte loads; the
    // ragged edges load 16-bit elements from clamped addresses and zero the
    // out-of-range ones with a select (no divergent branches around loads).
    const bool full_c = vec && (i0 + BM <= K) && (j0 + BM <= K);
    u32x4 v[4];
    auto gload = [&](int64_t t0) {
        if (!loader) return;
        if (full_c && t0 + BKT <= T) {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = *(const u32x4 *)(X + (t0 + 4 * q + r) * K + cbase);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + 4 * q + r;
                unsigned w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t c0 = cbase + 2 * e;
                    const bool ok0 = t < T && c0 < K, ok1 = t < T && c0 + 1 < K;
                    const unsigned lo = X[ok0 ? t * K + c0 : 0];
                    const unsigned hi = X[ok1 ? t * K + c0 + 1 : 0];
                    w[e] = (ok0 ? lo : 0u) | ((ok1 ? hi : 0u) << 16);
                }
                v[r] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    };
    auto sstore = [&](int buf) {
        if (!loader) return;
        // channel 8o + c gets tokens 4q..4q+3 as one 8-byte word
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // dword e of each token row holds channels 2e (low half) and 2e+1 (high half)
            const unsigned a0 = v[0][e], a1 = v[1][e], a2 = v[2][e], a3 = v[3][e];
            const unsigned lo_c0 = (a0 & 0xFFFFu) | (a1 << 16);
            const unsigned hi_c0 = (a2 & 0xFFFFu) | (a3 << 16);
            const unsigned lo_c1 = (a0 >> 16) | (a1 & 0xFFFF0000u);
            const unsigned hi_c1 = (a2 >> 16) | (a3 & 0xFFFF0000u);
            uint2 *p0 = (uint2 *)&Ps[buf][panel][8 * o + 2 * e][4 * q];
            uint2 *p1 = (uint2 *)&Ps[buf][panel][8 * o + 2 * e + 1][4 * q];
            *p0 = make_uint2(lo_c0, hi_c0);
            *p1 = make_uint2(lo_c1, hi_c1);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int pb = diag ? 0 : 1;
    const int64_t nk = (T + BKT - 1) / BKT;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int buf = (int)(kt & 1);
            if (kt + 1 < nk) gload((kt + 1) * BKT);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int tok = 16 * kh + 8 * (lane >> 5);
                bf16x8 a[2], b[2];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    a[bi] = *(const bf16x8 *)&Ps[buf][0][wr * 64 + bi * 32 + (lane & 31)][tok];
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    b[bj] = *(const bf16x8 *)&Ps[buf][pb][wc * 64 + bj * 32 + (lane & 31)][tok];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < 2; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
            }
            if (kt + 1 < nk) sstore(buf ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gi = i0 + wr * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t gj = j0 + wc * 64 + bj * 32 + (lane & 31);
                if (gi < K && gj < K && gi >= gj) H[gi * K + gj] += acc[bi][bj][r];
            }
}

}  // namespace

hipError_t launch_gram_bf16(float *H, const uint16_t *X, int64_t T, int64_t K, hipStream_t s)
{
    if (T <= 0 || K <= 0) return hipSuccess;
    const int64_t nt = (K + BM - 1) / BM;
    const int vec = (K % 8 == 0) && (((uintptr_t)X & 15) == 0);
    hipLaunchKernelGGL(gram_bf16_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(NT), 0, s, H, X,
                       T, K, vec);
    return hipGetLastError();
}

}  // namespace gq
