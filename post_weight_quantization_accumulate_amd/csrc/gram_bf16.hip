// gram_bf16.hip -- H_lower += X^T X for bf16 activations on the bf16 matrix cores.
//
// The calibration Hessian is the Gram matrix of the activations, summed over
// tokens, and chunk sums add (hipfire-calib-data, "Hessian storage"; AtomicChat
// GGUF page, "The importance matrix").  Products of two bf16 values are exact
// in fp32; each launch accumulates its chunk in fp32 registers from zero and adds
// the result to H once, so streaming many chunks rounds once per chunk and the
// result does not depend on scheduling.
//
// One workgroup per lower 256 x 256 tile (tile order as in the int8 product:
// XCD-contiguous, grouped by tile rows), 8 waves of 64 x 128 (4 x 2), each 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16.  The instruction computes X Y^T for
// 32-row panels X and Y of 16 k: lane l feeds k = 8 (l / 32) + 0..7 of row
// l % 32 of each, and result e of lane l is (X Y^T)[8 (e/4) + 4 (l/32) + e%4][l % 32].
//
// X is token-major, the instruction wants 8 consecutive tokens of one channel
// per lane: the transpose happens on the way into LDS.  A stage is 32 tokens;
// each of the 256 loader threads of a panel loads a 4-token x 8-channel patch
// (four 16-byte loads, three stages ahead into registers) and stores 8 words of
// 4 tokens, one per channel.  A panel in LDS is 256 rows of 64 bytes (32
// tokens); channel rho lives in physical row 32 (rho % 8) + rho / 8 and its
// 16-byte token chunk c at position c ^ (rho % 4) ^ (rho / 64 % 4).  A wave
// loads 2 token rows x 512 bytes per instruction (X rows are far apart, so
// wide contiguous segments keep many L2 channels busy); with that placement its
// 8-byte stores of one channel index spread over all banks, and so do the
// 16-byte matrix-operand reads of 32 consecutive channels.
#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 256;                    // tile edge (channels)
constexpr int GBT = 32;                     // tokens per stage
constexpr int GNT = 512;                    // threads
constexpr int kPanelBytes = GBM * GBT * 2;  // 16 KiB
// dynamic LDS: two slots of the A and B panels
constexpr size_t kGramLds = (size_t)4 * kPanelBytes;
// lgkmcnt(0) only: loads in flight to registers are not waited for
constexpr int kWaitLgkm0 = 0xC07F;

// VEC: K % 8 == 0 and X 16-byte aligned, so that every 8-channel octet is
// wholly inside or wholly outside [0, K) and loads as one 16-byte word.
template <bool VEC>
__global__ __launch_bounds__(GNT, 1) void gram_bf16_kernel(float *__restrict__ H,
                                                           const uint16_t *__restrict__ X,
                                                           int64_t T, int64_t K)
{
    extern __shared__ __attribute__((aligned(1024))) int8_t g_lds[];
    const int64_t nt = (K + GBM - 1) / GBM;
    int64_t ti, tj;
    lower_tile_grouped(xcd_order(blockIdx.x, gridDim.x), nt, ti, tj);
    const int64_t i0 = ti * GBM, j0 = tj * GBM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // loader role: threads 0..255 -> panel A (channels i0..), 256..511 -> panel B
    // (channels j0.., which on a diagonal tile are A's again); channels
    // 8 o .. 8 o + 7, tokens 4 q .. 4 q + 3 of each stage
    const int panel = tid >> 8, u = tid & 255;
    const int o = u & 31, q = u >> 5;        // a wave instruction: 2 token rows x 512 bytes
    const int64_t cbase = (panel ? j0 : i0) + 8 * o;
    // byte offset of this thread's patch from the start of its stage's first
    // token row (below 2^32 for K < 2^24), and whether its octet is in range
    const unsigned voff = (unsigned)((4 * q * K + cbase) * 2);
    const bool c_in = cbase < K;
    // Stages past T load zeros: the stage count is rounded up to a multiple of
    // 6 (the pipeline's period), so that the pipeline below needs no run-time cases.
    const int64_t nk = ((T + GBT - 1) / GBT + 5) / 6 * 6 > 0 ? ((T + GBT - 1) / GBT + 5) / 6 * 6 : 6;

    u32x4 g[3][4];
    auto gload = [&](auto P, int64_t kt) {
        constexpr int p = decltype(P)::value;
        const int64_t t0 = kt * GBT + 4 * q;
        if constexpr (VEC) {
            // Address = uniform row base (clamped into X) + per-thread byte
            // offset; out-of-range rows read the first 8 channels of a valid row
            // and lstore replaces them by zeros (a select here would wait for
            // the load at once).
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = kt * GBT + r < T ? kt * GBT + r : T - 1;
                const char *sb = (const char *)X + row * K * 2;
                const unsigned off = (c_in && t0 + r < T) ? voff : 0u;
                g[p][r] = *(const u32x4 *)(sb + off);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + r;
                unsigned w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t c0 = cbase + 2 * e;
                    const bool ok0 = t < T && c0 < K, ok1 = t < T && c0 + 1 < K;
                    const unsigned lo = X[ok0 ? t * K + c0 : 0];
                    const unsigned hi = X[ok1 ? t * K + c0 + 1 : 0];
                    w[e] = (ok0 ? lo : 0u) | ((ok1 ? hi : 0u) << 16);
                }
                g[p][r] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    };
    // channel rho = 8 o + c gets tokens 4 q .. 4 q + 3 as one 8-byte word, at
    // byte 8 (q % 2) of chunk q / 2 of its row: physical row 32 c + o, chunk
    // position (q / 2) ^ (c % 4) ^ (o / 8 % 4), i.e. byte 2048 c + sbase[c % 4]
    int sbase[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        sbase[x] = panel * kPanelBytes + 64 * o + 16 * ((q >> 1) ^ x ^ ((o >> 3) & 3)) + 8 * (q & 1);
    auto lstore = [&](auto P, auto SLOT, int64_t kt) {
        constexpr int p = decltype(P)::value;
        int8_t *base = g_lds + 2 * decltype(SLOT)::value * kPanelBytes;
        if constexpr (VEC) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (!(c_in && kt * GBT + 4 * q + r < T)) g[p][r] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // dword e of each token row holds channels 2e (low half) and 2e+1 (high half)
            const unsigned a0 = g[p][0][e], a1 = g[p][1][e], a2 = g[p][2][e], a3 = g[p][3][e];
            const uint2 w0 = make_uint2((a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16));
            const uint2 w1 = make_uint2((a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 2 * e + h;
                *(uint2 *)(base + 2048 * c + sbase[c & 3]) = h ? w1 : w0;
            }
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.0f;

    // operand read offsets (bytes within a panel) for the two k16 halves of a
    // stage: channel rho = r0 + 32 bb + m (r0 a multiple of 32) sits in physical
    // row 32 (m % 8) + r0 / 8 + 4 bb + m / 8, chunk ch at position
    // ch ^ (m % 4) ^ (rho / 64 % 4).  A wave's A rows share rho / 64 = wr; its B
    // rows have rho / 64 = 2 wc + bb / 2.
    const int m = lane & 31;
    int offa[2], offb[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = 2 * h + (lane >> 5);
        const int row = 64 * (32 * (m & 7) + (m >> 3));
        offa[h] = row + 16 * (ch ^ (m & 3) ^ wr) + 512 * wr;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            offb[h][hb] = row + 16 * (ch ^ (m & 3) ^ ((2 * wc + hb) & 3)) + 1024 * wc + 512 * hb;
    }

    // Stage kt: the barrier publishes stage kt (stored during stage kt - 1) and
    // frees the other LDS slot (read during stage kt - 1).  Register set
    // (kt + 1) % 3 holds stage kt + 1 (loaded during stage kt - 3): it goes to
    // LDS, then receives stage kt + 4, so global loads have three stages to
    // land.  The operands of the two k16 halves are read one half at a time
    // (the second while the first half's matrix instructions run).  P (LDS
    // parity), S (register set) and the flags are compile-time, so that the
    // loop body has no branches and the compiler's wait counts stay exact.
    auto step = [&](auto P, auto S, auto STORE, auto LOAD, int64_t kt) {
        constexpr int p = decltype(P)::value, sset = decltype(S)::value;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int8_t *Aq = g_lds + (2 * p) * kPanelBytes, *Bq = g_lds + (2 * p + 1) * kPanelBytes;
        bf16x8 a[2], b[4];
        auto rd = [&](int h) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) a[bb] = *(const bf16x8 *)(Aq + offa[h] + 256 * bb);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) b[bb] = *(const bf16x8 *)(Bq + offb[h][bb >> 1] + 256 * (bb & 1));
        };
        auto mm = [&]() {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
        };
        rd(0);
        if constexpr (decltype(STORE)::value)
            lstore(std::integral_constant<int, sset>{}, std::integral_constant<int, 1 - p>{}, kt + 1);
        if constexpr (decltype(LOAD)::value) gload(std::integral_constant<int, sset>{}, kt + 4);
        __builtin_amdgcn_sched_barrier(0);
        mm();
        __builtin_amdgcn_sched_barrier(0);
        rd(1);
        __builtin_amdgcn_sched_barrier(0);
        mm();
        __builtin_amdgcn_sched_barrier(0);
    };
    using Y = std::true_type;
    using N = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    gload(I0{}, 0);
    gload(I1{}, 1);
    gload(I2{}, 2);
    lstore(I0{}, I0{}, 0);
    gload(I0{}, 3);
    // stage kt uses LDS parity kt % 2 and register set (kt + 1) % 3: a period of 6
    for (int64_t kt = 0; kt < nk - 6; kt += 6) {
        step(I0{}, I1{}, Y{}, Y{}, kt);
        step(I1{}, I2{}, Y{}, Y{}, kt + 1);
        step(I0{}, I0{}, Y{}, Y{}, kt + 2);
        step(I1{}, I1{}, Y{}, Y{}, kt + 3);
        step(I0{}, I2{}, Y{}, Y{}, kt + 4);
        step(I1{}, I0{}, Y{}, Y{}, kt + 5);
    }
    step(I0{}, I1{}, Y{}, Y{}, nk - 6);
    step(I1{}, I2{}, Y{}, Y{}, nk - 5);
    step(I0{}, I0{}, Y{}, N{}, nk - 4);
    step(I1{}, I1{}, Y{}, N{}, nk - 3);
    step(I0{}, I2{}, Y{}, N{}, nk - 2);
    step(I1{}, I0{}, N{}, N{}, nk - 1);

    // H += acc on the lower triangle
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = i0 + wr * 64 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int64_t gj = j0 + wc * 128 + bj * 32 + m;
                if (gi < K && gj < K && gi >= gj) H[gi * K + gj] += acc[bi][bj][e];
            }
}

}  // namespace

hipError_t launch_gram_bf16(float *H, const uint16_t *X, int64_t T, int64_t K, hipStream_t s)
{
    if (T <= 0 || K <= 0) return hipSuccess;
    static const bool lds_ok =
        hipFuncSetAttribute((const void *)gram_bf16_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kGramLds) == hipSuccess &&
        hipFuncSetAttribute((const void *)gram_bf16_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kGramLds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int64_t nt = (K + GBM - 1) / GBM;
    const dim3 grid((unsigned)(nt * (nt + 1) / 2));
    if ((K % 8 == 0) && (((uintptr_t)X & 15) == 0))
        hipLaunchKernelGGL(gram_bf16_kernel<true>, grid, dim3(GNT), kGramLds, s, H, X, T, K);
    else
        hipLaunchKernelGGL(gram_bf16_kernel<false>, grid, dim3(GNT), kGramLds, s, H, X, T, K);
    return hipGetLastError();
}

}  // namespace gq
