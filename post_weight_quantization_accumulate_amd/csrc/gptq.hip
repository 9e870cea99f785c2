// gptq.hip -- the GPTQ error-feedback sweep over one lazy block of 128 columns,
// and the qerr reduction (ork-driver wiki, "Exp 2026-08-18 GPTQ Int4": error-
// compensated column-sequential int4 rounding emitting symmetric codes in
// [-8, 7] with a per-(row, group) scale absmax/7; qerr definition).
//
// Two sweep kernels share one arithmetic.  sweep4_kernel (4 lanes per row,
// described at its definition) runs static groups and groups of 32 columns or
// more, the common case; sweep_block_kernel runs dynamic groups shorter than 32.
//
// sweep_block_kernel: rows are independent given U, so a wave holds 4 rows, 16 lanes
// per row, 8 consecutive columns per lane (the whole 128-column block of a row
// lives in registers).  Column i of the block is owned by lane i/8 of each
// 16-lane row group; a DPP row broadcast hands its current value to the row
// group, every lane takes the same rounding decision, and each lane then
// applies the error to its own 8 columns with one 32-byte LDS read of U's row i
// (the 128 x 128 block of U sits in LDS; zeros below its diagonal make the
// update a no-op for columns already done).  The 128 columns are unrolled with
// the group size fixed at compile time, so the column loop is straight-line code
// the scheduler can overlap.  Group maxima are a 16-lane xor-shuffle reduction.
// The per-column errors leave the kernel transposed (k-major) through LDS, as
// the A operand of the matrix-core block update that follows.
//
// Variants (the MODE template bits): static groups read every scale from
// `scales`, written before the sweep from the original weights; NF4 takes scale
// absmax and the nearest of the 16 codebook levels.  For NF4, lane j < 15 of a
// row group compares the broadcast quotient with midpoint j, and the count of
// true lanes in the row group (a ballot and a popcount) is the level index; the
// level's value comes from a 16-entry LDS table.
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int BW = kSweepBlock;        // 128
constexpr int SW_NT = 1024;            // 16 waves
constexpr int ROWS_WG = 64;            // 4 rows per wave
constexpr int UPITCH = BW + 4;

// Value of register x in lane `src` of each 16-lane row, to every lane of it.
template <int src> __device__ inline float row_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + src, 0xF, 0xF, false));
}

// Midpoint j of the NF4 levels in fp32 (j = 15: above every value).
__device__ inline float nf4_mid(int j) { return j < 15 ? (kNF4[j] + kNF4[j + 1]) * 0.5f : INFINITY; }

// U's 128 x 128 diagonal block at (b0, b0) into LDS, element (r, c) at
// r * UP + (c / 32) * QP + c % 32, zero outside the bw x bw corner (past bw the
// reciprocal diagonal is 0, so padded columns carry zero error and change
// nothing).  Each thread takes 16-byte pieces 32 / (NT / 128) apart and issues
// 8 loads before it stores any, so the block costs a few memory round trips
// rather than one per element.  Pieces that are not whole inside the corner, or
// a K or U that does not allow 16-byte loads, go element by element.
template <int NT, int UP, int QP>
__device__ __attribute__((always_inline)) inline void load_u_block(float *Us, const float *__restrict__ U, int64_t K, int64_t b0, int bw, int tid)
{
    constexpr int PIECES = BW * BW / 4;             // 16-byte pieces in the block
    constexpr int PER = PIECES / NT;                // per thread
    constexpr int BATCH = PER < 8 ? PER : 8;
    const bool vec = (K % 4) == 0 && (((uintptr_t)U) & 15) == 0;
#pragma unroll
    for (int b = 0; b < PER; b += BATCH) {
        float4 v[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int p = tid + NT * (b + j);
            const int r = p / (BW / 4), c = 4 * (p % (BW / 4));
            const float *src = U + (b0 + r) * K + b0 + c;
            if (vec && r < bw && c + 4 <= bw) {
                v[j] = *(const float4 *)src;
            } else {
                v[j].x = (r < bw && c < bw) ? src[0] : 0.0f;
                v[j].y = (r < bw && c + 1 < bw) ? src[1] : 0.0f;
                v[j].z = (r < bw && c + 2 < bw) ? src[2] : 0.0f;
                v[j].w = (r < bw && c + 3 < bw) ? src[3] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int p = tid + NT * (b + j);
            const int r = p / (BW / 4), c = 4 * (p % (BW / 4));
            *(float4 *)(Us + r * UP + (c >> 5) * QP + (c & 31)) = v[j];
        }
    }
}

// Four waves per SIMD (one workgroup of 16 waves per CU): the grid has one
// workgroup per 64 rows, 160 for ten thousand rows, so each block of U is read
// from memory half as often as with 32 rows, and CUs stay free for the update
// products that run beside the sweep on a second stream.
template <int G, int MODE>
__global__ __launch_bounds__(SW_NT, 4) void sweep_block_kernel(float *__restrict__ Wk, float *__restrict__ ET,
                                                           uint8_t *__restrict__ codes,
                                                           float *__restrict__ scales,
                                                           const float *__restrict__ U, int64_t N,
                                                           int64_t K, int64_t b0, const int *__restrict__ gidx)
{
    constexpr bool STATIC = (MODE & MODE_STATIC) != 0, NF4 = (MODE & MODE_NF4) != 0;
    __shared__ __attribute__((aligned(16))) float Us[BW * UPITCH];
    __shared__ float rdiag[BW];
    __shared__ float lev[16];
    const int tid = threadIdx.x;
    const int bw = (int)((K - b0) < BW ? (K - b0) : BW);
    if (NF4 && tid < 16) lev[tid] = kNF4[tid];

    load_u_block<SW_NT, UPITCH, 32>(Us, U, K, b0, bw, tid);
    if (tid < BW) rdiag[tid] = tid < bw ? 1.0f / U[(b0 + tid) * K + b0 + tid] : 0.0f;
    __syncthreads();

    const int lane = tid & 63, wave = tid >> 6;
    const int g16 = lane & 15;
    const int rloc = wave * 4 + (lane >> 4);
    const int64_t row = (int64_t)blockIdx.x * ROWS_WG + rloc;
    const bool rv = row < N;
    const int cb = g16 * 8;
    const int64_t ngroups = K / G;

    float w[8];
    unsigned cdw = 0;          // the lane's 8 codes, column cb + t in nibble t
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int col = cb + t;
        w[t] = (rv && col < bw) ? Wk[row * K + b0 + col] : 0.0f;
    }

    // static groups: the scale of column cb + t's group -- group gidx[column]
    // when a group map is given (act order), else column / G -- its power-of-two
    // guard factor (below) and RN(1 / (scale * factor)) (0 for a zero scale);
    // columns past bw have none
    float sl[8], yl[8], fl[8];
    if constexpr (STATIC) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t col = b0 + cb + t;
            const bool ok = rv && cb + t < bw;
            const int64_t gi = ok ? (gidx ? (int64_t)gidx[col] : col / G) : 0;
            sl[t] = ok ? scales[row * ngroups + gi] : 0.0f;
            fl[t] = sl[t] < 0x1p-60f ? 0x1p64f : 1.0f;
            yl[t] = sl[t] != 0.0f ? 1.0f / (sl[t] * fl[t]) : 0.0f;
        }
    }
    // NF4: this lane's midpoint and the lanes 0..14 of its row group
    const float mymid = nf4_mid(g16);
    const unsigned long long rowmask = 0x7FFFull << (lane & 48);

    // the group's scale s (1 for an all-zero group), its guard factor f, and
    // y = RN(1 / (s f)) (0 there).  A scale below 2^-60 (weights all below about
    // 2^-57) is scaled by f = 2^64 for the quotient, exactly, with the value
    // scaled alike, so the correction step's remainder cannot underflow and
    // 1/s cannot overflow: the quotient stays the IEEE one.
    float s = 1.0f, y = 0.0f, f = 1.0f;
    float4 nu0 = *(const float4 *)&Us[cb], nu1 = *(const float4 *)&Us[cb + 4];
    // one column: the static index lets the broadcast source and the group test
    // be immediates
    auto column = [&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int q = i / 8, t = i % 8;
        const float wi = row_bcast<q>(w[t]);
        if constexpr (STATIC) {
            // every column takes its own group's scale from the lane holding it
            const float sc = row_bcast<q>(sl[t]);
            s = sc != 0.0f ? sc : 1.0f;
            y = row_bcast<q>(yl[t]);
            f = row_bcast<q>(fl[t]);
        } else if constexpr (i % G == 0) {
            float sc;
            {
                float m = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int col = cb + u;
                    m = (col >= i && col < i + G) ? fmaxf(m, fabsf(w[u])) : m;
                }
                m = fmaxf(m, __shfl_xor(m, 1, 16));
                m = fmaxf(m, __shfl_xor(m, 2, 16));
                m = fmaxf(m, __shfl_xor(m, 4, 16));
                m = fmaxf(m, __shfl_xor(m, 8, 16));
                sc = NF4 ? m : m / 7.0f;
                if (g16 == 0 && rv && i < bw) scales[row * ngroups + (b0 + i) / G] = sc;
            }
            // A group whose scale is 0 takes the zero code: y = 0 makes the
            // quotient 0 for any value, and with s = 1 the error is the value
            // itself (with dynamic scales every value met there is 0; with
            // static ones feedback may have moved it, and it passes on whole).
            s = sc != 0.0f ? sc : 1.0f;
            f = sc < 0x1p-60f ? 0x1p64f : 1.0f;
            y = sc != 0.0f ? 1.0f / (s * f) : 0.0f;
        }
        // x = RN(wi / s) by Markstein's correction step (Markstein 1990; Muller
        // et al., Handbook of Floating-Point Arithmetic, division via FMA): with
        // y = RN(1/s) and q0 = RN(wi y), r = wi - s q0 is exact and RN(q0 + r y)
        // is the correctly rounded quotient (normal range), so the code is the
        // same as from an IEEE division, in three dependent operations instead
        // of the division's dozen.  Value and scale enter scaled by f.
        const float wq = wi * f;
        const float q0 = wq * y;
        const float rr = fmaf(-(s * f), q0, wq);
        const float x = fmaf(rr, y, q0);
        float c;                   // the value's multiple of s: the code, or its level
        unsigned nib;
        if constexpr (NF4) {
            const unsigned long long gt = __ballot(x > mymid);
            const int ci = __popcll(gt & rowmask);
            c = lev[ci];
            nib = (unsigned)ci;
        } else {
            c = fminf(fmaxf(rintf(x), -8.0f), 7.0f);
            nib = (unsigned)(int)c & 0xFu;
        }
        const float e = fmaf(-c, s, wi) * rdiag[i];
        // U's row i was read one column ahead; read row i + 1 now
        const float4 u0 = nu0, u1 = nu1;
        if constexpr (i + 1 < BW) {
            nu0 = *(const float4 *)&Us[(i + 1) * UPITCH + cb];
            nu1 = *(const float4 *)&Us[(i + 1) * UPITCH + cb + 4];
        }
        w[0] = fmaf(-e, u0.x, w[0]);
        w[1] = fmaf(-e, u0.y, w[1]);
        w[2] = fmaf(-e, u0.z, w[2]);
        w[3] = fmaf(-e, u0.w, w[3]);
        w[4] = fmaf(-e, u1.x, w[4]);
        w[5] = fmaf(-e, u1.y, w[5]);
        w[6] = fmaf(-e, u1.z, w[6]);
        w[7] = fmaf(-e, u1.w, w[7]);
        const bool own = (g16 == q);
        w[t] = own ? e : w[t];
        cdw |= own ? nib << (4 * t) : 0u;
        asm("" : "+v"(cdw));       // pack now: sunk to the end, the 128 codes would all stay live
    };
    static_for<BW>(column);

    // codes: two per byte, column 2m in the low nibble
    if (rv) {
        uint8_t *crow = codes + row * (K / 2) + (b0 + cb) / 2;
        const unsigned packed = cdw;
        if (cb + 8 <= bw && (((uintptr_t)crow & 3) == 0)) {
            *(unsigned *)crow = packed;
        } else {
            for (int m = 0; m < 4; ++m)
                if (cb + 2 * m < bw) crow[m] = (uint8_t)(packed >> (8 * m));
        }
    }

    // errors, transposed through LDS: ET[k][n] for the block's k = 0..bw-1
    __syncthreads();
    float *Es = Us;                        // reuse: [BW][ROWS_WG + 1]
#pragma unroll
    for (int t = 0; t < 8; ++t) Es[(cb + t) * (ROWS_WG + 1) + rloc] = w[t];
    __syncthreads();
    const int64_t n0 = (int64_t)blockIdx.x * ROWS_WG;
    for (int e = tid; e < BW * ROWS_WG; e += SW_NT) {
        const int k = e / ROWS_WG, r = e % ROWS_WG;
        if (k < bw && n0 + r < N) ET[k * N + n0 + r] = Es[k * (ROWS_WG + 1) + r];
    }
}

// The same sweep with 4 lanes per row, 32 consecutive columns per lane, for
// static groups and for groups of 32 columns or more.  The block's columns fall
// in 4 quarters of 32; lane q of a row's 4-lane group starts with quarter q, and
// after each quarter the 4 lanes pass their state (weights, codes, static
// scales) one lane down the group, so the quarter being decided always sits in
// the group's first lane and one body of 32 columns serves all four quarters.
// Column i's value reaches the group from that lane by one DPP quad broadcast,
// the 4 lanes take the same rounding decision, and each applies the error to
// the 32 columns it holds from 8 16-byte LDS reads of U's row i, issued one
// column ahead.  U's block sits in LDS as 4 quarters of 32 columns per row, 36
// floats apart, so the 4 quarters a quad reads fall on different banks (the 16
// rows of a wave read the same addresses).  A dynamic group starts with a
// quarter; its absmax combines 1, 2 or 4 lanes by quad exchanges before the
// quarter's columns, which then run without branches.  NF4 takes the level
// index as the count of midpoints the quotient exceeds, as the ballot form
// counts.  Decisions and arithmetic are those of sweep_block_kernel, column by
// column.  Against 16 lanes per row, each decision is taken by 4 lanes instead
// of 16 and a wave holds 16 rows instead of 4.
constexpr int S4_NT = 128;              // 2 waves
constexpr int S4_ROWS = 32;             // 16 rows per wave
constexpr int S4_QP = 36;               // floats from one quarter of a U row to the next
constexpr int S4_UP = 4 * S4_QP;        // floats per U row in LDS

template <int src> __device__ inline float quad_bcast(float x)
{
    constexpr int ctrl = src | (src << 2) | (src << 4) | (src << 6);   // quad_perm [src, src, src, src]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
}

template <int ctrl> __device__ inline float quad_perm_f(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
}

// Lane p of each quad takes the value of lane p + 1 (lane 3 that of lane 0).
__device__ inline unsigned quad_next(unsigned x)
{
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 1 | (2 << 2) | (3 << 4) | (0 << 6), 0xF, 0xF, false);
}
__device__ inline float quad_next(float x) { return __uint_as_float(quad_next(__float_as_uint(x))); }

template <int MODE>
__global__ __launch_bounds__(S4_NT, 1) void sweep4_kernel(float *__restrict__ Wk, float *__restrict__ ET,
                                                          uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                          const float *__restrict__ U, int64_t N, int64_t K,
                                                          int lg, int64_t b0, const int *__restrict__ gidx)
{
    constexpr bool STATIC = (MODE & MODE_STATIC) != 0, NF4 = (MODE & MODE_NF4) != 0;
    __shared__ __attribute__((aligned(16))) float Us[BW * S4_UP];
    __shared__ __attribute__((aligned(16))) float rdiag[BW];
    __shared__ float lev[16];
    const int tid = threadIdx.x;
    const int G = 1 << lg;                // 32, 64 or 128
    const int bw = (int)((K - b0) < BW ? (K - b0) : BW);
    if (NF4 && tid < 16) lev[tid] = kNF4[tid];
    load_u_block<S4_NT, S4_UP, S4_QP>(Us, U, K, b0, bw, tid);
    if (tid < BW) rdiag[tid] = tid < bw ? 1.0f / U[(b0 + tid) * K + b0 + tid] : 0.0f;
    __syncthreads();

    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane & 3;
    const int rloc = wave * 16 + (lane >> 2);
    const int64_t row = (int64_t)blockIdx.x * S4_ROWS + rloc;
    const bool rv = row < N;
    const int cb = 32 * q;
    const int64_t ngroups = K >> lg;

    float w[32];
    {
        const float *wr = Wk + row * K + b0 + cb;
        if (rv && cb + 32 <= bw && (((uintptr_t)wr) & 15) == 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float4 v = *(const float4 *)(wr + 4 * k);
                w[4 * k] = v.x;
                w[4 * k + 1] = v.y;
                w[4 * k + 2] = v.z;
                w[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 32; ++t) w[t] = (rv && cb + t < bw) ? wr[t] : 0.0f;
        }
    }

    // static groups: each column's scale (group gidx[column] when a group map is
    // given, else column / G) and RN(1 / (scale * guard factor))
    float sl[STATIC ? 32 : 1], yl[STATIC ? 32 : 1];
    if constexpr (STATIC) {
        // every group index, then every scale, loaded from clamped addresses
        // before any is used: two waits on memory instead of one per column
        int64_t gi[32];
        if (gidx) {
            int gv[32];
#pragma unroll
            for (int t = 0; t < 32; ++t) gv[t] = gidx[(rv && cb + t < bw) ? b0 + cb + t : 0];
#pragma unroll
            for (int t = 0; t < 32; ++t) gi[t] = gv[t];
        } else {
#pragma unroll
            for (int t = 0; t < 32; ++t) gi[t] = (b0 + cb + t) >> lg;
        }
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const bool ok = rv && cb + t < bw;
            sl[t] = scales[ok ? row * ngroups + gi[t] : 0];
        }
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const bool ok = rv && cb + t < bw;
            sl[t] = ok ? sl[t] : 0.0f;
            const float ft = sl[t] < 0x1p-60f ? 0x1p64f : 1.0f;
            yl[t] = sl[t] != 0.0f ? 1.0f / (sl[t] * ft) : 0.0f;
        }
    }
    // NF4 midpoints, ascending
    float mids[NF4 ? 15 : 1];
    if constexpr (NF4) {
#pragma unroll
        for (int j = 0; j < 15; ++j) mids[j] = nf4_mid(j);
    }

    float s = 1.0f, y = 0.0f, f = 1.0f;   // as in sweep_block_kernel
    unsigned cdw[4] = {0u, 0u, 0u, 0u};   // codes of the lane's quarter, column t in nibble t % 8 of word t / 8
    const bool own = (q == 0);            // the group's first lane holds the quarter being decided
#pragma unroll 1
    for (int qi = 0; qi < 4; ++qi) {
        // this lane now holds quarter (q + qi) % 4; the group's first lane holds quarter qi
        const float *uq = Us + 32 * qi * S4_UP + ((q + qi) & 3) * S4_QP;
        // the quarter's reciprocal diagonal, in registers
        float rd[32];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 r4 = *(const float4 *)(rdiag + 32 * qi + 4 * k);
            rd[4 * k] = r4.x;
            rd[4 * k + 1] = r4.y;
            rd[4 * k + 2] = r4.z;
            rd[4 * k + 3] = r4.w;
        }
        // a group starts with the quarter: its scale from the absmax of the
        // group's quarters, which sit in lanes 0 (G = 32), 0-1 (64) or 0-3 (128)
        // of the quad
        if (!STATIC && ((32 * qi) & (G - 1)) == 0) {
            float m = 0.0f;
#pragma unroll
            for (int v = 0; v < 32; ++v) m = fmaxf(m, fabsf(w[v]));
            if (G >= 64) m = fmaxf(m, quad_perm_f<1 | (0 << 2) | (3 << 4) | (2 << 6)>(m));
            if (G == 128) m = fmaxf(m, quad_perm_f<2 | (3 << 2) | (0 << 4) | (1 << 6)>(m));
            m = quad_bcast<0>(m);
            const float sc = NF4 ? m : m / 7.0f;
            if (q == 0 && rv && 32 * qi < bw) scales[row * ngroups + ((b0 + 32 * qi) >> lg)] = sc;
            s = sc != 0.0f ? sc : 1.0f;
            f = sc < 0x1p-60f ? 0x1p64f : 1.0f;
            y = sc != 0.0f ? 1.0f / (s * f) : 0.0f;
        }

        // the rounding decision of column ti of the quarter: packs its code and
        // returns its scaled error
        auto decide = [&](auto T) -> float {
            constexpr int ti = decltype(T)::value;
            const float wi = quad_bcast<0>(w[ti]);
            if constexpr (STATIC) {
                const float sc = quad_bcast<0>(sl[ti]);
                s = sc != 0.0f ? sc : 1.0f;
                y = quad_bcast<0>(yl[ti]);
                f = sc < 0x1p-60f ? 0x1p64f : 1.0f;
            }
            // x = RN(wi / s) by Markstein's correction step, value and scale scaled by f
            const float wq = wi * f;
            const float q0 = wq * y;
            const float rr = fmaf(-(s * f), q0, wq);
            const float x = fmaf(rr, y, q0);
            float c;
            unsigned nib;
            if constexpr (NF4) {
                int ci = 0;
#pragma unroll
                for (int j = 0; j < 15; ++j) ci += x > mids[j] ? 1 : 0;
                c = lev[ci];
                nib = (unsigned)ci;
            } else {
                c = fminf(fmaxf(rintf(x), -8.0f), 7.0f);
                nib = (unsigned)(int)c & 0xFu;
            }
            cdw[ti / 8] |= own ? nib << (4 * (ti % 8)) : 0u;
            asm("" : "+v"(cdw[ti / 8]));      // pack now, not at the end
            return fmaf(-c, s, wi) * rd[ti];
        };

        // U's rows are read one column ahead, so a whole column covers the LDS
        // latency, and the columns are pipelined: column ti first updates the
        // value column ti + 1 decides on, takes that decision, and then
        // finishes its other 31 updates beside it.
        float nu[32];
        auto read_row = [&](int r) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float4 v = *(const float4 *)(uq + r * S4_UP + 4 * k);
                nu[4 * k] = v.x;
                nu[4 * k + 1] = v.y;
                nu[4 * k + 2] = v.z;
                nu[4 * k + 3] = v.w;
            }
        };
        read_row(0);
        float e = decide(std::integral_constant<int, 0>{});
        auto column = [&](auto T) {
            constexpr int ti = decltype(T)::value;
            float u[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) u[j] = nu[j];
            if constexpr (ti + 1 < 32) read_row(ti + 1);
            constexpr int nx = ti + 1 < 32 ? ti + 1 : -1;   // the value decided next
            float en = 0.0f;
            if constexpr (nx >= 0) {
                w[nx] = fmaf(-e, u[nx], w[nx]);
                en = decide(std::integral_constant<int, nx>{});
            }
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (j != nx) w[j] = fmaf(-e, u[j], w[j]);
            w[ti] = own ? e : w[ti];
            e = en;
            // nothing crosses: the next row's reads stay a column ahead of their use
            __builtin_amdgcn_sched_barrier(0);
        };
        static_for<32>(column);
        // pass the state one lane down the group: lane p then holds quarter (p + qi + 1) % 4
#pragma unroll
        for (int t = 0; t < 32; ++t) w[t] = quad_next(w[t]);
#pragma unroll
        for (int k = 0; k < 4; ++k) cdw[k] = quad_next(cdw[k]);
        if constexpr (STATIC) {
#pragma unroll
            for (int t = 0; t < 32; ++t) {
                sl[t] = quad_next(sl[t]);
                yl[t] = quad_next(yl[t]);
            }
        }
    }
    // after four passes lane q holds its own quarter again

    // codes: two per byte, column 2m in the low nibble
    if (rv) {
        uint8_t *crow = codes + row * (K / 2) + (b0 + cb) / 2;
        if (cb + 32 <= bw && (((uintptr_t)crow & 3) == 0)) {
#pragma unroll
            for (int k = 0; k < 4; ++k) ((unsigned *)crow)[k] = cdw[k];
        } else {
            for (int m = 0; m < 16; ++m)
                if (cb + 2 * m < bw) crow[m] = (uint8_t)(cdw[m / 4] >> (8 * (m % 4)));
        }
    }

    // errors, transposed through LDS: ET[k][n] for the block's k = 0..bw-1
    __syncthreads();
    float *Es = Us;                        // reuse: [BW][S4_ROWS + 1]
#pragma unroll
    for (int t = 0; t < 32; ++t) Es[(cb + t) * (S4_ROWS + 1) + rloc] = w[t];
    __syncthreads();
    const int64_t n0 = (int64_t)blockIdx.x * S4_ROWS;
    for (int e = tid; e < BW * S4_ROWS; e += S4_NT) {
        const int k = e / S4_ROWS, r = e % S4_ROWS;
        if (k < bw && n0 + r < N) ET[k * N + n0 + r] = Es[k * (S4_ROWS + 1) + r];
    }
}

__global__ __launch_bounds__(256) void copy_check_kernel(float *__restrict__ dst, const float *__restrict__ src,
                                                        int64_t n, unsigned *status)
{
    bool bad = false;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n / 4;
    const bool al = ((((uintptr_t)dst) | ((uintptr_t)src)) & 15) == 0;
    if (al) {
        for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
            const float4 v = ((const float4 *)src)[i];
            if (!isfinite(v.x) || !isfinite(v.y) || !isfinite(v.z) || !isfinite(v.w)) bad = true;
            ((float4 *)dst)[i] = v;
        }
        for (int64_t i = 4 * n4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
            const float v = src[i];
            if (!isfinite(v)) bad = true;
            dst[i] = v;
        }
    } else {
        for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
            const float v = src[i];
            if (!isfinite(v)) bad = true;
            dst[i] = v;
        }
    }
    if (bad) atomicOr(status, ST_NONFINITE);
}

__global__ __launch_bounds__(256) void check_finite_kernel(const float *__restrict__ x, int64_t n,
                                                          unsigned *status)
{
    bool bad = false;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        if (!isfinite(x[i])) bad = true;
    if (bad) atomicOr(status, ST_NONFINITE);
}

constexpr int QNT = 256;
constexpr int64_t QPARTS = 1024;

__device__ void block_sum2(double &a, double &b, double *sh)
{
    const int t = threadIdx.x;
    sh[t] = a;
    sh[QNT + t] = b;
    __syncthreads();
    for (int s = QNT / 2; s > 0; s >>= 1) {
        if (t < s) {
            sh[t] += sh[t + s];
            sh[QNT + t] += sh[QNT + t + s];
        }
        __syncthreads();
    }
    a = sh[0];
    b = sh[QNT];
}

// Partial sums over a fixed row range per workgroup: sum imp (w - c s)^2, sum imp w^2,
// with c the signed code, or with NF4 the level its unsigned index names.
template <bool NF4>
__global__ __launch_bounds__(QNT) void qerr_kernel(double *__restrict__ partials, const float *__restrict__ W,
                                                  const uint8_t *__restrict__ codes,
                                                  const float *__restrict__ scales,
                                                  const float *__restrict__ imp, int64_t N, int64_t K,
                                                  int64_t G, int64_t rows_per)
{
    __shared__ double sh[2 * QNT];
    __shared__ float lev[16];
    if (NF4 && threadIdx.x < 16) lev[threadIdx.x] = kNF4[threadIdx.x];
    __syncthreads();
    const int64_t r0 = blockIdx.x * rows_per;
    const int64_t r1 = (r0 + rows_per < N) ? r0 + rows_per : N;
    const int64_t half = K / 2, ng = K / G;
    double num = 0.0, den = 0.0;
    for (int64_t n = r0; n < r1; ++n) {
        for (int64_t m = threadIdx.x; m < half; m += QNT) {
            const unsigned b = codes[n * half + m];
            float c0, c1;
            if constexpr (NF4) {
                c0 = lev[b & 0xFu];
                c1 = lev[b >> 4];
            } else {
                c0 = (float)((int)(b & 0xFu) - ((b & 0x8u) ? 16 : 0));
                c1 = (float)((int)(b >> 4) - ((b & 0x80u) ? 16 : 0));
            }
            const int64_t k0 = 2 * m, k1 = 2 * m + 1;
            const float w0 = W[n * K + k0], w1 = W[n * K + k1];
            const float s0 = scales[n * ng + k0 / G], s1 = scales[n * ng + k1 / G];
            const double i0 = imp ? (double)imp[k0] : 1.0, i1 = imp ? (double)imp[k1] : 1.0;
            // exact products in fp64, one rounding in the difference
            const double d0 = (double)w0 - (double)c0 * (double)s0, d1 = (double)w1 - (double)c1 * (double)s1;
            num += i0 * d0 * d0 + i1 * d1 * d1;
            den += i0 * (double)w0 * (double)w0 + i1 * (double)w1 * (double)w1;
        }
    }
    block_sum2(num, den, sh);
    if (threadIdx.x == 0) {
        partials[2 * blockIdx.x] = num;
        partials[2 * blockIdx.x + 1] = den;
    }
}

// The same sums for K a multiple of 8 with W (and imp) 16-byte and the codes
// 4-byte aligned: a thread takes 8 consecutive columns of a row at a time (two
// 16-byte loads of W, one 4-byte word of codes), the grid strides over the flat
// index of the rows' 8-column chunks, and each workgroup folds its sums in the
// fixed-order tree.  The next pass's loads are issued before this pass's
// arithmetic, so that two passes' loads are in flight.
template <bool NF4>
__global__ __launch_bounds__(QNT) void qerr8_kernel(double *__restrict__ partials, const float *__restrict__ W,
                                                   const uint8_t *__restrict__ codes,
                                                   const float *__restrict__ scales,
                                                   const float *__restrict__ imp, int64_t N, int64_t K, int64_t G)
{
    __shared__ double sh[2 * QNT];
    __shared__ float lev[16];
    if (NF4 && threadIdx.x < 16) lev[threadIdx.x] = kNF4[threadIdx.x];
    __syncthreads();
    const int64_t chunks = K / 8, ng = K / G;
    const int lg = __builtin_ctzll((unsigned long long)G);   // G is a power of two
    const int64_t total = N * chunks;
    const int64_t S = (int64_t)gridDim.x * QNT;
    const int64_t dq2 = 2 * S / chunks, dr2 = 2 * S - dq2 * chunks;
    double num = 0.0, den = 0.0;
    // two chunks per pass, the grid's stride apart, and the next pass's loads
    // issued before this pass's arithmetic: four chunks' loads in flight
    float4 a0, b0, ia0, ib0, a1, b1, ia1, ib1;
    unsigned cw0, cw1;
    float s0, s1;
    auto load = [&](int64_t row, int64_t c, bool ok, float4 &a, float4 &b, float4 &ia, float4 &ib, unsigned &cw,
                    float &s8) __attribute__((always_inline)) {
        const int64_t r = ok ? row : 0, c8 = ok ? c : 0;
        a = *(const float4 *)(W + r * K + 8 * c8);
        b = *(const float4 *)(W + r * K + 8 * c8 + 4);
        cw = *(const unsigned *)(codes + r * (K / 2) + 4 * c8);
        if (imp) {
            ia = *(const float4 *)(imp + 8 * c8);
            ib = *(const float4 *)(imp + 8 * c8 + 4);
        } else {
            ia = ib = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        }
        s8 = G >= 8 ? scales[r * ng + ((8 * c8) >> lg)] : 0.0f;   // one group holds all 8 columns
    };
    auto advance = [&](int64_t &rw, int64_t &cl) __attribute__((always_inline)) {
        rw += dq2;
        cl += dr2;
        if (cl >= chunks) {
            cl -= chunks;
            ++rw;
        }
    };
    auto accumulate = [&](float4 a, float4 b, float4 ia, float4 ib, unsigned cw, float s8, int64_t prow,
                          int64_t c) __attribute__((always_inline)) {
        const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const float iw[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        const float *srow = scales + prow * ng;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const unsigned nib = (cw >> (4 * t)) & 0xFu;
            const float cv = NF4 ? lev[nib] : (float)((int)nib - ((nib & 8u) ? 16 : 0));
            const float sc = G >= 8 ? s8 : srow[(8 * c + t) >> lg];
            const double d = (double)w[t] - (double)cv * (double)sc;
            num += (double)iw[t] * d * d;
            den += (double)iw[t] * (double)w[t] * (double)w[t];
        }
    };
    int64_t g0 = (int64_t)blockIdx.x * QNT + threadIdx.x;
    int64_t r0 = g0 / chunks, c0 = g0 - r0 * chunks;
    int64_t r1 = (g0 + S) / chunks, c1 = g0 + S - r1 * chunks;
    load(r0, c0, g0 < total, a0, b0, ia0, ib0, cw0, s0);
    load(r1, c1, g0 + S < total, a1, b1, ia1, ib1, cw1, s1);
    for (; g0 < total; g0 += 2 * S) {
        const float4 pa0 = a0, pb0 = b0, pia0 = ia0, pib0 = ib0, pa1 = a1, pb1 = b1, pia1 = ia1, pib1 = ib1;
        const unsigned pcw0 = cw0, pcw1 = cw1;
        const float ps0 = s0, ps1 = s1;
        const int64_t pr0 = r0, pc0 = c0, pr1 = r1, pc1 = c1;
        advance(r0, c0);
        advance(r1, c1);
        // the next pass (clamped to chunk 0 past the end: in bounds, unused)
        load(r0, c0, g0 + 2 * S < total, a0, b0, ia0, ib0, cw0, s0);
        load(r1, c1, g0 + 3 * S < total, a1, b1, ia1, ib1, cw1, s1);
        accumulate(pa0, pb0, pia0, pib0, pcw0, ps0, pr0, pc0);
        if (g0 + S < total) accumulate(pa1, pb1, pia1, pib1, pcw1, ps1, pr1, pc1);
    }
    block_sum2(num, den, sh);
    if (threadIdx.x == 0) {
        partials[2 * blockIdx.x] = num;
        partials[2 * blockIdx.x + 1] = den;
    }
}

__global__ __launch_bounds__(QNT) void qerr_reduce_kernel(double *out2, const double *partials, int64_t nparts)
{
    __shared__ double sh[2 * QNT];
    double a = 0.0, b = 0.0;
    for (int64_t i = threadIdx.x; i < nparts; i += QNT) {
        a += partials[2 * i];
        b += partials[2 * i + 1];
    }
    block_sum2(a, b, sh);
    if (threadIdx.x == 0) {
        out2[0] = a;
        out2[1] = b;
    }
}

unsigned grid_for(int64_t n)
{
    int64_t g = (n + 255) / 256;
    if (g > 16384) g = 16384;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// ---------------------------------------------------------------- round to nearest
// The same int4 grid without error feedback: per (row, group) scale s = absmax/7
// from the weights themselves, code = clamp(rint(w / s), -8, 7) (IEEE fp32
// division, ties to even; 0 for an all-zero group), packed as the sweep packs
// them.  The comparator the GPTQ codes are judged against, and a uniform pack
// that still records qerr (ork-driver wiki, "Exp 2026-08-18 GPTQ Int4", the
// producer for a pack's qerr field).
__device__ inline float rtn_code(float w, float s)
{
    return s == 0.0f ? 0.0f : fminf(fmaxf(rintf(w / s), -8.0f), 7.0f);
}

// NF4: the index of the level nearest to x (x in units of the scale), by a
// four-step binary search over the 15 midpoints (mid[15] = +inf) held in LDS.
__device__ inline int nf4_index(float x, const float *mid)
{
    int c = x > mid[7] ? 8 : 0;
    c += x > mid[c + 3] ? 4 : 0;
    c += x > mid[c + 1] ? 2 : 0;
    c += x > mid[c] ? 1 : 0;
    return c;
}

// One thread per 8 consecutive columns of a row at a time (K % 8 == 0, 16-byte
// aligned W, 4-byte aligned codes): two 16-byte loads, one 4-byte store of 8
// codes; the grid strides over the rows' 8-column chunks with the same trip
// count in every thread of a workgroup.  A group of G >= 8 spans G/8
// consecutive threads, aligned within the wave (the row length K/8 in threads
// is a multiple of G/8 <= 16), and takes its maximum by lane exchanges; for
// G < 8 a thread holds whole groups.  The code is rint of the correctly rounded
// fp32 quotient w / s, formed from y = RN(1/s) by one Markstein correction
// (Markstein 1990; Muller et al., Handbook of Floating-Point Arithmetic,
// division via FMA): q0 = RN(w y), r = w - s q0 exactly, RN(q0 + r y) = RN(w / s)
// while the quotient and 1/s stay normal, so a group with s below 2^-60 (whose
// weights are all below 2^-57) is first scaled by 2^64, exactly.  Non-finite
// weights set ST_NONFINITE.  With partials set, the workgroup also writes its
// pair (sum imp (w - c s)^2, sum imp w^2) in fp64, as qerr_kernel defines them,
// to partials[2 blockIdx.x ..] (a fixed-order tree, so the sums are
// deterministic): no second pass over W.
// The kernel takes 91 VGPRs (five waves per SIMD, five 256-lane workgroups per
// CU), and the grid is at most one such round of the 256 CUs: every workgroup
// is resident from the start and takes the same number of passes, so no second
// round runs on a partly idle chip.
constexpr int RTN_NT = QNT;
constexpr int RTN_MAX_WG = 5 * 256;
__device__ inline float rtn_quot_y(float w, float s, float y)
{
    const float q0 = w * y;
    const float r = fmaf(-s, q0, w);
    return fmaf(r, y, q0);
}
// NF4 (template flag): scale absmax, code the nearest level's index (nf4_index of
// the same correctly rounded quotient), and qerr from the level's value.
template <bool NF4>
__global__ __launch_bounds__(RTN_NT) void rtn8_kernel(const float *__restrict__ W, uint8_t *__restrict__ codes,
                                                      float *__restrict__ scales, int64_t N, int64_t K, int G,
                                                      unsigned *status, const float *__restrict__ imp,
                                                      double *__restrict__ partials)
{
    __shared__ float mid[16], lev[16];
    if (NF4 && threadIdx.x < 16) {
        mid[threadIdx.x] = nf4_mid(threadIdx.x);
        lev[threadIdx.x] = kNF4[threadIdx.x];
    }
    if (NF4) __syncthreads();
    const int64_t chunks = K / 8;
    const int64_t ngroups = K / G;
    const int lg = __builtin_ctz((unsigned)G);               // G is a power of two
    double num = 0.0, den = 0.0;
    bool bad = false;
    // Passes over the flat index of the 8-column chunks (row-major, N x K/8 of
    // them): the workgroup's 256 consecutive chunks, then the grid's stride on.
    // Every lane takes part in each pass, those past the end with a dummy
    // chunk; a group of G/8 lanes is wholly in or out, since the stride and the
    // row's chunk count are multiples of G/8.  The next pass's weights are
    // loaded before this pass's arithmetic, so that two passes' loads are in
    // flight.
    const int64_t total = N * chunks;
    const int64_t stride = (int64_t)gridDim.x * RTN_NT;
    const int64_t dq = stride / chunks, dr = stride - dq * chunks;
    auto wload = [&](int64_t row, int64_t cc, bool ok, float4 &a, float4 &b, float4 &ia, float4 &ib) {
        const int64_t r = ok ? row : 0, c8 = ok ? cc : 0;
        a = *(const float4 *)(W + r * K + 8 * c8);
        b = *(const float4 *)(W + r * K + 8 * c8 + 4);
        if (partials && imp) {                       // 16-byte aligned (checked at launch)
            ia = *(const float4 *)(imp + 8 * c8);
            ib = *(const float4 *)(imp + 8 * c8 + 4);
        } else {
            ia = ib = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        }
    };
    float4 na, nbv, nia, nib;
    int64_t base = (int64_t)blockIdx.x * RTN_NT;     // the workgroup's first chunk of the pass
    int64_t gi = base + threadIdx.x;
    int64_t row = gi / chunks, cn = gi - row * chunks;
    bool nvalid = gi < total;
    if (base < total) wload(row, cn, nvalid, na, nbv, nia, nib);
    for (; base < total;) {
        const bool valid = nvalid;
        const int64_t c = valid ? cn : 0, prow = valid ? row : 0;
        const float4 a = na, b = nbv, i0 = nia, i1 = nib;
        base += stride;
        gi += stride;
        row += dq;
        cn += dr;
        if (cn >= chunks) {
            cn -= chunks;
            ++row;
        }
        nvalid = gi < total;
        if (base < total) wload(row, cn, nvalid, na, nbv, nia, nib);
        const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) bad = bad || (valid && !isfinite(w[t]));
        float sc[8], cv[8];                          // each column's scale and multiple of it
        unsigned nb[8];                              // each column's nibble
        // the codes of columns t0 .. t1-1 under the group scale sg
        auto codes_of = [&](float sg, int t0, int t1) {
            const bool tiny = sg < 0x1p-60f;
            const float f = tiny ? 0x1p64f : 1.0f;
            const float ss = sg == 0.0f ? 1.0f : sg * f;
            const float y = sg == 0.0f ? 0.0f : 1.0f / ss;    // quotient 0 in an all-zero group
            for (int t = t0; t < t1; ++t) {
                sc[t] = sg;
                const float x = rtn_quot_y(w[t] * f, ss, y);
                if constexpr (NF4) {
                    const int ci = nf4_index(x, mid);
                    cv[t] = lev[ci];
                    nb[t] = (unsigned)ci;
                } else {
                    cv[t] = fminf(fmaxf(rintf(x), -8.0f), 7.0f);
                    nb[t] = (unsigned)(int)cv[t] & 0xFu;
                }
            }
        };
        if (G >= 8) {
            float m = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(w[t]));
            for (int o = 1; o < G / 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
            const float sg = NF4 ? m : m / 7.0f;
            if (valid && (c & ((G >> 3) - 1)) == 0) scales[prow * ngroups + ((8 * c) >> lg)] = sg;
            codes_of(sg, 0, 8);
        } else {
            for (int g0 = 0; g0 < 8; g0 += G) {
                float m = 0.0f;
                for (int t = g0; t < g0 + G; ++t) m = fmaxf(m, fabsf(w[t]));
                const float sg = NF4 ? m : m / 7.0f;
                if (valid) scales[prow * ngroups + ((8 * c + g0) >> lg)] = sg;
                codes_of(sg, g0, g0 + G);
            }
        }
        unsigned dw = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) dw |= nb[t] << (4 * t);
        if (valid) *(unsigned *)(codes + prow * (K / 2) + 4 * c) = dw;
        if (partials && valid) {
            const float iw[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const double wi = (double)iw[t];
                const double d = (double)w[t] - (double)cv[t] * (double)sc[t];
                num += wi * d * d;
                den += wi * (double)w[t] * (double)w[t];
            }
        }
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(status, ST_NONFINITE);
    if (partials) {                                  // uniform: every thread reaches the tree
        __shared__ double sh[2 * QNT];
        block_sum2(num, den, sh);
        if (threadIdx.x == 0) {
            partials[2 * blockIdx.x] = num;
            partials[2 * blockIdx.x + 1] = den;
        }
    }
}

// Any other shape: one thread per unit of P = max(2, G) columns (whole groups,
// whole code bytes), scalar loads and byte stores; NF4 as in rtn8_kernel.
template <bool NF4>
__global__ __launch_bounds__(RTN_NT) void rtn_any_kernel(const float *__restrict__ W, uint8_t *__restrict__ codes,
                                                         float *__restrict__ scales, int64_t N, int64_t K, int G,
                                                         unsigned *status)
{
    __shared__ float mid[16];
    if (NF4 && threadIdx.x < 16) mid[threadIdx.x] = nf4_mid(threadIdx.x);
    if (NF4) __syncthreads();
    const int P = G > 2 ? G : 2;
    const int64_t units = K / P, idx = (int64_t)blockIdx.x * RTN_NT + threadIdx.x;
    if (idx >= N * units) return;
    const int64_t row = idx / units, k0 = (idx - row * units) * P;
    const float *w = W + row * K + k0;
    bool bad = false;
    float sc = 0.0f;
    unsigned lo = 0;
    for (int t = 0; t < P; ++t) {
        if (t % G == 0) {                           // a group starts: its scale
            float m = 0.0f;
            for (int u = t; u < t + G; ++u) {
                bad = bad || !isfinite(w[u]);
                m = fmaxf(m, fabsf(w[u]));
            }
            sc = NF4 ? m : m / 7.0f;
            scales[row * (K / G) + (k0 + t) / G] = sc;
        }
        const unsigned nib = NF4 ? (unsigned)nf4_index(sc == 0.0f ? 0.0f : w[t] / sc, mid)
                                 : (unsigned)(int)rtn_code(w[t], sc) & 0xFu;
        if (t & 1) codes[row * (K / 2) + (k0 + t) / 2] = (uint8_t)(lo | nib << 4);
        else lo = nib;
    }
    if (bad) atomicOr(status, ST_NONFINITE);
}

}  // namespace

int64_t qerr_partials(int64_t N)
{
    const int64_t np = N < QPARTS ? N : QPARTS;
    const int64_t rows_per = (N + np - 1) / np;
    return (N + rows_per - 1) / rows_per;
}

hipError_t launch_copy_check(float *dst, const float *src, int64_t n, unsigned *status, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_check_kernel, dim3(grid_for(n / 4 + 1)), dim3(256), 0, s, dst, src, n, status);
    return hipGetLastError();
}

hipError_t launch_check_finite(const float *x, int64_t n, unsigned *status, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_finite_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, n, status);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_sweep_mode(float *Wk, float *ET, uint8_t *codes, float *scales, const float *U, int64_t N,
                             int64_t K, int64_t G, int64_t b0, const int *gidx, hipStream_t s)
{
    // the API admits powers of two up to 128 only
    if (G < 1 || G > BW || (G & (G - 1))) return hipErrorInvalidValue;
    const int lg = __builtin_ctzll((unsigned long long)G);
    const int64_t nwg = (N + S4_ROWS - 1) / S4_ROWS;
    if constexpr (!(MODE & MODE_STATIC)) {
        // groups shorter than a quarter start inside it: the 16-lane form, with
        // the group size fixed at compile time
        if (G < 32) {
            const dim3 grid((unsigned)((N + ROWS_WG - 1) / ROWS_WG)), block(SW_NT);
#define GQ_SWEEP_CASE(g)                                                                                      \
    case g:                                                                                                   \
        hipLaunchKernelGGL((sweep_block_kernel<g, MODE>), grid, block, 0, s, Wk, ET, codes, scales, U, N, K, b0, \
                           gidx);                                                                             \
        break;
            switch (G) {
                GQ_SWEEP_CASE(1)
                GQ_SWEEP_CASE(2)
                GQ_SWEEP_CASE(4)
                GQ_SWEEP_CASE(8)
                GQ_SWEEP_CASE(16)
            }
#undef GQ_SWEEP_CASE
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sweep4_kernel<MODE>), dim3((unsigned)nwg), dim3(S4_NT), 0, s, Wk, ET, codes, scales, U,
                       N, K, lg, b0, gidx);
    return hipGetLastError();
}

hipError_t launch_sweep_block(float *Wk, float *ET, uint8_t *codes, float *scales, const float *U,
                              int64_t N, int64_t K, int64_t G, int64_t b0, int mode, const int *gidx,
                              hipStream_t s)
{
    if (gidx && !(mode & MODE_STATIC)) return hipErrorInvalidValue;
    switch (mode) {
    case 0: return launch_sweep_mode<0>(Wk, ET, codes, scales, U, N, K, G, b0, nullptr, s);
    case MODE_STATIC: return launch_sweep_mode<MODE_STATIC>(Wk, ET, codes, scales, U, N, K, G, b0, gidx, s);
    case MODE_NF4: return launch_sweep_mode<MODE_NF4>(Wk, ET, codes, scales, U, N, K, G, b0, nullptr, s);
    case MODE_STATIC | MODE_NF4:
        return launch_sweep_mode<MODE_STATIC | MODE_NF4>(Wk, ET, codes, scales, U, N, K, G, b0, gidx, s);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- act order
// Column a of the act order is the column with the a-th largest diagonal entry
// of H, equal entries in increasing column order.  Column i's rank counts the
// columns that come before it in that strict total order (NaN entries after all
// others, so the ranks stay a permutation whatever H holds; the factor refuses
// such an H anyway).  perm[rank] = i, inv[i] = rank, gidx[rank] = i / G.
__device__ inline bool act_before(float dj, int j, float di, int i)
{
    const bool nj = dj != dj, ni = di != di;
    if (nj != ni) return ni;
    if (nj) return j < i;
    return dj > di || (dj == di && j < i);
}

// rank[i] += the number of columns j in chunk blockIdx.y (AP_NT columns) that
// come before i; rank starts at zero, and integer sums do not depend on order.
constexpr int AP_NT = 256;
__global__ __launch_bounds__(AP_NT) void act_rank_kernel(int *__restrict__ rank, const float *__restrict__ H,
                                                         int64_t K)
{
    __shared__ float dt[AP_NT];
    const int64_t i = (int64_t)blockIdx.x * AP_NT + threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.y * AP_NT;
    const float di = i < K ? H[i * K + i] : 0.0f;
    dt[threadIdx.x] = j0 + threadIdx.x < K ? H[(j0 + threadIdx.x) * K + j0 + threadIdx.x] : 0.0f;
    __syncthreads();
    const int n = (int)((K - j0) < AP_NT ? (K - j0) : AP_NT);
    int c = 0;
    for (int u = 0; u < n; ++u) c += act_before(dt[u], (int)(j0 + u), di, (int)i) ? 1 : 0;
    if (i < K && c) atomicAdd(&rank[i], c);
}

// perm[rank[i]] = i, gidx[rank[i]] = i / G (rank is the inverse permutation).
__global__ __launch_bounds__(AP_NT) void act_scatter_kernel(int *__restrict__ perm, int *__restrict__ gidx,
                                                            const int *__restrict__ rank, int64_t K, int64_t G)
{
    const int64_t i = (int64_t)blockIdx.x * AP_NT + threadIdx.x;
    if (i < K) {
        perm[rank[i]] = (int)i;
        gidx[rank[i]] = (int)(i / G);
    }
}

// Hp[a][b] = H[perm[a]][perm[b]] from H's lower triangle (both triangles of Hp).
__global__ __launch_bounds__(256) void perm_sym_kernel(float *__restrict__ Hp, const float *__restrict__ H,
                                                       const int *__restrict__ perm, int64_t K)
{
    for (int64_t a = blockIdx.y; a < K; a += gridDim.y) {
        const int64_t i = perm[a];
        for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < K; b += (int64_t)gridDim.x * 256) {
            const int64_t j = perm[b];
            Hp[a * K + b] = i >= j ? H[i * K + j] : H[j * K + i];
        }
    }
}

// Wk[n][a] = W[n][perm[a]], with the finite check of the plain copy.
__global__ __launch_bounds__(256) void gather_cols_kernel(float *__restrict__ Wk, const float *__restrict__ W,
                                                          const int *__restrict__ perm, int64_t N, int64_t K,
                                                          unsigned *status)
{
    bool bad = false;
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y)
        for (int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x; a < K; a += (int64_t)gridDim.x * 256) {
            const float v = W[n * K + perm[a]];
            bad = bad || !isfinite(v);
            Wk[n * K + a] = v;
        }
    if (bad) atomicOr(status, ST_NONFINITE);
}

// out[a][b] = in[rowperm[a]][perm[b]] (rowperm null: row a itself) for K-wide
// rows: each workgroup holds one source row in LDS (read once, coalesced) and
// writes the output row in order, so neither side is a scattered access.  With
// status set, non-finite values set ST_NONFINITE.  K <= kRowGatherMaxK.
constexpr int64_t kRowGatherMaxK = 32768;          // 128 KB of LDS
constexpr int RG_NT = 512;
__global__ __launch_bounds__(RG_NT) void row_gather_kernel(float *__restrict__ out, const float *__restrict__ in,
                                                           const int *__restrict__ rowperm,
                                                           const int *__restrict__ perm, int64_t rows, int64_t K,
                                                           unsigned *status)
{
    extern __shared__ float rowbuf[];
    bool bad = false;
    for (int64_t a = blockIdx.x; a < rows; a += gridDim.x) {
        const float *src = in + (rowperm ? (int64_t)rowperm[a] : a) * K;
        for (int64_t k = threadIdx.x; k < K; k += RG_NT) rowbuf[k] = src[k];
        __syncthreads();
        for (int64_t b = threadIdx.x; b < K; b += RG_NT) {
            const float v = rowbuf[perm[b]];
            bad = bad || !isfinite(v);
            out[a * K + b] = v;
        }
        __syncthreads();
    }
    if (status && bad) atomicOr(status, ST_NONFINITE);
}

// S = the full symmetric matrix whose lower triangle is H's (K x K, row stride
// K): each 64 x 64 tile on or below the diagonal is read once and written to
// its place and, transposed through LDS, to the mirrored place.
__global__ __launch_bounds__(256) void sym_full_kernel(float *__restrict__ S, const float *__restrict__ H, int64_t K)
{
    const int64_t bi = blockIdx.y, bj = blockIdx.x;
    if (bj > bi) return;
    __shared__ float t[64][65];
    const int64_t r0 = bi * 64, c0 = bj * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4)
        if (r0 + r < K && c0 + tx < K) t[r][tx] = H[(r0 + r) * K + c0 + tx];
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t gr = r0 + r, gc = c0 + tx;
        if (gr < K && gc < K) S[gr * K + gc] = (bi != bj || r >= tx) ? t[r][tx] : t[tx][r];
    }
    if (bi != bj)
        for (int c = ty; c < 64; c += 4)
            if (c0 + c < K && r0 + tx < K) S[(c0 + c) * K + r0 + tx] = t[tx][c];
}

// codes[n][k] = cperm[n][inv[k]] for packed nibbles (two columns per byte).
__global__ __launch_bounds__(256) void unpermute_codes_kernel(uint8_t *__restrict__ codes,
                                                              const uint8_t *__restrict__ cperm,
                                                              const int *__restrict__ inv, int64_t N, int64_t K)
{
    const int64_t half = K / 2;
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
        const uint8_t *src = cperm + n * half;
        for (int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x; m < half; m += (int64_t)gridDim.x * 256) {
            const int a0 = inv[2 * m], a1 = inv[2 * m + 1];
            const unsigned lo = (src[a0 >> 1] >> (4 * (a0 & 1))) & 0xFu;
            const unsigned hi = (src[a1 >> 1] >> (4 * (a1 & 1))) & 0xFu;
            codes[n * half + m] = (uint8_t)(lo | (hi << 4));
        }
    }
}

unsigned cols_grid(int64_t cols)
{
    int64_t g = (cols + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 64 ? 64 : g));
}

// rows of a row-strided launch: at most 65535 (the y limit), the kernels stride
unsigned rows_grid(int64_t rows) { return (unsigned)(rows < 1 ? 1 : (rows > 65535 ? 65535 : rows)); }
hipError_t launch_qerr(double *partials, const float *W, const uint8_t *codes, const float *scales,
                       const float *imp, int64_t N, int64_t K, int64_t G, int mode, hipStream_t s, int64_t *nparts)
{
    const bool wide = K % 8 == 0 && ((uintptr_t)W & 15) == 0 && ((uintptr_t)codes & 3) == 0 &&
                      ((uintptr_t)imp & 15) == 0;
    if (wide) {
        const int64_t need = (N * (K / 8) + QNT - 1) / QNT;
        const int64_t nwg = need < QPARTS ? (need < 1 ? 1 : need) : QPARTS;
        if (mode & MODE_NF4)
            hipLaunchKernelGGL(qerr8_kernel<true>, dim3((unsigned)nwg), dim3(QNT), 0, s, partials, W, codes, scales,
                               imp, N, K, G);
        else
            hipLaunchKernelGGL(qerr8_kernel<false>, dim3((unsigned)nwg), dim3(QNT), 0, s, partials, W, codes, scales,
                               imp, N, K, G);
        if (nparts) *nparts = nwg;
        return hipGetLastError();
    }
    if (nparts) *nparts = qerr_partials(N);
    const int64_t np = N < QPARTS ? N : QPARTS;
    const int64_t rows_per = (N + np - 1) / np;
    const int64_t nwg = qerr_partials(N);
    if (mode & MODE_NF4)
        hipLaunchKernelGGL(qerr_kernel<true>, dim3((unsigned)nwg), dim3(QNT), 0, s, partials, W, codes, scales, imp,
                           N, K, G, rows_per);
    else
        hipLaunchKernelGGL(qerr_kernel<false>, dim3((unsigned)nwg), dim3(QNT), 0, s, partials, W, codes, scales, imp,
                           N, K, G, rows_per);
    return hipGetLastError();
}

hipError_t launch_qerr_reduce(double *out2, const double *partials, int64_t nparts, hipStream_t s)
{
    hipLaunchKernelGGL(qerr_reduce_kernel, dim3(1), dim3(QNT), 0, s, out2, partials, nparts);
    return hipGetLastError();
}

int64_t rtn_workgroups(int64_t N, int64_t K)
{
    const int64_t need = (N * (K / 8) + RTN_NT - 1) / RTN_NT;
    return need < RTN_MAX_WG ? need : RTN_MAX_WG;
}

int64_t rtn_partials(int64_t N, int64_t K)
{
    const int64_t fused = rtn_workgroups(N, K), sep = qerr_partials(N);
    return fused > sep ? fused : sep;
}

hipError_t launch_rtn(const float *W, uint8_t *codes, float *scales, const float *imp, double *partials, int64_t N,
                      int64_t K, int64_t G, int mode, unsigned *status, hipStream_t s, int64_t *nparts)
{
    if (G < 1 || G > 128 || (G & (G - 1)) || K % G || K % 2) return hipErrorInvalidValue;
    const bool nf4 = (mode & MODE_NF4) != 0;
    const bool wide = K % 8 == 0 && ((uintptr_t)W & 15) == 0 && ((uintptr_t)codes & 3) == 0 &&
                      ((uintptr_t)imp & 15) == 0;
    if (wide) {
        const int64_t nwg = rtn_workgroups(N, K);
        if (nf4)
            hipLaunchKernelGGL(rtn8_kernel<true>, dim3((unsigned)nwg), dim3(RTN_NT), 0, s, W, codes, scales, N, K,
                               (int)G, status, imp, partials);
        else
            hipLaunchKernelGGL(rtn8_kernel<false>, dim3((unsigned)nwg), dim3(RTN_NT), 0, s, W, codes, scales, N, K,
                               (int)G, status, imp, partials);
        if (nparts) *nparts = nwg;
        return hipGetLastError();
    }
    const int64_t threads = N * (K / (G > 2 ? G : 2));
    const dim3 grid((unsigned)((threads + RTN_NT - 1) / RTN_NT));
    if (nf4)
        hipLaunchKernelGGL(rtn_any_kernel<true>, grid, dim3(RTN_NT), 0, s, W, codes, scales, N, K, (int)G, status);
    else
        hipLaunchKernelGGL(rtn_any_kernel<false>, grid, dim3(RTN_NT), 0, s, W, codes, scales, N, K, (int)G, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !partials) return e;
    return launch_qerr(partials, W, codes, scales, imp, N, K, G, mode, s, nparts);
}

hipError_t launch_act_perm(int *perm, int *inv, int *gidx, const float *H, int64_t K, int64_t G, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    const unsigned nb = (unsigned)((K + AP_NT - 1) / AP_NT);
    hipError_t e = launch_fill_u32((unsigned *)inv, K, 0u, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(act_rank_kernel, dim3(nb, nb), dim3(AP_NT), 0, s, inv, H, K);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(act_scatter_kernel, dim3(nb), dim3(AP_NT), 0, s, perm, gidx, inv, K, G);
    return hipGetLastError();
}

namespace {
bool row_gather_ready()
{
    static const bool ok = hipFuncSetAttribute((const void *)row_gather_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(kRowGatherMaxK * sizeof(float))) == hipSuccess;
    return ok;
}

hipError_t launch_row_gather(float *out, const float *in, const int *rowperm, const int *perm, int64_t rows,
                             int64_t K, unsigned *status, hipStream_t s)
{
    const int64_t g = rows < 4096 ? rows : 4096;
    hipLaunchKernelGGL(row_gather_kernel, dim3((unsigned)g), dim3(RG_NT), (size_t)K * sizeof(float), s, out, in,
                       rowperm, perm, rows, K, status);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_perm_sym(float *Hp, const float *H, const int *perm, float *tmp, int64_t K, hipStream_t s)
{
    if (K <= 0) return hipSuccess;
    if (tmp && K <= kRowGatherMaxK && row_gather_ready()) {
        const unsigned nt = (unsigned)((K + 63) / 64);
        hipLaunchKernelGGL(sym_full_kernel, dim3(nt, nt), dim3(256), 0, s, tmp, H, K);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_row_gather(Hp, tmp, perm, perm, K, K, nullptr, s);
    }
    hipLaunchKernelGGL(perm_sym_kernel, dim3(cols_grid(K), rows_grid(K)), dim3(256), 0, s, Hp, H, perm, K);
    return hipGetLastError();
}

hipError_t launch_gather_cols(float *Wk, const float *W, const int *perm, int64_t N, int64_t K, unsigned *status,
                              hipStream_t s)
{
    if (N <= 0 || K <= 0) return hipSuccess;
    if (K <= kRowGatherMaxK && row_gather_ready()) return launch_row_gather(Wk, W, nullptr, perm, N, K, status, s);
    hipLaunchKernelGGL(gather_cols_kernel, dim3(cols_grid(K), rows_grid(N)), dim3(256), 0, s, Wk, W, perm, N, K,
                       status);
    return hipGetLastError();
}

hipError_t launch_unpermute_codes(uint8_t *codes, const uint8_t *cperm, const int *inv, int64_t N, int64_t K,
                                  hipStream_t s)
{
    if (N <= 0 || K <= 0) return hipSuccess;
    hipLaunchKernelGGL(unpermute_codes_kernel, dim3(cols_grid(K / 2), rows_grid(N)), dim3(256), 0, s, codes, cperm,
                       inv, N, K);
    return hipGetLastError();
}

}  // namespace gq
