// ozaki.hip -- products of symmetric fp64 matrices on the int8 matrix cores, in
// exact integer arithmetic (the modular "Ozaki scheme II": Ozaki, Uchino and
// Imamura, emulation of floating-point matrix products with integer matrix
// units and the Chinese remainder theorem).
//
// The sign iteration of psd_project multiplies symmetric matrices whose entries
// are bounded by their spectral norm (<= 1 after scaling).  For such a product
// C = A B:
//   1. split: every row i of A is scaled by a power of two 2^(beta - e_i) (e_i
//      the binary exponent of the row's largest magnitude) and rounded to an
//      integer, |a_ik| <= 2^beta; likewise B by rows j.  Because both matrices
//      are symmetric, C_ij = 2^(e_i + e_j - 2 beta) sum_k a_ik b_jk: the integer
//      operands are read row by row, k contiguous, which is the layout the int8
//      matrix instruction wants for both of its operands.
//   2. each integer matrix is stored as its residues modulo oz_mods(K) pairwise
//      coprime moduli m_r <= 256, each residue centred to fit int8;
//   3. per modulus, one int8 GEMM with exact int32 accumulation gives
//      sum_k a_ik b_jk mod m_r (|sum| < K 128^2 < 2^31 for K < 2^17);
//   4. the Chinese remainder theorem recovers the integer sum exactly from its
//      residues, since |sum| <= K 2^(2 beta) < M / 2, M = prod m_r; it is then
//      scaled back and rounded to fp64 once.
// The only rounding is the truncation of step 1 (relative 2^-beta per entry of
// the row's scale) and the final conversion.  Up to K = 8192 a product uses 12
// moduli (M ~ 2^94.8, beta = 40 at K = 5120), above that 13 (M ~ 2^102.5, beta =
// 43 at K = 17408).  The int8 products, one per modulus, run at the int8
// matrix rate, 64 times the fp64 one.
#include "gq_internal.h"

namespace gq {

namespace {

// The moduli: the largest pairwise coprime values whose residues, centred,
// fit int8.  A product uses the first oz_mods(K) of them.
constexpr int kMods[kOzMaxMods] = {256, 255, 253, 251, 247, 241, 239, 233, 229, 227, 223, 217, 211};

typedef unsigned __int128 u128;
typedef __int128 i128;

// The reconstruction's constants for the first NM moduli, at compile time:
// M = prod m_r and the weights W_r = (M / m_r) ((M / m_r)^-1 mod m_r) (so that
// sum_r c_r W_r = x mod M for the residues c_r of x), each as limbs of 16 bits
// (6 for 12 moduli, M ~ 2^94.8; 7 for 13, M ~ 2^102.5), which keeps every limb
// product c_r w below 2^24 (a full-rate 24-bit multiply).
template <int NM> constexpr u128 oz_modulus()
{
    u128 M = 1;
    for (int r = 0; r < NM; ++r) M *= (u128)kMods[r];
    return M;
}
template <int NM> constexpr int oz_limb_count()
{
    int bits = 0;
    for (u128 m = oz_modulus<NM>(); m; m >>= 1) ++bits;
    return (bits + 16) / 16;                  // one spare bit: signed limbs of values up to M
}
template <int NM> struct OzLimbs {
    static constexpr int L = oz_limb_count<NM>();
    unsigned short w[NM][L];
    unsigned short M[L];
    double invM;
};
template <int NM> constexpr OzLimbs<NM> oz_limbs()
{
    OzLimbs<NM> L{};
    const u128 M = oz_modulus<NM>();
    for (int r = 0; r < NM; ++r) {
        const u128 Mr = M / (u128)kMods[r];
        const int t = (int)(Mr % (u128)kMods[r]);
        int y = 1;
        while ((t * y) % kMods[r] != 1) ++y;
        const u128 W = Mr * (u128)y;                    // y < m_r, so W < M
        for (int k = 0; k < OzLimbs<NM>::L; ++k) L.w[r][k] = (unsigned short)(W >> (16 * k));
    }
    for (int k = 0; k < OzLimbs<NM>::L; ++k) L.M[k] = (unsigned short)(M >> (16 * k));
    L.invM = 1.0 / ((double)(unsigned long long)(M >> 64) * 18446744073709551616.0 +
                    (double)(unsigned long long)M);
    return L;
}
template <int NM> constexpr OzLimbs<NM> kOzLimbs = oz_limbs<NM>();
struct OzInv { double v[kOzMaxMods]; };
constexpr OzInv oz_inverses()
{
    OzInv t{};
    for (int r = 0; r < kOzMaxMods; ++r) t.v[r] = 1.0 / (double)kMods[r];
    return t;
}
constexpr OzInv kOzInv = oz_inverses();
// 1/M scaled by the weight of limb L - 3 (a power of two: exact)
template <int NM>
constexpr double kOzInvMTop = kOzLimbs<NM>.invM * (double)((u128)1 << (16 * (OzLimbs<NM>::L - 3)));
// The weight limbs of moduli 2j and 2j+1 side by side (u16 pairs), for
// v_dot2_u32_u16: one instruction adds both moduli's products into a limb sum.
// With an odd number of moduli the last pair's second half is a residue of 0
// with a weight of 0.
template <int NM> struct OzPairs {
    static constexpr int N = (NM + 1) / 2;
    static constexpr int RES = 2 * N;               // residues per output, the pad included
    unsigned w[N][OzLimbs<NM>::L];
};
template <int NM> constexpr OzPairs<NM> oz_pairs()
{
    OzPairs<NM> P{};
    for (int j = 0; j < OzPairs<NM>::N; ++j)
        for (int k = 0; k < OzLimbs<NM>::L; ++k)
            P.w[j][k] = (unsigned)kOzLimbs<NM>.w[2 * j][k] |
                        (2 * j + 1 < NM ? ((unsigned)kOzLimbs<NM>.w[2 * j + 1][k] << 16) : 0u);
    return P;
}
template <int NM> constexpr OzPairs<NM> kOzPairs = oz_pairs<NM>();
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
static_assert(OzLimbs<12>::L >= 3 && OzLimbs<13>::L >= 3, "quotient estimate from the top three limbs");
static_assert((oz_modulus<12>() >> (16 * OzLimbs<12>::L - 1)) == 0, "M fits the limbs");
static_assert((oz_modulus<13>() >> (16 * OzLimbs<13>::L - 1)) == 0, "M fits the limbs");

// sum_k D[k] 2^(16 k) for signed limbs |D[k]| < 2^31
template <int L> __device__ inline i128 from_signed_limbs(const int (&D)[L])
{
    // two's complement sums in unsigned arithmetic (wrapping, shifts defined),
    // limbs paired into 64-bit words first
    u128 x = 0;
    static_for<(L + 1) / 2>([&](auto P) {
        constexpr int k = 2 * decltype(P)::value;
        unsigned long long pk = (unsigned long long)(long long)D[k];
        if constexpr (k + 1 < L) pk += (unsigned long long)(long long)D[k + 1] << 16;
        x += (u128)(i128)(long long)pk << (16 * k);
    });
    return (i128)x;
}

// Residues of the integers z[0..3] (|z| <= 2^48) modulo kMods[r], packed as the
// int8 bytes the products use (byte t from z[t]).  Odd m: z (1/m) + 1.5 2^52,
// rounded once by the fma, is 1.5 2^52 plus the integer q nearest z / m (z / m
// lies at least 1/(2m) > 2^-9 from a half-integer, and the fp64 1/m moves it by
// under 2^-12), so z - m q is the centred residue, exactly; plus 1.5 2^52 it
// sits, in two's complement, in the low 32 bits.  m = 256: the low byte of
// z + 1.5 2^52 is z mod 256.
constexpr double kOzMagic = 6755399441055744.0;   // 1.5 2^52
__device__ inline unsigned residue_word(const double (&z)[4], int r)
{
    unsigned b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        double v;
        if (r == 0) {
            v = z[t] + kOzMagic;
        } else {
            const double q = fma(z[t], kOzInv.v[r], kOzMagic) - kOzMagic;
            v = fma(-(double)kMods[r], q, z[t]) + kOzMagic;
        }
        b[t] = (unsigned)__builtin_bit_cast(unsigned long long, v);
    }
    const unsigned x01 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
    const unsigned x23 = __builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u);
    return __builtin_amdgcn_perm(x23, x01, 0x05040100u);
}

// ---------------------------------------------------------------- split
constexpr int SPL_NT = 256;

__device__ inline int64_t poff(int64_t row, int64_t k, int64_t Kp);

template <int NM>
__global__ __launch_bounds__(SPL_NT) void oz_split_kernel(const double *__restrict__ Z, int64_t K, int64_t Kp,
                                                          int beta, int8_t *__restrict__ planes,
                                                          int *__restrict__ rowexp,
                                                          const unsigned long long *__restrict__ rowmax)
{
    __shared__ double red[SPL_NT / 64];
    __shared__ int e_sh;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t plane = Kp * Kp;
    if (i >= K) {                       // padding rows: zero in every plane
        for (int64_t k = 8 * tid; k < Kp; k += 8 * SPL_NT)
#pragma unroll
            for (int r = 0; r < NM; ++r) *(uint2 *)(planes + r * plane + poff(i, k, Kp)) = make_uint2(0u, 0u);
        if (tid == 0) rowexp[i] = 0;
        return;
    }
    const double *zr = Z + i * K;
    if (!rowmax) {
        double mx = 0.0;
        for (int64_t k = tid; k < K; k += SPL_NT) mx = fmax(mx, fabs(zr[k]));
        for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
        if ((tid & 63) == 0) red[tid >> 6] = mx;
    }
    __syncthreads();
    if (tid == 0) {
        double m = rowmax ? __longlong_as_double((long long)rowmax[i]) : red[0];
        if (!rowmax)
            for (int w = 1; w < SPL_NT / 64; ++w) m = fmax(m, red[w]);
        int e = 0;
        if (m > 0.0) frexp(m, &e);      // m = f 2^e, f in [1/2, 1): |z| <= 2^e
        e_sh = e;
        rowexp[i] = e;
    }
    __syncthreads();
    const double sc = ldexp(1.0, beta - e_sh);
    for (int64_t k0 = 8 * tid; k0 < Kp; k0 += 8 * SPL_NT) {
        double z[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) z[t] = (k0 + t < K) ? rint(zr[k0 + t] * sc) : 0.0;   // exact integers
        const double z0[4] = {z[0], z[1], z[2], z[3]}, z1[4] = {z[4], z[5], z[6], z[7]};
#pragma unroll
        for (int r = 0; r < NM; ++r)
            *(uint2 *)(planes + r * plane + poff(i, k0, Kp)) = make_uint2(residue_word(z0, r), residue_word(z1, r));
    }
}

// ---------------------------------------------------------------- int8 GEMM
// P_r = RA_r RB_r^T mod m_r over the lower 256 x 256 tiles, all moduli in one
// launch (blockIdx.y = modulus).  4 waves of 128 x 128 (2 x 2), one per SIMD,
// each 4 x 4 blocks of v_mfma_i32_32x32x32_i8 per k32 half, the sums in AGPRs.
// The instruction computes X Y^T for 32-row panels X and Y of 32 k: lane l
// feeds k = 16 (l / 32) + 0..15 of row l % 32 of each, and result e of lane l
// is (X Y^T)[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].  The B panel goes first,
// so that e % 4 runs along a row of the output tile and each lane holds 4
// consecutive residues of a row, one dword.
//
// Each stage (64 k) of an operand is one contiguous 16 KiB block of the tiled
// plane layout, already in the order LDS wants.  It goes straight from memory
// to one of 4 LDS slots with 16-byte global_load_lds (no registers), three
// stages ahead; the 16-byte chunk c of block row rho sits at position
// c ^ swz(rho), so 16 consecutive rows read one chunk without bank conflicts.
// One barrier per stage, between its two k32 halves: the second half's
// instructions run while the next stage's first-half operands are read.  Every
// LDS read and every copy is issued right after one matrix instruction, so the
// wave never stalls on a full LDS or memory queue while its SIMD's matrix pipe
// runs dry (the compiler's order is pinned by scheduling barriers).
constexpr int OBM = 256, OBK = 64, ONT = 256, OSLOTS = 4;
constexpr int kOzBlock = OBM * OBK;             // bytes of one stage of one operand
constexpr int kOzSlot = 2 * kOzBlock;           // one stage of both operands
constexpr int kOzEpiRow = 272;                  // LDS row stride of the output tile
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ inline int swz(int r) { return (r >> 2) & 3; }

// Byte offset of element (row, k) in a plane of the tiled layout: blocks of
// 256 rows x 64 bytes, block (row / 256, k / 64) at index (row / 256) (Kp / 64)
// + k / 64, rows of 64 bytes inside, chunk c of row rho at position c ^ swz(rho).
__device__ inline int64_t poff(int64_t row, int64_t k, int64_t Kp)
{
    return ((((row >> 8) * (Kp >> 6)) + (k >> 6)) << 14) + ((row & 255) << 6) +
           ((((k >> 4) & 3) ^ ((row >> 2) & 3)) << 4) + (k & 15);
}

// Waits with an immediate: lgkmcnt(0) only (vmcnt and expcnt left at their
// maxima), so that copies in flight are not waited for.
constexpr int kWaitLgkm0 = 0xC07F;

// 64 lanes x 16 bytes from g (per lane) to LDS at l + 16 lane.  Written as
// inline asm so that the compiler, which would otherwise wait for every such
// copy before any LDS read, leaves the waits to wait_vm; the kernel issues no
// other vector-memory loads while copies are in flight.  M0 is set right
// before each copy and used by nothing else in the kernel.
__device__ inline void copy16_lds(const int8_t *g, unsigned l)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l) : "memory");
}
template <int N> __device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// SPLIT: the epilogue's quotient with 1/m in two fp32 parts (|P| up to 2^30,
// Kp > 32768); one part suffices for |P| <= 2^29.
template <bool SPLIT>
__global__ __launch_bounds__(ONT, 1) void oz_gemm_kernel(const int8_t *__restrict__ RA,
                                                        const int8_t *__restrict__ RB, int64_t Kp,
                                                        uint8_t *__restrict__ Cres, OzConst c)
{
    extern __shared__ __attribute__((aligned(1024))) int8_t oz_lds[];
    constexpr int S = OSLOTS;
    const int r = blockIdx.y;
    const int64_t nt = Kp / OBM;
    int64_t ti, tj;
    lower_tile_grouped(xcd_order(blockIdx.x, gridDim.x), nt, ti, tj);
    const int64_t i0 = ti * OBM, j0 = tj * OBM;
    const int64_t plane = Kp * Kp;
    const int nk = (int)(Kp / OBK);                  // >= 4 = S
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    // this wave copies chunks 4 wave + u / 2 (1 KiB each) of both operands' blocks
    const int8_t *ga = RA + r * plane + ((ti * (Kp / OBK)) << 14) + 4096 * wave + 16 * lane;
    const int8_t *gb = RB + r * plane + ((tj * (Kp / OBK)) << 14) + 4096 * wave + 16 * lane;
    const unsigned lbase = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void *)oz_lds + 4096u * wave;
    // copy u of stage kt (u even: A chunk u / 2, odd: B chunk u / 2) into a slot
    auto copy = [&](int kt, int slot, int u) {
        const int64_t kb = (int64_t)kt * kOzBlock + 1024 * (u >> 1);
        copy16_lds(((u & 1) ? gb : ga) + kb, lbase + slot * kOzSlot + 1024 * (u >> 1) + (u & 1) * kOzBlock);
    };

    v16i acc[4][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0;
    // LDS read offsets within a slot: row wr 128 + 32 bb + m of A (wc 128 + ... of
    // B), chunk 2h + lane / 32 at position chunk ^ swz(row) = chunk ^ swz(m).
    const int m = lane & 31;
    int oa[2], ob[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = (2 * h + (lane >> 5)) ^ swz(m);
        oa[h] = (wr * 128 + m) * OBK + 16 * ch;
        ob[h] = kOzBlock + (wc * 128 + m) * OBK + 16 * ch;
    }
    // operand read u of half h, in the order the instructions first use them:
    // a0, b0 .. b3, a1 .. a3
    auto read = [&](v4i (&a)[4], v4i (&b)[4], int slot, int h, int u) {
        const int8_t *q = oz_lds + slot * kOzSlot;
        if (u == 0) a[0] = *(const v4i *)(q + oa[h]);
        else if (u <= 4) b[u - 1] = *(const v4i *)(q + ob[h] + 2048 * (u - 1));
        else a[u - 4] = *(const v4i *)(q + oa[h] + 2048 * (u - 4));
    };
    // the 16 instructions of one k32 half, side(i) issued after instruction i
    auto mma = [&](const v4i (&a)[4], const v4i (&b)[4], auto &&side) {
        static_for<16>([&](auto I) {
            constexpr int i = decltype(I)::value;
            acc[i / 4][i % 4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[i % 4], a[i / 4], acc[i / 4][i % 4], 0, 0, 0);
            side(I);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    v4i a0[4], b0[4], a1[4], b1[4];
    // Stage kt, entered with stage kt published and its first-half operands in
    // a0/b0 (or on their way): first half, reading the second half's operands;
    // wait for this wave's copies of stage kt + 1 and barrier (stage kt + 1
    // published, every wave past its reads of stage kt - 1); second half,
    // reading stage kt + 1's first-half operands.  Stage j's A chunks are copied
    // in the second half of stage j - S + 1 (after the barrier that frees slot
    // j % S), its B chunks in the first half of stage j - S + 2 (nothing reads
    // the slot before stage j - 1's barrier).  WN: copies that may stay in
    // flight at the barrier; CA / CB: copy A / B chunks; NEXT: not the last stage.
    auto step = [&](auto WN, auto CA, auto CB, auto NEXT, int kt, int slot) {
        const int nslot = slot == S - 1 ? 0 : slot + 1;
        const int fslot = slot == 0 ? S - 1 : slot - 1;    // slot of stages kt - 1 and kt + S - 1
        const int bslot = fslot == 0 ? S - 1 : fslot - 1;  // slot of stage kt + S - 2
        mma(a0, b0, [&](auto I) {
            constexpr int i = decltype(I)::value;
            if constexpr (i % 2 == 0) read(a1, b1, slot, 1, i / 2);
            else if constexpr (decltype(CB)::value && i % 4 == 1) copy(kt + S - 2, bslot, 2 * (i / 4) + 1);
        });
        if constexpr (decltype(NEXT)::value) {
            wait_vm<decltype(WN)::value>();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        __builtin_amdgcn_sched_barrier(0);
        mma(a1, b1, [&](auto I) {
            constexpr int i = decltype(I)::value;
            if constexpr (decltype(NEXT)::value) {
                if constexpr (i % 2 == 0) read(a0, b0, nslot, 0, i / 2);
                else if constexpr (decltype(CA)::value && i % 4 == 1) copy(kt + S - 1, fslot, 2 * (i / 4));
            }
        });
    };
    using T = std::true_type;
    using F = std::false_type;
    // prologue: stages 0 .. S - 3 whole, stage S - 2's A chunks
#pragma unroll
    for (int st = 0; st < S - 2; ++st)
#pragma unroll
        for (int u = 0; u < 8; ++u) copy(st, st, u);
#pragma unroll
    for (int u = 0; u < 8; u += 2) copy(S - 2, S - 2, u);
    wait_vm<8 * (S - 3) + 4>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) read(a0, b0, 0, 0, u);
    int slot = 0, kt = 0;
    for (; kt <= nk - S; ++kt) {
        step(std::integral_constant<int, 8 * (S - 3)>{}, T{}, T{}, T{}, kt, slot);
        slot = slot == S - 1 ? 0 : slot + 1;
    }
    static_for<S - 2>([&](auto J) {
        constexpr int j = decltype(J)::value;
        step(std::integral_constant<int, 8 * (S - 3 - j)>{}, F{}, std::integral_constant<bool, j == 0>{}, T{}, kt,
             slot);
        ++kt;
        slot = slot == S - 1 ? 0 : slot + 1;
    });
    step(std::integral_constant<int, 0>{}, F{}, F{}, F{}, kt, slot);

    // Residues mod m in [0, m), 4 columns to a dword, through LDS to 16-byte
    // row stores.  With |P| <= Kp 2^14, the fp32 value P / m - 1/2 (one fma) is
    // within 1/2 of the exact one (checked on the CPU at and near the bounds),
    // so q = floor of it is floor(P / m) or one below, P - q m lies in [0, 2m),
    // and min(r, r - m) over unsigned ints lands in [0, m).  Diagonal tiles are
    // written whole: entries above the diagonal are residues of the symmetric
    // product too.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int mi = c.m[r];
    const float inv_hi = (float)c.inv_m[r];
    const float inv_lo = (float)(c.inv_m[r] - (double)inv_hi);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned w = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int pv = acc[bi][bj][4 * q + t];
                    const float pf = (float)pv;
                    const float y = SPLIT ? fmaf(pf, inv_hi, fmaf(pf, inv_lo, -0.5f)) : fmaf(pf, inv_hi, -0.5f);
                    int qq;
                    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(qq) : "v"(y));
                    const unsigned rr = (unsigned)(__mul24(qq, -mi) + pv);
                    w |= min(rr, rr - (unsigned)mi) << (8 * t);
                }
                const int li = wr * 128 + bi * 32 + m;
                const int lj = wc * 128 + bj * 32 + 8 * q + 4 * (lane >> 5);
                *(unsigned *)(oz_lds + li * kOzEpiRow + lj) = w;
            }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    uint8_t *out = Cres + r * plane + i0 * Kp + j0;
#pragma unroll
    for (int u = 0; u < OBM * OBM / 16 / ONT; ++u) {
        const int cidx = tid + ONT * u;
        const int row = cidx >> 4, col = 16 * (cidx & 15);
        *(v4i *)(out + row * Kp + col) = *(const v4i *)(oz_lds + row * kOzEpiRow + col);
    }
}

// dynamic LDS: the 4-slot ring (128 KiB); the output tile (68 KiB) reuses it
constexpr size_t kOzGemmLds = (size_t)OSLOTS * kOzSlot;
static_assert(kOzGemmLds >= (size_t)OBM * kOzEpiRow, "output tile");

// ---------------------------------------------------------------- CRT
// One 64 x 64 lower tile per workgroup: reconstruct sum_k a_ik b_jk from its
// residues (128-bit integers), scale to fp64, apply alpha / beta / cin, and
// write the tile and, through LDS, its mirror.  An operand without a row
// exponent array has the same exponent on every row (entries below 2^exp in
// magnitude).  With o.planes set the kernel also writes the split form of its
// own (symmetric) output, plus o.diag_shift on the diagonal, for the next
// product at the exponent o.exp: an entry of 2^o.exp or more in magnitude
// would break the bound the reconstruction relies on and sets ST_RANGE.
constexpr int CT = 64, CNT = 256;


template <int NM, typename OutT>
__global__ __launch_bounds__(CNT) void oz_crt_kernel(GemmDesc d, const uint8_t *__restrict__ Cres, int64_t Kp,
                                                    OzOperand A, OzOperand B, int twobeta, OzOut o,
                                                    int beta, unsigned *status)
{
    const int *__restrict__ ea = A.rowexp;
    const int *__restrict__ eb = B.rowexp;
    int8_t *__restrict__ planes = o.planes;
    const double bound = ldexp(1.0, o.exp);
    __shared__ double tile[CT][CT + 1];
    const int64_t K = d.M;
    int64_t ti = 0, tj = 0;
    {
        // tile index -> (ti >= tj) in row order.  A tile row of one residue plane
        // is 64 bytes, half a cache line: the tile beside it reads the other
        // half.  Workgroups are dealt to the XCDs in turn, so the index is taken
        // through xcd_order, which gives each XCD a contiguous run of tiles: the
        // two tiles of a line then run together on one XCD and share its L2.
        const int64_t id = xcd_order(blockIdx.x, gridDim.x);
        int64_t t = (int64_t)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
        while (t * (t + 1) / 2 > id) --t;
        while ((t + 1) * (t + 2) / 2 <= id) ++t;
        ti = t;
        tj = id - t * (t + 1) / 2;
    }
    const bool diag = (ti == tj);
    const int64_t i0 = ti * CT, j0 = tj * CT;
    double alpha = d.alpha, beta_c = d.beta;
    if (d.alpha_dev) { for (int p = 0; p < d.alpha_pow; ++p) alpha *= *d.alpha_dev; }
    if (d.beta_dev) { for (int p = 0; p < d.beta_pow; ++p) beta_c *= *d.beta_dev; }
    const double *cin = (const double *)d.cin;
    const int64_t plane = Kp * Kp;
    const int tid = threadIdx.x;
    // thread -> 4 consecutive columns c4 .. c4+3 of rows lr, lr+16, lr+32, lr+48
    const int lr = tid >> 4, c4 = 4 * (tid & 15);
    bool range_bad = false;
    // residues of 4 consecutive outputs of row li = 16 rr + lr: one dword per
    // plane (Kp is a multiple of 256, j0 + c4 of 4: aligned)
    constexpr int kLimbs = OzLimbs<NM>::L, kOzPairN = OzPairs<NM>::N, kOzRes = OzPairs<NM>::RES;
    auto load_row = [&](unsigned (&rs)[kOzRes], int rr) {
        const int64_t gi = i0 + rr * 16 + lr;
        const uint8_t *p = Cres + (gi < K ? gi : 0) * Kp + j0 + c4;
#pragma unroll
        for (int r = 0; r < NM; ++r) rs[r] = *(const unsigned *)(p + r * plane);
#pragma unroll
        for (int r = NM; r < kOzRes; ++r) rs[r] = 0u;
    };
    auto do_row = [&](const unsigned (&rs)[kOzRes], int rr) {
        const int li = rr * 16 + lr;
        const int64_t gi = i0 + li;
        const bool row_in = gi < K;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t gj = j0 + c4 + t;
            double v = 0.0;
            if (row_in && gj < K && gi >= gj) {
                // S = sum_r c_r W_r by 16-bit limbs of W_r: each limb sum is below
                // NM * 255 * 2^16 < 2^28.  The residues of moduli 2j, 2j+1 (byte
                // t of rs[2j], rs[2j+1]) are put side by side as u16s by one byte
                // permute, and each limb takes one dot2 per pair.
                u16x2 cp[kOzPairN];
#pragma unroll
                for (int j = 0; j < kOzPairN; ++j)
                    cp[j] = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(rs[2 * j + 1], rs[2 * j],
                                                                            0x0C000C00u | ((4u + t) << 16) | (unsigned)t));
                unsigned L[kLimbs] = {};
#pragma unroll
                for (int k = 0; k < kLimbs; ++k)
#pragma unroll
                    for (int j = 0; j < kOzPairN; ++j)
                        L[k] = __builtin_amdgcn_udot2(cp[j], __builtin_bit_cast(u16x2, kOzPairs<NM>.w[j][k]), L[k], false);
                // The centred value is x = S - q M with q the integer nearest S / M:
                // |x| <= K 2^(2 beta) < 0.497 M (the choice of beta).  S / M < 2^12 is
                // estimated from the top three limbs (the rest adds below 2^-19 to
                // it) within 2^-19 + 2^-38, far inside the 0.003 margin.  x by signed
                // limbs L[k] - q M[k] (q M[k] < 2^28), one carry pass in 128 bits.
                const double St = fma(fma((double)L[kLimbs - 1], 65536.0, (double)L[kLimbs - 2]), 65536.0,
                                      (double)L[kLimbs - 3]);
                const int nq = -(int)rint(St * kOzInvMTop<NM>);
                int D[kLimbs];
#pragma unroll
                for (int k = 0; k < kLimbs; ++k) D[k] = __mul24(nq, (int)kOzLimbs<NM>.M[k]) + (int)L[k];
                const i128 x = from_signed_limbs(D);
                const double xd = ldexp((double)(long long)(x >> 64), 64) + (double)(unsigned long long)x;
                const int e = (ea ? ea[gi] : A.exp) + (eb ? eb[gj] : B.exp);
                v = alpha * ldexp(xd, e - twobeta);
                if (beta_c != 0.0) v += beta_c * cin[gi * d.ldc + gj];
                if (gi == gj) v += o.diag_shift;
                range_bad = range_bad || !(fabs(v) < bound);
            }
            tile[li][c4 + t] = v;
        }
    };
    // two rows in flight: each row's residues are loaded while the one before is
    // reconstructed (the last load repeats row 3, in bounds and unused)
    unsigned ra[kOzRes], rb[kOzRes];
    load_row(ra, 0);
#pragma unroll 1
    for (int rr = 0; rr < CT / 16; rr += 2) {
        load_row(rb, rr + 1);
        do_row(ra, rr);
        load_row(ra, rr + 2 < CT / 16 ? rr + 2 : rr + 1);
        do_row(rb, rr + 1);
    }
    __syncthreads();
    OutT *out = (OutT *)d.out;
    OutT *out_t = (OutT *)d.out_t;
    if (out) {
        const int cj = tid & (CT - 1), rg = tid >> 6;
        const int64_t gj = j0 + cj;
        for (int rr = 0; rr < CT / 4; ++rr) {
            const int li = rg * (CT / 4) + rr;
            const int64_t gi = i0 + li;
            if (gi < K && gj < K && gi >= gj) out[gi * d.ldo + gj] = (OutT)tile[li][cj];
            // mirror: element (j0 + li, i0 + cj) of the transposed block
            const int64_t mi = i0 + cj, mj = j0 + li;        // source (mi, mj) with mi >= mj
            if (out_t && mi < K && mj < K && mi >= mj) out_t[mj * d.ldo + mi] = (OutT)tile[cj][li];
        }
    }
    if (!planes) return;
    if (range_bad) atomicOr(status, ST_RANGE);
    // Split form of the symmetric output at exponent o.exp: each element's
    // residues are computed once, written to rows i0.. (this block) and, off the
    // diagonal, staged in LDS (7 moduli at a time, in the space of the fp64
    // tile) and written transposed to rows j0.. (the mirror).  On the diagonal
    // tile, entries above its diagonal come from their mirror.  Entries past K
    // are 0 and keep the padding zero.
    const double sc = ldexp(1.0, beta - o.exp);
    double z[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int li = rr * 16 + lr, cc = c4 + t;
            const double v = (diag && cc > li) ? tile[cc][li] : tile[li][cc];
            z[rr][t] = rint(v * sc);
        }
    constexpr int kBatch = 7;
    static_assert(sizeof(unsigned) * kBatch * CT * (CT / 4 + 1) <= sizeof(double) * CT * (CT + 1), "LDS reuse");
    unsigned (*rt)[CT][CT / 4 + 1] = reinterpret_cast<unsigned (*)[CT][CT / 4 + 1]>(&tile[0][0]);
    __syncthreads();                    // the fp64 tile is no longer read
#pragma unroll 1
    for (int batch = 0; batch < (NM + kBatch - 1) / kBatch; ++batch) {
        const int nq = NM - kBatch * batch < kBatch ? NM - kBatch * batch : kBatch;
#pragma unroll 1
        for (int q = 0; q < nq; ++q) {
            const int r = kBatch * batch + q;
            int8_t *pl = planes + r * plane;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const unsigned w = residue_word(z[rr], r);
                const int li = rr * 16 + lr;
                rt[q][li][c4 >> 2] = w;
                if (i0 + li < K) *(unsigned *)(pl + poff(i0 + li, j0 + c4, Kp)) = w;
            }
        }
        if (diag) continue;
        __syncthreads();
        // mirror rows j0 + li: bytes (i0 + c4 + t) come from rt[q][c4 + t][li]
#pragma unroll 1
        for (int q = 0; q < nq; ++q) {
            int8_t *pl = planes + (kBatch * batch + q) * plane;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int li = rr * 16 + lr;
                unsigned w = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) w |= ((rt[q][c4 + t][li >> 2] >> (8 * (li & 3))) & 0xFFu) << (8 * t);
                if (j0 + li < K) *(unsigned *)(pl + poff(j0 + li, i0 + c4, Kp)) = w;
            }
        }
        __syncthreads();
    }
}

// The bytes of a split form that oz_crt_kernel never writes: rows K .. Kp - 1,
// and in rows below K the 64-byte row segments from column ceil(K / 64) 64 on
// (the CRT's tiles end there).  One 16-byte chunk per thread and step.
__global__ void oz_pad_kernel(int8_t *__restrict__ planes, int64_t K, int64_t Kp, int64_t per_plane, int nm)
{
    const int64_t kseg = Kp >> 6, c0 = (K + 63) >> 6;
    const int64_t low = K * (kseg - c0);                // padding segments in rows below K
    const int64_t total = per_plane * nm * 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t sg = e >> 2, r = sg / per_plane;
        int64_t rem = sg - r * per_plane, row, seg;
        if (rem < low) {
            row = rem / (kseg - c0);
            seg = c0 + (rem - row * (kseg - c0));
        } else {
            rem -= low;
            row = K + rem / kseg;
            seg = rem - (row - K) * kseg;
        }
        *(uint4 *)(planes + r * Kp * Kp + poff(row, 64 * seg + 16 * (e & 3), Kp)) = make_uint4(0u, 0u, 0u, 0u);
    }
}

}  // namespace

int oz_mods(int64_t K) { return K <= kOzFewModsMaxK ? 12 : 13; }

const OzConst &oz_const(int nm)
{
    auto make = [](int n) {
        OzConst k{};
        k.nm = n;
        for (int r = 0; r < n; ++r) {
            k.m[r] = kMods[r];
            k.inv_m[r] = 1.0 / (double)kMods[r];
        }
        const u128 M = n == 12 ? oz_modulus<12>() : oz_modulus<13>();
        k.M_lo = (unsigned long long)M;
        k.M_hi = (unsigned long long)(M >> 64);
        return k;
    };
    static const OzConst c12 = make(12), c13 = make(13);
    return nm == 12 ? c12 : c13;
}

int oz_beta(int64_t K)
{
    // largest beta with K 2^(2 beta) <= 0.497 M, i.e. 2 beta <= log2 M - 1.01 - log2 K
    // (the reconstruction rounds S / M to the nearest integer and needs the
    // centred sum to stay clear of M / 2), and at most 48, where residue_word's
    // quotient is exact (40 at K = 5120 with 12 moduli, 43 at K = 17408 with 13)
    const OzConst &c = oz_const(oz_mods(K));
    const double log2M = std::log2(ldexp((double)c.M_hi, 64) + (double)c.M_lo);
    const double room = log2M - 1.01 - std::log2((double)(K > 1 ? K : 1));
    const int b = (int)std::floor(room / 2.0);
    return b < 48 ? b : 48;
}

int64_t oz_padded(int64_t K) { return (K + OBM - 1) / OBM * OBM; }

size_t oz_planes_bytes(int64_t K)
{
    const int64_t Kp = oz_padded(K);
    return (size_t)oz_mods(K) * (size_t)Kp * (size_t)Kp;
}

hipError_t oz_split(const double *Z, int64_t K, int beta, int8_t *planes, int *rowexp, hipStream_t s,
                    const unsigned long long *rowmax)
{
    const int64_t Kp = oz_padded(K);
    if (oz_mods(K) == 12)
        hipLaunchKernelGGL(oz_split_kernel<12>, dim3((unsigned)Kp), dim3(SPL_NT), 0, s, Z, K, Kp, beta, planes, rowexp,
                           rowmax);
    else
        hipLaunchKernelGGL(oz_split_kernel<13>, dim3((unsigned)Kp), dim3(SPL_NT), 0, s, Z, K, Kp, beta, planes, rowexp,
                           rowmax);
    return hipGetLastError();
}

hipError_t oz_product(const GemmDesc &d, const OzOperand &A, const OzOperand &B, int beta, uint8_t *Cres,
                      bool out_f32, const OzOut &o, unsigned *status, hipStream_t s, hipEvent_t after_gemm)
{
    const int64_t K = d.M;
    if (K <= 0) return hipSuccess;
    if (d.N != K || d.Kd != K) return hipErrorInvalidValue;
    const int64_t Kp = oz_padded(K);
    const int64_t nt = Kp / OBM;
    static bool lds_ok = hipFuncSetAttribute((const void *)oz_gemm_kernel<false>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kOzGemmLds) == hipSuccess &&
                         hipFuncSetAttribute((const void *)oz_gemm_kernel<true>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kOzGemmLds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int nm = oz_mods(K);
    // residues centred in [-128, 128): |P| <= Kp 2^14, within 2^29 up to Kp = 32768
    if (Kp <= 32768)
        hipLaunchKernelGGL(oz_gemm_kernel<false>, dim3((unsigned)(nt * (nt + 1) / 2), (unsigned)nm), dim3(ONT),
                           kOzGemmLds, s, A.planes, B.planes, Kp, Cres, oz_const(nm));
    else
        hipLaunchKernelGGL(oz_gemm_kernel<true>, dim3((unsigned)(nt * (nt + 1) / 2), (unsigned)nm), dim3(ONT),
                           kOzGemmLds, s, A.planes, B.planes, Kp, Cres, oz_const(nm));
    if (after_gemm) {
        const hipError_t e = hipEventRecord(after_gemm, s);
        if (e != hipSuccess) return e;
    }
    const dim3 cg((unsigned)(((K + CT - 1) / CT) * ((K + CT - 1) / CT + 1) / 2));
    if (nm == 12) {
        if (out_f32)
            hipLaunchKernelGGL((oz_crt_kernel<12, float>), cg, dim3(CNT), 0, s, d, Cres, Kp, A, B, 2 * beta, o, beta,
                               status);
        else
            hipLaunchKernelGGL((oz_crt_kernel<12, double>), cg, dim3(CNT), 0, s, d, Cres, Kp, A, B, 2 * beta, o, beta,
                               status);
    } else {
        if (out_f32)
            hipLaunchKernelGGL((oz_crt_kernel<13, float>), cg, dim3(CNT), 0, s, d, Cres, Kp, A, B, 2 * beta, o, beta,
                               status);
        else
            hipLaunchKernelGGL((oz_crt_kernel<13, double>), cg, dim3(CNT), 0, s, d, Cres, Kp, A, B, 2 * beta, o, beta,
                               status);
    }
    return hipGetLastError();
}

hipError_t oz_clear_padding(int8_t *planes, int64_t K, hipStream_t s)
{
    const int64_t Kp = oz_padded(K), kseg = Kp / 64, c0 = (K + 63) / 64;
    const int64_t per_plane = K * (kseg - c0) + (Kp - K) * kseg;
    if (per_plane == 0) return hipSuccess;
    const int nm = oz_mods(K);
    const int64_t n = per_plane * nm * 4;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(oz_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, planes, K, Kp, per_plane, nm);
    return hipGetLastError();
}

}  // namespace gq
